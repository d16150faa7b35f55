// Log-sum-exp merge of one output row from its partial attentions (LongSpec
// summary pages, "Fast Tree Attention": the cached and speculative parts are
// aggregated with the log-sum-exp trick, which keeps the result exact).
//
// For one output row with partials (o_k normalised, lse_k) over disjoint key
// sets: lse = log2(sum_k 2^lse_k) and out = sum_k 2^(lse_k - lse) o_k. Parts
// with lse_k = -inf contribute nothing; a row with no part at all gets
// out = 0, lse = -inf. Internally every LSE is base 2; the stored lse is
// natural log.
//
// One wave per output row. Its 64 lanes are PG part groups x (D/8) lanes of
// 8 dims: part group p takes parts p, p+PG, p+2PG, ... and keeps its own
// running max and weighted sum, so each lane has up to 8 independent loads in
// flight; the groups are then combined with cross-lane exchanges. Used by the
// merge kernel and by the split-KV kernel's fused merge.
#pragma once

#include "common.h"

namespace hta {

constexpr int kMergeUnroll = 9;  // parts per part group per pass (36 parts at D = 128)

// 8 consecutive elements of a partial row as floats.
__device__ __forceinline__ void merge_load8(const float* p, float* o) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
  o[0] = a[0]; o[1] = a[1]; o[2] = a[2]; o[3] = a[3];
  o[4] = b[0]; o[5] = b[1]; o[6] = b[2]; o[7] = b[3];
}
__device__ __forceinline__ void merge_load8(const unsigned short* p, float* o) {
  const u32x4 a = *(const u32x4*)p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(a[i] << 16);
    o[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
  }
}

// Merges output row `row` (of D values at out + row * D, its lse at lse[row])
// from p_count parts: load_o(k, v) reads this lane's 8 dims of part k's row
// into v (floats), load_l(k) part k's base-2 LSE. dead(k) tells, before any
// load, that part k holds nothing. bad poisons the row (NaN out and lse).
template <int D, bool OUT_BF16, typename LoadO, typename LoadL, typename DeadFn>
__device__ __forceinline__ void merge_row(int lane, int p_count, LoadO load_o, LoadL load_l, DeadFn dead, bool bad,
                                          void* out, float* lse, int64_t row) {
  constexpr int LPR = D / 8;    // lanes per part group (8 dims each)
  constexpr int PG = 64 / LPR;  // part groups per row
  const int pg = lane / LPR;
  const int dl = lane % LPR;
  // This lane's part group: running max m, weighted sum s and accumulator acc.
  float m = -__builtin_inff(), s = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int k0 = pg; k0 < p_count; k0 += PG * kMergeUnroll) {
    float lk[kMergeUnroll], ov[kMergeUnroll][8];
    // Which of this step's parts hold nothing is known before any load, so
    // every load of the step is issued before the first wait.
    bool dead_u[kMergeUnroll];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u)
      dead_u[u] = k0 + u * PG >= p_count || dead(min(k0 + u * PG, p_count - 1));
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int k = min(k0 + u * PG, p_count - 1);  // in-bounds; ignored past the end
      lk[u] = load_l(k);
      load_o(k, ov[u]);
    }
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) lk[u] = dead_u[u] ? -__builtin_inff() : lk[u];
    // No branch on the loaded values: while every part so far is empty, m and
    // mc are -inf, alpha is 0 and every weight is 0, so s and acc stay 0.
    float mc = m;
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) mc = fmaxf(mc, lk[u]);
    const float alpha = m == -__builtin_inff() ? 0.f : fast_exp2(m - mc);
    s *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const bool live = lk[u] != -__builtin_inff();  // an empty part's o is never used
      const float wk = live ? fast_exp2(lk[u] - mc) : 0.f;
      s += wk;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += live ? wk * ov[u][e] : 0.f;
    }
    m = mc;
  }
  // Combine the part groups (lanes dl, dl + LPR, ... hold the same dims).
  float mt = m;
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) mt = fmaxf(mt, __shfl_xor(mt, off));
  const float sc = (m == -__builtin_inff()) ? 0.f : fast_exp2(m - mt);
  s *= sc;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] *= sc;
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
    s += __shfl_xor(s, off);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off);
  }
  float lse_out;
  if (mt == -__builtin_inff()) {
    lse_out = -__builtin_inff();
  } else {
    const float inv = 1.0f / s;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    lse_out = (mt + fast_log2(s)) * kLn2;
  }
  if (bad) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = __builtin_nanf("");
    lse_out = __builtin_nanf("");
  }
  if (pg != 0) return;
  if (OUT_BF16) {
    u32x4 pk;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pk[i] = (unsigned)float_to_bf16_bits(acc[2 * i]) | ((unsigned)float_to_bf16_bits(acc[2 * i + 1]) << 16);
    *(u32x4*)(static_cast<unsigned short*>(out) + (size_t)row * D + dl * 8) = pk;
  } else {
    float* op = static_cast<float*>(out) + (size_t)row * D + dl * 8;
    f32x4 v0 = {acc[0], acc[1], acc[2], acc[3]}, v1 = {acc[4], acc[5], acc[6], acc[7]};
    *(f32x4*)op = v0;
    *(f32x4*)(op + 4) = v1;
  }
  if (dl == 0) lse[row] = lse_out;
}

// The same for RB rows at once (row[rb], or none where row[rb] < 0) of bf16
// partials, with UNR parts per part group per pass: every load of a pass (RB x
// UNR parts per lane, kept as raw bf16 words until all are issued) goes out
// before the first wait, so a wave with a few rows and up to UNR * PG parts
// pays one memory round trip. load_o(rb, k) returns this lane's 8 bf16 of row
// rb's part k, load_l(rb, k) its base-2 LSE.
template <int D, int RB, int UNR, bool OUT_BF16, typename LoadO, typename LoadL, typename DeadFn>
__device__ __forceinline__ void merge_rows(int lane, int p_count, LoadO load_o, LoadL load_l, DeadFn dead, bool bad,
                                           void* out, float* lse, const int64_t (&row)[RB]) {
  constexpr int LPR = D / 8;
  constexpr int PG = 64 / LPR;
  const int pg = lane / LPR;
  const int dl = lane % LPR;
  float m[RB], s[RB], acc[RB][8];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = -__builtin_inff();
    s[rb] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[rb][e] = 0.f;
  }
  for (int k0 = pg; k0 < p_count; k0 += PG * UNR) {
    float lk[RB][UNR];
    u32x4 raw[RB][UNR];
    bool dead_u[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) dead_u[u] = k0 + u * PG >= p_count || dead(min(k0 + u * PG, p_count - 1));
#pragma unroll
    for (int u = 0; u < UNR; ++u)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int k = min(k0 + u * PG, p_count - 1);
        lk[rb][u] = load_l(rb, k);
        raw[rb][u] = load_o(rb, k);
      }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mc = m[rb];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        lk[rb][u] = dead_u[u] ? -__builtin_inff() : lk[rb][u];
        mc = fmaxf(mc, lk[rb][u]);
      }
      const float alpha = m[rb] == -__builtin_inff() ? 0.f : fast_exp2(m[rb] - mc);
      s[rb] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[rb][e] *= alpha;
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const bool live = lk[rb][u] != -__builtin_inff();
        const float wk = live ? fast_exp2(lk[rb][u] - mc) : 0.f;
        s[rb] += wk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[rb][2 * i] += live ? wk * __uint_as_float(raw[rb][u][i] << 16) : 0.f;
          acc[rb][2 * i + 1] += live ? wk * __uint_as_float(raw[rb][u][i] & 0xffff0000u) : 0.f;
        }
      }
      m[rb] = mc;
    }
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float mt = m[rb];
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) mt = fmaxf(mt, __shfl_xor(mt, off));
    const float sc = (m[rb] == -__builtin_inff()) ? 0.f : fast_exp2(m[rb] - mt);
    float sr = s[rb] * sc, a8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a8[e] = acc[rb][e] * sc;
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
      sr += __shfl_xor(sr, off);
#pragma unroll
      for (int e = 0; e < 8; ++e) a8[e] += __shfl_xor(a8[e], off);
    }
    float lse_out;
    if (mt == -__builtin_inff()) {
      lse_out = -__builtin_inff();
    } else {
      const float inv = 1.0f / sr;
#pragma unroll
      for (int e = 0; e < 8; ++e) a8[e] *= inv;
      lse_out = (mt + fast_log2(sr)) * kLn2;
    }
    if (bad) {
#pragma unroll
      for (int e = 0; e < 8; ++e) a8[e] = __builtin_nanf("");
      lse_out = __builtin_nanf("");
    }
    if (pg != 0 || row[rb] < 0) continue;
    if (OUT_BF16) {
      u32x4 pk;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pk[i] = (unsigned)float_to_bf16_bits(a8[2 * i]) | ((unsigned)float_to_bf16_bits(a8[2 * i + 1]) << 16);
      *(u32x4*)(static_cast<unsigned short*>(out) + (size_t)row[rb] * D + dl * 8) = pk;
    } else {
      float* op = static_cast<float*>(out) + (size_t)row[rb] * D + dl * 8;
      f32x4 v0 = {a8[0], a8[1], a8[2], a8[3]}, v1 = {a8[4], a8[5], a8[6], a8[7]};
      *(f32x4*)op = v0;
      *(f32x4*)(op + 4) = v1;
    }
    if (dl == 0) lse[row[rb]] = lse_out;
  }
}

}  // namespace hta
