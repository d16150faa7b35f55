// Log-sum-exp merge of partial attentions (LongSpec summary pages, "Fast
// Tree Attention": the cached and speculative parts are aggregated with the
// log-sum-exp trick, which keeps the result exact).
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
// flight; the groups are then combined with cross-lane exchanges.
#include "common.h"
#include "hta_internal.h"

namespace hta {
namespace {

constexpr int UNROLL = 8;

struct MergeArgs {
  // slot mode: partials of one split-KV launch
  const int* prefix_len;
  const void* slot_o;
  const float* slot_lse2;
  const int* err_b;
  int* status;
  int nk, nwg, tree_tiles;
  // parts mode: n_parts caller arrays, natural-log lse
  const float* o_parts;
  const float* lse_parts;
  int n_parts;
  // common
  void* out;
  float* lse;
  int B, Hq, Hkv, G, T, Lcap, M;
};

// 8 consecutive elements of a partial row as floats.
__device__ __forceinline__ void load8(const float* p, float* o) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
  o[0] = a[0]; o[1] = a[1]; o[2] = a[2]; o[3] = a[3];
  o[4] = b[0]; o[5] = b[1]; o[6] = b[2]; o[7] = b[3];
}
__device__ __forceinline__ void load8(const unsigned short* p, float* o) {
  const u32x4 a = *(const u32x4*)p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(a[i] << 16);
    o[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
  }
}

template <int D, bool SLOTS, typename TSlot, bool OUT_BF16>
__global__ void __launch_bounds__(256) merge_kernel(MergeArgs a) {
  constexpr int LPR = D / 8;   // lanes per part group (8 dims each)
  constexpr int PG = 64 / LPR;  // part groups per row
  const int lane = threadIdx.x & 63;
  const int pg = lane / LPR;
  const int dl = lane % LPR;
  const int64_t rows_total = (int64_t)a.B * a.Hq * a.T;
  // Rows are ordered (b, head, node), so a (sequence, KV head) segment's rows
  // are contiguous; the same XCD mapping as the split-KV kernel puts them on
  // the XCD whose L2 holds that segment's partials.
  const int64_t row = (int64_t)xcd_remap((int)blockIdx.x, (int)gridDim.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows_total) return;
  const int b = (int)(row / ((int64_t)a.Hq * a.T));
  const int rem = (int)(row % ((int64_t)a.Hq * a.T));
  const int h = rem / a.T;
  const int node = rem % a.T;
  const int g = h / a.G;
  const int r = (h - g * a.G) * a.T + node;  // row within the KV head's M rows

  bool bad = false;
  int p_count = 0;
  unsigned w_first = 0, TT = 1;
  bool maybe_empty = false;
  const TSlot* o_base;
  const float* l_base;
  size_t o_stride, l_stride;
  float l_scale;
  if (SLOTS) {
    // One pass over the batch's prefix lengths gives the total tile count and
    // segment (b, g)'s first tile and count (the values total_tiles and
    // segment_tiles compute); err_b is requested beside it, so the row pays one
    // round trip here rather than one per quantity.
    // (a pointer select, not a branch, so the load is not waited on before the loop below)
    const int err_raw = *(a.err_b != nullptr ? a.err_b + b : a.prefix_len + b);
    unsigned seq_tiles = 0, before = 0;
    int count = 0, Lraw = 0;
#pragma unroll 4
    for (int bb = 0; bb < a.B; ++bb) {
      const int Lb = a.prefix_len[bb];
      const int nt = tiles_of((Lb < 0 || Lb > a.Lcap) ? 0 : Lb, a.nk) + a.tree_tiles;
      seq_tiles += (unsigned)nt;
      if (bb < b) before += (unsigned)nt;
      if (bb == b) {
        count = nt;
        Lraw = Lb;
      }
    }
    const bool bad_prefix = Lraw < 0 || Lraw > a.Lcap;
    bad = bad_prefix || (a.err_b != nullptr && err_raw != 0);
    if (bad_prefix && h == 0 && node == 0 && lane == 0) atomicOr(a.status, kStatusBadPrefix);
    TT = seq_tiles * (unsigned)a.Hkv;
    const unsigned first = before * (unsigned)a.Hkv + (unsigned)(g * count);
    int p_first = 0;
    if (count > 0) {
      w_first = split_owner(first, a.nwg, TT);
      const unsigned wl = split_owner(first + (unsigned)count - 1, a.nwg, TT);
      p_first = (int)w_first + b * a.Hkv + g;
      p_count = (int)(wl - w_first) + 1;
    }
    // with more workgroups than tiles, some own no tile and wrote nothing
    maybe_empty = TT < (unsigned)a.nwg;
    o_base = static_cast<const TSlot*>(a.slot_o) + ((size_t)p_first * a.M + r) * D + dl * 8;
    l_base = a.slot_lse2 + (size_t)p_first * a.M + r;
    o_stride = (size_t)a.M * D;
    l_stride = (size_t)a.M;
    l_scale = 1.0f;
  } else {
    p_count = a.n_parts;
    o_base = reinterpret_cast<const TSlot*>(a.o_parts) + (size_t)row * D + dl * 8;
    l_base = a.lse_parts + row;
    o_stride = (size_t)rows_total * D;
    l_stride = (size_t)rows_total;
    l_scale = kLog2e;
  }

  // This lane's part group: running max m, weighted sum s and accumulator acc.
  float m = -__builtin_inff(), s = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int k0 = pg; k0 < p_count; k0 += PG * UNROLL) {
    float lk[UNROLL], ov[UNROLL][8];
    // Which of this step's parts hold nothing (past the end, or a workgroup
    // that owns no tile) is known before any load, so every load of the step
    // is issued before the first wait.
    bool dead[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      dead[u] = k0 + u * PG >= p_count;
      if (SLOTS && maybe_empty) {
        const unsigned wk = w_first + (unsigned)min(k0 + u * PG, p_count - 1);
        dead[u] = dead[u] || split_begin(wk, a.nwg, TT) == split_begin(wk + 1, a.nwg, TT);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int k = min(k0 + u * PG, p_count - 1);  // in-bounds; ignored past the end
      lk[u] = l_base[(size_t)k * l_stride];
      load8(o_base + (size_t)k * o_stride, ov[u]);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) lk[u] = dead[u] ? -__builtin_inff() : lk[u] * l_scale;
    // No branch on the loaded values: while every part so far is empty, m and
    // mc are -inf, alpha is 0 and every weight is 0, so s and acc stay 0.
    float mc = m;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) mc = fmaxf(mc, lk[u]);
    const float alpha = m == -__builtin_inff() ? 0.f : fast_exp2(m - mc);
    s *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
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
    *(u32x4*)(static_cast<unsigned short*>(a.out) + (size_t)row * D + dl * 8) = pk;
  } else {
    float* op = static_cast<float*>(a.out) + (size_t)row * D + dl * 8;
    f32x4 v0 = {acc[0], acc[1], acc[2], acc[3]}, v1 = {acc[4], acc[5], acc[6], acc[7]};
    *(f32x4*)op = v0;
    *(f32x4*)(op + 4) = v1;
  }
  if (dl == 0) a.lse[row] = lse_out;
}

typedef void (*MergeFn)(MergeArgs);

template <bool SLOTS, typename TSlot, bool OUT_BF16>
MergeFn pick(int D) {
  if (D == 128) return merge_kernel<128, SLOTS, TSlot, OUT_BF16>;
  if (D == 64) return merge_kernel<64, SLOTS, TSlot, OUT_BF16>;
  return nullptr;
}

MergeArgs base_args(const Dims& d) {
  MergeArgs a = {};
  a.B = d.B;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.G;
  a.T = d.T;
  a.Lcap = d.Lcap;
  a.M = d.M;
  return a;
}

// Four rows per workgroup, rounded up to a multiple of 8 workgroups (one per
// XCD) so that xcd_remap applies.
unsigned grid_for(const Dims& d) {
  const int64_t rows = (int64_t)d.B * d.Hq * d.T;
  return (unsigned)(((rows + 3) / 4 + 7) / 8 * 8);
}

}  // namespace

hipError_t launch_merge_slots(const Dims& d, int tile_tokens, int nwg, int tree_tiles, const int* prefix_len,
                              Slots slots, const int* err_b, void* out, bool out_bf16, float* lse, int* status,
                              hipStream_t s) {
  MergeFn k;
  if (slots.o_bf16)
    k = out_bf16 ? pick<true, unsigned short, true>(d.D) : pick<true, unsigned short, false>(d.D);
  else
    k = out_bf16 ? pick<true, float, true>(d.D) : pick<true, float, false>(d.D);
  if (!k) return hipErrorInvalidValue;
  MergeArgs a = base_args(d);
  a.prefix_len = prefix_len;
  a.slot_o = slots.o;
  a.slot_lse2 = slots.lse2;
  a.err_b = err_b;
  a.status = status;
  a.nk = tile_tokens;
  a.nwg = nwg;
  a.tree_tiles = tree_tiles;
  a.out = out;
  a.lse = lse;
  hipLaunchKernelGGL(k, dim3(grid_for(d)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_merge_parts(const Dims& d, int n_parts, const float* o_parts,
                              const float* lse_parts, float* out, float* lse, hipStream_t s) {
  MergeFn k = pick<false, float, false>(d.D);
  if (!k) return hipErrorInvalidValue;
  MergeArgs a = base_args(d);
  a.o_parts = o_parts;
  a.lse_parts = lse_parts;
  a.n_parts = n_parts;
  a.out = out;
  a.lse = lse;
  hipLaunchKernelGGL(k, dim3(grid_for(d)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hta
