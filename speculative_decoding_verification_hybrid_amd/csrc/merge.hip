// Log-sum-exp merge of partial attentions (LongSpec summary pages, "Fast
// Tree Attention": the cached and speculative parts are aggregated with the
// log-sum-exp trick, which keeps the result exact).
//
// For one output row with partials (o_k normalised, lse_k) over disjoint key
// sets: lse = log2(sum_k 2^lse_k) and out = sum_k 2^(lse_k - lse) o_k, done
// as one max pass over the lse values and one weighted pass over the o rows.
// Parts with lse_k = -inf contribute nothing; a row with no part at all gets
// out = 0, lse = -inf. Internally every LSE is base 2; the stored lse is
// natural log.
//
// 32 threads per row, each owning D/32 consecutive dims (16-byte loads for
// D = 128), 8 rows per 256-thread workgroup.
#include "common.h"
#include "hta_internal.h"

namespace hta {
namespace {

constexpr int NK = kTileTokens;

struct MergeArgs {
  // slot mode: partials of the prefix kernel + optional tree partial
  const int* prefix_len;
  const float* slot_o;
  const float* slot_lse2;
  const float* o_tree;
  const float* lse2_tree;
  const int* err_b;
  int* status;
  int nwg;
  // parts mode: n_parts caller arrays, natural-log lse
  const float* o_parts;
  const float* lse_parts;
  int n_parts;
  // common
  void* out;
  float* lse;
  int B, Hq, Hkv, G, T, Lcap, M;
};

template <int D>
struct Vec;
template <>
struct Vec<128> {
  typedef f32x4 T;
};
template <>
struct Vec<64> {
  typedef float __attribute__((ext_vector_type(2))) T;
};

template <int D, bool SLOTS, bool OUT_BF16>
__global__ void __launch_bounds__(256) merge_kernel(MergeArgs a) {
  constexpr int DV = D / 32;
  typedef typename Vec<D>::T VT;
  const int tid = threadIdx.x;
  const int dq = tid & 31;
  const int64_t rows_total = (int64_t)a.B * a.Hq * a.T;
  const int64_t row = (int64_t)blockIdx.x * 8 + (tid >> 5);
  if (row >= rows_total) return;
  const int b = (int)(row / ((int64_t)a.Hq * a.T));
  const int rem = (int)(row % ((int64_t)a.Hq * a.T));
  const int h = rem / a.T;
  const int node = rem % a.T;
  const int g = h / a.G;
  const int r = (h - g * a.G) * a.T + node;  // row within the KV head's M rows

  bool bad = false;
  int p_first = 0, p_count = 0;  // slot range (SLOTS) or part range
  int64_t w_first = 0, TT = 1;   // SLOTS: first workgroup of the range, total tiles
  bool with_tree = false;
  if (SLOTS) {
    const int Lraw = a.prefix_len[b];
    const bool bad_prefix = Lraw < 0 || Lraw > a.Lcap;
    bad = bad_prefix || (a.err_b != nullptr && a.err_b[b] != 0);
    if (bad_prefix && h == 0 && node == 0 && dq == 0) atomicOr(a.status, kStatusBadPrefix);
    TT = total_tiles(a.prefix_len, a.B, a.Hkv, a.Lcap, NK);
    int64_t first;
    int count;
    segment_tiles(a.prefix_len, a.Hkv, a.Lcap, NK, b, g, &first, &count);
    if (count > 0) {
      const int64_t wf = split_owner(first, a.nwg, TT);
      const int64_t wl = split_owner(first + count - 1, a.nwg, TT);
      p_first = (int)wf + b * a.Hkv + g;
      p_count = (int)(wl - wf) + 1;
      w_first = wf;
    }
    with_tree = a.o_tree != nullptr;
  } else {
    p_first = 0;
    p_count = a.n_parts;
  }

  // With more workgroups than tiles some workgroups own no tile; they sit
  // between the owners of a segment's first and last tile and wrote nothing.
  auto part_lse2 = [&](int k) -> float {
    if (SLOTS) {
      const int64_t w = w_first + k;
      if (split_begin(w, a.nwg, TT) == split_begin(w + 1, a.nwg, TT)) return -__builtin_inff();
      return a.slot_lse2[(size_t)(p_first + k) * a.M + r];
    }
    return a.lse_parts[(size_t)k * rows_total + row] * kLog2e;
  };
  auto part_o = [&](int k) -> const float* {
    if (SLOTS) return a.slot_o + ((size_t)(p_first + k) * a.M + r) * D;
    return a.o_parts + ((size_t)k * rows_total + row) * D;
  };

  float mx = -__builtin_inff();
  for (int k = 0; k < p_count; ++k) mx = fmaxf(mx, part_lse2(k));
  float lt2 = -__builtin_inff();
  if (with_tree) {
    lt2 = a.lse2_tree[row];
    mx = fmaxf(mx, lt2);
  }

  float acc[DV];
#pragma unroll
  for (int e = 0; e < DV; ++e) acc[e] = 0.f;
  float lse_out;
  if (mx == -__builtin_inff()) {
    lse_out = -__builtin_inff();
  } else {
    float sum = 0.f;
    for (int k = 0; k < p_count; ++k) {
      const float lk = part_lse2(k);
      if (lk == -__builtin_inff()) continue;  // empty part: its o is never read
      const float wk = fast_exp2(lk - mx);
      const VT ov = *(const VT*)(part_o(k) + dq * DV);
      sum += wk;
#pragma unroll
      for (int e = 0; e < DV; ++e) acc[e] = fmaf(wk, ov[e], acc[e]);
    }
    if (with_tree) {
      const float wk = fast_exp2(lt2 - mx);
      const VT ov = *(const VT*)(a.o_tree + (size_t)row * D + dq * DV);
      sum += wk;
#pragma unroll
      for (int e = 0; e < DV; ++e) acc[e] = fmaf(wk, ov[e], acc[e]);
    }
    const float inv = 1.0f / sum;
#pragma unroll
    for (int e = 0; e < DV; ++e) acc[e] *= inv;
    lse_out = (mx + fast_log2(sum)) * kLn2;
  }
  if (bad) {
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int e = 0; e < DV; ++e) acc[e] = nan;
    lse_out = nan;
  }
  if (OUT_BF16) {
    unsigned short* op = static_cast<unsigned short*>(a.out) + (size_t)row * D + dq * DV;
#pragma unroll
    for (int e = 0; e < DV; ++e) op[e] = float_to_bf16_bits(acc[e]);
  } else {
    float* op = static_cast<float*>(a.out) + (size_t)row * D + dq * DV;
    VT v;
#pragma unroll
    for (int e = 0; e < DV; ++e) v[e] = acc[e];
    *(VT*)op = v;
  }
  if (dq == 0) a.lse[row] = lse_out;
}

typedef void (*MergeFn)(MergeArgs);

template <bool SLOTS, bool OUT_BF16>
MergeFn pick(int D) {
  if (D == 128) return merge_kernel<128, SLOTS, OUT_BF16>;
  if (D == 64) return merge_kernel<64, SLOTS, OUT_BF16>;
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

unsigned grid_for(const Dims& d) {
  const int64_t rows = (int64_t)d.B * d.Hq * d.T;
  return (unsigned)((rows + 7) / 8);
}

}  // namespace

hipError_t launch_merge_slots(const Dims& d, int nwg, const int* prefix_len, Slots slots,
                              const float* o_tree, const float* lse2_tree, const int* err_b,
                              void* out, bool out_bf16, float* lse, int* status, hipStream_t s) {
  MergeFn k = out_bf16 ? pick<true, true>(d.D) : pick<true, false>(d.D);
  if (!k) return hipErrorInvalidValue;
  MergeArgs a = base_args(d);
  a.prefix_len = prefix_len;
  a.slot_o = slots.o;
  a.slot_lse2 = slots.lse2;
  a.o_tree = o_tree;
  a.lse2_tree = lse2_tree;
  a.err_b = err_b;
  a.status = status;
  a.nwg = nwg;
  a.out = out;
  a.lse = lse;
  hipLaunchKernelGGL(k, dim3(grid_for(d)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_merge_parts(const Dims& d, int n_parts, const float* o_parts,
                              const float* lse_parts, float* out, float* lse, hipStream_t s) {
  MergeFn k = pick<false, false>(d.D);
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
