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
// D = 128), 8 rows per 256-thread workgroup. The weighted pass is unrolled
// and branch-free so that the loads of several parts are in flight together.
#include "common.h"
#include "hta_internal.h"

namespace hta {
namespace {

constexpr int NK = kTileTokens;
constexpr int UNROLL = 8;

struct MergeArgs {
  // slot mode: partials of one split-KV launch
  const int* prefix_len;
  const float* slot_o;
  const float* slot_lse2;
  const int* err_b;
  int* status;
  int nwg, tree_tiles;
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
  int p_count = 0;
  unsigned w_first = 0, TT = 1;
  const float* o_base;
  const float* l_base;
  size_t o_stride, l_stride;
  float l_scale;
  if (SLOTS) {
    const int Lraw = a.prefix_len[b];
    const bool bad_prefix = Lraw < 0 || Lraw > a.Lcap;
    bad = bad_prefix || (a.err_b != nullptr && a.err_b[b] != 0);
    if (bad_prefix && h == 0 && node == 0 && dq == 0) atomicOr(a.status, kStatusBadPrefix);
    TT = total_tiles(a.prefix_len, a.B, a.Hkv, a.Lcap, NK, a.tree_tiles);
    unsigned first;
    int count;
    segment_tiles(a.prefix_len, a.Hkv, a.Lcap, NK, a.tree_tiles, b, g, &first, &count);
    int p_first = 0;
    if (count > 0) {
      w_first = split_owner(first, a.nwg, TT);
      const unsigned wl = split_owner(first + (unsigned)count - 1, a.nwg, TT);
      p_first = (int)w_first + b * a.Hkv + g;
      p_count = (int)(wl - w_first) + 1;
    }
    o_base = a.slot_o + ((size_t)p_first * a.M + r) * D + dq * DV;
    l_base = a.slot_lse2 + (size_t)p_first * a.M + r;
    o_stride = (size_t)a.M * D;
    l_stride = (size_t)a.M;
    l_scale = 1.0f;
  } else {
    p_count = a.n_parts;
    o_base = a.o_parts + (size_t)row * D + dq * DV;
    l_base = a.lse_parts + row;
    o_stride = (size_t)rows_total * D;
    l_stride = (size_t)rows_total;
    l_scale = kLog2e;
  }

  // LSE of part k in log2 units; -inf for an empty part. With more workgroups
  // than tiles some workgroups own no tile: they sit between the owners of a
  // segment's first and last tile and wrote nothing to their slot.
  auto part_lse2 = [&](int k) -> float {
    if (SLOTS) {
      const unsigned wk = w_first + (unsigned)k;
      if (split_begin(wk, a.nwg, TT) == split_begin(wk + 1, a.nwg, TT)) return -__builtin_inff();
    }
    return l_base[(size_t)k * l_stride] * l_scale;
  };

  float mx = -__builtin_inff();
  for (int k = 0; k < p_count; ++k) mx = fmaxf(mx, part_lse2(k));

  float acc[DV];
#pragma unroll
  for (int e = 0; e < DV; ++e) acc[e] = 0.f;
  float lse_out;
  if (mx == -__builtin_inff()) {
    lse_out = -__builtin_inff();
  } else {
    float sum = 0.f;
    for (int k0 = 0; k0 < p_count; k0 += UNROLL) {
      float wk[UNROLL];
      VT ov[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int k = min(k0 + u, p_count - 1);  // in-bounds load; weight 0 past the end
        const float lk = part_lse2(k);
        wk[u] = (k0 + u < p_count && lk != -__builtin_inff()) ? fast_exp2(lk - mx) : 0.f;
        ov[u] = *(const VT*)(o_base + (size_t)k * o_stride);
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        sum += wk[u];
#pragma unroll
        for (int e = 0; e < DV; ++e) acc[e] += wk[u] == 0.f ? 0.f : wk[u] * ov[u][e];
      }
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

hipError_t launch_merge_slots(const Dims& d, int nwg, int tree_tiles, const int* prefix_len, Slots slots,
                              const int* err_b, void* out, bool out_bf16, float* lse, int* status,
                              hipStream_t s) {
  MergeFn k = out_bf16 ? pick<true, true>(d.D) : pick<true, false>(d.D);
  if (!k) return hipErrorInvalidValue;
  MergeArgs a = base_args(d);
  a.prefix_len = prefix_len;
  a.slot_o = slots.o;
  a.slot_lse2 = slots.lse2;
  a.err_b = err_b;
  a.status = status;
  a.nwg = nwg;
  a.tree_tiles = tree_tiles;
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
