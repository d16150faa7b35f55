// Merge kernel: the log-sum-exp merge of partial attentions (merge_row.h)
// as its own launch, one wave per output row, over either the slots of one
// split-KV launch (each (sequence, KV head) segment's partials are the slots
// of the workgroups that own its tiles) or caller-provided part arrays.
#include "common.h"
#include "hta_internal.h"
#include "merge_row.h"

namespace hta {
namespace {

struct MergeArgs {
  // slot mode: partials of one split-KV launch
  const int* prefix_len;
  const void* slot_o;
  const float* slot_lse2;
  const int* err_b;
  int* status;
  int nk, nwg, tree_tiles, tree_weight;
  // parts mode: n_parts caller arrays, natural-log lse
  const float* o_parts;
  const float* lse_parts;
  int n_parts;
  // common
  void* out;
  float* lse;
  int B, Hq, Hkv, G, T, Lcap, M;
};

template <int D, bool SLOTS, typename TSlot, bool OUT_BF16>
__global__ void __launch_bounds__(256) merge_kernel(MergeArgs a) {
  constexpr int LPR = D / 8;  // lanes per part group (8 dims each)
  const int lane = threadIdx.x & 63;
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
    // (segments as the split sees them: prefix tiles, tree tiles and the
    // empty tiles that weigh the tree tiles; count is the real ones)
    unsigned seq_tiles = 0, before = 0;
    int count = 0, span = 0, Lraw = 0;
#pragma unroll 4
    for (int bb = 0; bb < a.B; ++bb) {
      const int Lb = a.prefix_len[bb];
      const int nr = tiles_of((Lb < 0 || Lb > a.Lcap) ? 0 : Lb, a.nk) + a.tree_tiles;
      const int nt = nr + a.tree_tiles * (a.tree_weight - 1);
      seq_tiles += (unsigned)nt;
      if (bb < b) before += (unsigned)nt;
      if (bb == b) {
        count = nr;
        span = nt;
        Lraw = Lb;
      }
    }
    const bool bad_prefix = Lraw < 0 || Lraw > a.Lcap;
    bad = bad_prefix || (a.err_b != nullptr && err_raw != 0);
    if (bad_prefix && h == 0 && node == 0 && lane == 0) atomicOr(a.status, kStatusBadPrefix);
    TT = seq_tiles * (unsigned)a.Hkv;
    const unsigned first = before * (unsigned)a.Hkv + (unsigned)(g * span);
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

  auto load_o = [&](int k, float* v) { merge_load8(o_base + (size_t)k * o_stride, v); };
  auto load_l = [&](int k) { return l_base[(size_t)k * l_stride] * l_scale; };
  if (SLOTS && maybe_empty) {
    const unsigned nwg = (unsigned)a.nwg;
    merge_row<D, OUT_BF16>(
        lane, p_count, load_o, load_l,
        [&](int k) { return split_begin(w_first + (unsigned)k, nwg, TT) == split_begin(w_first + (unsigned)k + 1, nwg, TT); },
        bad, a.out, a.lse, row);
  } else {
    merge_row<D, OUT_BF16>(lane, p_count, load_o, load_l, [](int) { return false; }, bad, a.out, a.lse, row);
  }
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

hipError_t launch_merge_slots(const Dims& d, int tile_tokens, int nwg, int tree_tiles, int tree_weight,
                              const int* prefix_len,
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
  a.tree_weight = tree_weight;
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
