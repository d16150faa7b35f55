// Split-KV attention kernel on the vector ALUs, for float32 inputs and for
// bf16 layers whose G*T query rows per KV head are too few to fill a 32-row
// MFMA block. Same work split, fused tree tile and partial-result slots as the
// MFMA kernel (see common.h and prefix_mfma.hip); everything in float32.
//
// A workgroup of 256 threads owns 16 query rows (grid.y picks which 16 of
// the M rows of a KV head). Thread (r, c), r = tid/16, c = tid%16, works on
// row r: it scores tokens c, c+16, c+32, c+48 of each 64-token tile against
// that row, and accumulates output dims c, c+16, ... (so neighbouring lanes
// touch neighbouring LDS words). Row max and sum are reduced over the 16
// lanes of a row with cross-lane exchanges. Online softmax in the log2 domain.
#include "common.h"
#include "hta_internal.h"

namespace hta {
namespace {

constexpr int NK = kTileTokens;

struct ValuArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* kt;
  const void* vt;
  const int* parent;
  const int* prefix_len;
  float* slot_o;  // float partials
  float* slot_lse2;
  int* err_b;
  int* status;
  int B, Hq, Hkv, G, T, Lcap, M;
  int nwg, tree_tiles;
  float scale_log2;
};

template <int D, typename TIn>
__global__ void __launch_bounds__(256) prefix_valu_kernel(ValuArgs a) {
  constexpr int DS = D / 16;
  constexpr int KROW = D + 1;
  __shared__ float Qs[16][D + 1];
  __shared__ float Ks[NK * KROW];
  __shared__ float Vs[NK * D];
  __shared__ float Ps[16][NK];
  __shared__ int par_s[64];
  __shared__ unsigned long long anc_s[64];
  __shared__ int bad_s;

  const TIn* qg = static_cast<const TIn*>(a.q);
  const TIn* kg = static_cast<const TIn*>(a.k);
  const TIn* vg = static_cast<const TIn*>(a.v);
  const TIn* ktg = static_cast<const TIn*>(a.kt);
  const TIn* vtg = static_cast<const TIn*>(a.vt);
  const int tid = threadIdx.x;
  const int rl = tid >> 4;
  const int sl = tid & 15;

  const int w = xcd_remap(blockIdx.x, a.nwg);
  const unsigned TT = total_tiles(a.prefix_len, a.B, a.Hkv, a.Lcap, NK, a.tree_tiles);
  if (TT == 0) return;
  unsigned x = split_begin(w, a.nwg, TT);
  const unsigned x_end = split_begin(w + 1, a.nwg, TT);
  if (x >= x_end) return;
  SegmentWalk sw;
  if (!walk_start(&sw, x, a.prefix_len, a.B, a.Hkv, a.Lcap, NK, a.tree_tiles)) return;

  const int row = blockIdx.y * 16 + rl;
  const bool row_ok = row < a.M;
  const int node = row_ok ? row % a.T : 0;

  while (true) {
    const int b = sw.b, g = sw.g;
    const unsigned s_first = sw.seq_first + (unsigned)(g * sw.nt);
    const int tile0 = (int)(x - s_first);
    const unsigned piece_end = min(x_end, s_first + (unsigned)sw.nt);
    const int ntiles = (int)(piece_end - x);
    const int L = sw.L;
    const int n_prefix = sw.nt - a.tree_tiles;
    const bool has_tree = a.tree_tiles && tile0 + ntiles > n_prefix;
    const int slot = w + b * a.Hkv + g;
    const size_t kv_off = (size_t)(b * a.Hkv + g) * (size_t)a.Lcap * D;
    const size_t kt_off = (size_t)(b * a.Hkv + g) * a.T * D;
    const TIn* qp = qg + (size_t)(b * a.Hq + g * a.G) * a.T * D;

    __syncthreads();  // LDS of the previous piece is no longer read
    if (has_tree) {
      if (tid == 0) bad_s = 0;
      if (tid < a.T) par_s[tid] = a.parent[(size_t)b * a.T + tid];
      __syncthreads();
      if (tid < a.T) {
        bool ok = true;
        anc_s[tid] = ancestor_word(par_s, tid, &ok);
        if (!ok) bad_s = 1;
      }
    }
#pragma unroll
    for (int e = 0; e < DS; ++e) {
      const int d = sl + 16 * e;
      Qs[rl][d] = row_ok ? load_elem(qp + (size_t)row * D + d) : 0.f;
    }
    float o[DS];
#pragma unroll
    for (int e = 0; e < DS; ++e) o[e] = 0.f;
    float m = -__builtin_inff(), l = 0.f;

    for (int t = 0; t < ntiles; ++t) {
      const int ti = tile0 + t;
      const bool tree = ti >= n_prefix;
      const TIn* ks = tree ? ktg + kt_off : kg + kv_off + (size_t)ti * NK * D;
      const TIn* vs = tree ? vtg + kt_off : vg + kv_off + (size_t)ti * NK * D;
      const int nvalid = tree ? a.T : min(NK, L - ti * NK);  // >= 1 for every tile that exists
      // All of this thread's loads of the tile are issued before the first is
      // waited on (one memory round trip per tile, not one per element). Rows
      // past the valid tokens read the last valid row, so every read is in
      // bounds; they are stored as zeros.
      constexpr int PER = NK * D / 256;
      float kval[PER], vval[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int idx = tid + 256 * i;
        const int tk = idx / D, d = idx % D;
        const int src = min(tk, nvalid - 1) * D + d;
        kval[i] = load_elem(ks + src);
        vval[i] = load_elem(vs + src);
      }
      __syncthreads();  // every thread is done with the previous tile's Ks, Vs and Ps
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int idx = tid + 256 * i;
        const int tk = idx / D, d = idx % D;
        const bool ok = tk < nvalid;
        Ks[tk * KROW + d] = ok ? kval[i] : 0.f;
        Vs[tk * D + d] = ok ? vval[i] : 0.f;
      }
      __syncthreads();
      const unsigned long long vis = tree ? anc_s[node] : 0ull;
      float s[4];
      float mx = -__builtin_inff();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tk = sl + 16 * j;
        float acc = 0.f;
        for (int d = 0; d < D; ++d) acc = fmaf(Qs[rl][d], Ks[tk * KROW + d], acc);
        const bool seen = tree ? ((vis >> tk) & 1ull) != 0ull : tk < nvalid;
        s[j] = seen ? acc * a.scale_log2 : -__builtin_inff();
        mx = fmaxf(mx, s[j]);
      }
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float mn = fmaxf(m, mx);
      const float alpha = m == -__builtin_inff() ? 0.f : fast_exp2(m - mn);
      m = mn;
      const float msafe = m == -__builtin_inff() ? 0.f : m;
      float ls = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = fast_exp2(s[j] - msafe);
        Ps[rl][sl + 16 * j] = p;
        ls += p;
      }
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) ls += __shfl_xor(ls, off);
      l = l * alpha + ls;
#pragma unroll
      for (int e = 0; e < DS; ++e) o[e] *= alpha;
      __syncthreads();
      for (int tk = 0; tk < nvalid; ++tk) {
        const float p = Ps[rl][tk];
#pragma unroll
        for (int e = 0; e < DS; ++e) o[e] = fmaf(p, Vs[tk * D + sl + 16 * e], o[e]);
      }
    }

    if (row_ok) {
      const float inv = 1.0f / l;
      float* op = a.slot_o + ((size_t)slot * a.M + row) * D;
#pragma unroll
      for (int e = 0; e < DS; ++e) op[sl + 16 * e] = o[e] * inv;
      if (sl == 0) a.slot_lse2[(size_t)slot * a.M + row] = m + fast_log2(l);
    }
    if (has_tree && g == 0 && blockIdx.y == 0 && tid == 0) {
      a.err_b[b] = bad_s;
      if (bad_s) atomicOr(a.status, kStatusBadTree);
    }

    x = piece_end;
    if (x >= x_end) break;
    if (!walk_next(&sw, a.prefix_len, a.B, a.Hkv, a.Lcap, NK, a.tree_tiles)) break;
  }
}

typedef void (*KernelFn)(ValuArgs);

KernelFn pick(int D, bool bf16) {
  if (D == 128) return bf16 ? prefix_valu_kernel<128, unsigned short> : prefix_valu_kernel<128, float>;
  if (D == 64) return bf16 ? prefix_valu_kernel<64, unsigned short> : prefix_valu_kernel<64, float>;
  return nullptr;
}

}  // namespace

int prefix_valu_occupancy(int D, bool bf16) {
  KernelFn k = pick(D, bf16);
  if (!k) return 0;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(k), 256, 0) !=
      hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}

hipError_t launch_prefix_valu(const Dims& d, const PrefixLaunch& pl, const PrefixInputs& in, Slots slots,
                              int* err_b, int* status, hipStream_t s) {
  KernelFn k = pick(d.D, d.bf16);
  if (!k) return hipErrorInvalidValue;
  ValuArgs a;
  a.q = in.q;
  a.k = in.k_cache;
  a.v = in.v_cache;
  a.kt = in.k_tree;
  a.vt = in.v_tree;
  a.parent = in.parent;
  a.prefix_len = in.prefix_len;
  a.slot_o = static_cast<float*>(slots.o);
  a.slot_lse2 = slots.lse2;
  a.err_b = err_b;
  a.status = status;
  a.B = d.B;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.G;
  a.T = d.T;
  a.Lcap = d.Lcap;
  a.M = d.M;
  a.nwg = pl.nwg;
  a.tree_tiles = in.k_tree ? 1 : 0;
  a.scale_log2 = d.scale_log2;
  hipLaunchKernelGGL(k, dim3(pl.nwg, pl.row_groups), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hta
