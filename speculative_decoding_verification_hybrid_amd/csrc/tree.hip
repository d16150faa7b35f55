// Tree mask and the masked speculative part of Hybrid Tree Attention.
//
// LongSpec summary pages, "Fast Tree Attention": the few speculative tokens
// are handled by their own masked kernel. LogitSpec summary page, "draft
// tree construction and verification": the tree mask lets every branch of
// the draft tree be verified in the same pass, i.e. node i sees exactly the
// nodes on its root path. Here the mask is one 64-bit word per node, bit j
// set iff node j is i or an ancestor of i, built in LDS from parent[] by a
// walk up the tree; parent[j] < j makes every walk finish within T steps.
// A parent array that breaks -1 <= parent[i] < i marks the whole sequence
// bad: NaN outputs and a sticky status bit, never an out-of-range access.
#include "common.h"
#include "hta_internal.h"

namespace hta {
namespace {

__global__ void __launch_bounds__(64) tree_mask_kernel(const int* parent, unsigned long long* out,
                                                       int* status, int T) {
  __shared__ int par[64];
  __shared__ int bad;
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  if (i == 0) bad = 0;
  if (i < T) par[i] = parent[(size_t)b * T + i];
  __syncthreads();
  bool ok = true;
  unsigned long long wd = 0ull;
  if (i < T) wd = ancestor_word(par, i, &ok);
  if (!ok) bad = 1;
  __syncthreads();
  if (i < T) out[(size_t)b * T + i] = bad ? 0ull : wd;
  if (i == 0 && bad) atomicOr(status, kStatusBadTree);
}

struct TreeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int* parent;
  float* o;
  float* lse;
  int* err_b;
  int* status;
  int Hq, Hkv, G, T, M;
  float scale_log2;
  float lse_scale;
};

// grid (B*Hkv, ceil(M/16)); thread (r, c) = (tid/16, tid%16) works on row r of
// the block's 16 rows: tree keys c, c+16, ... and output dims c, c+16, ...
template <int D, typename TIn>
__global__ void __launch_bounds__(256) tree_attn_kernel(TreeArgs a) {
  constexpr int DS = D / 16;
  constexpr int KROW = D + 1;
  __shared__ int par[64];
  __shared__ unsigned long long anc[64];
  __shared__ int bad;
  __shared__ float Ks[64 * KROW];
  __shared__ float Vs[64 * D];
  __shared__ float Qs[16][D + 1];
  __shared__ float Ps[16][64];

  const TIn* qg = static_cast<const TIn*>(a.q);
  const TIn* kg = static_cast<const TIn*>(a.k);
  const TIn* vg = static_cast<const TIn*>(a.v);
  const int tid = threadIdx.x;
  const int rl = tid >> 4, sl = tid & 15;
  const int b = blockIdx.x / a.Hkv;
  const int g = blockIdx.x % a.Hkv;
  const int T = a.T;

  if (tid == 0) bad = 0;
  if (tid < T) par[tid] = a.parent[(size_t)b * T + tid];
  __syncthreads();
  if (tid < T) {
    bool ok = true;
    anc[tid] = ancestor_word(par, tid, &ok);
    if (!ok) bad = 1;
  }
  const size_t kv_off = (size_t)(b * a.Hkv + g) * T * D;
  for (int idx = tid; idx < T * D; idx += 256) {
    const int j = idx / D, d = idx % D;
    Ks[j * KROW + d] = load_elem(kg + kv_off + idx);
    Vs[j * D + d] = load_elem(vg + kv_off + idx);
  }
  const int row = blockIdx.y * 16 + rl;
  const bool row_ok = row < a.M;
  const int hl = row_ok ? row / T : 0;
  const int node = row_ok ? row % T : 0;
  const size_t orow = (size_t)(b * a.Hq + g * a.G + hl) * T + node;  // row of [B,Hq,T]
#pragma unroll
  for (int e = 0; e < DS; ++e) {
    const int d = sl + 16 * e;
    Qs[rl][d] = row_ok ? load_elem(qg + orow * D + d) : 0.f;
  }
  __syncthreads();

  if (bad) {
    if (row_ok) {
      const float nan = __builtin_nanf("");
#pragma unroll
      for (int e = 0; e < DS; ++e) a.o[orow * D + sl + 16 * e] = nan;
      if (sl == 0) a.lse[orow] = nan;
    }
    if (tid == 0 && g == 0 && blockIdx.y == 0) {
      if (a.err_b) a.err_b[b] = 1;
      atomicOr(a.status, kStatusBadTree);
    }
    return;
  }
  if (tid == 0 && g == 0 && blockIdx.y == 0 && a.err_b) a.err_b[b] = 0;

  const unsigned long long vis = anc[node];
  float s[4];
  float mx = -__builtin_inff();
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int j = sl + 16 * jj;
    float sc = -__builtin_inff();
    if (j < T && ((vis >> j) & 1ull)) {
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc = fmaf(Qs[rl][d], Ks[j * KROW + d], acc);
      sc = acc * a.scale_log2;
    }
    s[jj] = sc;
    mx = fmaxf(mx, sc);
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float ls = 0.f;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int j = sl + 16 * jj;
    const float p = fast_exp2(s[jj] - mx);  // exp2(-inf) = 0 for hidden nodes
    if (j < 64) Ps[rl][j] = p;
    ls += p;
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) ls += __shfl_xor(ls, off);
  __syncthreads();
  float o[DS];
#pragma unroll
  for (int e = 0; e < DS; ++e) o[e] = 0.f;
  for (int j = 0; j < T; ++j) {
    const float p = Ps[rl][j];
#pragma unroll
    for (int e = 0; e < DS; ++e) o[e] = fmaf(p, Vs[j * D + sl + 16 * e], o[e]);
  }
  if (row_ok) {
    const float inv = 1.0f / ls;
#pragma unroll
    for (int e = 0; e < DS; ++e) a.o[orow * D + sl + 16 * e] = o[e] * inv;
    if (sl == 0) a.lse[orow] = (mx + fast_log2(ls)) * a.lse_scale;
  }
}

typedef void (*TreeFn)(TreeArgs);

TreeFn pick(int D, bool bf16) {
  if (D == 128) return bf16 ? tree_attn_kernel<128, unsigned short> : tree_attn_kernel<128, float>;
  if (D == 64) return bf16 ? tree_attn_kernel<64, unsigned short> : tree_attn_kernel<64, float>;
  return nullptr;
}

__global__ void clear_status_kernel(int* status) {
  if (threadIdx.x == 0) *status = 0;
}

}  // namespace

hipError_t launch_tree_mask(const Dims& d, const int* parent, uint64_t* mask_out, int* status,
                            hipStream_t s) {
  hipLaunchKernelGGL(tree_mask_kernel, dim3(d.B), dim3(64), 0, s, parent,
                     reinterpret_cast<unsigned long long*>(mask_out), status, d.T);
  return hipGetLastError();
}

hipError_t launch_tree_attn(const Dims& d, const void* q, const void* k_tree, const void* v_tree,
                            const int* parent, float* o_tree, float* lse_tree, float lse_scale,
                            int* err_b, int* status, hipStream_t s) {
  TreeFn k = pick(d.D, d.bf16);
  if (!k) return hipErrorInvalidValue;
  TreeArgs a;
  a.q = q;
  a.k = k_tree;
  a.v = v_tree;
  a.parent = parent;
  a.o = o_tree;
  a.lse = lse_tree;
  a.err_b = err_b;
  a.status = status;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.G;
  a.T = d.T;
  a.M = d.M;
  a.scale_log2 = d.scale_log2;
  a.lse_scale = lse_scale;
  hipLaunchKernelGGL(k, dim3(d.B * d.Hkv, (d.M + 15) / 16), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_clear_status(int* status, hipStream_t s) {
  hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(64), 0, s, status);
  return hipGetLastError();
}

}  // namespace hta
