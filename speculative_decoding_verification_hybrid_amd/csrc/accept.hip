// Accepting a verified draft tree and committing its accepted nodes
// (LogitSpec summary pages, "draft tree construction and verification": the
// tree is rooted at x_{i+1} and the target verifies every branch at once;
// LongSpec summary pages: decoding stays lossless, the target keeps only what
// it would have produced itself).
//
// Greedy reading: the target's prediction at node j is the token with the
// largest logit at j (lowest index among equal maxima); from the root the
// accepted path moves to the child whose draft token equals the prediction at
// its parent (the lowest-numbered such child), and the prediction at the last
// accepted node is the bonus token. Committing appends the accepted nodes'
// K/V rows at prefix_len and advances it.
//
// Kernels:
//  * argmax_partial_kernel: rows = B*T logit rows of V entries, each split
//    over `split` workgroups; every workgroup reduces its slice to one 64-bit
//    key (order-preserving bits of the value above, V-1-index below, so the
//    largest key is the largest value at the lowest index) -- a pure HBM
//    stream of the logits.
//  * accept_kernel: one wave per sequence, lane i = tree node i. The node's
//    prediction is the max of its row's keys; a node's edge is accepted when
//    its token equals its parent's prediction and no lower-numbered sibling's
//    does; a node is on the accepted path when every edge from the root to it
//    is accepted (its ancestor word has no bit outside the accepted-edge
//    ballot). The accepted nodes form one root path in increasing index
//    order, so path[k] is the k-th set bit.
//  * commit_kernel: one workgroup per (sequence, KV head, K or V) copies the
//    accepted rows with 16-byte loads/stores; commit_len_kernel then advances
//    prefix_len (a separate launch, so that every copy has read the old value).
#include "common.h"
#include "hta_internal.h"

namespace hta {
namespace {

constexpr int kArgmaxThreads = 256;

// Order-preserving map of a float's bits to an unsigned int (larger float,
// larger key); NaN inputs are not ordered meaningfully.
__device__ __forceinline__ unsigned ordered_bits(float x) {
  const unsigned u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned long long make_key(float x, unsigned idx) {
  return ((unsigned long long)ordered_bits(x) << 32) | (unsigned long long)(0xffffffffu - idx);
}

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}

__device__ __forceinline__ unsigned long long wave_max64(unsigned long long k) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const unsigned lo = __shfl_xor((unsigned)k, off), hi = __shfl_xor((unsigned)(k >> 32), off);
    k = umax64(k, ((unsigned long long)hi << 32) | lo);
  }
  return k;
}

// VEC: the row starts 16-byte aligned and the chunk is a multiple of the
// vector width, so every thread reads whole 16-byte vectors.
template <bool BF16, bool VEC>
__global__ void __launch_bounds__(kArgmaxThreads) argmax_partial_kernel(const void* logits, int V, int split,
                                                                        int chunk, unsigned long long* part) {
  __shared__ unsigned long long red[kArgmaxThreads / 64];
  const int64_t row = blockIdx.x / split;
  const int s = blockIdx.x % split;
  const int lo = s * chunk;
  const int hi = min(V, lo + chunk);
  unsigned long long best = 0ull;  // below every real key
  if (BF16) {
    const unsigned short* p = static_cast<const unsigned short*>(logits) + row * (int64_t)V;
    if (VEC) {
      for (int i = lo + 8 * (int)threadIdx.x; i < hi; i += 8 * kArgmaxThreads) {
        const u32x4 v = *(const u32x4*)(p + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          best = umax64(best, make_key(__uint_as_float(v[e] << 16), (unsigned)(i + 2 * e)));
          best = umax64(best, make_key(__uint_as_float(v[e] & 0xffff0000u), (unsigned)(i + 2 * e + 1)));
        }
      }
    } else {
      for (int i = lo + (int)threadIdx.x; i < hi; i += kArgmaxThreads)
        best = umax64(best, make_key(bf16_bits_to_float(p[i]), (unsigned)i));
    }
  } else {
    const float* p = static_cast<const float*>(logits) + row * (int64_t)V;
    if (VEC) {
      for (int i = lo + 4 * (int)threadIdx.x; i < hi; i += 4 * kArgmaxThreads) {
        const f32x4 v = *(const f32x4*)(p + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) best = umax64(best, make_key(v[e], (unsigned)(i + e)));
      }
    } else {
      for (int i = lo + (int)threadIdx.x; i < hi; i += kArgmaxThreads)
        best = umax64(best, make_key(p[i], (unsigned)i));
    }
  }
  best = wave_max64(best);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long k = red[0];
#pragma unroll
    for (int w = 1; w < kArgmaxThreads / 64; ++w) k = umax64(k, red[w]);
    part[blockIdx.x] = k;
  }
}

__global__ void __launch_bounds__(64) accept_kernel(const unsigned long long* part, int split, const int* parent,
                                                    const int* tree_tokens, int T, int* target_out,
                                                    int* accept_len, int* accept_path, int* bonus,
                                                    int* status) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;  // tree node of this lane
  const bool node = i < T;
  unsigned long long key = 0ull;
  int p = -1, tok = 0;
  if (node) {
    const unsigned long long* kp = part + ((size_t)b * T + i) * split;
    for (int s = 0; s < split; ++s) key = umax64(key, kp[s]);
    p = parent[(size_t)b * T + i];
    tok = tree_tokens[(size_t)b * T + i];
  }
  const int target = (int)(0xffffffffu - (unsigned)(key & 0xffffffffull));
  if (node) target_out[(size_t)b * T + i] = target;
  const bool bad = __any(node && (p < -1 || p >= i));
  if (bad) {
    if (node) accept_path[(size_t)b * T + i] = -1;
    if (i == 0) {
      accept_len[b] = 0;
      bonus[b] = -1;
      atomicOr(status, kStatusBadTree);
    }
    return;
  }
  // edge i accepted: token i equals the prediction at its parent, and no
  // lower-numbered sibling's token does
  const int ptarget = __shfl(target, p < 0 ? 0 : p);
  const bool match = node && p >= 0 && tok == ptarget;
  bool first = true;
  for (int j = 0; j < T; ++j) {
    const int pj = __shfl(p, j);
    const bool mj = __shfl((int)match, j) != 0;
    if (j < i && pj == p && mj) first = false;
  }
  const unsigned long long edges = __ballot(!node || i == 0 || (match && first));
  // ancestor word of node i (node i and every node up to its root)
  unsigned long long anc = 0ull;
  int cur = node ? i : -1;
  for (int k = 0; k < T; ++k) {
    const int nxt = __shfl(p, cur < 0 ? 0 : cur);
    if (cur >= 0) {
      anc |= 1ull << cur;
      cur = nxt;
    }
  }
  const bool ok = node && (anc & 1ull) && (anc & ~edges) == 0ull;
  const unsigned long long okm = __ballot(ok);
  const int n = __popcll(okm);
  if (ok) accept_path[(size_t)b * T + __popcll(okm & ((1ull << i) - 1ull))] = i;
  if (node && i >= n) accept_path[(size_t)b * T + i] = -1;
  const int last = 63 - __clzll(okm);  // node 0 is always accepted, so okm != 0
  const int bt = __shfl(target, last);
  if (i == 0) {
    accept_len[b] = n;
    bonus[b] = bt;
  }
}

// grid: B*Hkv workgroups x 2 (K, V). Rows of D elements of elem_bytes each.
__global__ void __launch_bounds__(256) commit_kernel(const void* k_tree, const void* v_tree, const int* accept_len,
                                                     const int* accept_path, void* k_cache, void* v_cache,
                                                     const int* prefix_len, int Hkv, int T, int Lcap,
                                                     int row_bytes, int* status) {
  const int bg = blockIdx.x;
  const int b = bg / Hkv;
  const int n = accept_len[b];
  const int L = prefix_len[b];
  if (n <= 0 || n > T || L < 0 || L > Lcap - n) return;  // commit_len_kernel reports the overflow
  const unsigned char* src = static_cast<const unsigned char*>(blockIdx.y == 0 ? k_tree : v_tree) +
                             (size_t)bg * T * row_bytes;
  unsigned char* dst = static_cast<unsigned char*>(blockIdx.y == 0 ? k_cache : v_cache) +
                       ((size_t)bg * Lcap + L) * row_bytes;
  const int per_row = row_bytes / 16;
  for (int u = threadIdx.x; u < n * per_row; u += blockDim.x) {
    const int k = u / per_row, c = u % per_row;
    const int node = accept_path[(size_t)b * T + k];
    if (node < 0 || node >= T) {
      atomicOr(status, kStatusBadPath);
      continue;
    }
    *(u32x4*)(dst + (size_t)k * row_bytes + 16 * c) = *(const u32x4*)(src + (size_t)node * row_bytes + 16 * c);
  }
}

__global__ void __launch_bounds__(64) commit_len_kernel(const int* accept_len, int* prefix_len, int B, int T,
                                                        int Lcap, int* status) {
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const int n = accept_len[b];
    const int L = prefix_len[b];
    if (n <= 0) continue;
    if (n > T || L < 0 || L > Lcap - n) {
      atomicOr(status, kStatusCommitOverflow);
      continue;
    }
    prefix_len[b] = L + n;
  }
}

}  // namespace

int argmax_split_for(int64_t rows, int V) {
  // enough workgroups to cover the device several times, each reading >= 16 KB
  int split = (int)((2048 + rows - 1) / rows);
  const int max_by_size = max(1, V / 8192);
  split = min(split, max_by_size);
  return max(1, min(split, kArgmaxMaxSplit));
}

hipError_t launch_accept(const Dims& d, const void* logits, int V, bool logits_bf16, const int* parent,
                         const int* tree_tokens, unsigned long long* part, int* target_out, int* accept_len,
                         int* accept_path, int* bonus, int* status, hipStream_t s) {
  const int64_t rows = (int64_t)d.B * d.T;
  const int split = argmax_split_for(rows, V);
  const int width = logits_bf16 ? 8 : 4;  // elements per 16-byte vector
  int chunk = (V + split - 1) / split;
  chunk = (chunk + width - 1) / width * width;
  const bool vec = (V % width) == 0 && ((uintptr_t)logits & 15) == 0;
  const dim3 grid((unsigned)(rows * split));
  if (logits_bf16) {
    if (vec)
      hipLaunchKernelGGL((argmax_partial_kernel<true, true>), grid, dim3(kArgmaxThreads), 0, s, logits, V, split,
                         chunk, part);
    else
      hipLaunchKernelGGL((argmax_partial_kernel<true, false>), grid, dim3(kArgmaxThreads), 0, s, logits, V, split,
                         chunk, part);
  } else {
    if (vec)
      hipLaunchKernelGGL((argmax_partial_kernel<false, true>), grid, dim3(kArgmaxThreads), 0, s, logits, V,
                         split, chunk, part);
    else
      hipLaunchKernelGGL((argmax_partial_kernel<false, false>), grid, dim3(kArgmaxThreads), 0, s, logits, V,
                         split, chunk, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(accept_kernel, dim3(d.B), dim3(64), 0, s, part, split, parent, tree_tokens, d.T, target_out,
                     accept_len, accept_path, bonus, status);
  return hipGetLastError();
}

hipError_t launch_commit(const Dims& d, const void* k_tree, const void* v_tree, const int* accept_len,
                         const int* accept_path, void* k_cache, void* v_cache, int* prefix_len, int* status,
                         hipStream_t s) {
  const int row_bytes = d.D * (d.bf16 ? 2 : 4);
  hipLaunchKernelGGL(commit_kernel, dim3(d.B * d.Hkv, 2), dim3(256), 0, s, k_tree, v_tree, accept_len,
                     accept_path, k_cache, v_cache, prefix_len, d.Hkv, d.T, d.Lcap, row_bytes, status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(commit_len_kernel, dim3(1), dim3(64), 0, s, accept_len, prefix_len, d.B, d.T, d.Lcap,
                     status);
  return hipGetLastError();
}

}  // namespace hta
