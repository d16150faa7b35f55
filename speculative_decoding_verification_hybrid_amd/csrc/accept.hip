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
//  * argmax_kernel: the B*T logit rows of V entries are each split over
//    `split` workgroups; a workgroup reduces its slice to one 64-bit key
//    (order-preserving bits of the value above, V-1-index below, so the
//    largest key is the largest value at the lowest index) with all of its
//    16-byte loads issued before any compare -- a pure HBM stream of the
//    logits.
//  * accept_kernel: one workgroup per sequence gathers the split keys of its
//    T rows (all loads in flight at once, four waves) and walks the tree in
//    one wave, lane i = node i: a node's edge is
//    accepted when its token equals its parent's prediction and no
//    lower-numbered sibling's does; a node is on the accepted path when every
//    edge from the root to it is accepted (its ancestor word, built by
//    pointer jumping in six rounds, has no bit outside the accepted-edge
//    ballot). The accepted nodes form one root path in increasing index
//    order, so path[k] is the k-th set bit.
//  * commit_kernel: one workgroup per (sequence, KV head, K or V) copies the
//    accepted rows with 16-byte loads/stores; the last of a sequence's
//    workgroups to finish advances prefix_len (every workgroup has read the
//    old value before it arrives).
#include "common.h"
#include "hta_internal.h"

namespace hta {
namespace {

constexpr int kArgmaxThreads = 256;
constexpr int kArgmaxVecs = 2;  // 16-byte vectors per thread in the unrolled part of a slice
constexpr int kMaxKeyLoads = (kArgmaxMaxSplit + 3) / 4;  // per thread of the walking workgroup

// Order-preserving map of a float's bits to an unsigned int (larger float,
// larger key); NaN inputs are not ordered meaningfully.
__device__ __forceinline__ unsigned ordered_bits(float x) {
  unsigned u = __float_as_uint(x);
  u = u == 0x80000000u ? 0u : u;  // -0 and +0 compare equal, so they share a key
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned long long make_key(float x, unsigned idx) {
  return ((unsigned long long)ordered_bits(x) << 32) | (unsigned long long)(0xffffffffu - idx);
}

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}

__device__ __forceinline__ unsigned long long shfl64(unsigned long long k, int src) {
  const unsigned lo = __shfl((unsigned)k, src), hi = __shfl((unsigned)(k >> 32), src);
  return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ unsigned long long wave_max64(unsigned long long k) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const unsigned lo = __shfl_xor((unsigned)k, off), hi = __shfl_xor((unsigned)(k >> 32), off);
    k = umax64(k, ((unsigned long long)hi << 32) | lo);
  }
  return k;
}

// Keys of the 16-byte vector holding elements i .. i+W-1.
template <bool BF16>
__device__ __forceinline__ unsigned long long vec_max(const u32x4& v, int i) {
  unsigned long long best = 0ull;
  if (BF16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      best = umax64(best, make_key(__uint_as_float(v[e] << 16), (unsigned)(i + 2 * e)));
      best = umax64(best, make_key(__uint_as_float(v[e] & 0xffff0000u), (unsigned)(i + 2 * e + 1)));
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) best = umax64(best, make_key(__uint_as_float(v[e]), (unsigned)(i + e)));
  }
  return best;
}

// Largest key of elements [lo, hi) of one logit row, reduced over the workgroup
// (valid in every thread of wave 0; 0 = below every real key for an empty slice).
// VEC: the row starts 16-byte aligned and lo is a multiple of the vector width.
template <bool BF16, bool VEC>
__device__ unsigned long long slice_max(const void* row_ptr, int lo, int hi, unsigned long long* red) {
  const int tid = (int)threadIdx.x;
  unsigned long long best = 0ull;
  if (VEC) {
    constexpr int W = BF16 ? 8 : 4;  // elements per 16-byte vector
    const unsigned char* base = static_cast<const unsigned char*>(row_ptr);
    u32x4 v[kArgmaxVecs];
    bool ok[kArgmaxVecs];
#pragma unroll
    for (int it = 0; it < kArgmaxVecs; ++it) {  // every load in flight before the first compare
      const int i = lo + W * (tid + it * kArgmaxThreads);
      ok[it] = i < hi;
      if (ok[it]) v[it] = *(const u32x4*)(base + (size_t)i * (BF16 ? 2 : 4));
    }
#pragma unroll
    for (int it = 0; it < kArgmaxVecs; ++it)
      if (ok[it]) best = umax64(best, vec_max<BF16>(v[it], lo + W * (tid + it * kArgmaxThreads)));
    for (int i = lo + W * (tid + kArgmaxVecs * kArgmaxThreads); i < hi; i += W * kArgmaxThreads)
      best = umax64(best, vec_max<BF16>(*(const u32x4*)(base + (size_t)i * (BF16 ? 2 : 4)), i));
  } else if (BF16) {
    const unsigned short* p = static_cast<const unsigned short*>(row_ptr);
    for (int i = lo + tid; i < hi; i += kArgmaxThreads) best = umax64(best, make_key(bf16_bits_to_float(p[i]), (unsigned)i));
  } else {
    const float* p = static_cast<const float*>(row_ptr);
    for (int i = lo + tid; i < hi; i += kArgmaxThreads) best = umax64(best, make_key(p[i], (unsigned)i));
  }
  best = wave_max64(best);
  if ((tid & 63) == 0) red[tid >> 6] = best;
  __syncthreads();
  unsigned long long k = red[0];
#pragma unroll
  for (int w = 1; w < kArgmaxThreads / 64; ++w) k = umax64(k, red[w]);
  return k;
}

// grid: B*T*split workgroups; workgroup x reduces slice x % split of row x / split.
template <bool BF16, bool VEC>
__global__ void __launch_bounds__(kArgmaxThreads) argmax_kernel(const void* logits, int V, int split, int chunk,
                                                               unsigned long long* part) {
  __shared__ unsigned long long red[kArgmaxThreads / 64];
  const int64_t row = blockIdx.x / split;
  const int s = (int)(blockIdx.x % split);
  const int lo = s * chunk;
  const int hi = min(V, lo + chunk);
  const void* row_ptr = static_cast<const unsigned char*>(logits) + row * (int64_t)V * (BF16 ? 2 : 4);
  const unsigned long long key = slice_max<BF16, VEC>(row_ptr, lo, hi, red);
  if (threadIdx.x == 0) part[blockIdx.x] = key;
}

// grid: B workgroups of kArgmaxThreads; the tree walk runs in wave 0.
__global__ void __launch_bounds__(kArgmaxThreads) accept_kernel(const unsigned long long* part, int split,
                                                               const int* parent, const int* tree_tokens, int T,
                                                               int* target_out, int* accept_len,
                                                               int* accept_path, int* bonus, int* status) {
  __shared__ unsigned long long row_key[kArgmaxThreads / 64][64];
  const int tid = (int)threadIdx.x;
  const int b = (int)blockIdx.x;
  // Prediction per node: the largest of its row's split keys, gathered by all
  // four waves (node = lane, slices strided over the waves), then combined in wave 0.
  const int i = tid & 63, w = tid >> 6;
  const bool node = i < T;
  int p = -1, tok = 0;
  if (w == 0 && node) {
    p = parent[(size_t)b * T + i];
    tok = tree_tokens[(size_t)b * T + i];
  }
  unsigned long long k = 0ull;
  if (node) {
    const unsigned long long* kp = part + ((size_t)b * T + i) * split;
    unsigned long long v[kMaxKeyLoads];
#pragma unroll
    for (int j = 0; j < kMaxKeyLoads; ++j) v[j] = (w + 4 * j < split) ? kp[w + 4 * j] : 0ull;
#pragma unroll
    for (int j = 0; j < kMaxKeyLoads; ++j) k = umax64(k, v[j]);
  }
  row_key[w][i] = k;
  __syncthreads();
  if (w != 0) return;
  k = umax64(umax64(row_key[0][i], row_key[1][i]), umax64(row_key[2][i], row_key[3][i]));
  const int target = (int)(0xffffffffu - (unsigned)(k & 0xffffffffull));
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
  for (unsigned long long m = __ballot(match); m != 0ull; m &= m - 1ull) {  // matching nodes, few
    const int j = __ffsll((long long)m) - 1;
    const int pj = __shfl(p, j);
    if (j < i && pj == p) first = false;
  }
  const unsigned long long edges = __ballot(!node || i == 0 || (match && first));
  // ancestor word of node i (node i and every node up to its root): pointer
  // jumping, round r adds the ancestors at distances [2^r, 2^(r+1)); T <= 64
  // bounds a depth by 63, so six rounds reach every root.
  unsigned long long anc = node ? (1ull << i) : 0ull;
  int up = p;
#pragma unroll
  for (int r = 0; r < 6; ++r) {
    const int src = up < 0 ? i : up;
    const unsigned long long a = shfl64(anc, src);
    const int u = __shfl(up, src);
    if (up >= 0) {
      anc |= a;
      up = u;
    }
  }
  const bool ok = node && (anc & 1ull) && (anc & ~edges) == 0ull;
  const unsigned long long okm = __ballot(ok);
  const int n = __popcll(okm);
  if (ok) accept_path[(size_t)b * T + __popcll(okm & ((1ull << i) - 1ull))] = i;
  if (node && i >= n) accept_path[(size_t)b * T + i] = -1;
  const int last_node = 63 - __clzll(okm);  // node 0 is always accepted, so okm != 0
  const int bt = __shfl(target, last_node);
  if (i == 0) {
    accept_len[b] = n;
    bonus[b] = bt;
  }
}

// grid: B*Hkv workgroups x 2 (K, V). Rows of row_bytes bytes (a multiple of 16).
__global__ void __launch_bounds__(256) commit_kernel(const void* k_tree, const void* v_tree, const int* accept_len,
                                                     const int* accept_path, void* k_cache, void* v_cache,
                                                     int* prefix_len, int Hkv, int T, int Lcap, int row_bytes,
                                                     unsigned* count, int* status) {
  const int bg = blockIdx.x;
  const int b = bg / Hkv;
  const int n = accept_len[b];
  const int L = prefix_len[b];
  const bool fits = n > 0 && n <= T && L >= 0 && L <= Lcap - n;
  if (fits) {
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
  __syncthreads();  // every wave of this workgroup has read prefix_len[b]
  if (threadIdx.x == 0) {
    __threadfence();
    const unsigned old = atomicAdd(&count[b], 1u);
    if (old == 2u * (unsigned)Hkv - 1u) {  // the sequence's last workgroup
      count[b] = 0;
      if (L < 0 || L > Lcap)
        atomicOr(status, kStatusBadPrefix);  // no cache length to append to
      else if (n > 0) {
        if (fits)
          prefix_len[b] = L + n;
        else
          atomicOr(status, kStatusCommitOverflow);
      }
    }
  }
}

}  // namespace

int argmax_split_for(int V, bool logits_bf16) {
  // enough workgroups that each thread has kArgmaxVecs vectors in the unrolled part
  const int per_wg = kArgmaxVecs * kArgmaxThreads * (logits_bf16 ? 8 : 4);
  return max(1, min((V + per_wg - 1) / per_wg, kArgmaxMaxSplit));
}

hipError_t launch_accept(const Dims& d, const void* logits, int V, bool logits_bf16, const int* parent,
                         const int* tree_tokens, unsigned long long* part, int* target_out, int* accept_len,
                         int* accept_path, int* bonus, int* status, hipStream_t s) {
  const int64_t rows = (int64_t)d.B * d.T;
  const int split = argmax_split_for(V, logits_bf16);
  const int width = logits_bf16 ? 8 : 4;  // elements per 16-byte vector
  int chunk = (V + split - 1) / split;
  chunk = (chunk + width - 1) / width * width;
  const bool vec = (V % width) == 0 && ((uintptr_t)logits & 15) == 0;
  const dim3 grid((unsigned)(rows * split));
  const dim3 block(kArgmaxThreads);
  if (logits_bf16) {
    if (vec)
      hipLaunchKernelGGL((argmax_kernel<true, true>), grid, block, 0, s, logits, V, split, chunk, part);
    else
      hipLaunchKernelGGL((argmax_kernel<true, false>), grid, block, 0, s, logits, V, split, chunk, part);
  } else {
    if (vec)
      hipLaunchKernelGGL((argmax_kernel<false, true>), grid, block, 0, s, logits, V, split, chunk, part);
    else
      hipLaunchKernelGGL((argmax_kernel<false, false>), grid, block, 0, s, logits, V, split, chunk, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(accept_kernel, dim3(d.B), block, 0, s, part, split, parent, tree_tokens, d.T, target_out,
                     accept_len, accept_path, bonus, status);
  return hipGetLastError();
}

hipError_t launch_commit(const Dims& d, const void* k_tree, const void* v_tree, const int* accept_len,
                         const int* accept_path, void* k_cache, void* v_cache, int* prefix_len, unsigned* count,
                         int* status, hipStream_t s) {
  const int row_bytes = d.D * (d.bf16 ? 2 : 4);
  hipLaunchKernelGGL(commit_kernel, dim3(d.B * d.Hkv, 2), dim3(256), 0, s, k_tree, v_tree, accept_len,
                     accept_path, k_cache, v_cache, prefix_len, d.Hkv, d.T, d.Lcap, row_bytes, count, status);
  return hipGetLastError();
}

}  // namespace hta
