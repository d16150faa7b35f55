// Building the draft tree from the target's last logits (LogitSpec summary
// pages, §2 "LogitSpec workflow"): the greedy next token x1, the top-k
// next-next guesses without it, two kinds of n-gram query against the
// sequence's own tokens (query 1: the m tokens ending with x1; query 2 per
// guess: the m-1 tokens ending with x1, then the guess), and a tree rooted
// at x1 with one branch per guess, keeping keep[r] retrieved tokens for the
// guess of rank r (more for more confident guesses).
//
// Readings (as in the design notes): a match is the most recent earlier
// occurrence; retrieved tokens are those that follow it; ranking is by
// logit value, lower index first on ties. Node order: x1; query 1's tokens as
// a chain under it; then per guess by rank, the guess under x1 and its
// retrieved chain under the guess; nodes past T are dropped in that order and
// unused slots hold token -1 under the root.
//
// Kernels:
//  * topk_partial_kernel: B*split workgroups; each reduces its slice of a
//    logit row to its kk = k+1 largest 64-bit keys (order-preserving value
//    bits above, V-1-index below), by kk rounds of "largest key below the last
//    one" over keys held in registers.
//  * tree_build_kernel: one workgroup per sequence merges the split lists the
//    same way, then streams the sequence (history then x1) through LDS in
//    chunks. Every query-2 gram shares its first m-1 tokens (the m-1 tokens
//    ending with x1), so a position needs one compare of that tail plus a
//    lookup of its token among the guesses, and one compare for query 1;
//    the latest match per query is kept with an LDS atomic max. Thread 0
//    then lays out the tree (at most 64 nodes).
#include "common.h"
#include "hta_internal.h"

namespace hta {
namespace {

constexpr int kTopThreads = 256;
constexpr int kTopEPT = 16;                          // keys per thread in a slice
constexpr int kTopChunk = kTopThreads * kTopEPT;     // vocabulary entries per workgroup
constexpr int kHistChunk = 8192;                     // sequence tokens per LDS pass

__device__ __forceinline__ unsigned ordered_bits(float x) {
  const unsigned u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ unsigned long long make_key(float x, unsigned idx) {
  return ((unsigned long long)ordered_bits(x) << 32) | (unsigned long long)(0xffffffffu - idx);
}
__device__ __forceinline__ unsigned key_index(unsigned long long k) {
  return 0xffffffffu - (unsigned)(k & 0xffffffffull);
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

// kk rounds over the kTopEPT keys each thread holds (0 = no key): out[j] =
// j-th largest key of the workgroup (0 past the end). red: kTopThreads/64 slots.
__device__ void select_top(const unsigned long long* mine, int kk, unsigned long long* out,
                           unsigned long long* red, unsigned long long* bcast) {
  unsigned long long bound = ~0ull;  // every key is below it
  for (int j = 0; j < kk; ++j) {
    unsigned long long best = 0ull;
#pragma unroll
    for (int e = 0; e < kTopEPT; ++e)
      if (mine[e] < bound) best = umax64(best, mine[e]);
    best = wave_max64(best);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long k = red[0];
#pragma unroll
      for (int w = 1; w < kTopThreads / 64; ++w) k = umax64(k, red[w]);
      out[j] = k;
      *bcast = k;
    }
    __syncthreads();
    bound = *bcast;
    if (bound == 0ull) {  // fewer keys than kk: the rest stay 0
      for (int i = j + 1 + (int)threadIdx.x; i < kk; i += kTopThreads) out[i] = 0ull;
      break;
    }
  }
}

template <bool BF16>
__global__ void __launch_bounds__(kTopThreads) topk_partial_kernel(const void* logits, int V, int split, int kk,
                                                                   unsigned long long* part) {
  __shared__ unsigned long long red[kTopThreads / 64];
  __shared__ unsigned long long bcast;
  __shared__ unsigned long long out[kMaxTreeGuesses + 1];
  const int b = blockIdx.x / split, s = blockIdx.x % split;
  const int lo = s * kTopChunk;
  unsigned long long mine[kTopEPT];
#pragma unroll
  for (int e = 0; e < kTopEPT; ++e) {
    const int i = lo + (int)threadIdx.x + e * kTopThreads;
    float x = 0.f;
    if (i < V) {
      if (BF16) x = bf16_bits_to_float(static_cast<const unsigned short*>(logits)[(size_t)b * V + i]);
      else x = static_cast<const float*>(logits)[(size_t)b * V + i];
    }
    mine[e] = i < V ? make_key(x, (unsigned)i) : 0ull;
  }
  select_top(mine, kk, out, red, &bcast);
  __syncthreads();
  for (int j = threadIdx.x; j < kk; j += kTopThreads) part[((size_t)b * split + s) * (kMaxTreeGuesses + 1) + j] = out[j];
}

struct TreeArgs {
  const unsigned long long* part;
  int split, kk;
  const int* history;
  int hist_cap;
  const int* hist_len;
  TreeParams p;
  int T;
  int* tokens;
  int* parent;
  int* n_nodes;
  int* status;
};

__global__ void __launch_bounds__(kTopThreads) tree_build_kernel(TreeArgs a) {
  __shared__ unsigned long long red[kTopThreads / 64];
  __shared__ unsigned long long bcast;
  __shared__ unsigned long long top[kMaxTreeGuesses + 1];
  __shared__ int seqs[kHistChunk + kMaxNgram];
  __shared__ int q1s[kMaxNgram];   // query 1
  __shared__ int tail[kMaxNgram];  // the m-1 tokens ending with x1 (query 2 without its guess)
  __shared__ int best[kMaxTreeGuesses + 1];  // latest match end: [0] query 1, [1 + r] guess r
  const int b = blockIdx.x;
  const int tid = (int)threadIdx.x;
  const int T = a.T, k = a.p.k, m = a.p.m;
  const int L = a.hist_len[b];
  const int* hist = a.history + (size_t)b * a.hist_cap;
  int* tok_out = a.tokens + (size_t)b * T;
  int* par_out = a.parent + (size_t)b * T;

  if (L < 0 || L > a.hist_cap) {
    for (int i = tid; i < T; i += kTopThreads) {
      tok_out[i] = -1;
      par_out[i] = i == 0 ? -1 : 0;
    }
    if (tid == 0) {
      a.n_nodes[b] = 0;
      atomicOr(a.status, kStatusBadPrefix);
    }
    return;
  }

  // 1. merge the split lists: x1 and the ranked guesses
  unsigned long long mine[kTopEPT];
#pragma unroll
  for (int e = 0; e < kTopEPT; ++e) {
    const int i = tid + e * kTopThreads;  // entry i of split*kk
    mine[e] = i < a.split * a.kk
                  ? a.part[((size_t)b * a.split + i / a.kk) * (kMaxTreeGuesses + 1) + i % a.kk]
                  : 0ull;
  }
  select_top(mine, a.kk, top, red, &bcast);
  __syncthreads();
  const int x1 = (int)key_index(top[0]);
  // the sequence: hist[0 .. L-1], then x1 at position L; n = L + 1 tokens
  const int n = L + 1;
  auto seq_at = [&](int j) { return j < L ? hist[j] : x1; };
  if (tid < m) {
    q1s[tid] = n - m + tid >= 0 ? seq_at(n - m + tid) : -1;
    if (tid < m - 1) tail[tid] = n - (m - 1) + tid >= 0 ? seq_at(n - (m - 1) + tid) : -1;
  }
  if (tid <= k) best[tid] = -1;
  __syncthreads();

  // 2. one pass over the sequence, kHistChunk positions at a time (with the m-1
  // tokens before each chunk)
  const bool q1_possible = m <= n;
  const bool q2_possible = m - 1 <= n;
  for (int c0 = 0; c0 < n; c0 += kHistChunk) {
    const int lo = c0 - (m - 1);
    const int cnt = min(kHistChunk, n - c0) + (m - 1);
    for (int i = tid; i < cnt; i += kTopThreads) {
      const int j = lo + i;
      seqs[i] = j >= 0 ? seq_at(j) : -1;
    }
    __syncthreads();
    for (int i = tid; i < min(kHistChunk, n - c0); i += kTopThreads) {
      const int p = c0 + i;        // end position of the gram
      if (p < m - 1) continue;     // a gram needs m tokens
      const int* w = &seqs[i];     // w[0 .. m-1] = seq[p-m+1 .. p]
      if (q1_possible && p < n - 1) {  // query 1 may not match itself
        bool eq = true;
        for (int t = 0; t < m; ++t) eq &= w[t] == q1s[t];
        if (eq) atomicMax(&best[0], p);
      }
      if (q2_possible && k > 0) {
        bool eq = true;
        for (int t = 0; t < m - 1; ++t) eq &= w[t] == tail[t];
        if (eq) {
          const int tk = w[m - 1];
          for (int r = 0; r < k; ++r)
            if (tk == (int)key_index(top[1 + r])) atomicMax(&best[1 + r], p);
        }
      }
    }
    __syncthreads();
  }

  // 3. lay out the tree
  for (int i = tid; i < T; i += kTopThreads) {
    tok_out[i] = -1;
    par_out[i] = 0;
  }
  __syncthreads();
  if (tid == 0) {
    int used = 0;
    auto add = [&](int tokv, int par) {
      if (used >= T) return -1;
      tok_out[used] = tokv;
      par_out[used] = par;
      return used++;
    };
    add(x1, -1);
    if (best[0] >= 0) {
      int par = 0;
      for (int t = 0; t < a.p.keep_first && best[0] + 1 + t < n && par >= 0; ++t)
        par = add(seq_at(best[0] + 1 + t), par);
    }
    for (int r = 0; r < k; ++r) {
      const int node = add((int)key_index(top[1 + r]), 0);
      if (node < 0) break;
      const int pe = best[1 + r];
      if (pe < 0) continue;
      int par = node;
      for (int t = 0; t < a.p.keep[r] && pe + 1 + t < n && par >= 0; ++t) par = add(seq_at(pe + 1 + t), par);
    }
    a.n_nodes[b] = used;
  }
}

}  // namespace

int topk_split_for(int V) { return (V + kTopChunk - 1) / kTopChunk; }

hipError_t launch_build_tree(const Dims& d, const void* logits, int V, bool logits_bf16, const int* history,
                             int hist_cap, const int* hist_len, const TreeParams& p, unsigned long long* part,
                             int* tokens, int* parent, int* n_nodes, int* status, hipStream_t s) {
  const int split = topk_split_for(V);
  const int kk = p.k + 1;
  if (logits_bf16)
    hipLaunchKernelGGL(topk_partial_kernel<true>, dim3(d.B * split), dim3(kTopThreads), 0, s, logits, V, split, kk,
                       part);
  else
    hipLaunchKernelGGL(topk_partial_kernel<false>, dim3(d.B * split), dim3(kTopThreads), 0, s, logits, V, split,
                       kk, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  TreeArgs a;
  a.part = part;
  a.split = split;
  a.kk = kk;
  a.history = history;
  a.hist_cap = hist_cap;
  a.hist_len = hist_len;
  a.p = p;
  a.T = d.T;
  a.tokens = tokens;
  a.parent = parent;
  a.n_nodes = n_nodes;
  a.status = status;
  hipLaunchKernelGGL(tree_build_kernel, dim3(d.B), dim3(kTopThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hta
