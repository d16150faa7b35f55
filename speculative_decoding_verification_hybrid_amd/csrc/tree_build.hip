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
//    bits above, V-1-index below) by kk rounds of "largest key below the last
//    one", run per wave with DPP reductions (no barriers), then over the four
//    waves' lists. It also resets the sequence's match slots.
//  * tree_scan_kernel: (B, sequence/kScanChunk) workgroups; each merges the
//    split lists the same way (x1 and the guesses), stages its chunk of the
//    sequence (history then x1) in LDS and tests every gram ending in it.
//    Every query-2 gram shares its first m-1 tokens (the m-1 tokens ending
//    with x1), so a position needs one compare of that tail plus a lookup of
//    its token among the guesses, and one compare for query 1; the latest
//    match per query is kept with a device-wide atomic max.
//  * tree_layout_kernel: one workgroup per sequence sizes the branches, then
//    writes one node per thread.
//
// The indexed variant (hta_build_tree_indexed) answers the same queries from a
// hash index of each history's m-grams (LogitSpec summary pages, §4: the
// retrieval is hash-based). The index maps every distinct gram of the history
// to the largest position at which it ends. Query 1's own occurrence ends at
// x1, past the history, and a query-2 gram ends with a guess, never with x1,
// so the latest occurrence in the searched sequence (history then x1) that
// the scan finds is the latest one inside the history: exactly the index's
// entry. Two launches instead of three:
//  * topk_partial_kernel, with B * groups more workgroups that add the grams
//    ending at the history's new positions (lock-free: a slot's key is
//    claimed by compare-and-swap, its latest end raised by atomic max, and
//    the claimer copies the key's tokens into the slot);
//  * tree_layout_kernel<true>: wave 0 merges the split lists, lanes 0 .. k
//    probe the index for query 1 and the k query-2 grams (one slot read per
//    probe), then the layout as above; it records the length the index now
//    covers.
#include "common.h"
#include "hta_internal.h"

namespace hta {
namespace {

constexpr int kTopThreads = 256;
constexpr int kTopEPT = 16;                          // keys per thread in a slice
constexpr int kTopChunk = kTopThreads * kTopEPT;     // vocabulary entries per workgroup
constexpr int kScanChunk = 2048;                     // gram end positions per scan workgroup
constexpr int kInsertChunk = 4096;                   // history positions per index-insert workgroup
constexpr int kMaxInsertGroups = 32;                 // index-insert workgroups per sequence

__device__ __forceinline__ unsigned ordered_bits(float x) {
  unsigned u = __float_as_uint(x);
  u = u == 0x80000000u ? 0u : u;  // -0 and +0 compare equal, so they share a key
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
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp64(unsigned long long x) {
  const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)x, CTRL, 0xf, 0xf, false);
  const unsigned hi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)(x >> 32), CTRL, 0xf, 0xf, false);
  return ((unsigned long long)hi << 32) | lo;
}
// Largest key of the wave, in every lane: DPP within rows of 16 (partners at
// lane distance 1, 2, and rotations by 4 and 8), then the row swaps.
__device__ __forceinline__ unsigned long long wave_max64(unsigned long long k) {
  k = umax64(k, dpp64<0xB1>(k));   // quad_perm [1,0,3,2]
  k = umax64(k, dpp64<0x4E>(k));   // quad_perm [2,3,0,1]
  k = umax64(k, dpp64<0x124>(k));  // row_ror:4
  k = umax64(k, dpp64<0x128>(k));  // row_ror:8
  auto lo = __builtin_amdgcn_permlane16_swap((unsigned)k, (unsigned)k, false, false);
  auto hi = __builtin_amdgcn_permlane16_swap((unsigned)(k >> 32), (unsigned)(k >> 32), false, false);
  k = umax64(((unsigned long long)hi[0] << 32) | lo[0], ((unsigned long long)hi[1] << 32) | lo[1]);
  lo = __builtin_amdgcn_permlane32_swap((unsigned)k, (unsigned)k, false, false);
  hi = __builtin_amdgcn_permlane32_swap((unsigned)(k >> 32), (unsigned)(k >> 32), false, false);
  return umax64(((unsigned long long)hi[0] << 32) | lo[0], ((unsigned long long)hi[1] << 32) | lo[1]);
}

// kk rounds over the E keys each lane of one wave holds (0 = no key): lane 0
// writes out[j] = the j-th largest key of the wave (0 past the end). No
// barriers: every lane learns each round's maximum from wave_max64.
template <int E>
__device__ void select_top_wave(const unsigned long long* mine, int kk, unsigned long long* out) {
  unsigned long long bound = ~0ull;  // every key is below it
  for (int j = 0; j < kk; ++j) {
    unsigned long long best = 0ull;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (mine[e] < bound) best = umax64(best, mine[e]);
    best = wave_max64(best);
    if ((threadIdx.x & 63) == 0) out[j] = best;
    bound = best;  // 0 once the keys run out: later rounds write 0 too
  }
}

// bf16 logits within one 4096-entry slice: a 32-bit key holds the 16
// order-preserving value bits and the reversed slice index (12 bits) below,
// with bit 28 set (0 = no key), so its order is that of make_key on the same
// entries and the first selection runs on 32-bit compares and exchanges.
__device__ __forceinline__ unsigned ordered16(unsigned bits16) {
  bits16 = bits16 == 0x8000u ? 0u : bits16;  // -0 ranks as +0
  return (bits16 & 0x8000u) ? (~bits16 & 0xffffu) : (bits16 | 0x8000u);
}
__device__ __forceinline__ unsigned slice_key(unsigned bits16, int local) {
  return (1u << 28) | (ordered16(bits16) << 12) | (unsigned)(kTopChunk - 1 - local);
}
__device__ __forceinline__ unsigned long long slice_key_to_key(unsigned k, int lo) {
  if (k == 0u) return 0ull;
  const unsigned ord = (k >> 12) & 0xffffu;
  const unsigned bits16 = (ord & 0x8000u) ? (ord & 0x7fffu) : (~ord & 0xffffu);
  return make_key(bf16_bits_to_float(bits16), (unsigned)(lo + (kTopChunk - 1) - (int)(k & (kTopChunk - 1))));
}
static_assert(kTopChunk == 4096, "slice keys hold a 12-bit index");
__device__ __forceinline__ unsigned wave_max32(unsigned k) {
  k = max(k, (unsigned)__builtin_amdgcn_update_dpp(0, (int)k, 0xB1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
  k = max(k, (unsigned)__builtin_amdgcn_update_dpp(0, (int)k, 0x4E, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
  k = max(k, (unsigned)__builtin_amdgcn_update_dpp(0, (int)k, 0x124, 0xf, 0xf, false));  // row_ror:4
  k = max(k, (unsigned)__builtin_amdgcn_update_dpp(0, (int)k, 0x128, 0xf, 0xf, false));  // row_ror:8
  auto r = __builtin_amdgcn_permlane16_swap(k, k, false, false);
  k = max((unsigned)r[0], (unsigned)r[1]);
  r = __builtin_amdgcn_permlane32_swap(k, k, false, false);
  return max((unsigned)r[0], (unsigned)r[1]);
}
// select_top_wave on slice keys: lane 0 writes out[j] = the j-th largest slice key.
template <int E>
__device__ void select_top_wave32(const unsigned* mine, int kk, unsigned* out) {
  unsigned bound = ~0u;
  for (int j = 0; j < kk; ++j) {
    unsigned best = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (mine[e] < bound) best = max(best, mine[e]);
    best = wave_max32(best);
    if ((threadIdx.x & 63) == 0) out[j] = best;
    bound = best;
  }
}

// ---- n-gram hash index --------------------------------------------------
// w[0 .. m) = the gram. Knuth's multiplicative step per token, then
// MurmurHash3's 32-bit finaliser; the hash only picks the first slot to probe:
// keys are compared token by token, so its quality affects speed, not results.
__device__ __forceinline__ unsigned gram_hash(const int (&w)[kMaxNgram], int m) {
  unsigned x = 0x9e3779b9u;
#pragma unroll
  for (int t = 0; t < kMaxNgram; ++t)
    if (t < m) x = ((x ^ (unsigned)w[t]) * 0x9e3779b1u) ^ (x >> 15);
  x ^= x >> 16;
  x *= 0x85ebca6bu;
  x ^= x >> 13;
  x *= 0xc2b2ae35u;
  x ^= x >> 16;
  return x;
}
// Whether the gram of history row hist ending at position r is w[0 .. m).
__device__ __forceinline__ bool gram_ends_at(const int* hist, int r, int m, const int (&w)[kMaxNgram]) {
  bool eq = true;
#pragma unroll
  for (int t = 0; t < kMaxNgram; ++t)
    if (t < m) eq &= hist[r - m + 1 + t] == w[t];
  return eq;
}
// Slot layout, slot_ints(m) ints: [0] end position of the key occurrence
// (-1: empty), [1] largest end position, [2 .. 2+m) the key's tokens.
__host__ __device__ constexpr int slot_ints(int m) { return m + 2 <= 8 ? 8 : 16; }

// Adds the gram ending at position e (e >= m-1) to one sequence's table of
// mask+1 slots. Linear probing; an empty slot's key is claimed by a
// compare-and-swap of -1 to e, and the entry's latest end is raised by atomic
// max, so concurrent inserts of one gram meet in one slot. Inserts identify a
// slot's key through the history at its position; the claimer also copies
// the key's tokens into the slot for the lookups of later launches. The table
// holds at least twice as many slots as a history has positions: a free slot
// always exists, and the probe bound is never the exit taken.
__device__ void ngram_insert(int* tab, unsigned mask, int stride, const int* hist, int m, int e) {
  int w[kMaxNgram];
#pragma unroll
  for (int t = 0; t < kMaxNgram; ++t) w[t] = t < m ? hist[e - m + 1 + t] : 0;
  unsigned sl = gram_hash(w, m) & mask;
  for (unsigned probe = 0; probe <= mask; ++probe, sl = (sl + 1) & mask) {
    int* slot = tab + (size_t)stride * sl;
    int r = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (r < 0) {
      r = atomicCAS(slot, -1, e);
      if (r < 0) {
        atomicMax(slot + 1, e);
#pragma unroll
        for (int t = 0; t < kMaxNgram; ++t)
          if (t < m) slot[2 + t] = w[t];
        return;
      }
    }
    if (r == e || gram_ends_at(hist, r, m, w)) {
      atomicMax(slot + 1, e);
      return;
    }
  }
}
// Latest end position of gram w[0 .. m) in the table, -1 if absent: one
// slot read per probe (the key's tokens are inline). Runs in a launch after
// the inserts, so plain loads see them.
template <int SI>
__device__ int ngram_lookup(const int* tab, unsigned mask, int m, const int (&w)[kMaxNgram]) {
  unsigned sl = gram_hash(w, m) & mask;
  for (unsigned probe = 0; probe <= mask; ++probe, sl = (sl + 1) & mask) {
    const int4* slot = reinterpret_cast<const int4*>(tab + (size_t)SI * sl);
    int v[SI];
#pragma unroll
    for (int q = 0; q < SI / 4; ++q) {
      const int4 x = slot[q];
      v[4 * q] = x.x;
      v[4 * q + 1] = x.y;
      v[4 * q + 2] = x.z;
      v[4 * q + 3] = x.w;
    }
    if (v[0] < 0) return -1;
    bool eq = true;
#pragma unroll
    for (int t = 0; t < kMaxNgram; ++t)
      if (t < m) eq &= v[2 + t] == w[t];
    if (eq) return v[1];
  }
  return -1;
}

// Index work carried by the top-k launch (table == nullptr: none).
struct IndexInsert {
  int* table;
  const int* len;
  const int* history;
  const int* hist_len;
  int hist_cap, m, slots_log2, groups;
};

// Workgroup g of sequence b's insert groups adds the grams ending at its share
// of positions [max(len[b], m-1), history_len[b]). A history cut back below
// the covered length is re-indexed from position 0 by group 0 alone (the
// other groups leave it): clear, fence, insert.
__device__ void index_insert_group(const IndexInsert& ix, int b, int g) {
  const int L = ix.hist_len[b];
  if (L < 0 || L > ix.hist_cap) return;  // the layout kernel reports it
  const int cur = ix.len[b];
  const bool rebuild = L < cur;
  if (rebuild && g != 0) return;
  const unsigned mask = (1u << ix.slots_log2) - 1u;
  const int stride = slot_ints(ix.m);
  int* tab = ix.table + ((size_t)b << ix.slots_log2) * stride;
  const int* hist = ix.history + (size_t)b * ix.hist_cap;
  const int tid = (int)threadIdx.x;
  int first = max(cur, ix.m - 1), step = ix.groups * kTopThreads, off = g * kTopThreads;
  if (rebuild) {
    for (size_t i = (size_t)tid; i < (size_t)stride * ((size_t)mask + 1); i += kTopThreads) tab[i] = -1;
    __threadfence();
    __syncthreads();
    first = ix.m - 1;
    step = kTopThreads;
    off = 0;
  }
  for (int e = first + off + tid; e < L; e += step) ngram_insert(tab, mask, stride, hist, ix.m, e);
}

struct TreeArgs {
  const unsigned long long* part;
  int split, kk;
  bool bf16;  // the keys come from bf16 logits (the merge may use 32-bit keys)
  const int* history;
  int hist_cap;
  const int* hist_len;
  TreeParams p;
  int T;
  int* best_g;  // [B][kMaxTreeGuesses+1] latest match end per query ([0] query 1, [1+r] guess r)
  int* top_g;   // [B][kMaxTreeGuesses+1] x1 then the guesses
  int* tokens;
  int* parent;
  int* n_nodes;
  int* status;
  const int* ix_table;  // indexed build: the index and the length it covers
  int* ix_len;
  int ix_slots_log2;
};

// The split lists of sequence b (split * kk keys) merged by wave 0 into
// top[0 .. kk), with E keys per lane (64 E >= split * kk).
// bf16 logits: the keys' value bits are the 16 order-preserving bits of a
// bf16 number, and among equal values a lower list position (split, then
// rank in the split) is a lower vocabulary index. So the 32-bit key
// (value bits << 16 | 0xffff - position) orders the entries as the 64-bit
// keys do, and the rounds run on 32-bit compares and exchanges; the lane
// holding each winner writes its 64-bit key.
template <int E>
__device__ void merge_top_e(const TreeArgs& a, int b, unsigned long long* top) {
  unsigned long long mine[E];
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = lane + 64 * e;  // entry i of split*kk
    mine[e] = i < a.split * a.kk ? a.part[((size_t)b * a.split + i / a.kk) * (kMaxTreeGuesses + 1) + i % a.kk]
                                 : 0ull;
  }
  if (!a.bf16) {
    select_top_wave<E>(mine, a.kk, top);
    return;
  }
  static_assert(kMaxTreeSplit * (kMaxTreeGuesses + 1) <= 0x10000, "list positions fit 16 bits");
  unsigned m32[E];
#pragma unroll
  for (int e = 0; e < E; ++e)
    m32[e] = mine[e] ? ((unsigned)(mine[e] >> 48) << 16) | (0xffffu - (unsigned)(lane + 64 * e)) : 0u;
  unsigned bound = ~0u;
  for (int j = 0; j < a.kk; ++j) {
    unsigned best = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (m32[e] < bound) best = max(best, m32[e]);
    best = wave_max32(best);
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (best != 0u && m32[e] == best) top[j] = mine[e];
    if (best == 0u && lane == 0) top[j] = 0ull;
    bound = best;
  }
}
// Every selection round scans all E keys of a lane, so E follows the actual
// list length (a 128k vocabulary with 16 keys per split needs 8, not 32).
__device__ void merge_top(const TreeArgs& a, int b, unsigned long long* top) {
  if ((threadIdx.x >> 6) != 0) return;
  static_assert(kMaxTreeSplit * (kMaxTreeGuesses + 1) <= 64 * 32, "merge list fits 32 keys per lane");
  const int n = a.split * a.kk;
  if (n <= 64 * 4)
    merge_top_e<4>(a, b, top);
  else if (n <= 64 * 8)
    merge_top_e<8>(a, b, top);
  else if (n <= 64 * 16)
    merge_top_e<16>(a, b, top);
  else
    merge_top_e<32>(a, b, top);
}

// grid: B workgroups: sizes the branches, then writes one node per thread.
// INDEXED: the queries are answered here from the index (no scan launch).
template <bool INDEXED>
__global__ void __launch_bounds__(kTopThreads) tree_layout_kernel(TreeArgs a) {
  const int b = blockIdx.x;
  __shared__ int br_first[kMaxTreeGuesses + 2];
  __shared__ int best[kMaxTreeGuesses + 1];
  __shared__ int topt[kMaxTreeGuesses + 1];
  __shared__ unsigned long long top[kMaxTreeGuesses + 1];
  __shared__ int n_used;
  const int tid = (int)threadIdx.x;
  const int T = a.T, k = a.p.k;
  const int L = a.hist_len[b];
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
  const int n = L + 1;
  const int* hist = a.history + (size_t)b * a.hist_cap;
  if (INDEXED) {
    // tid 0: query 1 = seq[n-m .. n-1]; tid 1+r: query 2 = seq[n-m+1 .. n-1] + guess r.
    // The history part is requested before the merge; x1 and the guess after it.
    const int m = a.p.m;
    const int lead = tid == 0 ? m : m - 1;  // tokens taken from the sequence's end
    int w[kMaxNgram];
    if (tid <= k) {
#pragma unroll
      for (int t = 0; t < kMaxNgram; ++t) {
        const int j = n - lead + t;
        w[t] = t < lead && j >= 0 && j < L ? hist[j] : 0;
      }
    }
    merge_top(a, b, top);  // wave 0, which holds lanes 0 .. k
    __syncthreads();
    if (tid <= k) {
      const int x1t = (int)key_index(top[0]);
      const int tk = (int)key_index(top[tid]);
#pragma unroll
      for (int t = 0; t < kMaxNgram; ++t) {
        if (t < lead && n - lead + t == L) w[t] = x1t;
        if (t == lead) w[t] = tk;
      }
      const unsigned mask = (1u << a.ix_slots_log2) - 1u;
      int r = -1;
      if (lead <= n) {
        if (slot_ints(m) == 8)
          r = ngram_lookup<8>(a.ix_table + ((size_t)b << a.ix_slots_log2) * 8, mask, m, w);
        else
          r = ngram_lookup<16>(a.ix_table + ((size_t)b << a.ix_slots_log2) * 16, mask, m, w);
      }
      best[tid] = r;
      topt[tid] = tk;
    }
    if (tid == 0) a.ix_len[b] = L;  // the probes above read the history, not the length
  } else if (tid <= k) {
    best[tid] = a.best_g[b * (kMaxTreeGuesses + 1) + tid];
    topt[tid] = a.top_g[b * (kMaxTreeGuesses + 1) + tid];
  }
  __syncthreads();
  const int x1 = topt[0];
  auto seq_at = [&](int j) { return j < L ? hist[j] : x1; };
  if (tid == 0) {
    int used = 1;  // node 0 = x1
    const int c1 = best[0] >= 0 ? min(a.p.keep_first, n - 1 - best[0]) : 0;
    br_first[0] = used;
    used += c1;
    for (int r = 0; r < k; ++r) {
      br_first[1 + r] = used;
      used += 1 + (best[1 + r] >= 0 ? min(a.p.keep[r], n - 1 - best[1 + r]) : 0);
    }
    br_first[k + 1] = used;
    n_used = min(used, T);
    a.n_nodes[b] = n_used;
  }
  __syncthreads();
  for (int i = tid; i < T; i += kTopThreads) {
    int tv = -1, pv = 0;
    if (i == 0) {
      tv = x1;
      pv = -1;
    } else if (i < n_used) {
      int br = 0;
      while (i >= br_first[br + 1]) ++br;  // br_first is non-decreasing; i < br_first[k + 1]
      const int o = i - br_first[br];
      if (br == 0) {
        tv = seq_at(best[0] + 1 + o);
        pv = o == 0 ? 0 : i - 1;
      } else if (o == 0) {
        tv = topt[br];
        pv = 0;
      } else {
        tv = seq_at(best[br] + o);
        pv = i - 1;
      }
    }
    tok_out[i] = tv;
    par_out[i] = pv;
  }
}

// grid: B*split workgroups (plus B*ix.groups index-insert workgroups for the
// indexed build). Each wave selects the kk largest of its 1024 keys, then
// wave 0 selects the kk largest of the four lists. Workgroup 0 of a sequence
// also resets that sequence's match slots for the scan (best_g, absent on the
// indexed build).
template <bool BF16>
__global__ void __launch_bounds__(kTopThreads) topk_partial_kernel(const void* logits, int V, int B, int split,
                                                                   int kk, unsigned long long* part, int* best_g,
                                                                   IndexInsert ix) {
  __shared__ unsigned long long wave_top[kTopThreads / 64][kMaxTreeGuesses + 1];
  __shared__ unsigned wave_top32[kTopThreads / 64][kMaxTreeGuesses + 1];
  if (blockIdx.x >= (unsigned)(B * split)) {  // index-insert workgroups (indexed build only)
    const int i = (int)blockIdx.x - B * split;
    index_insert_group(ix, i / ix.groups, i % ix.groups);
    return;
  }
  const int b = blockIdx.x / split, s = blockIdx.x % split;
  const int lo = s * kTopChunk;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (best_g && s == 0 && threadIdx.x < kMaxTreeGuesses + 1) best_g[b * (kMaxTreeGuesses + 1) + threadIdx.x] = -1;
  if (BF16) {
    unsigned mine[kTopEPT];
#pragma unroll
    for (int e = 0; e < kTopEPT; ++e) {
      const int local = wv * (64 * kTopEPT) + lane + e * 64;
      const int i = lo + local;
      mine[e] = i < V ? slice_key(static_cast<const unsigned short*>(logits)[(size_t)b * V + i], local) : 0u;
    }
    select_top_wave32<kTopEPT>(mine, kk, wave_top32[wv]);
  } else {
    unsigned long long mine[kTopEPT];
#pragma unroll
    for (int e = 0; e < kTopEPT; ++e) {
      const int i = lo + wv * (64 * kTopEPT) + lane + e * 64;
      mine[e] = i < V ? make_key(static_cast<const float*>(logits)[(size_t)b * V + i], (unsigned)i) : 0ull;
    }
    select_top_wave<kTopEPT>(mine, kk, wave_top[wv]);
  }
  __syncthreads();
  constexpr int E2 = (kTopThreads / 64) * (kMaxTreeGuesses + 1) / 64;
  unsigned long long* out = part + ((size_t)b * split + s) * (kMaxTreeGuesses + 1);
  if (wv == 0) {
    if (BF16) {  // the four lists hold slice keys of the same slice: still 32-bit
      unsigned m2[E2];
#pragma unroll
      for (int e = 0; e < E2; ++e) {
        const int i = lane + 64 * e;  // entry i of the (kTopThreads/64) lists of kk
        m2[e] = i < (kTopThreads / 64) * kk ? wave_top32[i / kk][i % kk] : 0u;
      }
      unsigned* fin = wave_top32[0];  // lane 0 writes winner j after every lane has read entry j
      select_top_wave32<E2>(m2, kk, fin);
      if (lane < kk) out[lane] = slice_key_to_key(fin[lane], lo);
    } else {
      unsigned long long m2[E2];
#pragma unroll
      for (int e = 0; e < E2; ++e) {
        const int i = lane + 64 * e;
        m2[e] = i < (kTopThreads / 64) * kk ? wave_top[i / kk][i % kk] : 0ull;
      }
      select_top_wave<E2>(m2, kk, out);
    }
  }
}

// grid: (B, scan workgroups): workgroup c looks for the queries among the grams
// ending at positions [c*kScanChunk, (c+1)*kScanChunk) of the sequence.
__global__ void __launch_bounds__(kTopThreads) tree_scan_kernel(TreeArgs a) {
  __shared__ unsigned long long top[kMaxTreeGuesses + 1];
  __shared__ int seqs[kScanChunk + kMaxNgram];
  const int b = blockIdx.x, c = blockIdx.y;
  const int tid = (int)threadIdx.x;
  const int k = a.p.k, m = a.p.m;
  const int L = a.hist_len[b];
  if (L < 0 || L > a.hist_cap) return;  // the layout kernel reports it
  const int n = L + 1;                   // history, then x1
  const int c0 = c * kScanChunk;
  if (c0 >= n) return;
  const int* hist = a.history + (size_t)b * a.hist_cap;
  // this chunk's tokens (and the m-1 before it) are requested before the merge
  const int lo = c0 - (m - 1);
  const int cnt = min(kScanChunk, n - c0) + (m - 1);
  constexpr int kIters = (kScanChunk + kMaxNgram + kTopThreads - 1) / kTopThreads;
  int v[kIters];
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int i = tid + it * kTopThreads, j = lo + i;
    v[it] = (i < cnt && j >= 0 && j < L) ? hist[j] : -1;
  }
  merge_top(a, b, top);
  __syncthreads();
  const int x1 = (int)key_index(top[0]);
  if (c == 0 && tid <= k) a.top_g[b * (kMaxTreeGuesses + 1) + tid] = (int)key_index(top[tid]);
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int i = tid + it * kTopThreads;
    if (i < cnt) seqs[i] = lo + i == L ? x1 : v[it];
  }
  // query 1 = seq[n-m .. n-1]; query 2 = seq[n-m+1 .. n-1] + guess
  int q1r[kMaxNgram], tailr[kMaxNgram];
#pragma unroll
  for (int t = 0; t < kMaxNgram; ++t) {
    const int j1 = n - m + t, j2 = n - (m - 1) + t;
    q1r[t] = (t < m && j1 >= 0) ? (j1 < L ? hist[j1] : x1) : -1;
    tailr[t] = (t < m - 1 && j2 >= 0) ? (j2 < L ? hist[j2] : x1) : -1;
  }
  __syncthreads();
  const bool q1_possible = m <= n;
  const bool q2_possible = m - 1 <= n && k > 0;
  const int npos = min(kScanChunk, n - c0);
  int* bg = a.best_g + b * (kMaxTreeGuesses + 1);
#pragma unroll 4
  for (int it = 0; it < kScanChunk / kTopThreads; ++it) {
    const int i = tid + it * kTopThreads;
    const int p = c0 + i;  // end position of the gram; w[t] = seq[p-m+1+t]
    int w[kMaxNgram];
#pragma unroll
    for (int t = 0; t < kMaxNgram; ++t) w[t] = t < m ? seqs[i + t] : 0;
    const bool here = i < npos && p >= m - 1;
    bool e1 = here && q1_possible && p < n - 1;  // query 1 may not match itself
    bool e2 = here && q2_possible;
#pragma unroll
    for (int t = 0; t < kMaxNgram; ++t) {
      if (t < m) e1 &= w[t] == q1r[t];
      if (t < m - 1) e2 &= w[t] == tailr[t];
    }
    if (e1) atomicMax(&bg[0], p);
    if (e2) {
      int tk = w[0];
#pragma unroll
      for (int t = 1; t < kMaxNgram; ++t)
        if (t == m - 1) tk = w[t];
      for (int r = 0; r < k; ++r)
        if (tk == (int)key_index(top[1 + r])) atomicMax(&bg[1 + r], p);
    }
  }
}

}  // namespace

int topk_split_for(int V) { return (V + kTopChunk - 1) / kTopChunk; }

namespace {
TreeArgs tree_args(const Dims& d, int split, int kk, bool bf16, const int* history, int hist_cap,
                   const int* hist_len, const TreeParams& p, const unsigned long long* part, int* best_g, int* top_g,
                   int* tokens, int* parent, int* n_nodes, int* status) {
  TreeArgs a;
  a.part = part;
  a.split = split;
  a.kk = kk;
  a.bf16 = bf16;
  a.history = history;
  a.hist_cap = hist_cap;
  a.hist_len = hist_len;
  a.p = p;
  a.T = d.T;
  a.best_g = best_g;
  a.top_g = top_g;
  a.tokens = tokens;
  a.parent = parent;
  a.n_nodes = n_nodes;
  a.status = status;
  a.ix_table = nullptr;
  a.ix_len = nullptr;
  a.ix_slots_log2 = 0;
  return a;
}

hipError_t launch_topk(bool logits_bf16, dim3 grid, hipStream_t s, const void* logits, int V, int B, int split,
                       int kk, unsigned long long* part, int* best_g, const IndexInsert& ix) {
  if (logits_bf16)
    hipLaunchKernelGGL(topk_partial_kernel<true>, grid, dim3(kTopThreads), 0, s, logits, V, B, split, kk, part,
                       best_g, ix);
  else
    hipLaunchKernelGGL(topk_partial_kernel<false>, grid, dim3(kTopThreads), 0, s, logits, V, B, split, kk, part,
                       best_g, ix);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_build_tree(const Dims& d, const void* logits, int V, bool logits_bf16, const int* history,
                             int hist_cap, const int* hist_len, const TreeParams& p, unsigned long long* part,
                             int* aux, int* tokens, int* parent, int* n_nodes, int* status, hipStream_t s) {
  const int split = topk_split_for(V);
  const int kk = p.k + 1;
  int* best_g = aux;
  int* top_g = aux + (size_t)d.B * (kMaxTreeGuesses + 1);
  const TreeArgs a = tree_args(d, split, kk, logits_bf16, history, hist_cap, hist_len, p, part, best_g, top_g,
                               tokens, parent, n_nodes, status);
  const IndexInsert none = {};
  hipError_t e = launch_topk(logits_bf16, dim3(d.B * split), s, logits, V, d.B, split, kk, part, best_g, none);
  if (e != hipSuccess) return e;
  // positions 0 .. hist_cap (the longest sequence is the full history plus x1)
  const int chunks = (hist_cap + 1 + kScanChunk - 1) / kScanChunk;
  hipLaunchKernelGGL(tree_scan_kernel, dim3(d.B, chunks), dim3(kTopThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tree_layout_kernel<false>, dim3(d.B), dim3(kTopThreads), 0, s, a);
  return hipGetLastError();
}

// Two launches: the top-k workgroups with the index-insert workgroups, then
// per sequence the merge of the split lists, the index probes and the layout.
hipError_t launch_build_tree_indexed(const Dims& d, const void* logits, int V, bool logits_bf16, const int* history,
                                     const int* hist_len, const TreeParams& p, unsigned long long* part,
                                     const NgramIndex& ix, int* tokens, int* parent, int* n_nodes, int* status,
                                     hipStream_t s) {
  const int split = topk_split_for(V);
  const int kk = p.k + 1;
  IndexInsert ins;
  ins.table = ix.table;
  ins.len = ix.len;
  ins.history = history;
  ins.hist_len = hist_len;
  ins.hist_cap = ix.cap;
  ins.m = ix.m;
  ins.slots_log2 = ix.slots_log2;
  ins.groups = std::min(kMaxInsertGroups, std::max(1, (ix.cap + kInsertChunk - 1) / kInsertChunk));
  hipError_t e = launch_topk(logits_bf16, dim3(d.B * split + d.B * ins.groups), s, logits, V, d.B, split, kk, part,
                             nullptr, ins);
  if (e != hipSuccess) return e;
  TreeArgs a = tree_args(d, split, kk, logits_bf16, history, ix.cap, hist_len, p, part, nullptr, nullptr, tokens,
                         parent, n_nodes, status);
  a.ix_table = ix.table;
  a.ix_len = ix.len;
  a.ix_slots_log2 = ix.slots_log2;
  hipLaunchKernelGGL(tree_layout_kernel<true>, dim3(d.B), dim3(kTopThreads), 0, s, a);
  return hipGetLastError();
}

int ngram_slot_ints(int m) { return slot_ints(m); }

namespace {
// Sets the slots of sequence seq (seq < 0: of sequence blockIdx.y) to -1 and
// the length it covers to 0; n = the ints of one sequence's table.
__global__ void ngram_reset_kernel(int* table, int* len, size_t n, int seq) {
  const int b = seq >= 0 ? seq : (int)blockIdx.y;
  int* tab = table + (size_t)b * n;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    tab[i] = -1;
  if (blockIdx.x == 0 && threadIdx.x == 0) len[b] = 0;
}
}  // namespace

hipError_t launch_ngram_reset(const NgramIndex& ix, int seq, hipStream_t s) {
  const size_t n = (size_t)slot_ints(ix.m) << ix.slots_log2;
  const int blocks = (int)std::min<size_t>(256, (n + 255) / 256);
  hipLaunchKernelGGL(ngram_reset_kernel, dim3(blocks, seq >= 0 ? 1 : ix.B), dim3(256), 0, s, ix.table, ix.len, n,
                     seq);
  return hipGetLastError();
}

}  // namespace hta
