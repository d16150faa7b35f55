// Device-side helpers shared by the kernels of libhta.
//
// Split-KV work decomposition (used by the prefix kernels and the merge
// kernel, which must agree exactly). The cached part of every (sequence b,
// KV head g) pair -- a "segment" -- is cut into tiles of NK tokens; when the
// tree part is fused in, each segment gets one more tile holding its tree
// tokens (under the ancestor mask), placed last. All tiles of all segments
// are laid end to end (segments in order s = b*Hkv+g) and split into NWG
// nearly equal contiguous ranges, one per workgroup, so ragged prefixes still
// give every compute unit the same amount of KV to stream. A workgroup whose
// range crosses segment boundaries produces one partial result per segment
// piece; the partial of (workgroup w, segment s) lives in slot w + s, which
// is unique because ranges are contiguous and ordered. The merge finds the
// workgroups that cover a segment by inverting the split, so no index list
// is ever stored.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hta {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kStatusBadTree = 1;
constexpr int kStatusBadPrefix = 2;
constexpr int kStatusCommitOverflow = 4;
constexpr int kStatusBadPath = 8;
constexpr int kStatusMergeTimeout = 16;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float bf16_bits_to_float(unsigned int bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ float load_elem(const float* p) { return *p; }
__device__ __forceinline__ float load_elem(const unsigned short* p) {
  return bf16_bits_to_float(*p);
}

// Round-to-nearest-even float -> bf16 bits (the hardware conversion on gfx950).
__device__ __forceinline__ unsigned short float_to_bf16_bits(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(unsigned short, b);
}

__device__ __forceinline__ void store_elem(float* p, float x) { *p = x; }
__device__ __forceinline__ void store_elem(unsigned short* p, float x) { *p = float_to_bf16_bits(x); }

// Valid cached length of sequence b; an out-of-range prefix_len counts as empty
// here (the merge kernel reports it and fills the sequence's rows with NaN).
__device__ __forceinline__ int valid_prefix(const int* prefix_len, int b, int Lcap) {
  int L = prefix_len[b];
  return (L < 0 || L > Lcap) ? 0 : L;
}

__device__ __forceinline__ int tiles_of(int L, int NK) { return (L + NK - 1) / NK; }

// Tiles of each segment of sequence b in the split: its prefix tiles, its
// tree_tiles tree tiles, then (tree_weight - 1) * tree_tiles empty tiles that
// stand for the extra cost of the tree tiles (ancestor words, masks), so the
// workgroup holding them gets fewer prefix tiles. Kernels skip the empty
// tiles; a segment's last real tile is at index prefix tiles + tree_tiles - 1.
__device__ __forceinline__ int seg_tiles(const int* prefix_len, int b, int Lcap, int NK, int tree_tiles,
                                         int tree_weight = 1) {
  return tiles_of(valid_prefix(prefix_len, b, Lcap), NK) + tree_tiles * tree_weight;
}

// Tile counts and split arithmetic are 32-bit: the host keeps
// (largest possible tile count) * nwg below 2^32.
__device__ inline unsigned total_tiles(const int* prefix_len, int B, int Hkv, int Lcap, int NK,
                                       int tree_tiles, int tree_weight = 1) {
  unsigned t = 0;
  for (int b = 0; b < B; ++b) t += (unsigned)seg_tiles(prefix_len, b, Lcap, NK, tree_tiles, tree_weight);
  return t * (unsigned)Hkv;
}

// First tile (global index) owned by workgroup w of nwg.
__device__ __forceinline__ unsigned split_begin(unsigned w, unsigned nwg, unsigned TT) {
  return (w * TT) / nwg;
}

// Workgroup owning global tile x (0 <= x < TT): the largest w with split_begin(w) <= x.
__device__ __forceinline__ unsigned split_owner(unsigned x, unsigned nwg, unsigned TT) {
  return ((x + 1) * nwg - 1) / TT;
}

// Global index of the first tile of segment (b, g), and its count of real
// (non-empty) tiles.
__device__ inline void segment_tiles(const int* prefix_len, int Hkv, int Lcap, int NK, int tree_tiles,
                                     int b, int g, unsigned* first, int* count, int tree_weight = 1) {
  unsigned acc = 0;
  for (int bb = 0; bb < b; ++bb) acc += (unsigned)seg_tiles(prefix_len, bb, Lcap, NK, tree_tiles, tree_weight);
  const int nt = seg_tiles(prefix_len, b, Lcap, NK, tree_tiles, tree_weight);
  *first = acc * (unsigned)Hkv + (unsigned)(g * nt);
  *count = nt - tree_tiles * (tree_weight - 1);
}

// Walks a workgroup's tile range segment by segment.
struct SegmentWalk {
  int b, g, nt;        // current sequence, KV head, tiles per segment of b
  int L;               // valid cached length of sequence b
  unsigned seq_first;  // global index of the first tile of sequence b
};

// Positions the walk on the segment holding global tile x; false if x is past the end.
__device__ inline bool walk_start(SegmentWalk* sw, unsigned x, const int* prefix_len, int B, int Hkv,
                                  int Lcap, int NK, int tree_tiles, int tree_weight = 1) {
  unsigned first = 0;
  for (int b = 0; b < B; ++b) {
    const int L = valid_prefix(prefix_len, b, Lcap);
    const int nt = tiles_of(L, NK) + tree_tiles * tree_weight;
    const unsigned span = (unsigned)nt * (unsigned)Hkv;
    if (x < first + span) {
      sw->b = b;
      sw->nt = nt;
      sw->L = L;
      sw->seq_first = first;
      sw->g = (int)((x - first) / (unsigned)nt);
      return true;
    }
    first += span;
  }
  return false;
}

// Moves to the next segment that has tiles; false if there is none.
__device__ inline bool walk_next(SegmentWalk* sw, const int* prefix_len, int B, int Hkv, int Lcap, int NK,
                                 int tree_tiles, int tree_weight = 1) {
  if (++sw->g < Hkv) return true;
  sw->g = 0;
  sw->seq_first += (unsigned)sw->nt * (unsigned)Hkv;
  for (int b = sw->b + 1; b < B; ++b) {
    const int L = valid_prefix(prefix_len, b, Lcap);
    const int nt = tiles_of(L, NK) + tree_tiles * tree_weight;
    if (nt > 0) {
      sw->b = b;
      sw->nt = nt;
      sw->L = L;
      return true;
    }
  }
  return false;
}

// Ancestor word of tree node i from an LDS copy of its sequence's parent array:
// bit j set iff node j is i or an ancestor of i. parent[j] < j makes the walk
// end within T steps; a pointer that breaks -1 <= parent[j] < j clears *ok.
__device__ inline unsigned long long ancestor_word(const int* par, int i, bool* ok) {
  unsigned long long m = 0ull;
  int j = i;
  while (j >= 0) {
    const int pj = par[j];
    if (pj < -1 || pj >= j) {
      *ok = false;
      return 1ull << i;
    }
    m |= 1ull << j;
    j = pj;
  }
  return m;
}

// XCD-aware workgroup index: MI355X hands consecutive block ids to its 8
// XCDs in turn, so give XCD x a contiguous run of work ranges; neighbouring
// ranges share a KV head and hence its queries in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
  if ((nwg & 7) != 0) return bid;
  return (bid & 7) * (nwg >> 3) + (bid >> 3);
}

}  // namespace hta
