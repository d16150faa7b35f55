// Device-side helpers shared by the kernels of libhta.
//
// Split-KV work decomposition (used by the prefix kernels and the merge
// kernel, which must agree exactly). The cached part of every (sequence b,
// KV head g) pair -- a "segment" -- is cut into tiles of NK tokens. All
// tiles of all segments are laid end to end (segments in order s = b*Hkv+g)
// and split into NWG nearly equal contiguous ranges, one per workgroup, so
// ragged prefixes still give every compute unit the same amount of KV to
// stream. A workgroup whose range crosses segment boundaries produces one
// partial result per segment piece; the partial of (workgroup w, segment s)
// lives in slot w + s, which is unique because ranges are contiguous and
// ordered. The merge finds the workgroups that cover a segment by inverting
// the split, so no index list is ever stored.
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

struct SplitInfo {
  int64_t total_tiles;  // tiles over all segments
};

__device__ __forceinline__ int tiles_of(int L, int NK) { return (L + NK - 1) / NK; }

__device__ inline int64_t total_tiles(const int* prefix_len, int B, int Hkv, int Lcap, int NK) {
  int64_t t = 0;
  for (int b = 0; b < B; ++b) t += tiles_of(valid_prefix(prefix_len, b, Lcap), NK);
  return t * Hkv;
}

// First tile (global index) owned by workgroup w of nwg.
__device__ __forceinline__ int64_t split_begin(int64_t w, int64_t nwg, int64_t TT) {
  return (w * TT) / nwg;
}

// Workgroup owning global tile x (0 <= x < TT).
__device__ __forceinline__ int64_t split_owner(int64_t x, int64_t nwg, int64_t TT) {
  return ((x + 1) * nwg - 1) / TT;
}

// Global index of the first tile of segment (b, g), and its tile count.
__device__ inline void segment_tiles(const int* prefix_len, int Hkv, int Lcap, int NK, int b, int g,
                                     int64_t* first, int* count) {
  int64_t acc = 0;
  for (int bb = 0; bb < b; ++bb) acc += tiles_of(valid_prefix(prefix_len, bb, Lcap), NK);
  int nt = tiles_of(valid_prefix(prefix_len, b, Lcap), NK);
  *first = acc * Hkv + (int64_t)g * nt;
  *count = nt;
}

// XCD-aware workgroup index: MI355X hands consecutive block ids to its 8
// XCDs in turn, so give XCD x a contiguous run of work ranges; neighbouring
// ranges share a KV head and hence its queries in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
  if ((nwg & 7) != 0) return bid;
  return (bid & 7) * (nwg >> 3) + (bid >> 3);
}

}  // namespace hta
