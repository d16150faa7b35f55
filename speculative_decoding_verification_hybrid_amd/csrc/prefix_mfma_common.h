// Pieces shared by the split-KV MFMA kernels (prefix_mfma.hip: one 32-row
// query block per wave; prefix_mfma2.hip: two blocks per wave): the kernel
// arguments, the LDS layouts' index maps and the copy / wait / barrier
// primitives of the LDS pipeline.
#pragma once

#include "common.h"

namespace hta {
namespace mfma {

constexpr int NK = kTileTokens;
constexpr int NSTAGE = 4;

typedef short i16x4 __attribute__((ext_vector_type(4)));

struct PrefixArgs {
  const unsigned short* q;
  const unsigned short* k;
  const unsigned short* v;
  const unsigned short* kt;  // tree keys (fused tree part) or null
  const unsigned short* vt;
  const int* parent;
  const int* prefix_len;
  unsigned short* slot_o;  // bf16 partials
  float* slot_lse2;
  int* err_b;
  int* status;
  int B, Hq, Hkv, G, T, Lcap, M;
  int nwg, rows_per_group, tree_tiles;
  float scale_log2;
};

// XOR swizzle of the 16-byte chunks of K row r. D = 128: a row spans all 64
// banks and the swizzle is a bijection of r's low 4 bits, so the 16 rows of a
// K fragment read hit 16 different chunks. D = 64: two rows share the banks,
// and the same holds per half.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// MFMA row -> token within a 32-token sub-tile: swap bits 2 and 3.
__device__ __forceinline__ int kperm(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

__device__ __forceinline__ i16x4 lds_read_tr(const unsigned short* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

// Cross-half (lane l <-> l ^ 32) max and sum in VALU: the two results of the
// lane swap are this lane's value and its partner's, in some order.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(fmaxf(x, __uint_as_float(r[0])), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_waitcnt immediate that waits for vmcnt <= N only (gfx9 encoding: vmcnt
// in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maximum).
template <int N>
constexpr int vmcnt_only() {
  return (N & 15) | (((N >> 4) & 3) << 14) | (7 << 4) | (15 << 8);
}
constexpr int kLgkmZero = 15 | (7 << 4) | (3 << 14);  // lgkmcnt(0) only

// Workgroup barrier that orders LDS accesses only in the compiler: the
// hardware waits for the tile copies are the explicit ones before it (a memory
// fence here would drain every copy in flight).
__device__ __forceinline__ void tile_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One 16-byte-per-lane copy from global memory into LDS: lane i reads the 16
// bytes at base + off (base wave-uniform, in SGPRs; off a 32-bit per-lane byte
// offset) and they land at LDS byte address lds_base + 16 i. lds_base must be
// wave-uniform (it goes through M0, which needs one wait state before the
// copy). The "memory" clobber keeps the compiler from moving LDS accesses
// across the copy.
__device__ __forceinline__ void copy16_to_lds(const void* base, unsigned off, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(lds_base)
               : "memory", "m0");
}

__device__ __forceinline__ unsigned lds_addr(const unsigned short* p) {
  return (unsigned)(size_t)(const __attribute__((address_space(3))) unsigned short*)p;
}

typedef void (*KernelFn)(PrefixArgs);

// Two-block kernel instance for head dim D with nw computing waves (1..4), or null.
KernelFn prefix_mfma2_pick(int D, int nw);

}  // namespace mfma
}  // namespace hta
