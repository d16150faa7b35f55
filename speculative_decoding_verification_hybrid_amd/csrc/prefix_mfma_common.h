// Pieces of the split-KV MFMA kernel (prefix_mfma.hip): the kernel
// arguments, the LDS layouts' index maps and the copy / wait / barrier
// primitives of the LDS pipeline.
#pragma once

#include <type_traits>

#include "common.h"

namespace hta {
namespace mfma {

// Tokens per tile of the MFMA path's split (and per LDS pipeline stage).
constexpr int NK = kMfmaTileTokens;

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
  int nwg, rows_per_group, tree_tiles, tree_weight;
  float scale_log2;
  // Fused merge (fuse != 0): final out (bf16) and lse, and per (segment, row
  // group) words: seg_sync[2 i] arrivals and seg_sync[2 i + 1] departures
  // (zero between launches), seg_err[i] the segment's tree check.
  int fuse;
  void* out;
  float* lse;
  int* seg_sync;
  int* seg_err;
  unsigned slot_bytes_o, slot_bytes_l;  // slot array sizes (fused merge: buffer loads / stores)
};

// Cache policy of device-coherent accesses (sc1): stores write through to the
// point of coherence of the whole device, loads read from it, so workgroups on
// different XCDs (each with its own L2) see each other's data without
// cache-wide write-back or invalidation.
constexpr int kCpolDevice = 16;

// Raw buffer resource over `bytes` bytes at p (out-of-range accesses return 0
// or are dropped).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(const void* p, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

// XOR swizzle of the 16-byte chunks of K row r. D = 128: a row spans all 64
// banks and the swizzle is a bijection of r's low 4 bits, so the 16 rows of a
// K fragment read hit 16 different chunks. D = 64: two rows share the banks,
// and the same holds per half.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// MFMA row -> token within a 32-token tile: swap bits 2 and 3.
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
  static_assert(N >= 0 && N < 64, "vmcnt range");
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

// Score MFMAs S^T += K . Q^T. This file is compiled with MFMA results in
// VGPRs (the softmax reads them), so the compiler sees these MFMAs and
// inserts the wait states their results need; Q^T is kept in AGPRs.
__device__ __forceinline__ f32x16 mfma_s_first(const bf16x8& k, const bf16x8& q) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, q, f32x16{}, 0, 0, 0);
}
__device__ __forceinline__ void mfma_s_acc(f32x16& d, const bf16x8& k, const bf16x8& q) {
  d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, q, d, 0, 0, 0);
}

// P.V accumulation O^T += V^T . P^T with the accumulator pinned to AGPRs
// (the compiler would keep it in VGPRs between tiles and copy it into AGPRs
// before every MFMA). Its operands are V^T fragments (LDS reads, waited for
// explicitly) and bf16 probabilities written a tile earlier; the
// accumulators are only touched by VALU code after o_fence.
__device__ __forceinline__ void mfma_pv(f32x16& o, const bf16x8& v, const bf16x8& p) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(v), "v"(p));
}
// The same with the accumulator in VGPRs, as a compiler-visible MFMA (the
// compiler inserts the wait states its operands and result need).
__device__ __forceinline__ void mfma_pv_v(f32x16& o, const bf16x8& v, const bf16x8& p) {
  o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, p, o, 0, 0, 0);
}
// Keeps an accumulator in AGPRs at this point (no code).
__device__ __forceinline__ void o_tie(f32x16& o) { asm volatile("" : "+a"(o)); }
// The same with 3 wait states ahead of it, for places where the compiler may
// have just written the accumulator or an operand with VALU code (moving
// values between register files): a VALU write needs 2 before an MFMA reads
// the register.
__device__ __forceinline__ void mfma_pv_after_valu(f32x16& o, const bf16x8& v, const bf16x8& p) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(v), "v"(p));
}
// Ties an LDS-read result to the explicit wait before it: code that reads the
// value cannot be scheduled above this point (no code).
__device__ __forceinline__ void lds_tie(bf16x8& x) {
  u32x4 r = __builtin_bit_cast(u32x4, x);
  asm volatile("" : "+v"(r));
  x = __builtin_bit_cast(bf16x8, r);
}
// 24 wait states tied to one accumulator, before VALU code reads or writes
// it (or after VALU code wrote it, before the next MFMA reads it).
__device__ __forceinline__ void o_fence(f32x16& o) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(o)); }

// LDS reads of the tile loop, from inline assembly so that the compiler
// neither computes one address register per read nor inserts its own waits;
// their lgkmcnt waits are explicit and derived from the static slot
// schedule. K: one 16-byte read at a wave-uniform stage offset plus a
// per-lane address. V: one transposed 8-byte read at a per-lane base plus an
// immediate byte offset.
__device__ __forceinline__ bf16x8 lds_read_k(unsigned stage, unsigned addr) {
  u32x4 r;
  unsigned t;
  asm volatile("v_add_u32 %1, %2, %3\n\tds_read_b128 %0, %1" : "=v"(r), "=&v"(t) : "s"(stage), "v"(addr));
  return __builtin_bit_cast(bf16x8, r);
}
template <int OFF>
__device__ __forceinline__ i16x4 lds_read_v(unsigned addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return __builtin_bit_cast(i16x4, r);
}
// s_waitcnt lgkmcnt(N) only (N clamped to the 4-bit field: waiting for
// fewer outstanding operations than needed is always safe).
template <int N>
__device__ __forceinline__ void wait_lgkm() {
  constexpr int n = N < 0 ? 0 : N > 15 ? 15 : N;
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (n << 8) | (3 << 14));
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Keeps a Q fragment in AGPRs from here on (no code).
__device__ __forceinline__ void q_tie(bf16x8& q) { asm volatile("" : "+a"(q)); }

// The same copy with the LDS address formed as a wave-uniform base plus an
// immediate (one scalar add into M0).
// (s_add_u32 writes SCC, hence the clobber.)
template <int LOFF>
__device__ __forceinline__ void copy16_to_lds_at(const void* base, unsigned off, unsigned lds_base) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(lds_base), "i"(LOFF)
               : "memory", "m0", "scc");
}

// Two floats rounded to bf16 (round to nearest even) and packed, from inline
// assembly so the conversion stays in the slot it is written in.
__device__ __forceinline__ unsigned cvt_pk_bf16(float lo, float hi) {
  unsigned r;
  asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
  return r;
}

__device__ __forceinline__ unsigned lds_addr(const unsigned short* p) {
  return (unsigned)(size_t)(const __attribute__((address_space(3))) unsigned short*)p;
}

}  // namespace mfma
}  // namespace hta
