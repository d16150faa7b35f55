// The drafter's sliding-window self-attention (LongSpec summary pages, §2.A
// "memory-efficient architecture": self-attention over a window of 512
// positions, so the draft model's own cache has a fixed size).
//
// The draft cache is a ring of W slots (W = the handle's kv_capacity); slot
// s holds the newest position x with x mod W = s. Before a step, pos[b]
// positions have been written; the step's Tn new tokens (positions
// pos .. pos+Tn-1) come in k_new / v_new. New token j sees the positions
// max(0, pos+j-W+1) .. pos+j: in the ring, the entries whose age
// a = (pos-1-s) mod W (0 = newest) satisfies a < pos and a <= W-2-j; among
// the new tokens, 0 .. j. window_append then writes the new tokens into the
// ring and advances pos.
//
// window_attn_kernel: grid (B*Hkv, row groups of RB rows), NWV waves. The
// keys (ring slots, then the new tokens) are cut into 64-key chunks; wave w
// takes chunks w, w+NWV, ..., and requests its first chunk's K and V before
// anything else (the layout does not depend on pos). Per chunk, lane t scores key t against the RB
// rows (float32, q staged in LDS; half a K row of loads in flight at once),
// the wave keeps an online softmax per row, and P*V reads the chunk's V with
// coalesced 16-byte loads (lane (grp, c) takes dims 8c..8c+7 of keys grp,
// grp + 64/(D/8), ...), all in flight at once; the key groups are summed at the
// end. The eight waves' states are merged in LDS.
// Cost is negligible next to the cross-attention: W*D*2*2 bytes per KV head.
#include "common.h"
#include "hta_internal.h"

namespace hta {
namespace {

constexpr int RB = 1;       // query rows per workgroup
constexpr int NWV = 12;     // waves per workgroup: a 512-slot window plus new tokens is 9 chunks
constexpr int CH = 64;      // keys per chunk

struct WindowArgs {
  const void* q;
  const void* kr;
  const void* vr;
  const void* kn;
  const void* vn;
  const int* pos;
  void* out;
  float* lse;
  int* status;
  int B, Hq, Hkv, G, Tn, W, M;
  float scale_log2;
};

// 8 consecutive elements (16-byte aligned for bf16, 32 for float), kept in
// their stored form until used (bf16: one 16-byte register quad).
template <typename TIn>
struct Raw8;
template <>
struct Raw8<unsigned short> {
  u32x4 v;
  __device__ __forceinline__ void load(const unsigned short* p) { v = *(const u32x4*)p; }
  __device__ __forceinline__ float get(int e) const {
    return __uint_as_float((e & 1) ? (v[e >> 1] & 0xffff0000u) : (v[e >> 1] << 16));
  }
};
template <>
struct Raw8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *(const f32x4*)p;
    b = *(const f32x4*)(p + 4);
  }
  __device__ __forceinline__ float get(int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

template <int D, typename TIn>
__global__ void __launch_bounds__(NWV * 64) window_attn_kernel(WindowArgs a) {
  constexpr int LPR = D / 8;     // P*V: lanes per V row (8 dims each)
  constexpr int TPL = 64 / LPR;  // P*V: keys per load of the wave
  constexpr int NVL = 64 / TPL;  // P*V: loads per chunk
  __shared__ __align__(16) float qs[RB][D];
  __shared__ float ps[NWV][RB][CH];
  __shared__ float red_o[NWV][RB][D];
  __shared__ float red_m[NWV][RB];
  __shared__ float red_l[NWV][RB];

  const int bg = blockIdx.x;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int row0 = blockIdx.y * RB;
  const int tid = (int)threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const TIn* kr = static_cast<const TIn*>(a.kr) + (size_t)bg * a.W * D;
  const TIn* vr = static_cast<const TIn*>(a.vr) + (size_t)bg * a.W * D;
  const TIn* kn = static_cast<const TIn*>(a.kn) + (size_t)bg * a.Tn * D;
  const TIn* vn = static_cast<const TIn*>(a.vn) + (size_t)bg * a.Tn * D;
  const int pc = lane % LPR, pgrp = lane / LPR;  // P*V: lane takes dims 8pc.. of keys pgrp, pgrp+TPL, ...

  // Fixed chunk layout (it does not depend on pos, so the loads can start at
  // once): ring slots 0..W-1 in 64-key chunks, then the new tokens.
  const int ring_chunks = (a.W + CH - 1) / CH;
  const int nchunks = ring_chunks + (a.Tn + CH - 1) / CH;
  auto chunk_keys = [&](int ch, const TIn** kb, const TIn** vb, int* first) {
    const bool ring = ch < ring_chunks;
    *first = (ring ? ch : ch - ring_chunks) * CH;
    *kb = ring ? kr : kn;
    *vb = ring ? vr : vn;
    return ring ? a.W : a.Tn;  // keys of that kind in memory
  };
  // this wave's chunk keys: K rows (lane = key; for float inputs the first
  // half of each row, the second half is requested after it is used), V in
  // the P*V layout (requested once the scores are formed)
  constexpr int KV8 = sizeof(TIn) == 2 ? D / 8 : D / 16;  // 8-element K pieces held at once
  Raw8<TIn> kv[KV8], vv[NVL / 2];
  auto load_k = [&](int ch, int half) {
    const TIn *kb, *vb;
    int first;
    const int n = chunk_keys(ch, &kb, &vb, &first);
    const int kk = min(first + lane, n - 1);
#pragma unroll
    for (int e = 0; e < KV8; ++e) kv[e].load(kb + (size_t)kk * D + 8 * (e + half * KV8));
  };
  auto load_v = [&](int ch, int half) {  // half of the chunk's V loads
    const TIn *kb, *vb;
    int first;
    const int n = chunk_keys(ch, &kb, &vb, &first);
#pragma unroll
    for (int u = 0; u < NVL / 2; ++u)
      vv[u].load(vb + (size_t)min(first + (u + half * NVL / 2) * TPL + pgrp, n - 1) * D + 8 * pc);
  };
  if (wv < nchunks) load_k(wv, 0);

  const int P = a.pos[b];
  const bool bad = P < 0;
  // rows row0 .. row0+RB-1 of this KV head: head g*G + r / Tn, new token r % Tn
  const TIn* qp = static_cast<const TIn*>(a.q) + (size_t)(b * a.Hq + g * a.G) * a.Tn * D;
  for (int i = tid; i < RB * D; i += NWV * 64) {
    const int r = i / D, d = i % D;
    qs[r][d] = row0 + r < a.M ? load_elem(qp + (size_t)(row0 + r) * D + d) : 0.f;
  }
  __syncthreads();

  float m[RB], l[RB], o[RB][8];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    m[r] = -__builtin_inff();
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[r][e] = 0.f;
  }
  int jrow[RB];  // new-token index of each row (-1: no such row)
#pragma unroll
  for (int r = 0; r < RB; ++r) jrow[r] = row0 + r < a.M ? (row0 + r) % a.Tn : -1;

  // ring slots that hold a position: all W once P >= W, else slots 0 .. P-1
  // (the others may hold anything: masked, and their V is never multiplied)
  const int nring = bad ? 0 : min(P, a.W);
  const int p1 = bad ? 0 : (P > 0 ? (P - 1) % a.W : 0);  // slot of the newest ring entry
  for (int ch = wv; ch < nchunks && !bad; ch += NWV) {
    if (ch != wv) load_k(ch, 0);
    const bool ring = ch < ring_chunks;
    const TIn *kb, *vb;
    int first;
    chunk_keys(ch, &kb, &vb, &first);
    const int nvalid = ring ? nring : a.Tn;  // keys that may be seen
    const int key = first + lane;
    const bool exists = key < nvalid;
    // age of a ring entry (0 = newest); it holds a position iff age < P
    const int age = ring ? (p1 - key + a.W) % a.W : 0;
    float s[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) s[r] = 0.f;
#pragma unroll
    for (int e = 0; e < D; e += 4) {
      if (KV8 * 8 < D && e == KV8 * 8) load_k(ch, 1);  // float inputs: second half of the rows
      // one 4-dim step at a time: unbounded hoisting of the q reads from LDS
      // ahead of their use would need RB*D registers
      __builtin_amdgcn_sched_barrier(0);
      float k4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) k4[i] = kv[((e + i) >> 3) % KV8].get((e + i) & 7);
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const f32x4 qv = *(const f32x4*)&qs[r][e];
        s[r] = fmaf(qv[0], k4[0], s[r]);
        s[r] = fmaf(qv[1], k4[1], s[r]);
        s[r] = fmaf(qv[2], k4[2], s[r]);
        s[r] = fmaf(qv[3], k4[3], s[r]);
      }
    }
    // materialise the scores here: sinking their FMAs into the per-row
    // selects below would pull every q read ahead of them and spill
#pragma unroll
    for (int r = 0; r < RB; ++r) asm volatile("" : "+v"(s[r]));
    load_v(ch, 0);  // in flight during the softmax reductions
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int j = jrow[r];
      const bool seen = exists && j >= 0 && (ring ? (age < P && age <= a.W - 2 - j) : key <= j);
      const float sv = seen ? s[r] * a.scale_log2 : -__builtin_inff();
      float mx = sv;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float mn = fmaxf(m[r], mx);
      const float alpha = m[r] == -__builtin_inff() ? 0.f : fast_exp2(m[r] - mn);
      m[r] = mn;
      const float p = mn == -__builtin_inff() ? 0.f : fast_exp2(sv - mn);
      float ls = p;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) ls += __shfl_xor(ls, off);
      l[r] = l[r] * alpha + ls;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[r][e] *= alpha;
      ps[wv][r][lane] = p;  // 0 for every key not seen
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < NVL; ++u) {
      if (u == NVL / 2) load_v(ch, 1);
      __builtin_amdgcn_sched_barrier(0);
      const int t = u * TPL + pgrp;
      const bool vok = first + t < nvalid;  // a slot without a position may hold NaN
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const float p = ps[wv][r][t];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[r][e] = fmaf(p, vok ? vv[u % (NVL / 2)].get(e) : 0.f, o[r][e]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }

  // sum the key groups of the P*V layout (lanes with the same dims)
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) o[r][e] += __shfl_xor(o[r][e], off);
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    if (pgrp == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) red_o[wv][r][8 * pc + e] = o[r][e];
    }
    if (lane == 0) {
      red_m[wv][r] = m[r];
      red_l[wv][r] = l[r];
    }
  }
  __syncthreads();
  for (int i = tid; i < RB * D; i += NWV * 64) {
    const int r = i / D, d = i % D;
    const int row = row0 + r;
    if (row >= a.M) continue;
    const int h = g * a.G + row / a.Tn, j = row % a.Tn;
    const size_t orow = ((size_t)(b * a.Hq + h) * a.Tn + j);
    float ov, lv;
    if (bad) {
      ov = lv = __builtin_nanf("");
    } else {
      float ms = -__builtin_inff();
#pragma unroll
      for (int w = 0; w < NWV; ++w) ms = fmaxf(ms, red_m[w][r]);
      float lt = 0.f, ot = 0.f;
#pragma unroll
      for (int w = 0; w < NWV; ++w) {
        const float f = red_m[w][r] == -__builtin_inff() ? 0.f : fast_exp2(red_m[w][r] - ms);
        lt += f * red_l[w][r];
        ot += f * red_o[w][r][d];
      }
      ov = ot / lt;  // every row sees at least its own token: lt > 0
      lv = (ms + fast_log2(lt)) * kLn2;
    }
    store_elem(static_cast<TIn*>(a.out) + orow * D + d, ov);
    if (d == 0) a.lse[orow] = lv;
  }
  if (bad && tid == 0 && g == 0 && blockIdx.y == 0) atomicOr(a.status, kStatusBadPrefix);
}

// grid: B*Hkv workgroups x 2 (K, V): new token j goes to slot (pos+j) mod W; the
// last workgroup of a sequence to arrive advances pos (every workgroup has read
// the old value by then).
__global__ void __launch_bounds__(256) window_append_kernel(const void* k_new, const void* v_new, void* k_ring,
                                                            void* v_ring, int* pos, int Hkv, int Tn, int W,
                                                            int row_bytes, unsigned* count, int* status) {
  const int bg = blockIdx.x;
  const int b = bg / Hkv;
  const int P = pos[b];
  const bool ok = P >= 0;
  if (ok) {
    const unsigned char* src = static_cast<const unsigned char*>(blockIdx.y == 0 ? k_new : v_new) +
                               (size_t)bg * Tn * row_bytes;
    unsigned char* dst = static_cast<unsigned char*>(blockIdx.y == 0 ? k_ring : v_ring) + (size_t)bg * W * row_bytes;
    const int per_row = row_bytes / 16;
    const int p0 = P % W;
    for (int u = threadIdx.x; u < Tn * per_row; u += blockDim.x) {
      const int j = u / per_row, c = u % per_row;
      const int slot = (p0 + j) % W;
      *(u32x4*)(dst + (size_t)slot * row_bytes + 16 * c) = *(const u32x4*)(src + (size_t)j * row_bytes + 16 * c);
    }
  }
  __syncthreads();  // every wave has read pos[b]
  if (threadIdx.x == 0) {
    __threadfence();
    const unsigned old = atomicAdd(&count[b], 1u);
    if (old == 2u * (unsigned)Hkv - 1u) {
      count[b] = 0;
      if (ok)
        pos[b] = P + Tn;
      else
        atomicOr(status, kStatusBadPrefix);
    }
  }
}

typedef void (*KernelFn)(WindowArgs);

KernelFn pick(int D, bool bf16) {
  if (D == 128) return bf16 ? window_attn_kernel<128, unsigned short> : window_attn_kernel<128, float>;
  if (D == 64) return bf16 ? window_attn_kernel<64, unsigned short> : window_attn_kernel<64, float>;
  return nullptr;
}

}  // namespace

hipError_t launch_window_attn(const Dims& d, const void* q, const void* k_ring, const void* v_ring,
                              const void* k_new, const void* v_new, const int* pos, void* out, float* lse,
                              int* status, hipStream_t s) {
  KernelFn k = pick(d.D, d.bf16);
  if (!k) return hipErrorInvalidValue;
  WindowArgs a;
  a.q = q;
  a.kr = k_ring;
  a.vr = v_ring;
  a.kn = k_new;
  a.vn = v_new;
  a.pos = pos;
  a.out = out;
  a.lse = lse;
  a.status = status;
  a.B = d.B;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.G;
  a.Tn = d.T;
  a.W = d.Lcap;
  a.M = d.M;
  a.scale_log2 = d.scale_log2;
  hipLaunchKernelGGL(k, dim3(d.B * d.Hkv, (d.M + RB - 1) / RB), dim3(NWV * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_window_append(const Dims& d, const void* k_new, const void* v_new, void* k_ring, void* v_ring,
                                int* pos, unsigned* count, int* status, hipStream_t s) {
  const int row_bytes = d.D * (d.bf16 ? 2 : 4);
  hipLaunchKernelGGL(window_append_kernel, dim3(d.B * d.Hkv, 2), dim3(256), 0, s, k_new, v_new, k_ring, v_ring,
                     pos, d.Hkv, d.T, d.Lcap, row_bytes, count, status);
  return hipGetLastError();
}

}  // namespace hta
