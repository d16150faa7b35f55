// Split-KV attention for bf16 layers with few query rows per KV head
// (M = G*T <= 16, D = 128 or 64): the drafter's cross-attention over the target's KV cache
// (LongSpec summary pages, §2.A "memory-efficient architecture": the draft
// model reads the target model's cache instead of keeping its own), and
// verification of very small trees. With so few rows a 32-row MFMA block would
// be mostly padding, so scores and outputs are formed with v_dot2_f32_bf16 on
// the vector ALUs and reduced across lanes with DPP. Same work split,
// fused tree tile and partial-result slots (float) as the other split-KV
// kernels (common.h). Above 8 rows the rows are split into two groups of up
// to 8 (grid.y); the two workgroups of one range run side by side on one XCD,
// so the second reads the keys and values from its L2.
//
// Layout of one wave at D = 128 (64 lanes = 4 groups of 16; at D = 64, 8
// groups of 8): lane (grp, c) loads the 16 bytes at dims 8c..8c+7 of one
// token per load, so a single 16-byte load of the wave covers 4 (8)
// consecutive tokens, fully coalesced. A unit is 8 (4) such loads, 32
// tokens, of K and of V straight into registers; the four waves of a
// workgroup take the units of their range in turn. The next unit's K is
// requested right after the scores are formed and its V right after P*V, so
// one buffer each suffices and several waves fit per SIMD. No LDS staging.
//
// Per unit: every lane forms U*MR partial dot products (8 dims each) for its
// tokens and the MR query rows, then four halving exchange stages (partners
// at lane distance 8, mirrored within 8, 2, 1; the first is skipped at
// D = 64) sum them over the lanes of a token while halving the set each lane
// keeps: afterwards lane (grp, c) holds the full scores of token slot c/2
// for rows (c&1)*MR/2 .. +MR/2-1.
// Online softmax in the log2 domain with a lazy maximum (raised only when a
// row's unit maximum exceeds it by more than 8, so p <= 2^8). The
// probabilities go through a 256-byte LDS buffer per wave as bf16 pairs of
// neighbouring token slots, which v_dot2 multiplies into the output with the
// matching V pair (two tokens' values of one dim packed by v_perm). The token
// groups' outputs and the four waves' states are combined once per piece.
#include "common.h"
#include "hta_internal.h"

namespace hta {
namespace {

constexpr int NK = kTileTokens;  // 64-token tiles of the split
constexpr int UNIT = 32;         // tokens per unit of K (and of V)
constexpr int NWAVE = 4;
constexpr float kLazy = 8.f;     // log2 units a row maximum may lag behind

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct DotArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* kt;
  const void* vt;
  const int* parent;
  const int* prefix_len;
  float* slot_o;
  float* slot_lse2;
  int* err_b;
  int* status;
  int B, Hq, Hkv, G, T, Lcap, M;
  int nwg, tree_tiles;
  float scale_log2;
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kRor4 = 0x124, kRor8 = 0x128, kHalfMirror = 0x141, kXor1 = 0xB1, kXor2 = 0x4E;

__device__ __forceinline__ float dot2(unsigned a, unsigned b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc,
                                         false);
}

__device__ __forceinline__ float dot8(const u32x4& a, const u32x4& b) {
  float acc = dot2(a[0], b[0], 0.f);
  acc = dot2(a[1], b[1], acc);
  acc = dot2(a[2], b[2], acc);
  return dot2(a[3], b[3], acc);
}

// Sum (or max) over the 4 lane groups of 16 (bits 4 and 5 of the lane).
__device__ __forceinline__ float groups_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float groups_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// One halving stage: a lane with bit h set keeps the upper half of x[0..2n),
// the other the lower half, each adding its partner's copy of the kept half.
template <int CTRL, int N>
__device__ __forceinline__ void halve(float* x, bool h) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float keep = h ? x[N + i] : x[i];
    const float send = h ? x[i] : x[N + i];
    x[i] = keep + dpp<CTRL>(send);
  }
}

// s_waitcnt immediate: wait until at most N vector-memory loads of this wave
// are in flight (the other counters left alone).
template <int N>
constexpr int vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  return (N & 15) | (((N >> 4) & 3) << 14) | (7 << 4) | (15 << 8);
}

// Lanes of one token's row: CL = D/8 lanes of 8 dims each, so one 16-byte load
// of the wave covers TPL = 64/CL consecutive tokens and a unit is U = UNIT/TPL
// loads. Lane (grp, c) = (lane / CL, lane % CL).
template <int D, int MR>
__global__ void __launch_bounds__(256) prefix_dot_kernel(DotArgs a) {
  constexpr int CL = D / 8;     // lanes per token
  constexpr int TPL = 64 / CL;  // tokens per load
  constexpr int U = UNIT / TPL;  // loads per unit
  constexpr int NV = MR / 2;    // scores per lane per unit
  static_assert(MR == 2 || MR == 4 || MR == 8, "rows per KV head");
  static_assert(D == 128 || D == 64, "head dims");
  __shared__ __align__(16) unsigned short pbuf[NWAVE][TPL][U / 2][MR][2];  // bf16 P: [wave][grp][slot pair][row][slot&1]
  __shared__ __align__(16) float red_o[NWAVE][MR][D];
  __shared__ float red_m[NWAVE][MR];
  __shared__ float red_l[NWAVE][MR];
  __shared__ int par_s[64];
  __shared__ unsigned long long anc_s[64];
  __shared__ int bad_s;

  const unsigned short* qg = static_cast<const unsigned short*>(a.q);
  const unsigned short* kg = static_cast<const unsigned short*>(a.k);
  const unsigned short* vg = static_cast<const unsigned short*>(a.v);
  const unsigned short* ktg = static_cast<const unsigned short*>(a.kt);
  const unsigned short* vtg = static_cast<const unsigned short*>(a.vt);
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: tile bases stay scalar
  const int grp = lane / CL, c = lane % CL;
  const int slot_own = c >> 1;     // token slot of this lane's scores
  const int rbase = (c & 1) * NV;  // first row of this lane's scores
  const int r0 = (int)blockIdx.y * MR;  // this workgroup's first row

  const int w = xcd_remap(blockIdx.x, a.nwg);
  const unsigned TT = total_tiles(a.prefix_len, a.B, a.Hkv, a.Lcap, NK, a.tree_tiles);
  if (TT == 0) return;
  unsigned x = split_begin(w, a.nwg, TT);
  const unsigned x_end = split_begin(w + 1, a.nwg, TT);
  if (x >= x_end) return;
  SegmentWalk sw;
  if (!walk_start(&sw, x, a.prefix_len, a.B, a.Hkv, a.Lcap, NK, a.tree_tiles)) return;

  while (true) {
    const int b = sw.b, g = sw.g;
    const unsigned s_first = sw.seq_first + (unsigned)(g * sw.nt);
    const int tile0 = (int)(x - s_first);
    const unsigned piece_end = min(x_end, s_first + (unsigned)sw.nt);
    const int ntiles = (int)(piece_end - x);
    const int L = sw.L;
    const int n_prefix = sw.nt - a.tree_tiles;
    const bool has_tree = a.tree_tiles && tile0 + ntiles > n_prefix;
    const int slot = w + b * a.Hkv + g;
    const size_t kv_off = (size_t)(b * a.Hkv + g) * (size_t)a.Lcap * D;
    const size_t kt_off = (size_t)(b * a.Hkv + g) * a.T * D;
    const unsigned short* qp = qg + (size_t)(b * a.Hq + g * a.G) * a.T * D;

    __syncthreads();  // LDS of the previous piece is no longer read
    if (has_tree) {
      if (tid == 0) bad_s = 0;
      if (tid < a.T) par_s[tid] = a.parent[(size_t)b * a.T + tid];
      __syncthreads();
      if (tid < a.T) {
        bool ok = true;
        anc_s[tid] = ancestor_word(par_s, tid, &ok);
        if (!ok) bad_s = 1;
      }
      __syncthreads();
    }

    // this group's query rows of the KV head, dims 8c..8c+7 (rows past M are
    // zero; their loads read row M-1, so that every load is issued on every
    // path and the compiler's count of loads in flight stays exact)
    u32x4 qr[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      const u32x4 v = *(const u32x4*)(qp + (size_t)min(r0 + r, a.M - 1) * D + 8 * c);
      qr[r] = r0 + r < a.M ? v : u32x4{0u, 0u, 0u, 0u};
    }

    // ancestor word of the tree node behind each of this lane's rows
    unsigned long long vis_row[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j)
      vis_row[j] = (has_tree && r0 + rbase + j < a.M) ? anc_s[(r0 + rbase + j) % a.T] : 0ull;

    float o[MR][8];
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[r][e] = 0.f;
    float m[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) m[r] = -__builtin_inff();
    float l[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) l[j] = 0.f;

    // this wave's units: units wv, wv+4, ... of the piece (two 32-token units per tile)
    const int nu = 2 * ntiles;
    const int nun = nu > wv ? (nu - wv + NWAVE - 1) / NWAVE : 0;
    auto unit_of = [&](int i) { return wv + NWAVE * i; };  // piece unit of this wave's i-th unit

    // Loads of one unit's K (or V) rows; tokens past the end repeat the last
    // valid row. Branch-free, so that the loads write straight into the
    // registers the next unit reads: with a branch (or a conditional load) the
    // compiler merged the paths' results with register copies at the loop's
    // back edge, and those copies waited for every load in flight, so no load
    // ever overlapped the next unit.
    auto load_rows = [&](int pu, const unsigned short* base_tree, const unsigned short* base_cache, u32x4* dst) {
      const int ti = tile0 + (pu >> 1);
      const bool tree = ti >= n_prefix;
      const unsigned short* src = tree ? base_tree + kt_off : base_cache + kv_off + (size_t)ti * NK * D;
      const int nvalid = tree ? a.T : min(NK, L - ti * NK);  // >= 1 for every tile that exists
      const char* sb = reinterpret_cast<const char*>(src);
      const int t0 = (pu & 1) * UNIT;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const unsigned tk = (unsigned)min(t0 + TPL * u + grp, nvalid - 1);
        dst[u] = *(const u32x4*)(sb + (tk * D + 8u * c) * 2u);
      }
    };

    // K and V of one unit live in registers; the next unit's K is requested as
    // soon as the scores are formed, its V as soon as P*V is done (the last
    // unit requests itself again, which keeps the loop free of branches around
    // the loads).
    u32x4 kr[U], vr[U];
    if (nun > 0) {
      load_rows(unit_of(0), ktg, kg, kr);
      load_rows(unit_of(0), vtg, vg, vr);
    }
    // In flight at the top of unit i: K(i), then V(i) (U loads each, in that
    // order); K(i+1) goes out after the scores, V(i+1) after P*V. So each use
    // waits until at most U loads are left (explicit, because the compiler's
    // own count at the loop head is a full drain).
    for (int i = 0; i < nun; ++i) {
      __builtin_amdgcn_s_waitcnt(vm_wait<U>());  // K(i) has landed; V(i) may still be in flight
      __builtin_amdgcn_sched_barrier(0);
      const int pu = unit_of(i);
      const int ti = tile0 + (pu >> 1);
      const bool tree = ti >= n_prefix;
      const int nvalid = tree ? a.T : min(NK, L - ti * NK);
      // partial scores x[u*MR + r] over this lane's 8 dims
      float xs[U * MR];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < MR; ++r) xs[u * MR + r] = dot8(qr[r], kr[u]);
      // keep the scheduler from hoisting the next loads above their registers' last use
      // (that would need a second buffer and halve the waves per SIMD)
      __builtin_amdgcn_sched_barrier(0);
      load_rows(unit_of(min(i + 1, nun - 1)), ktg, kg, kr);
      // (at D = 64 the 8 lanes of a token start at the second stage, with
      // the same 4 * MR values left as after the first stage at D = 128)
      if constexpr (CL == 16) halve<kRor8, 4 * MR>(xs, (c >> 3) & 1);
      halve<kHalfMirror, 2 * MR>(xs, (c >> 2) & 1);
      halve<kXor2, MR>(xs, (c >> 1) & 1);
      halve<kXor1, MR / 2>(xs, c & 1);
      // xs[j], j < NV: score of token slot slot_own, row rbase + j
      const int tk = (pu & 1) * UNIT + TPL * slot_own + grp;
      float s[NV], um[NV];
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const bool seen = r0 + rbase + j < a.M && tk < nvalid && (!tree || ((vis_row[j] >> tk) & 1ull));
        s[j] = seen ? xs[j] * a.scale_log2 : -__builtin_inff();
        float v = s[j];
        v = fmaxf(v, dpp<kRor4>(v));
        v = fmaxf(v, dpp<kRor8>(v));
        v = fmaxf(v, dpp<kXor2>(v));
        um[j] = groups_max(v);
      }
      // every lane learns the unit maxima of all MR rows (the other half from lane c^1)
      float umax[MR];
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const float other = dpp<kXor1>(um[j]);
        umax[j] = (c & 1) ? other : um[j];
        umax[NV + j] = (c & 1) ? um[j] : other;
      }
      bool raise = false;
#pragma unroll
      for (int r = 0; r < MR; ++r) raise |= umax[r] > m[r] + kLazy;
      if (raise) {  // same decision in every lane
#pragma unroll
        for (int r = 0; r < MR; ++r) {
          const float mn = fmaxf(m[r], umax[r]);
          const float alpha = m[r] == -__builtin_inff() ? 0.f : fast_exp2(m[r] - mn);
          m[r] = mn;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[r][e] *= alpha;
          if (r < NV) l[r] *= (c & 1) ? 1.f : alpha;
          else l[r - NV] *= (c & 1) ? alpha : 1.f;
        }
      }
      // probabilities of this lane's scores, to LDS as bf16
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const float mr = (c & 1) ? m[NV + j] : m[j];
        const float p = mr == -__builtin_inff() ? 0.f : fast_exp2(s[j] - mr);
        l[j] += p;
        pbuf[wv][grp][slot_own >> 1][rbase + j][slot_own & 1] = float_to_bf16_bits(p);
      }
      // the other lanes of the wave wrote their P before these reads (LDS
      // executes one wave's accesses in order; the fence keeps the compiler's)
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_s_waitcnt(vm_wait<U>());  // V(i) has landed; K(i+1) may still be in flight
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int pr = 0; pr < U / 2; ++pr) {
        // P of slots 2pr, 2pr+1 for every row, as bf16x2
        unsigned pp[MR];
        if (MR >= 4) {
#pragma unroll
          for (int r = 0; r < MR; r += 4) {
            const u32x4 t4 = *(const u32x4*)&pbuf[wv][grp][pr][r][0];
#pragma unroll
            for (int e = 0; e < 4; ++e) pp[(r + e) % MR] = t4[e];
          }
        } else {
          const u32x2 t2 = *(const u32x2*)&pbuf[wv][grp][pr][0][0];
          pp[0] = t2[0];
          pp[MR - 1] = t2[1];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // dims 2i and 2i+1 of slots 2pr and 2pr+1 (low half = slot 2pr)
          const unsigned lo = __builtin_amdgcn_perm(vr[2 * pr + 1][i], vr[2 * pr][i], 0x05040100u);
          const unsigned hi = __builtin_amdgcn_perm(vr[2 * pr + 1][i], vr[2 * pr][i], 0x07060302u);
#pragma unroll
          for (int r = 0; r < MR; ++r) {
            o[r][2 * i] = dot2(lo, pp[r], o[r][2 * i]);
            o[r][2 * i + 1] = dot2(hi, pp[r], o[r][2 * i + 1]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      load_rows(unit_of(min(i + 1, nun - 1)), vtg, vg, vr);
      // the next unit's P writes come after these reads
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }

    // combine: groups within the wave, then the waves through LDS
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      float v = l[j];
      v += dpp<kRor4>(v);
      v += dpp<kRor8>(v);
      v += dpp<kXor2>(v);
      l[j] = groups_sum(v);
    }
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (CL == 8) o[r][e] += dpp<kRor8>(o[r][e]);  // lane bit 3 is a token group here
        o[r][e] = groups_sum(o[r][e]);
      }
    if (grp == 0) {
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        *(f32x4*)&red_o[wv][r][8 * c] = f32x4{o[r][0], o[r][1], o[r][2], o[r][3]};
        *(f32x4*)&red_o[wv][r][8 * c + 4] = f32x4{o[r][4], o[r][5], o[r][6], o[r][7]};
      }
      if (c < 2) {
#pragma unroll
        for (int j = 0; j < NV; ++j) red_l[wv][rbase + j] = l[j];
      }
      if (c == 0) {
#pragma unroll
        for (int r = 0; r < MR; ++r) red_m[wv][r] = m[r];
      }
    }
    __syncthreads();
    for (int idx = tid; idx < MR * D; idx += 256) {
      const int r = idx / D, d = idx % D;
      if (r0 + r >= a.M) continue;
      float ms = -__builtin_inff();
#pragma unroll
      for (int q = 0; q < NWAVE; ++q) ms = fmaxf(ms, red_m[q][r]);
      float lt = 0.f, ot = 0.f;
#pragma unroll
      for (int q = 0; q < NWAVE; ++q) {
        const float f = red_m[q][r] == -__builtin_inff() ? 0.f : fast_exp2(red_m[q][r] - ms);
        lt += f * red_l[q][r];
        ot += f * red_o[q][r][d];
      }
      a.slot_o[((size_t)slot * a.M + r0 + r) * D + d] = lt > 0.f ? ot / lt : 0.f;
      if (d == 0) a.slot_lse2[(size_t)slot * a.M + r0 + r] = lt > 0.f ? ms + fast_log2(lt) : -__builtin_inff();
    }
    if (has_tree && g == 0 && tid == 0) {
      a.err_b[b] = bad_s;
      if (bad_s) atomicOr(a.status, kStatusBadTree);
    }

    x = piece_end;
    if (x >= x_end) break;
    if (!walk_next(&sw, a.prefix_len, a.B, a.Hkv, a.Lcap, NK, a.tree_tiles)) break;
  }
}

typedef void (*KernelFn)(DotArgs);

// Rows per workgroup for M rows in all (two groups of up to 8 above 8 rows).
template <int D>
KernelFn pick_d(int M) {
  if (M <= 2) return prefix_dot_kernel<D, 2>;
  if (M <= 4) return prefix_dot_kernel<D, 4>;
  if (M <= kDotMaxRows) return prefix_dot_kernel<D, 8>;
  return nullptr;
}
KernelFn pick(int D, int M) { return D == 128 ? pick_d<128>(M) : D == 64 ? pick_d<64>(M) : nullptr; }

}  // namespace

bool prefix_dot_supported(int D, int M, bool bf16) {
  return bf16 && (D == 128 || D == 64) && M >= 1 && M <= kDotMaxRows;
}

int dot_row_groups(int M) { return M > 8 ? 2 : 1; }

int prefix_dot_occupancy(int D, int M) {
  KernelFn k = pick(D, M);
  if (!k) return 0;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(k), 256, 0) !=
      hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}

hipError_t launch_prefix_dot(const Dims& d, const PrefixLaunch& pl, const PrefixInputs& in, Slots slots,
                             int* err_b, int* status, hipStream_t s) {
  KernelFn k = pick(d.D, d.M);
  if (!k || !d.bf16 || pl.row_groups != dot_row_groups(d.M)) return hipErrorInvalidValue;
  DotArgs a;
  a.q = in.q;
  a.k = in.k_cache;
  a.v = in.v_cache;
  a.kt = in.k_tree;
  a.vt = in.v_tree;
  a.parent = in.parent;
  a.prefix_len = in.prefix_len;
  a.slot_o = static_cast<float*>(slots.o);
  a.slot_lse2 = slots.lse2;
  a.err_b = err_b;
  a.status = status;
  a.B = d.B;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.G;
  a.T = d.T;
  a.Lcap = d.Lcap;
  a.M = d.M;
  a.nwg = pl.nwg;
  a.tree_tiles = in.k_tree ? 1 : 0;
  a.scale_log2 = d.scale_log2;
  hipLaunchKernelGGL(k, dim3(pl.nwg, pl.row_groups), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hta
