// Split-KV attention kernel on bf16 MFMA, two 32-row query blocks per wave
// (gfx950). The work split, LDS layouts and copy pipeline are those of the
// one-block kernel in prefix_mfma.hip (see its header comment); this file
// differs in how a wave's time is spent. It is compiled with MFMA results in
// VGPRs (so the scores feed the softmax without copies), except the P.V
// accumulators, which mfma_acc() keeps in AGPRs.
#include "hta_internal.h"
#include "prefix_mfma_common.h"

namespace hta {
namespace mfma {
namespace {

// P.V accumulation of the two-block kernel with the accumulator pinned to
// AGPRs (keeping the 128 accumulator registers of a wave out of the VGPR file,
// which then holds Q, K, V, S and the softmax state without spilling). The
// compiler does not see this MFMA, so the asm carries the waits it would
// insert: 2 wait states after a VALU write of an operand (every call: the
// compiler may place such a write anywhere before it), and acc_fence() (24
// wait states, tying the accumulators) before any VALU access of them.
__device__ __forceinline__ void mfma_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
template <int DB>
__device__ __forceinline__ void acc_fence(f32x16* O) {
  if constexpr (DB == 4)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(O[0]), "+a"(O[1]), "+a"(O[2]), "+a"(O[3]));
  else
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(O[0]), "+a"(O[1]));
}

// Two-block variant: one wave per SIMD (4 waves, 256 threads), each owning
// two 32-row query blocks A and B (64 rows), so every K / V fragment read
// from LDS serves 64 rows and a wave always has independent MFMA work to put
// under its softmax. Per 32-token sub-tile j of the KV stream, a wave runs
//   PV_B(j-1), S_B(j)   while the softmax of block A on S_A(j) runs,
//   PV_A(j),   S_A(j+1) while the softmax of block B on S_B(j) runs,
// so the scores of A are always one sub-tile ahead of B. The softmax (lazy
// maximum, sum-bounded), the masks, the LDS layouts, the copy pipeline and the
// epilogue are those of the one-block kernel above. NW of the 4 waves compute;
// the others only copy and meet the barriers.
template <int D, int NW>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
prefix_mfma2_kernel(PrefixArgs a) {
  constexpr int NWAVE = 4;
  constexpr int KC = D / 16;
  constexpr int DB = D / 32;
  constexpr int DCH = D / 8;
  constexpr int DG = D / 16;
  constexpr int TILE = NK * D;
  constexpr int STAGE = 2 * TILE;
  constexpr int RPB = 64 / DCH;
  constexpr int NBLK = NK / RPB;
  constexpr int NBH = NBLK / NWAVE;
  constexpr int GRP = 2 * NBH;
  constexpr int SROW = D + 8;
  static_assert(NBLK % NWAVE == 0, "copy blocks split evenly over the waves");
  static_assert(NSTAGE * STAGE >= NWAVE * 64 * SROW, "epilogue staging fits in the tile buffers");
  static_assert(3 * GRP < 64, "vmcnt range");
  constexpr int NPV = 2 * DB;         // P.V MFMAs per block and sub-tile
  constexpr int NSLOT = NPV + KC;     // MFMA slots per pipeline block
  constexpr int EPS = 16 / NSLOT;     // probabilities per slot
  static_assert(EPS * NSLOT == 16 && NPV >= KC, "slot layout");

  __shared__ __attribute__((aligned(1024))) unsigned short lds[NSTAGE * STAGE];
  __shared__ int par_s[64];
  __shared__ unsigned long long anc_s[64];
  __shared__ int bad_s;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int grp = lane >> 4;
  const int gl = lane & 15;

  const int w = xcd_remap(blockIdx.x, a.nwg);
  const unsigned TT = total_tiles(a.prefix_len, a.B, a.Hkv, a.Lcap, NK, a.tree_tiles);
  if (TT == 0) return;
  unsigned x = split_begin(w, a.nwg, TT);
  const unsigned x_end = split_begin(w + 1, a.nwg, TT);
  if (x >= x_end) return;
  SegmentWalk sw;
  if (!walk_start(&sw, x, a.prefix_len, a.B, a.Hkv, a.Lcap, NK, a.tree_tiles)) return;

  const bool computes = wave < NW;
  const int row_a = blockIdx.y * a.rows_per_group + wave * 64 + l32;  // block A row of this lane
  const int row_b = row_a + 32;                                        // block B row
  const int row_limit = min(a.M, (int)(blockIdx.y + 1) * a.rows_per_group);
  const bool ok_a = computes && row_a < row_limit;
  const bool ok_b = computes && row_b < row_limit;
  const int node_a = ok_a ? row_a % a.T : 0;
  const int node_b = ok_b ? row_b % a.T : 0;

  int koff[KC];
  {
    const int kr = kperm(l32);
#pragma unroll
    for (int c = 0; c < KC; ++c) koff[c] = kr * D + (((2 * c + hh) ^ swz<D>(kr)) << 3);
  }
  const int voff = TILE + (2 * hh * DG + (grp & 1)) * 64 + 4 * gl;
  const int cp_row = lane / DCH;
  const int cp_kc = lane % DCH;
  const int cp_vt = ((lane >> 3) / DG) * 4 + ((lane & 7) >> 1);
  const int cp_vd = ((lane >> 3) % DG) * 16 + (lane & 1) * 8;

  while (true) {
    const int b = sw.b, g = sw.g;
    const unsigned s_first = sw.seq_first + (unsigned)(g * sw.nt);
    const int tile0 = (int)(x - s_first);
    const unsigned piece_end = min(x_end, s_first + (unsigned)sw.nt);
    const int ntiles = (int)(piece_end - x);
    const int L = valid_prefix(a.prefix_len, b, a.Lcap);
    const int n_prefix = sw.nt - a.tree_tiles;
    const bool has_tree = a.tree_tiles && tile0 + ntiles > n_prefix;
    const int slot = w + b * a.Hkv + g;
    const size_t kv_off = (size_t)(b * a.Hkv + g) * (size_t)a.Lcap * D;
    const unsigned short* kp = a.k + kv_off;
    const unsigned short* vp = a.v + kv_off;
    const size_t kt_off = (size_t)(b * a.Hkv + g) * a.T * D;
    const unsigned short* qp = a.q + (size_t)(b * a.Hq + g * a.G) * a.T * D;

    unsigned long long anc_a = 0ull, anc_b = 0ull;
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
      anc_a = anc_s[node_a];
      anc_b = anc_s[node_b];
    }

    // Q^T fragments of both blocks, loaded like the tile copies (see the
    // one-block kernel); rows past the limit load row 0 and are zeroed.
    bf16x8 qa[KC], qb[KC];
    {
      const unsigned short* qra = qp + (size_t)(ok_a ? row_a : 0) * D + 8 * hh;
      const unsigned short* qrb = qp + (size_t)(ok_b ? row_b : 0) * D + 8 * hh;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        u32x4 ra, rb;
        asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(ra) : "v"(qra + 16 * c) : "memory");
        asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(rb) : "v"(qrb + 16 * c) : "memory");
        qa[c] = __builtin_bit_cast(bf16x8, ra);
        qb[c] = __builtin_bit_cast(bf16x8, rb);
      }
    }
    auto copy_tile = [&](int t) __attribute__((always_inline)) {
      const int ti = tile0 + t;
      const bool tree = ti >= n_prefix;
      const unsigned short* ks = tree ? a.kt + kt_off : kp + (size_t)ti * NK * D;
      const unsigned short* vs = tree ? a.vt + kt_off : vp + (size_t)ti * NK * D;
      const int last = (tree ? a.T : min(NK, L - ti * NK)) - 1;
      unsigned short* dst = lds + (t % NSTAGE) * STAGE;
#pragma unroll
      for (int i = 0; i < NBH; ++i) {
        const int r0 = (wave + i * NWAVE) * RPB;
        const int r = r0 + cp_row;
        copy16_to_lds(ks, (unsigned)(min(r, last) * D + ((cp_kc ^ swz<D>(r)) << 3)) * 2u,
                      lds_addr(dst + r0 * D));
      }
#pragma unroll
      for (int i = 0; i < NBH; ++i) {
        const int r0 = (wave + i * NWAVE) * RPB;
        copy16_to_lds(vs, (unsigned)(min(r0 + cp_vt, last) * D + cp_vd) * 2u, lds_addr(dst + TILE + r0 * D));
      }
    };
    auto wait_tiles = [&](int n) __attribute__((always_inline)) {
      if (n >= 3)
        __builtin_amdgcn_s_waitcnt(vmcnt_only<3 * GRP>());
      else if (n == 2)
        __builtin_amdgcn_s_waitcnt(vmcnt_only<2 * GRP>());
      else if (n == 1)
        __builtin_amdgcn_s_waitcnt(vmcnt_only<GRP>());
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_only<0>());
    };

    for (int t = 0; t < min(ntiles, NSTAGE); ++t) copy_tile(t);
    wait_tiles(min(ntiles, NSTAGE) - 1);  // tile 0 and the older Q loads have landed
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      u32x4 ra = __builtin_bit_cast(u32x4, qa[c]);
      u32x4 rb = __builtin_bit_cast(u32x4, qb[c]);
      asm volatile("" : "+v"(ra), "+v"(rb));
      if (!ok_a) ra = u32x4{0u, 0u, 0u, 0u};
      if (!ok_b) rb = u32x4{0u, 0u, 0u, 0u};
      qa[c] = __builtin_bit_cast(bf16x8, ra);
      qb[c] = __builtin_bit_cast(bf16x8, rb);
    }
    tile_barrier();

    f32x16 OA[DB], OB[DB];
    float m_a = -__builtin_inff(), l_a = 0.f, m_b = -__builtin_inff(), l_b = 0.f;

    if (computes) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          OA[db][v] = 0.f;
          OB[db][v] = 0.f;
        }
      bf16x8 ka[KC], va[2][DB], PA[2], PB[2];
      f32x16 SA, SB;
      float prA[16], prB[16];
      auto load_k = [&](const unsigned short* kb) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < KC; ++c) ka[c] = *(const bf16x8*)(kb + koff[c]);
      };
      // V^T fragments of one 32-token sub-tile (vb: the sub-tile's V base plus voff).
      auto load_v = [&](const unsigned short* vb) __attribute__((always_inline)) {
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const i16x4 lo = lds_read_tr(vb + (4 * kc * DG + 2 * db) * 64);
            const i16x4 hi = lds_read_tr(vb + ((4 * kc + 1) * DG + 2 * db) * 64);
            va[kc][db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
      };
      auto scores = [&](const bf16x8* q) __attribute__((always_inline)) {
        f32x16 S;
#pragma unroll
        for (int v = 0; v < 16; ++v) S[v] = 0.f;
#pragma unroll
        for (int c = 0; c < KC; ++c) S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], q[c], S, 0, 0, 0);
        return S;
      };
      // Hidden scores of sub-tile h of a tree or ragged tile get -inf added.
      auto mask = [&](f32x16& S, unsigned long long anc, bool tree, int nvalid, int h)
                      __attribute__((always_inline)) {
        unsigned vis;
        const int j0 = h * 32 + 8 * hh;
        if (tree) {
          vis = (unsigned)((anc >> j0) & 0xffull) | ((unsigned)((anc >> (j0 + 16)) & 0xffull) << 8);
        } else {
          const int n0 = min(max(nvalid - j0, 0), 8), n1 = min(max(nvalid - j0 - 16, 0), 8);
          vis = ((1u << n0) - 1u) | (((1u << n1) - 1u) << 8);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) S[v] += __uint_as_float((((vis >> v) & 1u) - 1u) & 0xff800000u);
      };
      // p = 2^(S c - m) against the stored max (taken as 0 while m is -inf).
      auto probs = [&](const f32x16& S, float m, float* pr) __attribute__((always_inline)) {
        const float nm = m == -__builtin_inff() ? 0.f : -m;
#pragma unroll
        for (int v = 0; v < 16; ++v) pr[v] = fast_exp2(fmaf(S[v], a.scale_log2, nm));
      };
      auto row_sum = [&](const float* pr) __attribute__((always_inline)) {
        const float s0 = (pr[0] + pr[4]) + (pr[8] + pr[12]), s1 = (pr[1] + pr[5]) + (pr[9] + pr[13]);
        const float s2 = (pr[2] + pr[6]) + (pr[10] + pr[14]), s3 = (pr[3] + pr[7]) + (pr[11] + pr[15]);
        return (s0 + s1) + (s2 + s3);
      };
      // The sum bounds every term: while it stays <= 256 the stored max m can
      // stay. Otherwise (and while m is -inf) take the exact row max over both
      // half-rows; if it exceeds m by more than 8, raise m, rescale (l, O) and
      // recompute. Then l takes the sub-tile's sum.
      auto settle = [&](const f32x16& S, float& m, float& l, f32x16* O, float* pr, float ls)
                        __attribute__((always_inline)) {
        if (__any(!(ls <= 256.0f) || m == -__builtin_inff())) {
          float mx0 = fmaxf(fmaxf(S[0], S[1]), S[2]), mx1 = fmaxf(fmaxf(S[3], S[4]), S[5]);
          float mx2 = fmaxf(fmaxf(S[6], S[7]), S[8]), mx3 = fmaxf(fmaxf(S[9], S[10]), S[11]);
          float mx4 = fmaxf(fmaxf(S[12], S[13]), S[14]);
          float mx = fmaxf(fmaxf(fmaxf(mx0, mx1), fmaxf(mx2, mx3)), fmaxf(mx4, S[15]));
          mx = half_max(mx) * a.scale_log2;
          if (__any(mx > m + 8.0f)) {
            const float mn = fmaxf(m, mx);
            const float alpha = m == -__builtin_inff() ? 0.f : fast_exp2(m - mn);
            m = mn;
            l *= alpha;
            acc_fence<DB>(O);
#pragma unroll
            for (int db = 0; db < DB; ++db) O[db] *= alpha;
            probs(S, m, pr);
            ls = row_sum(pr);
          }
        }
        l += ls;
      };
      auto to_bf16 = [&](const float* pr, bf16x8* P) __attribute__((always_inline)) {
#pragma unroll
        for (int v = 0; v < 16; ++v) P[v >> 3][v & 7] = (__bf16)pr[v];
      };
      auto to_bf16_half = [&](const float* pr, bf16x8* P, int half) __attribute__((always_inline)) {
#pragma unroll
        for (int v = 0; v < 8; ++v) P[half][v] = (__bf16)pr[8 * half + v];
      };

      // One pipeline block: NSLOT slots of one MFMA each. Slots 0..NPV-1 add
      // P.V to O (P = bf16 of pr_in, converted up front), slots NPV.. compute
      // S_next = K . q^T. Alongside run the probabilities of S_cur against m,
      // EPS per slot and software-pipelined (the fma one slot ahead of its
      // exp, the sum one slot behind) so that no slot waits on its own VALU
      // results, and the LDS reads rd(k). All LDS reads before the block have
      // landed at its start; with wait_mid, those issued in the first slots
      // have landed before the first score MFMA. Returns the row sum.
      auto block = [&](f32x16* O, const float* pr_in, bf16x8* P, const bf16x8* q, f32x16& S_next,
                       const f32x16& S_cur, float m, float* pr_out, bool wait_mid, auto&& rd)
                       __attribute__((always_inline)) {
        const float nm = m == -__builtin_inff() ? 0.f : -m;
        float x[16];
        float ps[4] = {0.f, 0.f, 0.f, 0.f};
        to_bf16(pr_in, P);
#pragma unroll
        for (int e = 0; e < EPS; ++e) x[e] = fmaf(S_cur[e], a.scale_log2, nm);
        __builtin_amdgcn_s_waitcnt(kLgkmZero);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < NSLOT; ++k) {
          if (k < NPV) {
            mfma_acc(O[k % DB], va[k / DB][k % DB], P[k / DB]);
          } else {
            if (k == NPV && wait_mid) __builtin_amdgcn_s_waitcnt(kLgkmZero);
            S_next = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[k - NPV], q[k - NPV], k == NPV ? f32x16{} : S_next,
                                                             0, 0, 0);
          }
#pragma unroll
          for (int e = 0; e < EPS; ++e) {
            if (k + 1 < NSLOT) x[(k + 1) * EPS + e] = fmaf(S_cur[(k + 1) * EPS + e], a.scale_log2, nm);
            pr_out[k * EPS + e] = fast_exp2(x[k * EPS + e]);
            if (k >= 1) {
              float& acc = ps[((k - 1) * EPS + e) & 3];
              acc += pr_out[(k - 1) * EPS + e];
              asm volatile("" : "+v"(acc));  // keeps the sum in its slot
            }
          }
          rd(k);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int e = 0; e < EPS; ++e) ps[((NSLOT - 1) * EPS + e) & 3] += pr_out[(NSLOT - 1) * EPS + e];
        return (ps[0] + ps[1]) + (ps[2] + ps[3]);
      };

      // Pipeline over the piece's 32-token sub-tiles j = 2t + h. Entering
      // block X_j: prA = settled probabilities of A(j), SB = masked S_B(j),
      // va = V_j. X_j: PV_A(j), K_{j+1} -> S_A(j+1), softmax of B(j).
      // Y_j: PV_B(j), V_{j+1} -> S_B(j+1), softmax of A(j+1). The blocks past
      // the last sub-tile compute on stale LDS contents and are discarded.
      {
        const bool tree0 = tile0 >= n_prefix;
        const int nvalid0 = tree0 ? a.T : min(NK, L - tile0 * NK);
        load_k(lds);
        load_v(lds + voff);
        SA = scores(qa);
        SB = scores(qb);
        if (tree0 || nvalid0 < 32) {
          mask(SA, anc_a, tree0, nvalid0, 0);
          mask(SB, anc_b, tree0, nvalid0, 0);
        }
        probs(SA, m_a, prA);
        settle(SA, m_a, l_a, OA, prA, row_sum(prA));
      }
      for (int t = 0; t < ntiles; ++t) {
        const unsigned short* Ks = lds + (t % NSTAGE) * STAGE;
        const unsigned short* Kn = lds + ((t + 1) % NSTAGE) * STAGE;
        const bool has_next = t + 1 < ntiles;
        const int ti1 = tile0 + t + 1;
        const bool tree1 = ti1 >= n_prefix;
        const int nvalid1 = has_next ? (tree1 ? a.T : min(NK, L - ti1 * NK)) : 0;
        const int ti = tile0 + t;
        const bool tree = ti >= n_prefix;
        const int nvalid = tree ? a.T : min(NK, L - ti * NK);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          // the sub-tile after this one: (t, 1) or (t + 1, 0)
          const unsigned short* Kj1 = h == 0 ? Ks + 32 * D : Kn;
          const bool more = h == 0 || has_next;
          const bool masked1 = h == 0 ? (tree || nvalid < 64) : (tree1 || nvalid1 < 32);
          const bool tree_1 = h == 0 ? tree : tree1;
          const int nvalid_1 = h == 0 ? nvalid : nvalid1;
          if (h == 1 && has_next) {
            // Every wave's reads of tile t are done (V of its second sub-tile
            // landed) and tile t+1 has landed: refill tile t's stage.
            __builtin_amdgcn_s_waitcnt(kLgkmZero);
            wait_tiles(min(ntiles - 2 - t, 2));
            tile_barrier();
            if (t + NSTAGE < ntiles) copy_tile(t + NSTAGE);
          }
          // ---- X_j: PV_A(j), then S_A(j+1) from the K_{j+1} chunks read in
          // its first KC slots; alongside, the probabilities of B(j).
          const float lsB = block(OA, prA, PA, qa, SA, SB, m_b, prB, true, [&](int k) __attribute__((always_inline)) {
            if (k < KC) ka[k] = *(const bf16x8*)(Kj1 + koff[k]);
          });
          settle(SB, m_b, l_b, OB, prB, lsB);
          if (more && masked1) mask(SA, anc_a, tree_1, nvalid_1, 1 - h);
          // ---- Y_j: PV_B(j), then S_B(j+1); alongside, the probabilities of
          // A(j+1), and each V_{j+1} fragment read right behind the MFMA that
          // frees its registers.
          const unsigned short* vb = Kj1 + voff;
          const float lsA = block(OB, prB, PB, qb, SB, SA, m_a, prA, false, [&](int k) __attribute__((always_inline)) {
            if (k < NPV) {
              const int kc = k / DB, db = k % DB;
              const i16x4 lo = lds_read_tr(vb + (4 * kc * DG + 2 * db) * 64);
              const i16x4 hi = lds_read_tr(vb + ((4 * kc + 1) * DG + 2 * db) * 64);
              va[kc][db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
          });
          if (more) {
            settle(SA, m_a, l_a, OA, prA, lsA);
            if (masked1) mask(SB, anc_b, tree_1, nvalid_1, 1 - h);
          }
        }
      }
    } else {
      for (int t = 0; t + 1 < ntiles; ++t) {
        wait_tiles(min(ntiles - 2 - t, 2));
        tile_barrier();
        if (t + NSTAGE < ntiles) copy_tile(t + NSTAGE);
      }
    }
    __syncthreads();  // no wave reads the tile buffers any more

    // Epilogue: both blocks' rows, normalised and rounded to bf16, staged in
    // LDS (block A rows 0..31, block B rows 32..63 of this wave), then written
    // as whole rows.
    unsigned short* stg = lds + wave * 64 * SROW;
    if (computes) {
      acc_fence<DB>(OA);
      acc_fence<DB>(OB);
      const float lta = half_sum(l_a), ltb = half_sum(l_b);
      const float inva = 1.0f / lta, invb = 1.0f / ltb;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + 8 * g4 + 4 * hh;
          u32x2 pa, pb;
          pa[0] = (unsigned)float_to_bf16_bits(OA[db][4 * g4 + 0] * inva) |
                  ((unsigned)float_to_bf16_bits(OA[db][4 * g4 + 1] * inva) << 16);
          pa[1] = (unsigned)float_to_bf16_bits(OA[db][4 * g4 + 2] * inva) |
                  ((unsigned)float_to_bf16_bits(OA[db][4 * g4 + 3] * inva) << 16);
          pb[0] = (unsigned)float_to_bf16_bits(OB[db][4 * g4 + 0] * invb) |
                  ((unsigned)float_to_bf16_bits(OB[db][4 * g4 + 1] * invb) << 16);
          pb[1] = (unsigned)float_to_bf16_bits(OB[db][4 * g4 + 2] * invb) |
                  ((unsigned)float_to_bf16_bits(OB[db][4 * g4 + 3] * invb) << 16);
          *(u32x2*)(stg + l32 * SROW + d) = pa;
          *(u32x2*)(stg + (32 + l32) * SROW + d) = pb;
        }
      if (ok_a && hh == 0) a.slot_lse2[(size_t)slot * a.M + row_a] = m_a + fast_log2(lta);
      if (ok_b && hh == 0) a.slot_lse2[(size_t)slot * a.M + row_b] = m_b + fast_log2(ltb);
    }
    __syncthreads();
    const int wrow0 = blockIdx.y * a.rows_per_group + wave * 64;
#pragma unroll
    for (int i = 0; i < (computes ? 64 * DCH / 64 : 0); ++i) {
      const int u = i * 64 + lane;
      const int rr = u / DCH, c = u % DCH;
      const u32x4 val = *(const u32x4*)(stg + rr * SROW + c * 8);
      if (wrow0 + rr < row_limit) *(u32x4*)(a.slot_o + ((size_t)slot * a.M + wrow0 + rr) * D + c * 8) = val;
    }
    if (has_tree && g == 0 && blockIdx.y == 0 && tid == 0) {
      a.err_b[b] = bad_s;
      if (bad_s) atomicOr(a.status, kStatusBadTree);
    }

    x = piece_end;
    if (x >= x_end) break;
    if (!walk_next(&sw, a.prefix_len, a.B, a.Hkv, a.Lcap, NK, a.tree_tiles)) break;
    __syncthreads();
  }
}

template <int D>
KernelFn pick2_d(int nw) {
  switch (nw) {
    case 1: return prefix_mfma2_kernel<D, 1>;
    case 2: return prefix_mfma2_kernel<D, 2>;
    case 3: return prefix_mfma2_kernel<D, 3>;
    case 4: return prefix_mfma2_kernel<D, 4>;
    default: return nullptr;
  }
}

}  // namespace

KernelFn prefix_mfma2_pick(int D, int nw) {
  return D == 128 ? pick2_d<128>(nw) : D == 64 ? pick2_d<64>(nw) : nullptr;
}

}  // namespace mfma
}  // namespace hta
