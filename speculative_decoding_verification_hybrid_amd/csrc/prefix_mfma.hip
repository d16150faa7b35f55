// Split-KV attention kernel on bf16 MFMA (gfx950, v_mfma_f32_32x32x16_bf16).
//
// LongSpec summary pages, "Fast Tree Attention": every tree token attends to
// the whole cached KV prefix of its sequence with no mask (the cached part)
// and to its own root path among the tree tokens (the speculative part,
// masked); the parts are combined with the log-sum-exp trick. Here the G
// query heads that share a KV head and the T tree nodes form M = G*T query
// rows per KV head, so one pass over the KV serves all M rows. Each
// workgroup streams one contiguous range of 32-token tiles (see common.h) and
// leaves a normalised partial (o, log2-LSE) per row in a workspace slot for
// the merge kernel. When the tree part is fused in, each (sequence, KV head)
// ends with ceil(T/32) extra tiles holding its tree keys/values, scored under
// the ancestor mask built in LDS from parent[] -- the same online softmax
// then covers both parts, and the merge combines the pieces.
//
// Work per wave: one wave per SIMD, each owning QB blocks of 32 query rows
// (64 rows at QB = 2), so every K or V fragment read from LDS feeds QB MFMAs.
// A tile is processed in NSLOT "slots", each one MFMA plus the VALU work of
// one or two probabilities plus at most one or two LDS reads; tile j's slots
// run, in this order,
//   * P.V of tile j-1 (its V^T fragments and bf16 probabilities are already
//     in registers) while the K fragments of tile j+1 are read,
//   * the scores of tile j+1 (S^T = K . Q^T) while the V^T fragments of tile j
//     are read,
// and alongside both, the softmax of tile j (its scores were computed during
// tile j-1). The MFMA pipe therefore always has independent work queued
// under the exp/sum of the softmax, and every LDS read has at least half a
// tile of slots to land before its MFMA. Slots are fenced with
// sched_barrier so the compiler keeps this composition.
//
// Memory pipeline: K and V tiles go from HBM straight into LDS with
// global_load_lds_dwordx4 (no staging registers) through NS stages of 16 KB
// (D = 128). Tile j's K fragments are read during tile j-1 and its V
// fragments during tile j, and its V registers are consumed during tile j+1,
// so at the start of tile j the stage of tile j-2 is free everywhere: after
// one workgroup barrier (which also publishes every wave's copies of tile
// j+1) it is refilled with tile j-2+NS (with the NS = 4 stages used, tile
// j+2: one tile in flight while tile j runs, which keeps up, since the loop
// is bound by its own instruction stream rather than by the memory). Each
// wave waits for its own copies with an explicit vmcnt; the copies (and the Q
// loads, queued ahead of them) come from inline assembly so the compiler's
// wait insertion never drains the copy queue before an LDS read.
//
// Layouts: K rows keep their 16-byte chunks XOR-swizzled by row
// (conflict-free ds_read_b128 for the MFMA A operand); V is stored as
// 128-byte blocks of 4 tokens x 16 dims, exactly what one 16-lane group of
// ds_read_b64_tr_b16 consumes. Both come from permuting which global 16-byte
// chunk each lane of a copy fetches; the global side stays coalesced.
//
// MFMA mapping: scores are computed transposed, so each lane holds one query
// row (a column of the result) and 16 tokens; the row max needs one
// cross-half exchange and the running (m, l) live in lanes. K rows are fed
// with bits 2 and 3 of the row index swapped, which makes the 8 scores a
// half-wave holds per 16-token k-chunk belong to 8 consecutive tokens:
// converted to bf16 they are directly the B operand of O^T += V^T . P^T.
// The V^T operand comes from the transposed LDS read.
//
// Online softmax in the log2 domain with a lazily updated maximum: the stored
// max m only moves when a tile's max exceeds it by more than 8 (so each
// probability stays below 256), which is exact because the same stale max is
// used for both the sum and the output. The row max itself is only computed
// when the probabilities against the stored max sum to more than 256 (the
// sum bounds every term) or m is still -inf, which after a piece's first tile
// is rare; that check sits after the slots, where it also rescales O.
#include "hta_internal.h"
#include "merge_row.h"
#include "prefix_mfma_common.h"

namespace hta {
namespace mfma {
namespace {

// Static schedule of one tile's slots (see the header comment): slot k
// issues one MFMA (P.V for k < NPV, then scores), then its LDS reads. The KC
// K fragments of the next tile are read over the P.V slots from slot TOP on
// (the barrier that publishes the tile comes right before slot TOP) up to
// four slots before the first score MFMA, where they are waited for once. The 4*DB halves of V^T fragments of this tile are
// read over the score slots but the last two (their registers are free once
// the P.V MFMAs are done) and waited for once, at the top of the next tile.
template <int D, int QB>
struct SlotSchedule {
  static constexpr int KC = D / 16, DB = D / 32, NPV = 2 * DB * QB, NSC = KC * QB, NSLOT = NPV + NSC;
  static constexpr int TOP = NPV >= 8 ? 2 : 1;
  static constexpr int kslot(int c) { return TOP + c * (NPV - TOP - 4 > 0 ? NPV - TOP - 4 : 1) / KC; }
  static constexpr int vslot(int f, int h) { return NPV + (2 * f + h) * (NSC - 2) / (4 * DB); }
  static constexpr bool valid() {
    for (int f = 0; f < 2 * DB; ++f)
      for (int h = 0; h < 2; ++h)
        if (vslot(f, h) < NPV || vslot(f, h) >= NSLOT) return false;
    for (int c = 0; c < KC; ++c)
      if (kslot(c) < TOP || kslot(c) >= NPV) return false;
    return true;
  }
  static_assert(valid(), "slot schedule");
};

template <int D, int QB, int NWAVE, int NS>
__global__ void __launch_bounds__(NWAVE * 64) prefix_mfma_kernel(PrefixArgs a) {
  constexpr int KC = D / 16;               // 16-dim k-chunks of S^T = K.Q^T
  constexpr int DB = D / 32;               // 32-dim blocks of O^T
  constexpr int DCH = D / 8;               // 16-byte chunks per row
  constexpr int DG = D / 16;               // 16-dim groups (V blocks per 4 tokens)
  constexpr int TILE = NK * D;             // bf16 elements of one K (or V) tile
  constexpr int STAGE = 2 * TILE;          // K tile, then V tile
  constexpr int RPB = 64 / DCH;            // rows per 1 KB copy
  constexpr int NBLK = NK / RPB;           // copies per K (or V) tile
  constexpr int KPW = NBLK / NWAVE;        // K (and V) copies per wave per tile
  constexpr int CPW = 2 * KPW;             // copies per wave per tile
  constexpr int SROW = D;                  // epilogue staging row; 16-byte chunks XOR-swizzled by row
  constexpr int NPV = 2 * DB * QB;         // P.V MFMAs per tile
  constexpr int NSC = KC * QB;             // score MFMAs per tile
  constexpr int NSLOT = NPV + NSC;
  constexpr int EPS = 16 * QB / NSLOT;     // probabilities per slot
  using Sch = SlotSchedule<D, QB>;
  // Two waves per SIMD (eight per workgroup) leave each wave half the
  // register file: the P.V accumulators and Q then live in VGPRs with
  // compiler-visible MFMAs; with one wave per SIMD they sit in AGPRs.
  constexpr bool VACC = NWAVE == 8;
  static_assert(NBLK % NWAVE == 0, "copies split evenly over the waves");
  static_assert(EPS * NSLOT == 16 * QB, "slot layout");
  static_assert(NS >= 4, "stages: tiles j-1, j, j+1 in use plus one in flight");
  static_assert(NS * STAGE >= NWAVE * 32 * QB * SROW, "epilogue staging fits in the tile buffers");

  __shared__ __attribute__((aligned(1024))) unsigned short lds[NS * STAGE];
  __shared__ unsigned long long anc_s[64];
  __shared__ int bad_s;
  __shared__ int timed_out_s;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar control flow
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int grp = lane >> 4;  // 16-lane group (transposed V reads)
  const int gl = lane & 15;

  const int w = xcd_remap(blockIdx.x, a.nwg);
  const unsigned TT = total_tiles(a.prefix_len, a.B, a.Hkv, a.Lcap, NK, a.tree_tiles, a.tree_weight);
  if (TT == 0) return;
  unsigned x = split_begin(w, a.nwg, TT);
  const unsigned x_end = split_begin(w + 1, a.nwg, TT);
  if (x >= x_end) return;
  SegmentWalk sw;
  if (!walk_start(&sw, x, a.prefix_len, a.B, a.Hkv, a.Lcap, NK, a.tree_tiles, a.tree_weight)) return;

  const int row_limit = min(a.M, (int)(blockIdx.y + 1) * a.rows_per_group);
  const int wrow0 = blockIdx.y * a.rows_per_group + wave * 32 * QB;  // first row of this wave
  int rowq[QB];
  bool okq[QB];
#pragma unroll
  for (int X = 0; X < QB; ++X) {
    rowq[X] = wrow0 + 32 * X + l32;
    okq[X] = rowq[X] < row_limit;
  }

  // Lane-constant LDS offsets (elements, within a stage). K: the fragments of
  // this lane's MFMA row; the swizzle depends only on the row's low 4 bits.
  const unsigned lds_base = lds_addr(lds);
  unsigned kaddr[KC];  // LDS byte address of K fragment c in stage 0
  {
    const int kr = kperm(l32);
#pragma unroll
    for (int c = 0; c < KC; ++c) kaddr[c] = lds_base + (unsigned)(kr * D + (((2 * c + hh) ^ swz<D>(kr)) << 3)) * 2u;
  }
  // V block (4 tokens x 16 dims, 64 elements) of tokens 4u.., dims 16g..: (u * DG + g) * 64.
  // A transposed read of tokens 16kc + 8hh + 4rr, dims 32db + 16(grp&1) + 0..15
  // reads block ((4kc + 2hh + rr) * DG + 2db + (grp&1)), lane gl at 4 gl.
  const unsigned voff_b = (unsigned)(TILE + (2 * hh * DG + (grp & 1)) * 64 + 4 * gl) * 2u;  // bytes
  // This lane's part of a 1 KB copy. K: row within the copy and logical chunk.
  // V: token within the copy and dims (the V block layout above).
  // Copy i < KPW of a wave moves K rows (wave + i*NWAVE)*RPB .. +RPB-1 of the
  // tile, copy KPW + i the same V rows; for a full tile, each lane's byte
  // offsets into the tile's K and V rows (kofs, vofs) are fixed, and so is the
  // LDS offset of each copy relative to the stage (wave part in wlds).
  const int cp_row = lane / DCH;
  const int cp_kc = lane % DCH;
  const int cp_vt = ((lane >> 3) / DG) * 4 + ((lane & 7) >> 1);
  const int cp_vd = ((lane >> 3) % DG) * 16 + (lane & 1) * 8;
  unsigned kofs[KPW], vofs[KPW];
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int r0 = (wave + i * NWAVE) * RPB;
    kofs[i] = (unsigned)((r0 + cp_row) * D + ((cp_kc ^ swz<D>(r0 + cp_row)) << 3)) * 2u;
    vofs[i] = (unsigned)((r0 + cp_vt) * D + cp_vd) * 2u;
  }
  const unsigned wlds = __builtin_amdgcn_readfirstlane(lds_base + (unsigned)(wave * RPB * D * 2));

  int seg_lo = -1, seg_hi = -1;  // (sequence, KV head) segments this workgroup holds tiles of
  while (true) {
    const int b = sw.b, g = sw.g;
    const unsigned s_first = sw.seq_first + (unsigned)(g * sw.nt);
    const int tile0 = (int)(x - s_first);
    const unsigned piece_end = min(x_end, s_first + (unsigned)sw.nt);
    const int n_prefix = sw.nt - a.tree_tiles * a.tree_weight;  // tiles of cached KV; the tree tiles (if any) follow
    // Real tiles of this piece (the segment's empty tiles after its tree tiles
    // only weigh the split); a piece of empty tiles alone is skipped.
    const unsigned real_end = s_first + (unsigned)(n_prefix + a.tree_tiles);
    const int n = x < real_end ? (int)(min(piece_end, real_end) - x) : 0;
    if (n <= 0) {
      x = piece_end;
      if (x >= x_end) break;
      if (!walk_next(&sw, a.prefix_len, a.B, a.Hkv, a.Lcap, NK, a.tree_tiles, a.tree_weight)) break;
      continue;
    }
    if (seg_lo < 0) seg_lo = b * a.Hkv + g;
    seg_hi = b * a.Hkv + g;
    const int L = sw.L;
    const bool has_tree = a.tree_tiles && tile0 + n > n_prefix;
    const int slot = w + b * a.Hkv + g;
    const size_t kv_off = (size_t)(b * a.Hkv + g) * (size_t)a.Lcap * D;
    const unsigned short* kp = a.k + kv_off;
    const unsigned short* vp = a.v + kv_off;
    const size_t kt_off = (size_t)(b * a.Hkv + g) * a.T * D;
    const unsigned short* qp = a.q + (size_t)(b * a.Hq + g * a.G) * a.T * D;

    // Ancestor words of this sequence's tree (pieces holding tree tiles); the
    // parent array is loaded with the prologue's copies and Q, the words are
    // built once those have landed.
    unsigned long long anc[QB];
#pragma unroll
    for (int X = 0; X < QB; ++X) anc[X] = 0ull;

    // Tokens of tile t of the piece that hold keys (>= 1 for every tile).
    auto nvalid_of = [&](int t) __attribute__((always_inline)) {
      const int ti = tile0 + t;
      return ti >= n_prefix ? min(NK, a.T - (ti - n_prefix) * NK) : min(NK, L - ti * NK);
    };
    // Queue the copies of tile t of the piece into stage t % NS: this wave's
    // CPW of the tile's 2*NBLK 1 KB blocks (K blocks first, then V). Rows past
    // the tile's valid tokens repeat its last valid row, so every value read
    // is finite and in bounds; their scores are masked to -inf.
    auto copy_tile = [&](int t) __attribute__((always_inline)) {
      const int ti = tile0 + t;
      const bool tree = ti >= n_prefix;
      const size_t row0 = tree ? (size_t)(ti - n_prefix) * NK : (size_t)ti * NK;
      const unsigned short* ks = (tree ? a.kt + kt_off : kp) + row0 * D;
      const unsigned short* vs = (tree ? a.vt + kt_off : vp) + row0 * D;
      const int last = nvalid_of(t) - 1;
      const unsigned sb = wlds + (unsigned)((t % NS) * STAGE * 2);
      static_for<0, KPW>([&](auto ii) __attribute__((always_inline)) {
        constexpr int i = decltype(ii)::value;
        const int r0 = (wave + i * NWAVE) * RPB;
        const int r = r0 + cp_row;
        copy16_to_lds_at<i * NWAVE * RPB * D * 2>(ks, (unsigned)(min(r, last) * D + ((cp_kc ^ swz<D>(r)) << 3)) * 2u,
                                                 sb);
      });
      static_for<0, KPW>([&](auto ii) __attribute__((always_inline)) {
        constexpr int i = decltype(ii)::value;
        const int r0 = (wave + i * NWAVE) * RPB;
        copy16_to_lds_at<(TILE + i * NWAVE * RPB * D) * 2>(vs, (unsigned)(min(r0 + cp_vt, last) * D + cp_vd) * 2u,
                                                          sb);
      });
    };
    // The same for a full prefix tile whose K / V rows start at ks / vs, into
    // the stage at LDS byte offset sb (every offset precomputed).
    auto copy_full = [&](const unsigned short* ks, const unsigned short* vs, unsigned sb)
                         __attribute__((always_inline)) {
      static_for<0, KPW>([&](auto ii) __attribute__((always_inline)) {
        constexpr int i = decltype(ii)::value;
        copy16_to_lds_at<i * NWAVE * RPB * D * 2>(ks, kofs[i], sb);
      });
      static_for<0, KPW>([&](auto ii) __attribute__((always_inline)) {
        constexpr int i = decltype(ii)::value;
        copy16_to_lds_at<(TILE + i * NWAVE * RPB * D) * 2>(vs, vofs[i], sb);
      });
    };
    // Wait until at most `ahead` tiles' copies of this wave are in flight.
    auto wait_ahead = [&](int ahead) __attribute__((always_inline)) {
      switch (ahead) {
#define HTA_WAIT_CASE(k) \
  case k: __builtin_amdgcn_s_waitcnt(vmcnt_only<(k * CPW < 63 ? k * CPW : 63)>()); break;
        HTA_WAIT_CASE(1) HTA_WAIT_CASE(2) HTA_WAIT_CASE(3) HTA_WAIT_CASE(4) HTA_WAIT_CASE(5)
        HTA_WAIT_CASE(6) HTA_WAIT_CASE(7) HTA_WAIT_CASE(8) HTA_WAIT_CASE(9) HTA_WAIT_CASE(10)
#undef HTA_WAIT_CASE
        default: __builtin_amdgcn_s_waitcnt(vmcnt_only<0>()); break;
      }
    };
    static_assert(NS - 2 <= 10, "wait_ahead cases");

    // Hidden scores of tile t (tree tile, ragged last prefix tile) get -inf
    // added. Sc[X][v] scores token 16*(v/8) + 8*hh + v%8 of the tile.
    auto mask_scores = [&](f32x16* Sc, int t) __attribute__((always_inline)) {
      const int ti = tile0 + t;
      const bool tree = ti >= n_prefix;
      const int nv = nvalid_of(t);
      if (tree || nv < NK) {
        const int j0 = 8 * hh;
        const int n0 = min(max(nv - j0, 0), 8), n1 = min(max(nv - j0 - 16, 0), 8);
        const unsigned lim = ((1u << n0) - 1u) | (((1u << n1) - 1u) << 8);
        const int tb = tree ? (ti - n_prefix) * NK + j0 : 0;
#pragma unroll
        for (int X = 0; X < QB; ++X) {
          unsigned vis = lim;
          if (tree)
            vis &= (unsigned)((anc[X] >> tb) & 0xffull) | ((unsigned)((anc[X] >> (tb + 16)) & 0xffull) << 8);
#pragma unroll
          for (int v = 0; v < 16; ++v) Sc[X][v] += __uint_as_float((((vis >> v) & 1u) - 1u) & 0xff800000u);
        }
      }
    };

    f32x16 O[QB][DB];
    f32x16 S[QB];
    bf16x8 P[QB][2], vf[2][DB];
    float m[QB], l[QB];
#pragma unroll
    for (int X = 0; X < QB; ++X) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) O[X][db][v] = 0.f;
      m[X] = -__builtin_inff();
      l[X] = 0.f;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int e = 0; e < 8; ++e) P[X][kc][e] = (__bf16)0.f;
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[kc][db][e] = (__bf16)0.f;
    // The first tile's P.V operands are these zeros: hide their value from the
    // compiler, so it does not materialise them right before the (inline
    // assembly) MFMAs, whose operand hazards it cannot see.
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
      for (int X = 0; X < QB; ++X) {
        u32x4 r = __builtin_bit_cast(u32x4, P[X][kc]);
        asm volatile("" : "+v"(r));
        P[X][kc] = __builtin_bit_cast(bf16x8, r);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        u32x4 r = __builtin_bit_cast(u32x4, vf[kc][db]);
        asm volatile("" : "+v"(r));
        vf[kc][db] = __builtin_bit_cast(bf16x8, r);
      }
    }

    // Prologue: queue tile 0, the Q loads and tile 1 (P0 = NS - 2 tiles: the
    // steady refill of tile 0 then queues tile 2), wait for tile 0 and Q,
    // score tile 0.
    constexpr int P0 = 2;
    copy_tile(0);
    // Q^T fragments (B operand of S^T = K.Q^T): row rowq[X], dims 16c + 8hh .. +7.
    // Loaded from inline assembly, like the tile copies, so that one explicit
    // wait covers both: they are queued right after tile 0's copies and are
    // complete once every copy queued before tile 1's is. Rows past the limit
    // load row 0 and are zeroed.
    bf16x8 qf[QB][KC];
#pragma unroll
    for (int X = 0; X < QB; ++X) {
      const unsigned short* qr = qp + (size_t)(okq[X] ? rowq[X] : 0) * D + 8 * hh;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        u32x4 r;
        asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r) : "v"(qr + 16 * c) : "memory");
        qf[X][c] = __builtin_bit_cast(bf16x8, r);
      }
    }
    int par_r = 0;
    if (has_tree && tid < a.T)
      asm volatile("global_load_dword %0, %1, off" : "=v"(par_r) : "v"(a.parent + (size_t)b * a.T + tid) : "memory");
    for (int t = 1; t < min(n, P0); ++t) copy_tile(t);
    wait_ahead(min(n, P0) - 1);
    // Tie the Q registers to the wait: nothing below may read them earlier.
    // (The compiler still could copy them between the load and here; the CPU
    // test tests/test_q_load_isa.py checks the generated code for that.)
#pragma unroll
    for (int X = 0; X < QB; ++X)
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        u32x4 r = __builtin_bit_cast(u32x4, qf[X][c]);
        asm volatile("" : "+v"(r));
        if (!okq[X]) r = u32x4{0u, 0u, 0u, 0u};
        qf[X][c] = __builtin_bit_cast(bf16x8, r);
      }
    if (has_tree) {
      asm volatile("" : "+v"(par_r));  // landed with the copies waited for above
      // Ancestor words by pointer doubling in wave 0 (node i in lane i, T <= 64):
      // after round r a node's word holds its ancestors up to distance 2^r - 1
      // and p its ancestor at distance 2^r, so 6 rounds cover any depth. The
      // tree is valid iff every node has -1 <= parent < its own index.
      if (wave == 0) {
        const bool node = lane < a.T;
        int p = node ? par_r : -1;
        const bool ok = !node || (p >= -1 && p < lane);
        unsigned long long an = node ? 1ull << lane : 0ull;
#pragma unroll
        for (int r = 0; r < 6; ++r) {
          const int src = p >= 0 && p < 64 ? p : lane;
          const int pp = __shfl(p, src);
          const unsigned lo = __shfl((unsigned)an, src), hi = __shfl((unsigned)(an >> 32), src);
          if (src != lane) {
            an |= ((unsigned long long)hi << 32) | lo;
            p = pp;
          }
        }
        if (node) anc_s[lane] = ok ? an : 1ull << lane;
        const bool bad_tree = __any(!ok);
        if (lane == 0) bad_s = bad_tree;
      }
      // (LDS-only wait before the barrier: tile 1's copies stay in flight)
      wait_lgkm<0>();
      tile_barrier();
#pragma unroll
      for (int X = 0; X < QB; ++X) anc[X] = anc_s[okq[X] ? rowq[X] % a.T : 0];
    }
    tile_barrier();
    // Scores of the tile in the stage at LDS byte offset kb, straight from its
    // K tile in LDS (prologue and the rare recomputation of the max-raise path);
    // t is the tile's index in the piece, for its mask.
    auto scores_of = [&](f32x16* Sc, unsigned kb, int t) __attribute__((always_inline)) {
      bf16x8 kr[KC];
#pragma unroll
      for (int c = 0; c < KC; ++c) kr[c] = lds_read_k(kb, kaddr[c]);
      wait_lgkm<0>();
#pragma unroll
      for (int c = 0; c < KC; ++c) lds_tie(kr[c]);
#pragma unroll
      for (int X = 0; X < QB; ++X) {
        Sc[X] = mfma_s_first(kr[0], qf[X][0]);
#pragma unroll
        for (int c = 1; c < KC; ++c) mfma_s_acc(Sc[X], kr[c], qf[X][c]);
      }
      mask_scores(Sc, t);
    };
#pragma unroll
    for (int X = 0; X < QB; ++X)
#pragma unroll
      for (int c = 0; c < KC; ++c)
        if constexpr (!VACC) q_tie(qf[X][c]);
    scores_of(S, 0u, 0);
    // The stored max starts at tile 0's exact row max (so the first tile needs
    // no rescaling pass); rows that see nothing in tile 0 keep -inf. The
    // softmax adds nm = -m (0 while m is -inf); lim bounds a tile's
    // probability sum below which m may stay (-1 while m is -inf, so that the
    // first visible score takes the exact path).
    float nm[QB], lim[QB];
#pragma unroll
    for (int X = 0; X < QB; ++X) {
      float mx = S[X][0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, S[X][v]);
      m[X] = half_max(mx) * a.scale_log2;
      nm[X] = m[X] == -__builtin_inff() ? 0.f : -m[X];
      lim[X] = m[X] == -__builtin_inff() ? -1.f : 256.f;
    }

    // Tiles before jm are full prefix tiles (no mask). Tiles 0 .. issued-1
    // have been queued; at tile j a tile t may be queued once the stage it
    // takes (t % NS) is free everywhere, i.e. t <= j - 2 + NS. In the steady
    // state exactly that tile is queued and NS - 4 tiles stay in flight beyond
    // tile j+1; past the piece's last tile nothing is.
    const int jm = min(n, max(0, L / NK - tile0));
    int issued = min(n, P0);
    const unsigned short* kq = kp + (size_t)(tile0 + issued) * NK * D;  // rows of tile `issued`
    const unsigned short* vq = vp + (size_t)(tile0 + issued) * NK * D;
    constexpr unsigned SB = STAGE * 2;  // bytes per stage
    auto rot = [](unsigned o) __attribute__((always_inline)) { return o + SB == NS * SB ? 0u : o + SB; };
    unsigned op = 0u, oc = 0u, on = rot(0u);  // stage byte offsets of tiles j-1, j and j+1
    unsigned ocp = (unsigned)((NS - 2) % NS) * SB;  // stage byte offset of tile j-2+NS
    bool drained = false;                           // every copy of the piece has landed and been published
    // Probability sum of tile j-1, checked (and added to l) at the start of tile j.
    float lsp[QB];
#pragma unroll
    for (int X = 0; X < QB; ++X) lsp[X] = 0.f;

    // The lazy-max check of tile t's probabilities Pt (sum lst), before their
    // P.V: the sum bounds every term, so while it stays <= 256 the stored max
    // can stay. Otherwise (and while m is -inf) take the exact row max over
    // both half-rows; if it exceeds m by more than 8, raise m, rescale l and O,
    // and recompute the tile's probabilities from its scores, recomputed from
    // its K tile (still in LDS at stage byte offset ot: a stage is refilled
    // two tiles after its tile). Then the sum joins l.
    auto check = [&](int t, bf16x8(&Pt)[QB][2], float(&lst)[QB], unsigned ot) __attribute__((always_inline)) {
      bool need = false;
#pragma unroll
      for (int X = 0; X < QB; ++X) need |= !(lst[X] <= lim[X]);
      if (__any(need)) {
        f32x16 Sj[QB];
        wait_lgkm<0>();
        scores_of(Sj, ot, t);
#pragma unroll
        for (int X = 0; X < QB; ++X) {
          float mx = Sj[X][0];
#pragma unroll
          for (int v = 1; v < 16; ++v) mx = fmaxf(mx, Sj[X][v]);
          mx = half_max(mx) * a.scale_log2;
          if (__any(mx > m[X] + 8.0f)) {
            const float mn = fmaxf(m[X], mx);
            const float alpha = m[X] == -__builtin_inff() ? 0.f : fast_exp2(m[X] - mn);
            m[X] = mn;
            nm[X] = mn == -__builtin_inff() ? 0.f : -mn;
            lim[X] = mn == -__builtin_inff() ? -1.f : 256.f;
            l[X] *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              if constexpr (!VACC) o_fence(O[X][db]);
              O[X][db] *= alpha;
              if constexpr (!VACC) o_fence(O[X][db]);
            }
            float q4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const float p = fast_exp2(fmaf(Sj[X][v], a.scale_log2, nm[X]));
              q4[v & 3] += p;
              Pt[X][v >> 3][v & 7] = (__bf16)p;
            }
            lst[X] = (q4[0] + q4[1]) + (q4[2] + q4[3]);
          }
        }
      }
#pragma unroll
      for (int X = 0; X < QB; ++X) l[X] += lst[X];
    };

    // Tile j: its scores are in Sc, tile j-1's probabilities in Pc (sum in
    // lsp); leaves tile j+1's scores in Sn and tile j's probabilities in Pn
    // (sum in lsp). Two consecutive tiles swap the roles of the two register
    // sets, so no scores or probabilities are copied between tiles.
    constexpr int TOP = NPV >= 8 ? 2 : 1;  // P.V slots issued ahead of the barrier
    // A steady step (steady_c true) is one known to take the steady-state
    // refill below and to need no mask for tile j+1: its code tests neither.
    auto step = [&](auto steady_c, const int j, f32x16(&Sc)[QB], f32x16(&Sn)[QB], bf16x8(&Pc)[QB][2],
                    bf16x8(&Pn)[QB][2]) __attribute__((always_inline)) {
      constexpr bool kSteady = decltype(steady_c)::value;
      if (j > 0) check(j - 1, Pc, lsp, op);
#pragma unroll
      for (int X = 0; X < QB; ++X)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          if constexpr (!VACC) o_tie(O[X][db]);
      wait_lgkm<0>();  // this wave's V reads of tile j-1
      // (tied to the wait, for the compiler-visible MFMAs of the VGPR form)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int db = 0; db < DB; ++db) lds_tie(vf[kc][db]);
      // Top of the tile (after the first TOP P.V MFMAs, which run meanwhile):
      // tile j+1 has landed for every wave (each waits for its own copies and
      // the barrier publishes them), and every wave is done with the stage of
      // tile j-2 (its V registers were consumed during tile j-1): it takes
      // tile j-2+NS. In the steady state that is a full prefix tile with
      // NS - 4 tiles in flight beyond tile j+1 (one fixed wait, precomputed
      // copy offsets); otherwise (the ring filling up, masked copies, the
      // tail) up to two tiles are queued with the general copy.
      auto top = [&]() __attribute__((always_inline)) {
        const int t = j - 2 + NS;
        if (kSteady || (t < jm && issued == t)) {
          __builtin_amdgcn_s_waitcnt(vmcnt_only<((NS - 4) * CPW < 63 ? (NS - 4) * CPW : 63)>());
          tile_barrier();
          copy_full(kq, vq, wlds + ocp);
          ++issued;
          kq += NK * D;
          vq += NK * D;
        } else if (issued == n) {
          // Nothing left to queue: once every copy has landed and one barrier
          // has published them, the remaining tiles need neither.
          if (!drained) {
            __builtin_amdgcn_s_waitcnt(vmcnt_only<0>());
            tile_barrier();
            drained = true;
          }
        } else {
          wait_ahead(issued - j - 2);
          tile_barrier();
#pragma unroll
          for (int r = 0; r < 2; ++r)
            if (issued < n && issued <= t) {
              copy_tile(issued);
              ++issued;
            }
          kq = kp + (size_t)(tile0 + issued) * NK * D;
          vq = vp + (size_t)(tile0 + issued) * NK * D;
        }
      };

      const unsigned kn = on;                      // K tile j+1
      const unsigned vc = lds_base + voff_b + oc;  // V tile j
      float xs[16 * QB], pr[16 * QB], ps[QB];
      bf16x8 kf[KC];
      i16x4 vh[2][2][DB];     // V^T fragment halves of tile j: [low/high][kc][db]
      unsigned pk[QB][2][4];  // bf16 pairs of this tile's probabilities
      auto fma_p = [&](int p) __attribute__((always_inline)) {
        xs[p] = fmaf(Sc[p >> 4][p & 15], a.scale_log2, nm[p >> 4]);
      };
      // (the tie keeps each add in its slot: left alone, the compiler sinks
      // all of them into one dependent chain after the last slot)
      auto sum_p = [&](int p) __attribute__((always_inline)) {
        if ((p & 15) == 0)
          ps[p >> 4] = pr[p];
        else
          ps[p >> 4] += pr[p];
        asm volatile("" : "+v"(ps[p >> 4]));
        if (p & 1) pk[p >> 4][(p >> 3) & 1][(p & 7) >> 1] = cvt_pk_bf16(pr[p - 1], pr[p]);
      };
      // The scaled scores run two slots ahead of their exp (a transcendental
      // reading a VALU result of the previous instruction needs a wait state).
#pragma unroll
      for (int e = 0; e < 2 * EPS; ++e) fma_p(e);
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, NSLOT>([&](auto kk) __attribute__((always_inline)) {
        constexpr int k = decltype(kk)::value;
        if constexpr (k == TOP) {
          top();
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (k < NPV) {
          // P.V of tile j-1 (zeros before the first tile)
          constexpr int f = k / QB, X = k % QB, kc = f / DB, db = f % DB;
          if constexpr (VACC)
            mfma_pv_v(O[X][db], vf[kc][db], Pc[X][kc]);
          else
            mfma_pv(O[X][db], vf[kc][db], Pc[X][kc]);
          // This slot's exp waits for the MFMA issue (the compiler would put
          // the quarter-rate exp first and hold the MFMA up behind it).
#pragma unroll
          for (int e = 0; e < EPS; ++e) asm volatile("" : "+v"(xs[k * EPS + e]));
        } else {
          // scores of tile j+1 (computed on stale data past the piece's last tile, then unused)
          constexpr int c = (k - NPV) / QB, X = (k - NPV) % QB;
          if constexpr (k == NPV) {
            wait_lgkm<0>();
#pragma unroll
            for (int cc = 0; cc < KC; ++cc) lds_tie(kf[cc]);
          }
          if constexpr (c == 0)
            Sn[X] = mfma_s_first(kf[c], qf[X][c]);
          else
            mfma_s_acc(Sn[X], kf[c], qf[X][c]);
        }
        // V^T fragments of tile j into the registers the P.V above has freed.
        static_for<0, 2 * DB>([&](auto ff) __attribute__((always_inline)) {
          constexpr int f = decltype(ff)::value, kc = f / DB, db = f % DB;
          static_for<0, 2>([&](auto hh_) __attribute__((always_inline)) {
            constexpr int h = decltype(hh_)::value;
            if constexpr (Sch::vslot(f, h) == k)
              vh[h][kc][db] = lds_read_v<((4 * kc + h) * DG + 2 * db) * 128>(vc);
          });
        });
        // K fragments of tile j+1 (after the barrier that published it)
        static_for<0, KC>([&](auto cc) __attribute__((always_inline)) {
          constexpr int c = decltype(cc)::value;
          if constexpr (Sch::kslot(c) == k) kf[c] = lds_read_k(kn, kaddr[c]);
        });
#pragma unroll
        for (int e = 0; e < EPS; ++e) {
          if (k + 2 < NSLOT) fma_p((k + 2) * EPS + e);
          pr[k * EPS + e] = fast_exp2(xs[k * EPS + e]);
          if (k >= 1) sum_p((k - 1) * EPS + e);
        }
        if constexpr (k >= NPV) {
          // the score MFMA first in the slot, the VALU work after it
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x602, 16, 0);  // VALU and transcendental
        }
        __builtin_amdgcn_sched_barrier(0);
      });
#pragma unroll
      for (int e = 0; e < EPS; ++e) sum_p((NSLOT - 1) * EPS + e);
#pragma unroll
      for (int X = 0; X < QB; ++X) {
        lsp[X] = ps[X];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
          Pn[X][kc] = __builtin_bit_cast(bf16x8, u32x4{pk[X][kc][0], pk[X][kc][1], pk[X][kc][2], pk[X][kc][3]});
      }
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          vf[kc][db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vh[0][kc][db], vh[1][kc][db], 0, 1, 2, 3, 4,
                                                                           5, 6, 7));
      // Masks of tile j+1 (known now that its scores are).
      if (!kSteady && j + 1 >= jm && j + 1 < n) mask_scores(Sn, j + 1);
      op = oc;
      oc = on;
      on = rot(on);
      ocp = rot(ocp);
    };
    // Tiles in pairs (an odd count starts with a single tile and one copy).
    // Steps 0 .. n_st-1 are steady: tile j-2+NS is a full prefix tile, queued
    // in order (the prologue queued NS-2 tiles), so tile j+1 is full too.
    // The remaining steps take the general path.
    f32x16 S1[QB];
    bf16x8 P1[QB][2];
    auto swap_sets = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int X = 0; X < QB; ++X) {
        S[X] = S1[X];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) P[X][kc] = P1[X][kc];
      }
    };
    static_assert(P0 == NS - 2, "the steady steps start at tile 0");
    const int n_st = issued == P0 ? max(0, min(n, jm - P0)) : 0;
    constexpr std::integral_constant<bool, true> kSteadyStep{};
    constexpr std::integral_constant<bool, false> kGeneralStep{};
    int j = 0;
    if (n_st & 1) {
      step(kSteadyStep, 0, S, S1, P, P1);
      swap_sets();
      j = 1;
    }
    for (; j < n_st; j += 2) {
      step(kSteadyStep, j, S, S1, P, P1);
      step(kSteadyStep, j + 1, S1, S, P1, P);
    }
    if ((n - j) & 1) {
      step(kGeneralStep, j, S, S1, P, P1);
      swap_sets();
      ++j;
    }
    for (; j < n; j += 2) {
      step(kGeneralStep, j, S, S1, P, P1);
      step(kGeneralStep, j + 1, S1, S, P1, P);
    }
    check(n - 1, P, lsp, op);
    // P.V of the last tile.
    wait_lgkm<0>();
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int db = 0; db < DB; ++db) lds_tie(vf[kc][db]);
#pragma unroll
    for (int f = 0; f < 2 * DB; ++f)
#pragma unroll
      for (int X = 0; X < QB; ++X)
        if constexpr (VACC)
          mfma_pv_v(O[X][f % DB], vf[f / DB][f % DB], P[X][f / DB]);
        else
          mfma_pv_after_valu(O[X][f % DB], vf[f / DB][f % DB], P[X][f / DB]);
#pragma unroll
    for (int X = 0; X < QB; ++X)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        if constexpr (!VACC) o_fence(O[X][db]);
    __builtin_amdgcn_s_waitcnt(vmcnt_only<0>());
    __syncthreads();  // every copy has landed and no wave reads the tile buffers any more

    // Epilogue: O^T holds dims db*32 + 8*(v/4) + 4*hh + v%4 of row rowq[X].
    // Normalise, round to bf16 and stage this wave's rows in LDS (16-byte
    // chunk c of row r at chunk c ^ (r mod DCH), so the 32 rows a store
    // instruction touches spread over the banks), then write them out as
    // whole contiguous rows.
    unsigned short* stg = lds + wave * 32 * QB * SROW;
#pragma unroll
    for (int X = 0; X < QB; ++X) {
      const float lt = half_sum(l[X]);
      const float inv = 1.0f / lt;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + 8 * g4 + 4 * hh;
          u32x2 pk;
          pk[0] = cvt_pk_bf16(O[X][db][4 * g4 + 0] * inv, O[X][db][4 * g4 + 1] * inv);
          pk[1] = cvt_pk_bf16(O[X][db][4 * g4 + 2] * inv, O[X][db][4 * g4 + 3] * inv);
          const int r = 32 * X + l32;
          *(u32x2*)(stg + r * SROW + (((d >> 3) ^ (r & (DCH - 1))) << 3) + (d & 7)) = pk;
        }
      if (okq[X] && hh == 0) {
        const float v = m[X] + fast_log2(lt);
        if (a.fuse)
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), slot_rsrc(a.slot_lse2, a.slot_bytes_l),
                                                (unsigned)(slot * a.M + rowq[X]) * 4u, 0, kCpolDevice);
        else
          a.slot_lse2[(size_t)slot * a.M + rowq[X]] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 32 * QB * DCH / 64; ++i) {
      const int u = i * 64 + lane;
      const int rr = u / DCH, c = u % DCH;
      const u32x4 val = *(const u32x4*)(stg + rr * SROW + ((c ^ (rr & (DCH - 1))) << 3));
      if (wrow0 + rr < row_limit) {
        if (a.fuse)
          __builtin_amdgcn_raw_buffer_store_b128(val, slot_rsrc(a.slot_o, a.slot_bytes_o),
                                                 ((unsigned)(slot * a.M + wrow0 + rr) * D + (unsigned)c * 8) * 2u, 0,
                                                 kCpolDevice);
        else  // streamed past the caches: read once, by the merge
          __builtin_nontemporal_store(val, (u32x4*)(a.slot_o + ((size_t)slot * a.M + wrow0 + rr) * D + c * 8));
      }
    }
    // The workgroup holding the first tree tile of (b, KV head 0) reports the
    // tree check; for the fused merge, each segment's holder notes it too.
    if (has_tree && tile0 <= n_prefix && g == 0 && blockIdx.y == 0 && tid == 0) {
      a.err_b[b] = bad_s;
      if (bad_s) atomicOr(a.status, kStatusBadTree);
    }
    if (a.fuse && has_tree && tile0 <= n_prefix && tid == 0)
      __hip_atomic_store(a.seg_err + (b * a.Hkv + g) * (int)gridDim.y + (int)blockIdx.y, bad_s, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);

    x = piece_end;
    if (x >= x_end) break;
    if (!walk_next(&sw, a.prefix_len, a.B, a.Hkv, a.Lcap, NK, a.tree_tiles, a.tree_weight)) break;
    __syncthreads();  // staging area, anc_s / bad_s of this piece are no longer read
  }

  // Fused merge (verification attention, where every segment has tiles):
  // the workgroups holding tiles of a segment each merge a contiguous share
  // of its rows once all of them have left their partials. Each publishes
  // its partials (release), counts itself in every segment it holds, then per
  // segment waits until the count is complete -- every contributor is resident
  // (one launch no wider than the device), and the wait is bounded: past the
  // bound the share's rows come out NaN with HTA_STATUS_MERGE_TIMEOUT -- and
  // merges its rows (merge_row.h) from all contributors' slots. The last
  // contributor past the wait clears the segment's words for the next launch.
  if (a.fuse && seg_lo >= 0) {  // (a workgroup holding only empty tiles contributes to no segment)
    constexpr int kSpinLimit = 1 << 15;  // about 40 ms of polling
    const int RG = (int)gridDim.y;
    // The partials went out as device-coherent (write-through) stores: once
    // they are complete, every other workgroup's sc1 loads see them.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
      for (int sg = seg_lo; sg <= seg_hi; ++sg)
        __hip_atomic_fetch_add(a.seg_sync + 2 * (sg * RG + (int)blockIdx.y), 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    const int rows_lo = (int)blockIdx.y * a.rows_per_group;
    const int nrows = row_limit - rows_lo;
    const bool maybe_empty = TT < (unsigned)a.nwg;
    const __amdgpu_buffer_rsrc_t rs_o = slot_rsrc(a.slot_o, a.slot_bytes_o);
    const __amdgpu_buffer_rsrc_t rs_l = slot_rsrc(a.slot_lse2, a.slot_bytes_l);
    for (int sg = seg_lo; sg <= seg_hi; ++sg) {
      const int b = sg / a.Hkv, g = sg % a.Hkv;
      unsigned first;
      int count;
      segment_tiles(a.prefix_len, a.Hkv, a.Lcap, NK, a.tree_tiles, b, g, &first, &count, a.tree_weight);
      const unsigned w_first = split_owner(first, (unsigned)a.nwg, TT);
      const unsigned w_last = split_owner(first + (unsigned)count - 1, (unsigned)a.nwg, TT);
      const int n_range = (int)(w_last - w_first) + 1;  // slots of the segment (some empty when TT < nwg)
      // Contributors (workgroups owning tiles of the segment) and this one's
      // rank among them: with fewer tiles than workgroups some in the range
      // own none and never arrive.
      int nc = n_range, share = (int)((unsigned)w - w_first);
      if (maybe_empty) {
        nc = 0;
        share = 0;
        for (unsigned u = w_first; u <= w_last; ++u) {
          const int ne = split_begin(u, (unsigned)a.nwg, TT) < split_begin(u + 1, (unsigned)a.nwg, TT);
          nc += ne;
          if (u < (unsigned)w) share += ne;
        }
      }
      int* sync = a.seg_sync + 2 * (sg * RG + (int)blockIdx.y);
      if (tid == 0) {
        int it = 0;
        while (__hip_atomic_load(sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < nc && it < kSpinLimit) {
          __builtin_amdgcn_s_sleep(2);
          ++it;
        }
        timed_out_s = it >= kSpinLimit;
        if (timed_out_s) atomicOr(a.status, kStatusMergeTimeout);
        if (__hip_atomic_fetch_add(sync + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nc - 1) {
          __hip_atomic_store(sync, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(sync + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      __syncthreads();
      const int Lraw = a.prefix_len[b];
      const bool bad_prefix = Lraw < 0 || Lraw > a.Lcap;
      const bool bad = timed_out_s || bad_prefix ||
                       __hip_atomic_load(a.seg_err + sg * RG + (int)blockIdx.y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
      const int p_first = (int)w_first + b * a.Hkv + g;
      // This workgroup's rows, RB per wave at a time (rows of a wave batch
      // past the share are skipped: their loads are in bounds, their results
      // unused).
      constexpr int RB = 2, UNR = kMergeUnroll;  // the merge kernel's passes: the same bits
      const int r_beg = rows_lo + share * nrows / nc, r_end = rows_lo + (share + 1) * nrows / nc;
      if (bad_prefix && g == 0 && r_beg == 0 && tid == 0) atomicOr(a.status, kStatusBadPrefix);
      for (int r0 = r_beg + wave * RB; r0 < r_end; r0 += NWAVE * RB) {
        int64_t row[RB];
        unsigned o_off[RB], l_off[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int r = min(r0 + rb, r_end - 1);
          row[rb] = r0 + rb < r_end ? ((int64_t)b * a.Hq + g * a.G + r / a.T) * a.T + r % a.T : -1;
          // Device-coherent loads (sc1) of the slots other workgroups wrote through.
          o_off[rb] = ((unsigned)(p_first * a.M + r) * D + (unsigned)(lane % (D / 8)) * 8) * 2u;
          l_off[rb] = (unsigned)(p_first * a.M + r) * 4u;
        }
        auto load_o = [&](int rb, int k) {
          return __builtin_amdgcn_raw_buffer_load_b128(rs_o, o_off[rb] + (unsigned)k * (unsigned)(a.M * D * 2), 0,
                                                       kCpolDevice);
        };
        auto load_l = [&](int rb, int k) {
          return __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(rs_l, l_off[rb] + (unsigned)k * (unsigned)(a.M * 4), 0,
                                                          kCpolDevice));
        };
        if (maybe_empty) {
          const unsigned nwg = (unsigned)a.nwg;
          merge_rows<D, RB, UNR, true>(
              lane, n_range, load_o, load_l,
              [&](int k) { return split_begin(w_first + (unsigned)k, nwg, TT) == split_begin(w_first + (unsigned)k + 1, nwg, TT); },
              bad, a.out, a.lse, row);
        } else {
          merge_rows<D, RB, UNR, true>(lane, n_range, load_o, load_l, [](int) { return false; }, bad, a.out, a.lse, row);
        }
      }
      __syncthreads();  // timed_out_s is rewritten for the next segment
    }
  }
}

typedef void (*KernelFn)(PrefixArgs);

// Instances: every (QB, waves) the plan can pick -- QB = 2 with 1, 2 or 4
// waves, QB = 1 (on request, or for a single 32-row block) with 1, 2, 4 or 8
// at D = 128 -- at D = 128 and 64. Four stages: deeper rings (up to 9 at
// D = 128) measured no faster, since the loop is bound by instruction issue
// rather than by memory latency, and the smaller ring lets two workgroups
// share a CU where registers allow.
struct Inst {
  int D, qb, waves, stages;
  KernelFn fn;
};
constexpr int kStages = 4;
const Inst kInst[] = {
    {128, 1, 8, kStages, prefix_mfma_kernel<128, 1, 8, kStages>},
    {128, 2, 4, kStages, prefix_mfma_kernel<128, 2, 4, kStages>},
    {128, 2, 2, kStages, prefix_mfma_kernel<128, 2, 2, kStages>},
    {128, 2, 1, kStages, prefix_mfma_kernel<128, 2, 1, kStages>},
    {128, 1, 4, kStages, prefix_mfma_kernel<128, 1, 4, kStages>},
    {128, 1, 2, kStages, prefix_mfma_kernel<128, 1, 2, kStages>},
    {128, 1, 1, kStages, prefix_mfma_kernel<128, 1, 1, kStages>},
    {64, 2, 4, kStages, prefix_mfma_kernel<64, 2, 4, kStages>},
    {64, 2, 2, kStages, prefix_mfma_kernel<64, 2, 2, kStages>},
    {64, 2, 1, kStages, prefix_mfma_kernel<64, 2, 1, kStages>},
    {64, 1, 4, kStages, prefix_mfma_kernel<64, 1, 4, kStages>},
    {64, 1, 2, kStages, prefix_mfma_kernel<64, 1, 2, kStages>},
    {64, 1, 1, kStages, prefix_mfma_kernel<64, 1, 1, kStages>},
};

const Inst* find(int D, int qb, int waves) {
  for (const Inst& i : kInst)
    if (i.D == D && i.qb == qb && i.waves == waves) return &i;
  return nullptr;
}

}  // namespace
}  // namespace mfma

using mfma::PrefixArgs;

bool prefix_mfma_supported(int D, int waves, int qb) { return mfma::find(D, qb, waves) != nullptr; }

int prefix_mfma_occupancy(int D, int waves, int qb) {
  const mfma::Inst* in = mfma::find(D, qb, waves);
  if (!in) return 0;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(in->fn), waves * 64, 0) !=
      hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}

hipError_t launch_prefix_mfma(const Dims& d, const PrefixLaunch& pl, const PrefixInputs& in, Slots slots,
                              int* err_b, int* status, hipStream_t s, const FusedMerge& fuse) {
  const mfma::Inst* inst = mfma::find(d.D, pl.qb, pl.waves);
  if (!inst) return hipErrorInvalidValue;
  PrefixArgs a;
  a.q = static_cast<const unsigned short*>(in.q);
  a.k = static_cast<const unsigned short*>(in.k_cache);
  a.v = static_cast<const unsigned short*>(in.v_cache);
  a.kt = static_cast<const unsigned short*>(in.k_tree);
  a.vt = static_cast<const unsigned short*>(in.v_tree);
  a.parent = in.parent;
  a.prefix_len = in.prefix_len;
  a.slot_o = static_cast<unsigned short*>(slots.o);
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
  a.rows_per_group = pl.rows_per_group;
  a.tree_tiles = in.k_tree ? tree_tiles_for(d.T, mfma::NK) : 0;
  a.tree_weight = in.k_tree ? kTreeTileWeight : 1;
  a.scale_log2 = d.scale_log2;
  a.fuse = fuse.out != nullptr && in.k_tree != nullptr;
  a.out = fuse.out;
  a.lse = fuse.lse;
  a.seg_sync = fuse.seg_sync;
  a.seg_err = fuse.seg_err;
  a.slot_bytes_o = (unsigned)slots.o_bytes;
  a.slot_bytes_l = (unsigned)slots.lse2_bytes;
  hipLaunchKernelGGL(inst->fn, dim3(pl.nwg, pl.row_groups), dim3(pl.waves * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace hta
