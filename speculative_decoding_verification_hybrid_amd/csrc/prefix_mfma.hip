// Split-KV attention kernel on bf16 MFMA (gfx950, v_mfma_f32_32x32x16_bf16).
//
// LongSpec summary pages, "Fast Tree Attention": every tree token attends to
// the whole cached KV prefix of its sequence with no mask (the cached part)
// and to its own root path among the tree tokens (the speculative part,
// masked); the parts are combined with the log-sum-exp trick. Here the G
// query heads that share a KV head and the T tree nodes form M = G*T query
// rows per KV head, so one pass over the KV serves all M rows. Each
// workgroup streams one contiguous range of 64-token tiles (see common.h) and
// leaves a normalised partial (o, log2-LSE) per row in a workspace slot for
// the merge kernel. When the tree part is fused in, each (sequence, KV head)
// ends with one extra tile holding its tree keys/values, scored under the
// ancestor mask built in LDS from parent[] -- the same online softmax then
// covers both parts, and the merge combines the pieces.
//
// Memory pipeline: K and V tiles go from HBM straight into LDS with
// global_load_lds_dwordx4 (no staging registers), through 4 LDS stages, so up
// to 3 tiles (96 KB at D = 128) are in flight per workgroup while one is
// consumed. Each wave waits for its own copies (vmcnt), then all waves meet at
// one barrier per tile, after which the stage of the tile just finished is
// refilled. The copies are issued from inline assembly, so the compiler's wait
// insertion never sees them (it would otherwise drain the whole copy queue
// before LDS reads it cannot prove disjoint from a copy in flight); every wait
// on them is explicit (the Q fragments are loaded the same way, just before
// the first copies of a piece).
//
// One copy instruction moves 1 KB: 4 (D = 128) or 8 (D = 64) whole rows of K
// or V, read coalesced from HBM, with the lanes' 16-byte chunks permuted on
// the way into LDS. K rows keep their 16-byte chunks XOR-swizzled by row; V is
// stored as 128-byte blocks of 4 tokens x 16 dims, which is exactly what one
// 16-lane group of a transposed read consumes.
//
// Compute: WQ waves (two per SIMD at WQ = 8), each owning one block of 32
// query rows; the first wave of each SIMD runs at higher priority, so the pair
// drifts into alternating MFMA and softmax phases.
//   * scores are computed transposed, S^T = K . Q^T: each lane holds one
//     query row (a column of the MFMA result) and 16 tokens, so the row max
//     needs one cross-half exchange and the running (m, l) live in lanes;
//   * K rows are fed to the MFMA with bits 2 and 3 of the row index swapped,
//     which makes the 8 scores a half-wave holds for each 16-token k-chunk
//     belong to 8 consecutive tokens; converted to bf16 they are directly the
//     B operand of O^T += V^T . P^T;
//   * the V^T operand comes from ds_read_b64_tr_b16: in each 16-lane group,
//     lane i receives element i%4 of the 8-byte chunks read by lanes
//     4j + i/4 (j = 0..3), so lanes that read 4 dims of 4 consecutive tokens
//     hand each lane 4 consecutive tokens of one dim.
// LDS reads run ahead of their use: the V fragments of a 32-token sub-tile
// are read while its score MFMAs run, and the K fragments of the next
// sub-tile while the softmax runs.
// Online softmax runs in the log2 domain with a lazily updated maximum: the
// stored max only moves when a sub-tile's max exceeds it by more than 8 (so
// exp2 stays below 256), which is exact because the same stale max is used
// for both the sum and the output. The row max itself is only computed when
// the probabilities against the stored max sum to more than 256 (the sum
// bounds every term), which after the first sub-tile is rare.
#include <type_traits>

#include "hta_internal.h"
#include "prefix_mfma_common.h"

namespace hta {
namespace mfma {
namespace {

// Threads per workgroup: the WQ compute waves plus copy-only waves up to 4
// (WQ <= 4) or 8.
template <int WQ>
constexpr int threads_for() { return WQ <= 4 ? 256 : 512; }

template <int D, int WQ>
__global__ void __launch_bounds__(threads_for<WQ>()) prefix_mfma_kernel(PrefixArgs a) {
  constexpr int NWAVE = threads_for<WQ>() / 64;
  constexpr int KC = D / 16;          // k-chunks of K.Q^T
  constexpr int DB = D / 32;          // 32-dim blocks of O
  constexpr int DCH = D / 8;          // 16-byte chunks per row
  constexpr int DG = D / 16;          // 16-dim groups (V blocks per 4 tokens)
  constexpr int TILE = NK * D;        // bf16 elements of one K (or V) tile
  constexpr int STAGE = 2 * TILE;     // K tile, then V tile
  constexpr int RPB = 64 / DCH;       // rows per 1 KB copy block
  constexpr int NBLK = NK / RPB;      // copy blocks per K (or V) tile
  constexpr int NBH = NBLK / NWAVE;   // K (and V) copy instructions per wave per tile
  constexpr int GRP = 2 * NBH;        // copy instructions per wave per tile
  constexpr int SROW = D + 8;         // epilogue staging row (16-byte aligned rows)
  static_assert(NBLK % NWAVE == 0, "copy blocks split evenly over the waves");
  static_assert(NSTAGE * STAGE >= NWAVE * 32 * SROW, "epilogue staging fits in the tile buffers");
  static_assert(3 * GRP < 64, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) unsigned short lds[NSTAGE * STAGE];
  __shared__ int par_s[64];
  __shared__ unsigned long long anc_s[64];
  __shared__ int bad_s;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar control flow
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int grp = lane >> 4;  // 16-lane group (transposed V reads)
  const int gl = lane & 15;
  if (NWAVE == 8 && wave < 4) __builtin_amdgcn_s_setprio(2);

  const int w = xcd_remap(blockIdx.x, a.nwg);
  const unsigned TT = total_tiles(a.prefix_len, a.B, a.Hkv, a.Lcap, NK, a.tree_tiles);
  if (TT == 0) return;
  unsigned x = split_begin(w, a.nwg, TT);
  const unsigned x_end = split_begin(w + 1, a.nwg, TT);
  if (x >= x_end) return;
  SegmentWalk sw;
  if (!walk_start(&sw, x, a.prefix_len, a.B, a.Hkv, a.Lcap, NK, a.tree_tiles)) return;

  const bool computes = wave < WQ;  // copy-only waves issue copies and meet the barriers
  const int row = blockIdx.y * a.rows_per_group + wave * 32 + l32;  // this lane's query row
  const int row_limit = min(a.M, (int)(blockIdx.y + 1) * a.rows_per_group);
  const bool row_ok = computes && row < row_limit;
  const int node = row_ok ? row % a.T : 0;

  // Lane-constant LDS offsets (elements, within a stage). K: the fragments of
  // this lane's row; the swizzle depends only on the row's low 4 bits, which
  // are the same in both 32-token sub-tiles.
  int koff[KC];
  {
    const int kr = kperm(l32);
#pragma unroll
    for (int c = 0; c < KC; ++c) koff[c] = kr * D + (((2 * c + hh) ^ swz<D>(kr)) << 3);
  }
  // V block (4 tokens x 16 dims, 64 elements) of tokens 4u.., dims 16g..: (u * DG + g) * 64.
  // A transposed read of tokens 32st + 16kc + 8hh + 4rr, dims 32db + 16(grp&1) + 0..15
  // reads block ((8st + 4kc + 2hh + rr) * DG + 2db + (grp&1)), lane gl at 4 gl.
  const int voff = TILE + (2 * hh * DG + (grp & 1)) * 64 + 4 * gl;
  // This lane's part of a 1 KB copy block. K: row within the block and logical
  // chunk. V: token within the block and dims (the V block layout above).
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
    const int n_prefix = sw.nt - a.tree_tiles;  // tiles of cached KV; the tree tile (if any) follows
    const bool has_tree = a.tree_tiles && tile0 + ntiles > n_prefix;
    const int slot = w + b * a.Hkv + g;
    const size_t kv_off = (size_t)(b * a.Hkv + g) * (size_t)a.Lcap * D;
    const unsigned short* kp = a.k + kv_off;
    const unsigned short* vp = a.v + kv_off;
    const size_t kt_off = (size_t)(b * a.Hkv + g) * a.T * D;
    const unsigned short* qp = a.q + (size_t)(b * a.Hq + g * a.G) * a.T * D;

    unsigned long long anc_row = 0ull;
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
      anc_row = anc_s[node];
    }

    // Q^T fragments (B operand of S^T = K.Q^T): row `row`, dims 16c + 8hh .. +7.
    // Loaded from inline assembly, like the tile copies, so that one explicit
    // wait covers both: they are queued before the first tiles' copies and are
    // complete once tile 0 is. Rows past the limit load row 0 and are zeroed.
    bf16x8 qf[KC];
    {
      const unsigned short* qr = qp + (size_t)(row_ok ? row : 0) * D + 8 * hh;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        u32x4 r;
        asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r) : "v"(qr + 16 * c) : "memory");
        qf[c] = __builtin_bit_cast(bf16x8, r);
      }
    }
    // Queue the copies of tile t of the piece into stage t % NSTAGE: this
    // wave's NBH blocks of K and NBH blocks of V. Rows past the tile's valid
    // tokens repeat its last valid row, so every value read is finite and in
    // bounds; their scores are masked to -inf.
    auto copy_tile = [&](int t) __attribute__((always_inline)) {
      const int ti = tile0 + t;
      const bool tree = ti >= n_prefix;
      const unsigned short* ks = tree ? a.kt + kt_off : kp + (size_t)ti * NK * D;
      const unsigned short* vs = tree ? a.vt + kt_off : vp + (size_t)ti * NK * D;
      const int last = (tree ? a.T : min(NK, L - ti * NK)) - 1;
      unsigned short* dst = lds + (t % NSTAGE) * STAGE;
#pragma unroll
      for (int i = 0; i < NBH; ++i) {
        const int r0 = (wave + i * NWAVE) * RPB;  // first row of the block (wave-uniform)
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
    // Wait until at most n tiles' copies of this wave are still in flight.
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

    f32x16 O[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) O[db][v] = 0.f;
    float m = -__builtin_inff(), l = 0.f;

    bf16x8 ka[KC];
    auto load_k = [&](const unsigned short* kb) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < KC; ++c) ka[c] = *(const bf16x8*)(kb + koff[c]);
    };

    // Every stage starts filled: tile t goes to stage t % NSTAGE, and the stage
    // of tile t is refilled (with tile t + NSTAGE) once tile t is consumed.
    for (int t = 0; t < min(ntiles, NSTAGE); ++t) copy_tile(t);
    wait_tiles(min(ntiles, NSTAGE) - 1);  // tile 0 and the older Q loads have landed
    // Tie the Q registers to the wait: nothing below may read them earlier.
    // (The compiler still could copy them between the load and here; the CPU
    // test tests/test_q_load_isa.py checks the generated code for that.)
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      u32x4 r = __builtin_bit_cast(u32x4, qf[c]);
      asm volatile("" : "+v"(r));
      if (!row_ok) r = u32x4{0u, 0u, 0u, 0u};
      qf[c] = __builtin_bit_cast(bf16x8, r);
    }
    tile_barrier();
    if (computes) load_k(lds);

    for (int t = 0; t < ntiles; ++t) {
      const unsigned short* Ks = lds + (t % NSTAGE) * STAGE;
      const int ti = tile0 + t;
      const bool tree = ti >= n_prefix;
      const int nvalid = tree ? a.T : min(NK, L - ti * NK);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if (!computes || st * 32 >= nvalid) break;
        // S^T = K . Q^T for 32 tokens (K fragments already in registers).
        f32x16 S;
#pragma unroll
        for (int v = 0; v < 16; ++v) S[v] = 0.f;
#pragma unroll
        for (int c = 0; c < KC; ++c) S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], qf[c], S, 0, 0, 0);
        // V^T fragments of this sub-tile: tokens 16kc + 8hh + 0..7, dims 32db + lane%32.
        bf16x8 va[2][DB];
        {
          const unsigned short* vb = Ks + voff + 8 * st * DG * 64;
#pragma unroll
          for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const i16x4 lo = lds_read_tr(vb + (4 * kc * DG + 2 * db) * 64);
              const i16x4 hi = lds_read_tr(vb + ((4 * kc + 1) * DG + 2 * db) * 64);
              va[kc][db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        }
        // S[v] scores token st*32 + 16*(v/8) + 8*hh + v%8 of the tile. On the
        // tree tile and on a ragged last tile, bit v of `vis` says whether that
        // token is seen; hidden scores get -inf added (no compares, no masks).
        if (tree || st * 32 + 32 > nvalid) {
          unsigned vis;
          const int j0 = st * 32 + 8 * hh;
          if (tree) {
            vis = (unsigned)((anc_row >> j0) & 0xffull) | ((unsigned)((anc_row >> (j0 + 16)) & 0xffull) << 8);
          } else {
            const int n0 = min(max(nvalid - j0, 0), 8), n1 = min(max(nvalid - j0 - 16, 0), 8);
            vis = ((1u << n0) - 1u) | (((1u << n1) - 1u) << 8);
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) S[v] += __uint_as_float((((vis >> v) & 1u) - 1u) & 0xff800000u);
        }
        // Probabilities against the stored max m; the row sum adds them in fp32
        // (four partial sums), the P.V product takes them rounded to bf16. The
        // sum bounds every term, so if it stays <= 256 so does each
        // p = 2^(s - m) and m can stay. Otherwise (and always while m is still
        // -inf) take the exact row max over both half-rows; if it exceeds m by
        // more than 8, raise m, rescale l and O, and recompute.
        float pr[16];
        auto probs = [&]() __attribute__((always_inline)) {
          const float nm = m == -__builtin_inff() ? 0.f : -m;
#pragma unroll
          for (int v = 0; v < 16; ++v) pr[v] = fast_exp2(fmaf(S[v], a.scale_log2, nm));
        };
        auto row_sum = [&]() __attribute__((always_inline)) {
          const float s0 = (pr[0] + pr[4]) + (pr[8] + pr[12]), s1 = (pr[1] + pr[5]) + (pr[9] + pr[13]);
          const float s2 = (pr[2] + pr[6]) + (pr[10] + pr[14]), s3 = (pr[3] + pr[7]) + (pr[11] + pr[15]);
          return (s0 + s1) + (s2 + s3);
        };
        probs();
        float ls = row_sum();
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
#pragma unroll
            for (int db = 0; db < DB; ++db) O[db] *= alpha;
            probs();
            ls = row_sum();
          }
        }
        bf16x8 P[2];
#pragma unroll
        for (int v = 0; v < 16; ++v) P[v >> 3][v & 7] = (__bf16)pr[v];
        l += ls;
        // K fragments of the next sub-tile of this tile, read while P.V runs.
        if (st == 0 && nvalid > 32) load_k(Ks + 32 * D);
        // O^T += V^T . P^T over the two 16-token k-chunks of this sub-tile.
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
          for (int db = 0; db < DB; ++db)
            O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kc][db], P[kc], O[db], 0, 0, 0);
      }
      if (t + 1 < ntiles) {
        // Tile t+1 has landed for every wave (at most tiles t+2, t+3 still in
        // flight: tiles up to t+3 have been queued) and every wave's reads of
        // tile t are done: its stage takes tile t+4. Then the K fragments of
        // tile t+1.
        __builtin_amdgcn_s_waitcnt(kLgkmZero);
        wait_tiles(min(ntiles - 2 - t, 2));
        tile_barrier();
        if (t + NSTAGE < ntiles) copy_tile(t + NSTAGE);
        if (computes) load_k(lds + ((t + 1) % NSTAGE) * STAGE);
      }
    }
    __syncthreads();  // no wave reads the tile buffers any more (all copies landed before the last barrier)

    // Epilogue: O^T holds dims db*32 + 8*(v/4) + 4*hh + v%4 of query row `row`.
    // Normalise, round to bf16 and stage this wave's 32 rows in LDS (rows
    // padded by 16 bytes), then write them out as whole contiguous rows.
    const float lt = half_sum(l);
    const float inv = 1.0f / lt;
    unsigned short* stg = lds + wave * 32 * SROW;
    if (computes) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + 8 * g4 + 4 * hh;
          u32x2 pk;
          pk[0] = (unsigned)float_to_bf16_bits(O[db][4 * g4 + 0] * inv) |
                  ((unsigned)float_to_bf16_bits(O[db][4 * g4 + 1] * inv) << 16);
          pk[1] = (unsigned)float_to_bf16_bits(O[db][4 * g4 + 2] * inv) |
                  ((unsigned)float_to_bf16_bits(O[db][4 * g4 + 3] * inv) << 16);
          *(u32x2*)(stg + l32 * SROW + d) = pk;
        }
    }
    if (row_ok && hh == 0) a.slot_lse2[(size_t)slot * a.M + row] = m + fast_log2(lt);
    __syncthreads();
    const int wrow0 = blockIdx.y * a.rows_per_group + wave * 32;  // first row of this wave
#pragma unroll
    for (int i = 0; i < (computes ? 32 * DCH / 64 : 0); ++i) {
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
    __syncthreads();  // staging area, par_s / anc_s / bad_s of this piece are no longer read
  }
}

template <int D>
KernelFn pick_d(int wq) {
  switch (wq) {
    case 1: return prefix_mfma_kernel<D, 1>;
    case 2: return prefix_mfma_kernel<D, 2>;
    case 3: return prefix_mfma_kernel<D, 3>;
    case 4: return prefix_mfma_kernel<D, 4>;
    case 5: return prefix_mfma_kernel<D, 5>;
    case 6: return prefix_mfma_kernel<D, 6>;
    case 7: return prefix_mfma_kernel<D, 7>;
    case 8: return prefix_mfma_kernel<D, 8>;
    default: return nullptr;
  }
}

KernelFn pick(int D, int waves, int qb) {
  if (qb == 2) return prefix_mfma2_pick(D, waves);
  if (qb != 1) return nullptr;
  return D == 128 ? pick_d<128>(waves) : D == 64 ? pick_d<64>(waves) : nullptr;
}

int threads_of(int waves, int qb) { return qb == 2 || waves <= 4 ? 256 : 512; }

}  // namespace
}  // namespace mfma

using mfma::KernelFn;
using mfma::PrefixArgs;
using mfma::pick;
using mfma::threads_of;

bool prefix_mfma_supported(int D, int waves, int qb) { return pick(D, waves, qb) != nullptr; }

int prefix_mfma_occupancy(int D, int waves, int qb) {
  KernelFn k = pick(D, waves, qb);
  if (!k) return 0;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(k), threads_of(waves, qb), 0) !=
      hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}

hipError_t launch_prefix_mfma(const Dims& d, const PrefixLaunch& pl, const PrefixInputs& in, Slots slots,
                              int* err_b, int* status, hipStream_t s) {
  KernelFn k = pick(d.D, pl.waves, pl.qb);
  if (!k) return hipErrorInvalidValue;
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
  a.tree_tiles = in.k_tree ? 1 : 0;
  a.scale_log2 = d.scale_log2;
  hipLaunchKernelGGL(k, dim3(pl.nwg, pl.row_groups), dim3(threads_of(pl.waves, pl.qb)), 0, s, a);
  return hipGetLastError();
}

}  // namespace hta
