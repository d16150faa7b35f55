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
// Per workgroup: WQ waves, each owning one block of 32 query rows (two waves
// per SIMD at WQ = 8, so one wave's softmax overlaps the other's MFMA). Per
// tile, all waves share one copy of K and V in LDS, both row-major with each
// row's 16-byte chunks XOR-swizzled so that the reads below are free of bank
// conflicts:
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
// Online softmax runs in the log2 domain with a lazily updated maximum: the
// stored max only moves when a tile's max exceeds it by more than 8 (so
// exp2 stays below 256), which is exact because the same stale max is used
// for both the sum and the output.
#include "common.h"
#include "hta_internal.h"

namespace hta {
namespace {

constexpr int NK = kTileTokens;

typedef short i16x4 __attribute__((ext_vector_type(4)));

struct PrefixArgs {
  const unsigned short* q;
  const unsigned short* k;
  const unsigned short* v;
  const unsigned short* kt;  // tree keys (fused tree part) or null
  const unsigned short* vt;
  const int* parent;
  const int* prefix_len;
  float* slot_o;
  float* slot_lse2;
  int* err_b;
  int* status;
  int B, Hq, Hkv, G, T, Lcap, M;
  int nwg, rows_per_group, tree_tiles;
  float scale_log2;
};

// XOR swizzle of the 16-byte chunks of tile row r: D = 128 rows span all 64
// banks, D = 64 rows half of them. Conflict-free for the 16 distinct rows of a
// K read and for the 4 rows x 4 chunks of a transposed V read.
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

template <int D, int WQ>
__global__ void __launch_bounds__(64 * WQ) prefix_mfma_kernel(PrefixArgs a) {
  constexpr int NT = 64 * WQ;
  constexpr int KC = D / 16;          // k-chunks of K.Q^T
  constexpr int DB = D / 32;          // 32-dim blocks of O
  constexpr int DCH = D / 8;          // 16-byte chunks per row
  constexpr int TILE = NK * D;        // bf16 elements of one K (or V) tile
  constexpr int CH = 2 * NK * DCH;    // chunks of K + V per tile
  constexpr int NL = (CH + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) unsigned short lds[2 * 2 * TILE];
  __shared__ int par_s[64];
  __shared__ unsigned long long anc_s[64];
  __shared__ int bad_s;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;
  const int l32 = lane & 31;
  const int grp = lane >> 4;  // 16-lane group (transposed V reads)
  const int gl = lane & 15;

  const int w = xcd_remap(blockIdx.x, a.nwg);
  const unsigned TT = total_tiles(a.prefix_len, a.B, a.Hkv, a.Lcap, NK, a.tree_tiles);
  if (TT == 0) return;
  unsigned x = split_begin(w, a.nwg, TT);
  const unsigned x_end = split_begin(w + 1, a.nwg, TT);
  if (x >= x_end) return;
  SegmentWalk sw;
  if (!walk_start(&sw, x, a.prefix_len, a.B, a.Hkv, a.Lcap, NK, a.tree_tiles)) return;

  const int row = blockIdx.y * a.rows_per_group + wave * 32 + l32;  // this lane's query row
  const int row_limit = min(a.M, (int)(blockIdx.y + 1) * a.rows_per_group);
  const bool row_ok = row < row_limit;
  const int node = row_ok ? row % a.T : 0;

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

    if (has_tree) {
      if (tid == 0) bad_s = 0;
      if (tid < a.T) par_s[tid] = a.parent[(size_t)b * a.T + tid];
      __syncthreads();
      if (tid < a.T) {
        bool ok = true;
        anc_s[tid] = ancestor_word(par_s, tid, &ok);
        if (!ok) bad_s = 1;
      }
      // read after the barrier that follows the first tile store below
    }

    // Q^T fragments (B operand of S^T = K.Q^T): row `row`, dims 16c + 8hh .. +7.
    bf16x8 qf[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      u32x4 r = {0u, 0u, 0u, 0u};
      if (row_ok) r = *(const u32x4*)(qp + (size_t)row * D + 16 * c + 8 * hh);
      qf[c] = __builtin_bit_cast(bf16x8, r);
    }

    // Stage a tile through registers: chunk idx < NK*DCH is K, the rest V.
    // Rows past the tile's valid tokens are zero (V of a masked token must be 0).
    u32x4 reg[NL];
    auto load_tile = [&](int ti) {
      const bool tree = ti >= n_prefix;
      const unsigned short* ks = tree ? a.kt + kt_off : kp + (size_t)ti * NK * D;
      const unsigned short* vs = tree ? a.vt + kt_off : vp + (size_t)ti * NK * D;
      const int nv = tree ? a.T : min(NK, L - ti * NK);
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int idx = tid + i * NT;
        if (CH % NT == 0 || idx < CH) {
          const int is_v = idx >= NK * DCH;
          const int e = idx - is_v * NK * DCH;
          const int r = e / DCH, c = e % DCH;
          u32x4 val = {0u, 0u, 0u, 0u};
          if (r < nv) val = *(const u32x4*)((is_v ? vs : ks) + (size_t)r * D + c * 8);
          reg[i] = val;
        }
      }
    };
    auto store_tile = [&](int stage) {
      unsigned short* base = lds + stage * 2 * TILE;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int idx = tid + i * NT;
        if (CH % NT == 0 || idx < CH) {
          const int is_v = idx >= NK * DCH;
          const int e = idx - is_v * NK * DCH;
          const int r = e / DCH, c = e % DCH;
          *(u32x4*)(base + is_v * TILE + r * D + ((c ^ swz<D>(r)) << 3)) = reg[i];
        }
      }
    };

    f32x16 O[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) O[db][v] = 0.f;
    float m = -__builtin_inff(), l = 0.f;
    unsigned long long anc_row = 0ull;

    load_tile(tile0);
    store_tile(0);
    __syncthreads();
    if (has_tree) anc_row = anc_s[node];

    for (int t = 0; t < ntiles; ++t) {
      const int ti = tile0 + t;
      if (t + 1 < ntiles) load_tile(ti + 1);
      const unsigned short* Ks = lds + (t & 1) * 2 * TILE;
      const unsigned short* Vs = Ks + TILE;
      const bool tree = ti >= n_prefix;
      const int nvalid = tree ? a.T : min(NK, L - ti * NK);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if (st * 32 >= nvalid) break;
        f32x16 S;
#pragma unroll
        for (int v = 0; v < 16; ++v) S[v] = 0.f;
        const int kr = st * 32 + kperm(l32);
        const unsigned short* krow = Ks + kr * D;
        const int ksw = swz<D>(kr);
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const bf16x8 ka = *(const bf16x8*)(krow + (((2 * c + hh) ^ ksw) << 3));
          S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[c], S, 0, 0, 0);
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
          for (int v = 0; v < 16; ++v)
            S[v] += __uint_as_float((((vis >> v) & 1u) - 1u) & 0xff800000u);
        }
        float mx = fmaxf(fmaxf(S[0], S[1]), S[2]);
#pragma unroll
        for (int v = 3; v < 15; v += 2) mx = fmaxf(fmaxf(mx, S[v]), S[v + 1]);
        mx = fmaxf(mx, S[15]);
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * a.scale_log2;
        if (__any(mx > m + 8.0f)) {
          const float mn = fmaxf(m, mx);
          const float alpha = m == -__builtin_inff() ? 0.f : fast_exp2(m - mn);
          m = mn;
          l *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) O[db] *= alpha;
        }
        const float nm = m == -__builtin_inff() ? 0.f : -m;
        bf16x8 P[2];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = fast_exp2(fmaf(S[v], a.scale_log2, nm));
          l += p;
          P[v >> 3][v & 7] = (__bf16)p;
        }
        // O^T += V^T . P^T over the two 16-token k-chunks of this sub-tile.
#pragma unroll
        for (int kc2 = 0; kc2 < 2; ++kc2) {
          const int vr = st * 32 + 16 * kc2 + 8 * hh + (gl >> 2);  // rows vr and vr + 4
          const unsigned short* vrow0 = Vs + vr * D;
          const unsigned short* vrow1 = vrow0 + 4 * D;
          const int sw0 = swz<D>(vr), sw1 = swz<D>(vr + 4);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int dcol = db * 32 + 16 * (grp & 1) + 4 * (gl & 3);
            const int ch = dcol >> 3, half = (dcol >> 2) & 1;
            const i16x4 lo = lds_read_tr(vrow0 + (((ch ^ sw0) << 3) | (half << 2)));
            const i16x4 hi = lds_read_tr(vrow1 + (((ch ^ sw1) << 3) | (half << 2)));
            const bf16x8 va =
                __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, P[kc2], O[db], 0, 0, 0);
          }
        }
      }
      if (t + 1 < ntiles) store_tile((t + 1) & 1);
      __syncthreads();
    }

    // Epilogue: O^T holds dims db*32 + 8*(v/4) + 4*hh + v%4 of query row `row`.
    const float lt = l + __shfl_xor(l, 32);
    if (row_ok) {
      const float inv = 1.0f / lt;
      float* op = a.slot_o + ((size_t)slot * a.M + row) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          f32x4 val;
          val[0] = O[db][4 * g4 + 0] * inv;
          val[1] = O[db][4 * g4 + 1] * inv;
          val[2] = O[db][4 * g4 + 2] * inv;
          val[3] = O[db][4 * g4 + 3] * inv;
          *(f32x4*)(op + db * 32 + 8 * g4 + 4 * hh) = val;
        }
      if (hh == 0) a.slot_lse2[(size_t)slot * a.M + row] = m + fast_log2(lt);
    }
    if (has_tree && g == 0 && blockIdx.y == 0 && tid == 0) {
      a.err_b[b] = bad_s;
      if (bad_s) atomicOr(a.status, kStatusBadTree);
    }

    x = piece_end;
    if (x >= x_end) break;
    if (!walk_next(&sw, a.prefix_len, a.B, a.Hkv, a.Lcap, NK, a.tree_tiles)) break;
    __syncthreads();  // par_s / anc_s / bad_s of this piece are no longer read
  }
}

typedef void (*KernelFn)(PrefixArgs);

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

KernelFn pick(int D, int wq, int qb) {
  if (qb != 1) return nullptr;
  if (D == 128) return pick_d<128>(wq);
  if (D == 64) return pick_d<64>(wq);
  return nullptr;
}

}  // namespace

bool prefix_mfma_supported(int D, int waves, int qb) { return pick(D, waves, qb) != nullptr; }

int prefix_mfma_occupancy(int D, int waves, int qb) {
  KernelFn k = pick(D, waves, qb);
  if (!k) return 0;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(k), 64 * waves, 0) !=
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
  a.slot_o = slots.o;
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
  hipLaunchKernelGGL(k, dim3(pl.nwg, pl.row_groups), dim3(64 * pl.waves), 0, s, a);
  return hipGetLastError();
}

}  // namespace hta
