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
// tile, all waves share one copy of K and V in LDS, both row-major. K rows are
// padded by 16 bytes and V rows by 64 bytes, which makes the reads below free
// of bank conflicts while every read is a base register plus an immediate:
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
  unsigned short* slot_o;  // bf16 partials
  float* slot_lse2;
  int* err_b;
  int* status;
  int B, Hq, Hkv, G, T, Lcap, M;
  int nwg, rows_per_group, tree_tiles;
  float scale_log2;
};

// LDS row strides (bf16 elements). K: 16-byte pad, so the 16 rows of a K
// fragment read start 4 banks apart. V: 64-byte pad, so the 4 rows x 4 chunks
// of a transposed V read cover all 64 banks once (D = 128: rows 16 banks
// apart; D = 64: rows 48 banks apart).
template <int D>
struct Rows {
  static constexpr int K = D + 8;
  static constexpr int V = D + 32;
};

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

// MFMA row -> token within a 32-token sub-tile: swap bits 2 and 3.
__device__ __forceinline__ int kperm(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

__device__ __forceinline__ i16x4 lds_read_tr(const unsigned short* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

// Threads per workgroup: the WQ compute waves plus loader-only waves up to 4
// (WQ <= 4) or 8, so no wave stages more than 8 chunks of a tile.
template <int WQ>
constexpr int threads_for() { return WQ <= 4 ? 256 : 512; }

template <int D, int WQ>
__global__ void __launch_bounds__(threads_for<WQ>()) prefix_mfma_kernel(PrefixArgs a) {
  constexpr int NT = threads_for<WQ>();
  constexpr int KC = D / 16;          // k-chunks of K.Q^T
  constexpr int DB = D / 32;          // 32-dim blocks of O
  constexpr int DCH = D / 8;          // 16-byte chunks per row
  constexpr int KR = Rows<D>::K, VR = Rows<D>::V;
  constexpr int KT = NK * KR;         // bf16 elements of one K tile
  constexpr int STAGE = KT + NK * VR; // K tile + V tile
  constexpr int CH = 2 * NK * DCH;    // 16-byte chunks of K + V per tile
  constexpr int NL = (CH + NT - 1) / NT;
  static_assert(2 * STAGE >= WQ * 32 * D, "epilogue staging reuses the tile buffers");

  __shared__ __attribute__((aligned(16))) unsigned short lds[2 * STAGE];
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

  const bool computes = wave < WQ;  // loader-only waves stage tiles and hit the barriers
  const int row = blockIdx.y * a.rows_per_group + wave * 32 + l32;  // this lane's query row
  const int row_limit = min(a.M, (int)(blockIdx.y + 1) * a.rows_per_group);
  const bool row_ok = computes && row < row_limit;
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
      unsigned short* base = lds + stage * STAGE;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int idx = tid + i * NT;
        if (CH % NT == 0 || idx < CH) {
          const int is_v = idx >= NK * DCH;
          const int e = idx - is_v * NK * DCH;
          const int r = e / DCH, c = e % DCH;
          *(u32x4*)(base + (is_v ? KT + r * VR : r * KR) + c * 8) = reg[i];
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
      const unsigned short* Ks = lds + (t & 1) * STAGE;
      const unsigned short* Vs = Ks + KT;
      const bool tree = ti >= n_prefix;
      const int nvalid = tree ? a.T : min(NK, L - ti * NK);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if (!computes || st * 32 >= nvalid) break;
        // S^T = K . Q^T for 32 tokens: fetch all 8 K fragments, then the MFMA chain.
        const unsigned short* krow = Ks + (st * 32 + kperm(l32)) * KR + 8 * hh;
        bf16x8 ka[KC];
#pragma unroll
        for (int c = 0; c < KC; ++c) ka[c] = *(const bf16x8*)(krow + 16 * c);
        f32x16 S;
#pragma unroll
        for (int v = 0; v < 16; ++v) S[v] = 0.f;
#pragma unroll
        for (int c = 0; c < KC; ++c) S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], qf[c], S, 0, 0, 0);
        // keep the K reads ahead of the chain (the scheduler would otherwise sink
        // each read next to its MFMA and pay the LDS latency 8 times)
        __builtin_amdgcn_sched_group_barrier(0x100, KC, 0);  // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, KC, 0);  // MFMAs
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
        }
        const float nm = m == -__builtin_inff() ? 0.f : -m;
        bf16x8 P[2];
        float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = fast_exp2(fmaf(S[v], a.scale_log2, nm));
          ls[v & 3] += p;
          P[v >> 3][v & 7] = (__bf16)p;
        }
        l += (ls[0] + ls[1]) + (ls[2] + ls[3]);
        // O^T += V^T . P^T over the two 16-token k-chunks of this sub-tile.
#pragma unroll
        for (int kc2 = 0; kc2 < 2; ++kc2) {
          // rows vr and vr + 4 of the tile; dims of this lane's 4-dim group
          const int vr = st * 32 + 16 * kc2 + 8 * hh + (gl >> 2);
          const unsigned short* vp0 = Vs + vr * VR + 16 * (grp & 1) + 4 * (gl & 3);
          bf16x8 va[DB];
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const i16x4 lo = lds_read_tr(vp0 + db * 32);
            const i16x4 hi = lds_read_tr(vp0 + 4 * VR + db * 32);
            va[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
#pragma unroll
          for (int db = 0; db < DB; ++db)
            O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db], P[kc2], O[db], 0, 0, 0);
        }
      }
      if (t + 1 < ntiles) store_tile((t + 1) & 1);
      __syncthreads();
    }

    // Epilogue: O^T holds dims db*32 + 8*(v/4) + 4*hh + v%4 of query row `row`.
    // Normalise, round to bf16 and stage this wave's 32 rows in LDS (16-byte
    // units XOR-swizzled by row), then write them out as whole contiguous rows.
    const float lt = half_sum(l);
    const float inv = 1.0f / lt;
    unsigned short* stg = lds + wave * 32 * D;
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
        *(u32x2*)(stg + l32 * D + ((((d >> 3) ^ (l32 & (DCH - 1)))) << 3) + (d & 7)) = pk;
      }
    }
    if (row_ok && hh == 0) a.slot_lse2[(size_t)slot * a.M + row] = m + fast_log2(lt);
    __syncthreads();
    const int wrow0 = blockIdx.y * a.rows_per_group + wave * 32;  // first row of this wave
#pragma unroll
    for (int i = 0; i < (computes ? 32 * DCH / 64 : 0); ++i) {
      const int u = i * 64 + lane;
      const int rr = u / DCH, c = u % DCH;
      const u32x4 val = *(const u32x4*)(stg + rr * D + ((c ^ (rr & (DCH - 1))) << 3));
      if (wrow0 + rr < row_limit)
        *(u32x4*)(a.slot_o + ((size_t)slot * a.M + wrow0 + rr) * D + c * 8) = val;
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
  return D == 128 ? pick_d<128>(wq) : D == 64 ? pick_d<64>(wq) : nullptr;
}

int threads_of(int waves) { return waves <= 4 ? 256 : 512; }

}  // namespace

bool prefix_mfma_supported(int D, int waves, int qb) { return pick(D, waves, qb) != nullptr; }

int prefix_mfma_occupancy(int D, int waves, int qb) {
  KernelFn k = pick(D, waves, qb);
  if (!k) return 0;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(k),
                                                   threads_of(waves), 0) !=
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
  hipLaunchKernelGGL(k, dim3(pl.nwg, pl.row_groups), dim3(threads_of(pl.waves)), 0, s, a);
  return hipGetLastError();
}

}  // namespace hta
