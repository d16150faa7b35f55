// Split-KV prefix kernel on bf16 MFMA (gfx950, v_mfma_f32_32x32x16_bf16).
//
// The cached part of Hybrid Tree Attention (LongSpec summary pages, "Fast
// Tree Attention"): every tree token attends to the whole KV prefix of its
// sequence with no mask. The G query heads that share a KV head and the T
// tree nodes form M = G*T query rows per KV head, so one pass over the KV
// serves all M rows; each workgroup streams one contiguous range of prefix
// tiles (see common.h) and leaves a normalised partial (o, log2-LSE) per
// row in a workspace slot for the merge kernel.
//
// Per workgroup: WQ waves, each owning QB blocks of 32 query rows. Per
// 64-token tile, all waves share one copy of K and V in LDS:
//   * K is stored row-major with a 16-byte pad per row (conflict-free
//     128-bit reads);
//   * V is stored transposed (D rows of 64 tokens, 16-byte chunks XOR
//     swizzled), so each lane reads 8 consecutive tokens of one dim.
// Scores are computed transposed, S^T = K . Q^T, so that each lane holds
// one query row (column of the MFMA result) and 16 tokens: the row max
// needs one cross-half exchange and the running (m, l) live in lanes. K rows
// are fed to the MFMA with bits 2 and 3 of the row index swapped, which
// makes the 8 scores a half-wave holds for each 16-token k-chunk belong to 8
// consecutive tokens; converted to bf16 they are directly the B operand of
// O^T += V^T . P^T, whose A operand is the 128-bit V^T read above.
// Online softmax runs in the log2 domain with a lazily updated maximum: the
// stored max only moves when a tile's max exceeds it by more than 8 (so
// exp2 stays below 256), which is exact because the same stale max is used
// for both the sum and the output.
#include "common.h"
#include "hta_internal.h"

namespace hta {
namespace {

constexpr int NK = kTileTokens;

template <int D>
struct MfmaTile {
  static constexpr int KROW = D + 8;  // bf16 per K row in LDS
  static constexpr int K_ELEMS = NK * KROW;
  static constexpr int V_ELEMS = D * NK;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;  // bf16 elements per stage
};

struct PrefixArgs {
  const unsigned short* q;
  const unsigned short* k;
  const unsigned short* v;
  const int* prefix_len;
  float* slot_o;
  float* slot_lse2;
  int B, Hq, Hkv, G, T, Lcap, M;
  int nwg, rows_per_group;
  float scale_log2;
};

// Physical 16-byte chunk of V^T row d holding logical chunk c.
__device__ __forceinline__ int vt_chunk(int d, int c) { return c ^ (((d >> 1) ^ (d >> 4)) & 7); }
// MFMA row -> token within a 32-token sub-tile: swap bits 2 and 3.
__device__ __forceinline__ int kperm(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

template <int D, int QB, int WQ>
__global__ void __launch_bounds__(64 * WQ) prefix_mfma_kernel(PrefixArgs a) {
  using TL = MfmaTile<D>;
  constexpr int NT = 64 * WQ;
  constexpr int KC = D / 16;             // k-chunks of Q.K^T
  constexpr int DB = D / 32;             // 32-dim blocks of O
  constexpr int DCH = D / 8;             // 16-byte chunks per K/V row
  constexpr int KCH = NK * DCH;          // K chunks per tile
  constexpr int NLK = (KCH + NT - 1) / NT;
  constexpr int VU = (NK / 4) * DCH;     // V units (4 tokens x 8 dims) per tile
  constexpr int NLV = (VU + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) unsigned short lds[2 * TL::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;
  const int l32 = lane & 31;

  const int w = xcd_remap(blockIdx.x, a.nwg);
  const int64_t TT = total_tiles(a.prefix_len, a.B, a.Hkv, a.Lcap, NK);
  if (TT == 0) return;
  int64_t x = split_begin(w, a.nwg, TT);
  const int64_t x_end = split_begin(w + 1, a.nwg, TT);
  if (x >= x_end) return;

  // Locate the segment holding tile x.
  int b = 0, nt_b = 0;
  int64_t seq_first = 0;
  for (b = 0; b < a.B; ++b) {
    nt_b = tiles_of(valid_prefix(a.prefix_len, b, a.Lcap), NK);
    const int64_t span = (int64_t)nt_b * a.Hkv;
    if (x < seq_first + span) break;
    seq_first += span;
  }
  if (b >= a.B || nt_b == 0) return;  // unreachable while x < TT; keeps the walk in bounds
  int g = (int)((x - seq_first) / nt_b);

  const int row_base = blockIdx.y * a.rows_per_group;
  const int row_limit = min(a.M, row_base + a.rows_per_group);

  while (x < x_end) {
    const int64_t s_first = seq_first + (int64_t)g * nt_b;
    const int tile0 = (int)(x - s_first);
    const int64_t piece_end = min(x_end, s_first + nt_b);
    const int ntiles = (int)(piece_end - x);
    const int L = valid_prefix(a.prefix_len, b, a.Lcap);
    const int slot = w + b * a.Hkv + g;
    const int tok_begin = tile0 * NK;
    const int tok_end = min((tile0 + ntiles) * NK, L);
    const size_t kv_off = (size_t)(b * a.Hkv + g) * (size_t)a.Lcap * D;
    const unsigned short* kp = a.k + kv_off;
    const unsigned short* vp = a.v + kv_off;
    const unsigned short* qp = a.q + (size_t)(b * a.Hq + g * a.G) * a.T * D;

    // Q^T fragments (B operand): lane holds row l32 of each q-block, dims 16c + 8hh .. +7.
    bf16x8 qf[QB][KC];
#pragma unroll
    for (int nb = 0; nb < QB; ++nb) {
      const int row = row_base + (wave * QB + nb) * 32 + l32;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        u32x4 r = {0u, 0u, 0u, 0u};
        if (row < row_limit) r = *(const u32x4*)(qp + (size_t)row * D + 16 * c + 8 * hh);
        qf[nb][c] = __builtin_bit_cast(bf16x8, r);
      }
    }

    u32x4 kreg[NLK];
    u32x4 vreg[NLV][4];
    auto load_tile = [&](int t) {
      const int base = tok_begin + t * NK;
#pragma unroll
      for (int i = 0; i < NLK; ++i) {
        const int idx = tid + i * NT;
        if (KCH % NT == 0 || idx < KCH) {
          const int tk = base + idx / DCH;
          u32x4 r = {0u, 0u, 0u, 0u};
          if (tk < tok_end) r = *(const u32x4*)(kp + (size_t)tk * D + (idx % DCH) * 8);
          kreg[i] = r;
        }
      }
#pragma unroll
      for (int i = 0; i < NLV; ++i) {
        const int u = tid + i * NT;
        if (VU % NT == 0 || u < VU) {
          const int tk0 = base + 4 * (u / DCH);
          const int dc = u % DCH;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            u32x4 r = {0u, 0u, 0u, 0u};
            if (tk0 + j < tok_end) r = *(const u32x4*)(vp + (size_t)(tk0 + j) * D + dc * 8);
            vreg[i][j] = r;
          }
        }
      }
    };
    auto store_tile = [&](int stage) {
      unsigned short* Ks = lds + stage * TL::STAGE;
      unsigned short* Vt = Ks + TL::K_ELEMS;
#pragma unroll
      for (int i = 0; i < NLK; ++i) {
        const int idx = tid + i * NT;
        if (KCH % NT == 0 || idx < KCH)
          *(u32x4*)(Ks + (idx / DCH) * TL::KROW + (idx % DCH) * 8) = kreg[i];
      }
#pragma unroll
      for (int i = 0; i < NLV; ++i) {
        const int u = tid + i * NT;
        if (VU % NT == 0 || u < VU) {
          const int tg = u / DCH;  // 4-token group
          const int dg = u % DCH;  // 8-dim group
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int d = dg * 8 + e;
            const unsigned a0 = vreg[i][0][e >> 1], a1 = vreg[i][1][e >> 1];
            const unsigned a2 = vreg[i][2][e >> 1], a3 = vreg[i][3][e >> 1];
            u32x2 pk;
            if (e & 1) {
              pk[0] = (a0 >> 16) | (a1 & 0xffff0000u);
              pk[1] = (a2 >> 16) | (a3 & 0xffff0000u);
            } else {
              pk[0] = (a0 & 0xffffu) | (a1 << 16);
              pk[1] = (a2 & 0xffffu) | (a3 << 16);
            }
            *(u32x2*)(Vt + d * NK + vt_chunk(d, tg >> 1) * 8 + (tg & 1) * 4) = pk;
          }
        }
      }
    };

    f32x16 O[QB][DB];
#pragma unroll
    for (int nb = 0; nb < QB; ++nb)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) O[nb][db][v] = 0.f;
    float m[QB], l[QB];
#pragma unroll
    for (int nb = 0; nb < QB; ++nb) {
      m[nb] = -__builtin_inff();
      l[nb] = 0.f;
    }

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
      if (t + 1 < ntiles) load_tile(t + 1);
      const unsigned short* Ks = lds + (t & 1) * TL::STAGE;
      const unsigned short* Vt = Ks + TL::K_ELEMS;
      const int nvalid = min(NK, tok_end - (tok_begin + t * NK));
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if (st * 32 >= nvalid) break;
        f32x16 S[QB];
#pragma unroll
        for (int nb = 0; nb < QB; ++nb)
#pragma unroll
          for (int v = 0; v < 16; ++v) S[nb][v] = 0.f;
        const unsigned short* krow = Ks + (st * 32 + kperm(l32)) * TL::KROW + 8 * hh;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const bf16x8 ka = *(const bf16x8*)(krow + 16 * c);
#pragma unroll
          for (int nb = 0; nb < QB; ++nb)
            S[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[nb][c], S[nb], 0, 0, 0);
        }
        if (st * 32 + 32 > nvalid) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int tl = st * 32 + 16 * (v >> 3) + 8 * hh + (v & 7);
            if (tl >= nvalid) {
#pragma unroll
              for (int nb = 0; nb < QB; ++nb) S[nb][v] = -__builtin_inff();
            }
          }
        }
        float mx[QB];
        bool need = false;
#pragma unroll
        for (int nb = 0; nb < QB; ++nb) {
          float r = S[nb][0];
#pragma unroll
          for (int v = 1; v < 16; ++v) r = fmaxf(r, S[nb][v]);
          r = fmaxf(r, __shfl_xor(r, 32));
          mx[nb] = r * a.scale_log2;
          need |= mx[nb] > m[nb] + 8.0f;
        }
        if (__any(need)) {
#pragma unroll
          for (int nb = 0; nb < QB; ++nb) {
            const float mn = fmaxf(m[nb], mx[nb]);
            const float alpha = fast_exp2(m[nb] - mn);
            m[nb] = mn;
            l[nb] *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) O[nb][db] *= alpha;
          }
        }
        bf16x8 P[QB][2];
#pragma unroll
        for (int nb = 0; nb < QB; ++nb) {
          const float nm = -m[nb];
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float p = fast_exp2(fmaf(S[nb][v], a.scale_log2, nm));
            l[nb] += p;
            P[nb][v >> 3][v & 7] = (__bf16)p;
          }
        }
#pragma unroll
        for (int kc2 = 0; kc2 < 2; ++kc2) {
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int d = db * 32 + l32;
            const bf16x8 va = *(const bf16x8*)(Vt + d * NK + vt_chunk(d, st * 4 + kc2 * 2 + hh) * 8);
#pragma unroll
            for (int nb = 0; nb < QB; ++nb)
              O[nb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, P[nb][kc2], O[nb][db], 0, 0, 0);
          }
        }
      }
      if (t + 1 < ntiles) store_tile((t + 1) & 1);
      __syncthreads();
    }

    // Epilogue: O^T holds dims db*32 + 8*(v/4) + 4*hh + v%4 of query row l32.
#pragma unroll
    for (int nb = 0; nb < QB; ++nb) {
      const float lt = l[nb] + __shfl_xor(l[nb], 32);
      const float inv = 1.0f / lt;
      const float lse2 = m[nb] + fast_log2(lt);
      const int row = row_base + (wave * QB + nb) * 32 + l32;
      if (row < row_limit) {
        float* op = a.slot_o + ((size_t)slot * a.M + row) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            f32x4 val;
            val[0] = O[nb][db][4 * g4 + 0] * inv;
            val[1] = O[nb][db][4 * g4 + 1] * inv;
            val[2] = O[nb][db][4 * g4 + 2] * inv;
            val[3] = O[nb][db][4 * g4 + 3] * inv;
            *(f32x4*)(op + db * 32 + 8 * g4 + 4 * hh) = val;
          }
        if (hh == 0) a.slot_lse2[(size_t)slot * a.M + row] = lse2;
      }
    }

    // Next segment (skip sequences with no tiles).
    x = piece_end;
    if (x >= x_end) break;
    if (++g == a.Hkv) {
      g = 0;
      seq_first += (int64_t)nt_b * a.Hkv;
      do {
        ++b;
        nt_b = tiles_of(valid_prefix(a.prefix_len, b, a.Lcap), NK);
      } while (nt_b == 0 && b + 1 < a.B);
      if (nt_b == 0) break;
    }
  }
}

typedef void (*KernelFn)(PrefixArgs);

// Instantiated shapes: one 32-row block per wave for 1..8 waves, or two
// blocks per wave with 4 waves (256 rows). Two blocks per wave need ~500 of
// the 512 VGPR+AGPR registers, which only fits at one wave per SIMD.
template <int D>
KernelFn pick_d(int wq, int qb) {
  if (qb == 2) return wq == 4 ? prefix_mfma_kernel<D, 2, 4> : nullptr;
  if (qb != 1) return nullptr;
  switch (wq) {
    case 1: return prefix_mfma_kernel<D, 1, 1>;
    case 2: return prefix_mfma_kernel<D, 1, 2>;
    case 3: return prefix_mfma_kernel<D, 1, 3>;
    case 4: return prefix_mfma_kernel<D, 1, 4>;
    case 5: return prefix_mfma_kernel<D, 1, 5>;
    case 6: return prefix_mfma_kernel<D, 1, 6>;
    case 7: return prefix_mfma_kernel<D, 1, 7>;
    case 8: return prefix_mfma_kernel<D, 1, 8>;
    default: return nullptr;
  }
}

KernelFn pick(int D, int wq, int qb) {
  if (D == 128) return pick_d<128>(wq, qb);
  if (D == 64) return pick_d<64>(wq, qb);
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

hipError_t launch_prefix_mfma(const Dims& d, const PrefixLaunch& pl, const void* q,
                              const void* k_cache, const void* v_cache, const int* prefix_len,
                              Slots slots, hipStream_t s) {
  KernelFn k = pick(d.D, pl.waves, pl.qb);
  if (!k) return hipErrorInvalidValue;
  PrefixArgs a;
  a.q = static_cast<const unsigned short*>(q);
  a.k = static_cast<const unsigned short*>(k_cache);
  a.v = static_cast<const unsigned short*>(v_cache);
  a.prefix_len = prefix_len;
  a.slot_o = slots.o;
  a.slot_lse2 = slots.lse2;
  a.B = d.B;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.G;
  a.T = d.T;
  a.Lcap = d.Lcap;
  a.M = d.M;
  a.nwg = pl.nwg;
  a.rows_per_group = pl.rows_per_group;
  a.scale_log2 = d.scale_log2;
  hipLaunchKernelGGL(k, dim3(pl.nwg, pl.row_groups), dim3(64 * pl.waves), 0, s, a);
  return hipGetLastError();
}

}  // namespace hta
