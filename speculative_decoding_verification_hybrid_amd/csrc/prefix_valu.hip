// Split-KV prefix kernel on the vector ALUs, for float32 inputs and for bf16
// layers whose G*T query rows per KV head are too few to fill a 32-row MFMA
// block. Same work split and partial-result slots as the MFMA kernel (see
// common.h); this one keeps everything in float32.
//
// A workgroup of 256 threads owns 16 query rows (grid.y picks which 16 of
// the M rows of a KV head). Thread (r, c), r = tid/16, c = tid%16, works on
// row r: it scores tokens c, c+16, c+32, c+48 of each 64-token tile against
// that row, and accumulates output dims c, c+16, ... (so neighbouring lanes
// touch neighbouring LDS words). Row max and sum are reduced over the 16
// lanes of a row with cross-lane exchanges. Online softmax in the log2 domain.
#include "common.h"
#include "hta_internal.h"

namespace hta {
namespace {

constexpr int NK = kTileTokens;

struct ValuArgs {
  const void* q;
  const void* k;
  const void* v;
  const int* prefix_len;
  float* slot_o;
  float* slot_lse2;
  int B, Hq, Hkv, G, T, Lcap, M;
  int nwg;
  float scale_log2;
};

template <int D, typename TIn>
__global__ void __launch_bounds__(256) prefix_valu_kernel(ValuArgs a) {
  constexpr int DS = D / 16;
  constexpr int KROW = D + 1;
  __shared__ float Qs[16][D + 1];
  __shared__ float Ks[NK * KROW];
  __shared__ float Vs[NK * D];
  __shared__ float Ps[16][NK];

  const TIn* qg = static_cast<const TIn*>(a.q);
  const TIn* kg = static_cast<const TIn*>(a.k);
  const TIn* vg = static_cast<const TIn*>(a.v);
  const int tid = threadIdx.x;
  const int rl = tid >> 4;
  const int sl = tid & 15;

  const int w = xcd_remap(blockIdx.x, a.nwg);
  const int64_t TT = total_tiles(a.prefix_len, a.B, a.Hkv, a.Lcap, NK);
  if (TT == 0) return;
  int64_t x = split_begin(w, a.nwg, TT);
  const int64_t x_end = split_begin(w + 1, a.nwg, TT);
  if (x >= x_end) return;

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
  const int row = blockIdx.y * 16 + rl;
  const bool row_ok = row < a.M;

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
    const TIn* qp = qg + (size_t)(b * a.Hq + g * a.G) * a.T * D;

    __syncthreads();  // LDS of the previous piece is no longer read
#pragma unroll
    for (int e = 0; e < DS; ++e) {
      const int d = sl + 16 * e;
      Qs[rl][d] = row_ok ? load_elem(qp + (size_t)row * D + d) : 0.f;
    }
    float o[DS];
#pragma unroll
    for (int e = 0; e < DS; ++e) o[e] = 0.f;
    float m = -__builtin_inff(), l = 0.f;

    for (int t = 0; t < ntiles; ++t) {
      const int base = tok_begin + t * NK;
      const int nvalid = min(NK, tok_end - base);
      __syncthreads();
      for (int idx = tid; idx < NK * D; idx += 256) {
        const int tk = idx / D, d = idx % D;
        const bool ok = tk < nvalid;
        const size_t off = kv_off + (size_t)(base + tk) * D + d;
        Ks[tk * KROW + d] = ok ? load_elem(kg + off) : 0.f;
        Vs[tk * D + d] = ok ? load_elem(vg + off) : 0.f;
      }
      __syncthreads();
      float s[4];
      float mx = -__builtin_inff();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tk = sl + 16 * j;
        float acc = 0.f;
        for (int d = 0; d < D; ++d) acc = fmaf(Qs[rl][d], Ks[tk * KROW + d], acc);
        s[j] = tk < nvalid ? acc * a.scale_log2 : -__builtin_inff();
        mx = fmaxf(mx, s[j]);
      }
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float mn = fmaxf(m, mx);
      const float alpha = fast_exp2(m - mn);
      m = mn;
      float ls = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = fast_exp2(s[j] - m);
        Ps[rl][sl + 16 * j] = p;
        ls += p;
      }
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) ls += __shfl_xor(ls, off);
      l = l * alpha + ls;
#pragma unroll
      for (int e = 0; e < DS; ++e) o[e] *= alpha;
      __syncthreads();
      for (int tk = 0; tk < nvalid; ++tk) {
        const float p = Ps[rl][tk];
#pragma unroll
        for (int e = 0; e < DS; ++e) o[e] = fmaf(p, Vs[tk * D + sl + 16 * e], o[e]);
      }
    }

    if (row_ok) {
      const float inv = 1.0f / l;
      float* op = a.slot_o + ((size_t)slot * a.M + row) * D;
#pragma unroll
      for (int e = 0; e < DS; ++e) op[sl + 16 * e] = o[e] * inv;
      if (sl == 0) a.slot_lse2[(size_t)slot * a.M + row] = m + fast_log2(l);
    }

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

typedef void (*KernelFn)(ValuArgs);

KernelFn pick(int D, bool bf16) {
  if (D == 128) return bf16 ? prefix_valu_kernel<128, unsigned short> : prefix_valu_kernel<128, float>;
  if (D == 64) return bf16 ? prefix_valu_kernel<64, unsigned short> : prefix_valu_kernel<64, float>;
  return nullptr;
}

}  // namespace

int prefix_valu_occupancy(int D, bool bf16) {
  KernelFn k = pick(D, bf16);
  if (!k) return 0;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(k), 256, 0) !=
      hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}

hipError_t launch_prefix_valu(const Dims& d, const PrefixLaunch& pl, const void* q,
                              const void* k_cache, const void* v_cache, const int* prefix_len,
                              Slots slots, hipStream_t s) {
  KernelFn k = pick(d.D, d.bf16);
  if (!k) return hipErrorInvalidValue;
  ValuArgs a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
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
  a.scale_log2 = d.scale_log2;
  hipLaunchKernelGGL(k, dim3(pl.nwg, pl.row_groups), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hta
