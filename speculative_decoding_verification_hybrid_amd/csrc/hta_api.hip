// C ABI of libhta: handle, launch planning, workspace and the entry points
// declared in include/hta.h.
#include <math.h>
#include <new>
#include <stdint.h>
#include <stdlib.h>

#include "common.h"
#include "hta.h"
#include "hta_internal.h"

struct hta_handle_s {
  hta_config_t cfg;
  hta::Dims dims;
  hta::PrefixLaunch pl;
  hta_plan_t plan;
  void* ws;
  hta::Slots slots;
  int* err_b;        // [B] bad-tree flags of the last call
  int* status;       // sticky HTA_STATUS_* bits
  unsigned long long* argmax_part;  // [B*T*kArgmaxMaxSplit] partial argmax keys (hta_accept)
  unsigned* seq_count;              // [B] arrival counters of hta_commit; zero between calls
  unsigned long long* topk_part;    // [B * kMaxTreeSplit * (kMaxTreeGuesses + 1)] keys (hta_build_tree)
  int* tree_aux;                    // [2 * B * (kMaxTreeGuesses + 1)] match ends, x1 + guesses
  int* seg_sync;                    // [2 * B * Hkv * row_groups] fused-merge arrivals / departures
  int* seg_err;                     // [B * Hkv * row_groups] fused-merge tree checks
  bool fuse_merge;                  // hta_verify_attn merges inside the split-KV launch
};

struct hta_ngram_index_s {
  hta::NgramIndex ix;  // table [B][2^slots_log2][2], len [B], in one allocation
  int device;
};

namespace {

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Split weight of a tree tile in the handle's split-KV launches with tree tiles.
int tree_weight(const hta_handle_s* h) { return h->pl.path == HTA_PATH_MFMA ? hta::kTreeTileWeight : 1; }

int check_hip(hipError_t e) { return e == hipSuccess ? HTA_OK : HTA_ERR_HIP; }

// Tensor arguments are read with 16-byte vector loads.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
template <typename... P>
bool all_aligned(const P*... p) {
  return (aligned16(p) && ...);
}

int validate(const hta_config_t* c) {
  if (!c) return HTA_ERR_INVALID_ARG;
  if (c->batch < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 1 ||
      c->tree_nodes < 1 || c->kv_capacity < 1)
    return HTA_ERR_INVALID_ARG;
  if (c->n_q_heads % c->n_kv_heads != 0) return HTA_ERR_INVALID_ARG;
  if (c->dtype != HTA_F32 && c->dtype != HTA_BF16) return HTA_ERR_INVALID_ARG;
  if (c->num_workgroups < 0) return HTA_ERR_INVALID_ARG;
  if (c->force_path < HTA_PATH_AUTO || c->force_path > HTA_PATH_DOT) return HTA_ERR_INVALID_ARG;
  if (!(c->softmax_scale == c->softmax_scale)) return HTA_ERR_INVALID_ARG;  // NaN
  if (c->head_dim != 64 && c->head_dim != 128) return HTA_ERR_UNSUPPORTED;
  if (c->tree_nodes > 64) return HTA_ERR_UNSUPPORTED;
  if (c->force_path == HTA_PATH_MFMA && c->dtype != HTA_BF16) return HTA_ERR_UNSUPPORTED;
  if (c->force_path == HTA_PATH_DOT &&
      !hta::prefix_dot_supported(c->head_dim, (c->n_q_heads / c->n_kv_heads) * c->tree_nodes,
                                 c->dtype == HTA_BF16))
    return HTA_ERR_UNSUPPORTED;
  if (c->qblocks_per_wave < 0 || c->qblocks_per_wave > 2) return HTA_ERR_INVALID_ARG;
  if (c->fuse_merge != 0 && c->fuse_merge != 1) return HTA_ERR_INVALID_ARG;
  // Index arithmetic limits: rows and per-sequence KV spans stay within int32.
  const int64_t rows = (int64_t)c->batch * c->n_q_heads * c->tree_nodes;
  if (rows * c->head_dim > INT32_MAX) return HTA_ERR_UNSUPPORTED;
  if ((int64_t)c->kv_capacity * c->head_dim > INT32_MAX) return HTA_ERR_UNSUPPORTED;
  if ((int64_t)c->batch * c->n_kv_heads > (1 << 20)) return HTA_ERR_UNSUPPORTED;
  return HTA_OK;
}

// Split-KV kernel shape. MFMA path: query rows in blocks of 32; a wave owns
// qb blocks (one wave per SIMD, at most 4 per workgroup; 2, or 4 when fewer
// blocks would leave a wave count that is not 1, 2 or 4); more rows than
// one workgroup holds go to further row groups (grid.y). The plan takes qb = 2
// whenever there are two blocks or more, so every K / V fragment read from LDS
// feeds two MFMAs; qb = 1 is taken on request or for a single block, and at
// D = 128 it may use up to 8 waves (two per SIMD, accumulators in VGPRs).
// VALU path: 16 rows per workgroup. DOT path: up to 8 rows per workgroup of
// 4 waves (two row groups above 8 rows).
void plan_rows(const hta::Dims& d, int path, int qb_req, hta::PrefixLaunch* pl) {
  pl->path = path;
  if (path == HTA_PATH_MFMA) {
    pl->tile_tokens = hta::kMfmaTileTokens;
    const int nqb = (d.M + 31) / 32;
    const int qb = qb_req > 0 ? qb_req : (nqb >= 2 ? 2 : 1);
    const int max_waves = qb == 1 && d.D == 128 ? 8 : 4;  // qb = 1 at D = 128: up to two waves per SIMD
    const int max_blocks = max_waves * qb;      // blocks per workgroup
    const int rg = (nqb + max_blocks - 1) / max_blocks;
    const int per = (nqb + rg - 1) / rg;        // blocks per row group
    int waves = (per + qb - 1) / qb;
    waves = waves <= 1 ? 1 : waves <= 2 ? 2 : waves <= 4 ? 4 : 8;
    pl->row_groups = rg;
    pl->rows_per_group = per * 32;
    pl->waves = waves;
    pl->qb = qb;
  } else if (path == HTA_PATH_DOT) {
    pl->tile_tokens = hta::kTileTokens;
    pl->row_groups = hta::dot_row_groups(d.M);
    pl->rows_per_group = d.M > 8 ? 8 : d.M;
    pl->waves = 4;
    pl->qb = 0;
  } else {
    pl->tile_tokens = hta::kTileTokens;
    pl->row_groups = (d.M + 15) / 16;
    pl->rows_per_group = 16;
    pl->waves = 4;
    pl->qb = 0;
  }
}

#define HTA_TRY(expr)             \
  do {                            \
    int rc_ = (expr);             \
    if (rc_ != HTA_OK) return rc_; \
  } while (0)

}  // namespace

namespace hta {

int plan_launch(const hta_config_t* cfg, int cus, Dims* dp, PrefixLaunch* pl, int* occ_out) {
  Dims& d = *dp;
  d.B = cfg->batch;
  d.Hq = cfg->n_q_heads;
  d.Hkv = cfg->n_kv_heads;
  d.G = d.Hq / d.Hkv;
  d.T = cfg->tree_nodes;
  d.D = cfg->head_dim;
  d.Lcap = cfg->kv_capacity;
  d.M = d.G * d.T;
  d.bf16 = cfg->dtype == HTA_BF16;
  const float scale = cfg->softmax_scale > 0.f ? cfg->softmax_scale : 1.0f / sqrtf((float)d.D);
  d.scale_log2 = scale * kLog2e;

  int path = cfg->force_path;
  if (path == HTA_PATH_AUTO)
    path = (d.bf16 && d.M >= 16)                    ? HTA_PATH_MFMA
           : prefix_dot_supported(d.D, d.M, d.bf16) ? HTA_PATH_DOT
                                                    : HTA_PATH_VALU;
  plan_rows(d, path, cfg->qblocks_per_wave, pl);
  if (path == HTA_PATH_MFMA && !prefix_mfma_supported(d.D, pl->waves, pl->qb)) return HTA_ERR_UNSUPPORTED;
  const int occ = path == HTA_PATH_MFMA  ? prefix_mfma_occupancy(d.D, pl->waves, pl->qb)
                  : path == HTA_PATH_DOT ? prefix_dot_occupancy(d.D, d.M)
                                         : prefix_valu_occupancy(d.D, d.bf16);
  int64_t nwg = cfg->num_workgroups;
  if (nwg <= 0) {
    nwg = (int64_t)cus * (occ > 0 ? occ : 1) / pl->row_groups;
    // MFMA path with two or more workgroups per CU: one in eight fewer than
    // would fill every slot measured equal or faster on every shape tried
    // (up to 3.7 us per layer at 32k context), so take 7/8 of them.
    if (path == HTA_PATH_MFMA && occ >= 2) nwg = nwg * 7 / 8;
    nwg = nwg < 8 ? 8 : (nwg / 8) * 8;
  }
  // The kernels split tiles with 32-bit arithmetic: keep max_tiles * nwg < 2^32.
  const int nk = pl->tile_tokens;
  const int64_t max_tiles = (int64_t)d.B * d.Hkv *
                            ((d.Lcap + nk - 1) / nk +
                             tree_tiles_for(d.T, nk) * (path == HTA_PATH_MFMA ? kTreeTileWeight : 1));
  if (cfg->num_workgroups <= 0 && nwg > max_tiles) nwg = max_tiles;
  const int64_t nwg_cap = (int64_t)UINT32_MAX / max_tiles;
  if (nwg_cap < 1) return HTA_ERR_UNSUPPORTED;
  if (nwg > nwg_cap) nwg = nwg_cap;
  if (nwg > (1 << 20)) nwg = 1 << 20;
  pl->nwg = (int)nwg;
  *occ_out = occ;
  return HTA_OK;
}

int launch_split(const Dims& d, const PrefixLaunch& pl, const PrefixInputs& in, Slots slots, int* err_b,
                 int* status, hipStream_t s) {
  if (pl.path == HTA_PATH_MFMA) return check_hip(launch_prefix_mfma(d, pl, in, slots, err_b, status, s));
  if (pl.path == HTA_PATH_DOT) return check_hip(launch_prefix_dot(d, pl, in, slots, err_b, status, s));
  return check_hip(launch_prefix_valu(d, pl, in, slots, err_b, status, s));
}

}  // namespace hta

namespace {
// The tree-building arguments shared by hta_build_tree and its indexed form.
int tree_params(const hta_tree_params_t* params, int32_t vocab, int32_t logits_dtype, hta::TreeParams* p) {
  if (logits_dtype != HTA_F32 && logits_dtype != HTA_BF16) return HTA_ERR_INVALID_ARG;
  if (params->k < 0 || params->k > HTA_MAX_TREE_GUESSES || params->m < 1 || params->m > HTA_MAX_NGRAM ||
      params->keep_first < 0 || params->keep_first > 64)
    return HTA_ERR_INVALID_ARG;
  for (int r = 0; r < params->k; ++r)
    if (params->keep[r] < 0 || params->keep[r] > 64) return HTA_ERR_INVALID_ARG;
  if (vocab < params->k + 1) return HTA_ERR_INVALID_ARG;
  if (hta::topk_split_for(vocab) > hta::kMaxTreeSplit) return HTA_ERR_UNSUPPORTED;
  p->k = params->k;
  p->m = params->m;
  p->keep_first = params->keep_first;
  for (int r = 0; r < hta::kMaxTreeGuesses; ++r) p->keep[r] = r < params->k ? params->keep[r] : 0;
  return HTA_OK;
}
}  // namespace

static int launch_split(hta_handle_t h, const hta::PrefixInputs& in, hipStream_t s) {
  return hta::launch_split(h->dims, h->pl, in, h->slots, h->err_b, h->status, s);
}

extern "C" {

int hta_validate_config(const hta_config_t* cfg) { return validate(cfg); }

const char* hta_status_string(int status) {
  switch (status) {
    case HTA_OK: return "ok";
    case HTA_ERR_INVALID_ARG: return "invalid argument";
    case HTA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case HTA_ERR_NO_MEMORY: return "workspace allocation failed";
    case HTA_ERR_HIP: return "HIP runtime error";
    case HTA_ERR_BAD_TREE: return "parent array breaks -1 <= parent[i] < i";
    case HTA_ERR_BAD_PREFIX: return "prefix_len outside [0, kv_capacity]";
    case HTA_ERR_NO_DEVICE: return "no usable GPU";
    case HTA_ERR_TOO_LARGE: return "shape needs more than the no-allocation entry point's scratch memory";
    default: return "unknown status";
  }
}

int hta_create(hta_handle_t* out, const hta_config_t* cfg) {
  if (!out) return HTA_ERR_INVALID_ARG;
  *out = nullptr;
  HTA_TRY(validate(cfg));
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return HTA_ERR_NO_DEVICE;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return HTA_ERR_NO_DEVICE;

  hta_handle_s* h = new (std::nothrow) hta_handle_s();
  if (!h) return HTA_ERR_NO_MEMORY;
  h->cfg = *cfg;
  hta::Dims& d = h->dims;
  int occ = 0;
  const int rc = hta::plan_launch(cfg, cus, &d, &h->pl, &occ);
  if (rc != HTA_OK) {
    delete h;
    return rc;
  }
  const int path = h->pl.path;
  const int64_t nwg = h->pl.nwg;
  const int64_t max_slots = nwg + (int64_t)d.B * d.Hkv - 1;
  size_t off = 0;
  const size_t off_so = off;
  const bool slot_bf16 = path == HTA_PATH_MFMA;
  off = align256(off + (size_t)max_slots * d.M * d.D * (slot_bf16 ? 2 : 4));
  const size_t off_sl = off;
  off = align256(off + (size_t)max_slots * d.M * sizeof(float));
  const size_t off_ap = off;
  off = align256(off + (size_t)d.B * d.T * hta::kArgmaxMaxSplit * sizeof(unsigned long long));
  const size_t off_tk = off;
  off = align256(off + (size_t)d.B * hta::kMaxTreeSplit * (hta::kMaxTreeGuesses + 1) * sizeof(unsigned long long));
  const size_t off_ta = off;
  off = align256(off + 2 * (size_t)d.B * (hta::kMaxTreeGuesses + 1) * sizeof(int));
  const size_t off_eb = off;
  off = align256(off + (size_t)d.B * sizeof(int));
  const size_t off_ct = off;
  off = align256(off + (size_t)d.B * sizeof(unsigned));
  const size_t off_st = off;
  off = align256(off + sizeof(int));
  const size_t off_ss = off;
  const int64_t n_seg = (int64_t)d.B * d.Hkv * h->pl.row_groups;
  off = align256(off + (size_t)n_seg * 2 * sizeof(int));
  const size_t off_se = off;
  off = align256(off + (size_t)n_seg * sizeof(int));
  if (hipMalloc(&h->ws, off) != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    return HTA_ERR_NO_MEMORY;
  }
  char* base = static_cast<char*>(h->ws);
  h->slots.o = base + off_so;
  h->slots.o_bf16 = slot_bf16;
  h->slots.lse2 = reinterpret_cast<float*>(base + off_sl);
  h->slots.o_bytes = off_sl - off_so;
  h->slots.lse2_bytes = off_ap - off_sl;
  h->err_b = reinterpret_cast<int*>(base + off_eb);
  h->status = reinterpret_cast<int*>(base + off_st);
  h->argmax_part = reinterpret_cast<unsigned long long*>(base + off_ap);
  h->seq_count = reinterpret_cast<unsigned*>(base + off_ct);
  h->topk_part = reinterpret_cast<unsigned long long*>(base + off_tk);
  h->tree_aux = reinterpret_cast<int*>(base + off_ta);
  h->seg_sync = reinterpret_cast<int*>(base + off_ss);
  h->seg_err = reinterpret_cast<int*>(base + off_se);
  // The fused merge waits for all workgroups of a segment, so every workgroup
  // of the launch must be resident at once: only when the grid fits the
  // device (the default plan does; a larger num_workgroups does not).
  // (The fused merge addresses the slots with 32-bit buffer offsets.)
  h->fuse_merge = cfg->fuse_merge != 0 && path == HTA_PATH_MFMA &&
                  (int64_t)h->pl.nwg * h->pl.row_groups <= (int64_t)cus * (occ > 0 ? occ : 1) &&
                  h->slots.o_bytes < ((size_t)1 << 31);
  if (hipMemset(base + off_eb, 0, off - off_eb) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess) {
    (void)hipFree(h->ws);
    delete h;
    return HTA_ERR_HIP;
  }

  hta_plan_t& p = h->plan;
  p.path = path;
  p.num_workgroups = h->pl.nwg;
  p.row_groups = h->pl.row_groups;
  p.rows_per_group = h->pl.rows_per_group;
  p.waves_per_workgroup = h->pl.waves;
  p.qblocks_per_wave = h->pl.qb;
  p.tile_tokens = h->pl.tile_tokens;
  p.max_slots = (int32_t)max_slots;
  p.workspace_bytes = (int64_t)off;
  p.device = dev;
  p.compute_units = cus;
  *out = h;
  return HTA_OK;
}

int hta_destroy(hta_handle_t h) {
  if (!h) return HTA_OK;
  int rc = HTA_OK;
  int cur = 0;
  if (hipGetDevice(&cur) == hipSuccess && cur != h->plan.device) (void)hipSetDevice(h->plan.device);
  if (hipDeviceSynchronize() != hipSuccess) rc = HTA_ERR_HIP;
  if (hipFree(h->ws) != hipSuccess) rc = HTA_ERR_HIP;
  if (cur != h->plan.device) (void)hipSetDevice(cur);
  delete h;
  return rc;
}

int hta_get_plan(hta_handle_t h, hta_plan_t* plan) {
  if (!h || !plan) return HTA_ERR_INVALID_ARG;
  *plan = h->plan;
  return HTA_OK;
}

int hta_verify_attn(hta_handle_t h, const void* q, const void* k_cache, const void* v_cache,
                    const void* k_tree, const void* v_tree, const int32_t* parent,
                    const int32_t* prefix_len, void* out, float* lse, void* stream) {
  if (!h || !q || !k_cache || !v_cache || !k_tree || !v_tree || !parent || !prefix_len || !out || !lse)
    return HTA_ERR_INVALID_ARG;
  if (!all_aligned(q, k_cache, v_cache, k_tree, v_tree, out)) return HTA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hta::PrefixInputs in = {q, k_cache, v_cache, k_tree, v_tree, parent, prefix_len};
  if (h->fuse_merge) {
    hta::FusedMerge fm;
    fm.out = out;
    fm.lse = lse;
    fm.seg_sync = h->seg_sync;
    fm.seg_err = h->seg_err;
    return check_hip(hta::launch_prefix_mfma(h->dims, h->pl, in, h->slots, h->err_b, h->status, s, fm));
  }
  HTA_TRY(launch_split(h, in, s));
  return check_hip(hta::launch_merge_slots(h->dims, h->pl.tile_tokens, h->pl.nwg,
                                           hta::tree_tiles_for(h->dims.T, h->pl.tile_tokens), tree_weight(h), prefix_len,
                                           h->slots, h->err_b, out, h->dims.bf16, lse, h->status, s));
}

int hta_cross_attn(hta_handle_t h, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* prefix_len, void* out, float* lse, void* stream) {
  if (!h || !q || !k_cache || !v_cache || !prefix_len || !out || !lse) return HTA_ERR_INVALID_ARG;
  if (!all_aligned(q, k_cache, v_cache, out)) return HTA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hta::PrefixInputs in = {q, k_cache, v_cache, nullptr, nullptr, nullptr, prefix_len};
  HTA_TRY(launch_split(h, in, s));
  return check_hip(hta::launch_merge_slots(h->dims, h->pl.tile_tokens, h->pl.nwg, 0, 1, prefix_len, h->slots,
                                           nullptr, out, h->dims.bf16, lse, h->status, s));
}

int hta_window_attn(hta_handle_t h, const void* q, const void* k_ring, const void* v_ring, const void* k_new,
                    const void* v_new, const int32_t* pos, void* out, float* lse, void* stream) {
  if (!h || !q || !k_ring || !v_ring || !k_new || !v_new || !pos || !out || !lse) return HTA_ERR_INVALID_ARG;
  if (!all_aligned(q, k_ring, v_ring, k_new, v_new, out)) return HTA_ERR_INVALID_ARG;
  if (h->dims.T > h->dims.Lcap) return HTA_ERR_UNSUPPORTED;  // more new tokens than the window holds
  return check_hip(hta::launch_window_attn(h->dims, q, k_ring, v_ring, k_new, v_new, pos, out, lse, h->status,
                                           static_cast<hipStream_t>(stream)));
}

int hta_window_append(hta_handle_t h, const void* k_new, const void* v_new, void* k_ring, void* v_ring,
                      int32_t* pos, void* stream) {
  if (!h || !k_new || !v_new || !k_ring || !v_ring || !pos) return HTA_ERR_INVALID_ARG;
  if (!all_aligned(k_new, v_new, static_cast<const void*>(k_ring), static_cast<const void*>(v_ring)))
    return HTA_ERR_INVALID_ARG;
  if (h->dims.T > h->dims.Lcap) return HTA_ERR_UNSUPPORTED;
  return check_hip(hta::launch_window_append(h->dims, k_new, v_new, k_ring, v_ring, pos, h->seq_count, h->status,
                                             static_cast<hipStream_t>(stream)));
}

int hta_build_tree(hta_handle_t h, const void* logits, int32_t vocab, int32_t logits_dtype, const int32_t* history,
                   int32_t history_cap, const int32_t* history_len, const hta_tree_params_t* params,
                   int32_t* tree_tokens, int32_t* parent, int32_t* n_nodes, void* stream) {
  if (!h || !logits || !history || !history_len || !params || !tree_tokens || !parent || !n_nodes)
    return HTA_ERR_INVALID_ARG;
  if (history_cap < 1) return HTA_ERR_INVALID_ARG;
  hta::TreeParams p;
  const int rc = tree_params(params, vocab, logits_dtype, &p);
  if (rc != HTA_OK) return rc;
  return check_hip(hta::launch_build_tree(h->dims, logits, vocab, logits_dtype == HTA_BF16, history, history_cap,
                                          history_len, p, h->topk_part, h->tree_aux, tree_tokens, parent, n_nodes, h->status,
                                          static_cast<hipStream_t>(stream)));
}

int hta_ngram_index_create(hta_ngram_index_t* out, int32_t batch, int32_t history_cap, int32_t m) {
  if (!out) return HTA_ERR_INVALID_ARG;
  *out = nullptr;
  if (batch < 1 || history_cap < 1 || m < 1 || m > HTA_MAX_NGRAM) return HTA_ERR_INVALID_ARG;
  if (history_cap > (1 << 26) || batch > (1 << 20)) return HTA_ERR_UNSUPPORTED;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return HTA_ERR_NO_DEVICE;
  int lg = 6;  // at least 64 slots, and at least twice the positions of a history
  while (((int64_t)1 << lg) < 2 * (int64_t)history_cap) ++lg;
  const size_t tab_bytes = (size_t)batch * ((size_t)hta::ngram_slot_ints(m) << lg) * sizeof(int);
  const size_t bytes = align256(tab_bytes) + (size_t)batch * sizeof(int);
  hta_ngram_index_s* x = new (std::nothrow) hta_ngram_index_s();
  if (!x) return HTA_ERR_NO_MEMORY;
  void* mem = nullptr;
  if (hipMalloc(&mem, bytes) != hipSuccess) {
    (void)hipGetLastError();
    delete x;
    return HTA_ERR_NO_MEMORY;
  }
  x->ix.table = static_cast<int*>(mem);
  x->ix.len = reinterpret_cast<int*>(static_cast<char*>(mem) + align256(tab_bytes));
  x->ix.B = batch;
  x->ix.cap = history_cap;
  x->ix.m = m;
  x->ix.slots_log2 = lg;
  x->device = dev;
  if (hta::launch_ngram_reset(x->ix, -1, nullptr) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    (void)hipFree(mem);
    delete x;
    return HTA_ERR_HIP;
  }
  *out = x;
  return HTA_OK;
}

int hta_ngram_index_destroy(hta_ngram_index_t idx) {
  if (!idx) return HTA_OK;
  int rc = HTA_OK;
  int cur = 0;
  if (hipGetDevice(&cur) == hipSuccess && cur != idx->device) (void)hipSetDevice(idx->device);
  if (hipDeviceSynchronize() != hipSuccess) rc = HTA_ERR_HIP;
  if (hipFree(idx->ix.table) != hipSuccess) rc = HTA_ERR_HIP;
  if (cur != idx->device) (void)hipSetDevice(cur);
  delete idx;
  return rc;
}

int hta_ngram_index_reset(hta_ngram_index_t idx, int32_t seq, void* stream) {
  if (!idx || seq < -1 || seq >= idx->ix.B) return HTA_ERR_INVALID_ARG;
  return check_hip(hta::launch_ngram_reset(idx->ix, seq, static_cast<hipStream_t>(stream)));
}

int hta_build_tree_indexed(hta_handle_t h, hta_ngram_index_t idx, const void* logits, int32_t vocab,
                           int32_t logits_dtype, const int32_t* history, const int32_t* history_len,
                           const hta_tree_params_t* params, int32_t* tree_tokens, int32_t* parent, int32_t* n_nodes,
                           void* stream) {
  if (!h || !idx || !logits || !history || !history_len || !params || !tree_tokens || !parent || !n_nodes)
    return HTA_ERR_INVALID_ARG;
  hta::TreeParams p;
  const int rc = tree_params(params, vocab, logits_dtype, &p);
  if (rc != HTA_OK) return rc;
  if (idx->ix.B != h->dims.B || idx->ix.m != params->m) return HTA_ERR_INVALID_ARG;
  return check_hip(hta::launch_build_tree_indexed(h->dims, logits, vocab, logits_dtype == HTA_BF16, history,
                                                  history_len, p, h->topk_part, idx->ix, tree_tokens, parent,
                                                  n_nodes, h->status, static_cast<hipStream_t>(stream)));
}

int hta_tree_mask(hta_handle_t h, const int32_t* parent, uint64_t* mask_out, void* stream) {
  if (!h || !parent || !mask_out) return HTA_ERR_INVALID_ARG;
  return check_hip(hta::launch_tree_mask(h->dims, parent, mask_out, h->status,
                                         static_cast<hipStream_t>(stream)));
}

int hta_tree_attn(hta_handle_t h, const void* q, const void* k_tree, const void* v_tree,
                  const int32_t* parent, float* o_tree, float* lse_tree, void* stream) {
  if (!h || !q || !k_tree || !v_tree || !parent || !o_tree || !lse_tree) return HTA_ERR_INVALID_ARG;
  if (!all_aligned(q, k_tree, v_tree, o_tree)) return HTA_ERR_INVALID_ARG;
  return check_hip(hta::launch_tree_attn(h->dims, q, k_tree, v_tree, parent, o_tree, lse_tree, hta::kLn2,
                                         nullptr, h->status, static_cast<hipStream_t>(stream)));
}

int hta_prefix_attn(hta_handle_t h, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* prefix_len, float* o_prefix, float* lse_prefix, void* stream) {
  if (!h || !q || !k_cache || !v_cache || !prefix_len || !o_prefix || !lse_prefix)
    return HTA_ERR_INVALID_ARG;
  if (!all_aligned(q, k_cache, v_cache, o_prefix)) return HTA_ERR_INVALID_ARG;
  HTA_TRY(hta_prefix_partials(h, q, k_cache, v_cache, prefix_len, stream));
  return hta_merge_prefix(h, prefix_len, o_prefix, lse_prefix, stream);
}

int hta_prefix_partials(hta_handle_t h, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* prefix_len, void* stream) {
  if (!h || !q || !k_cache || !v_cache || !prefix_len) return HTA_ERR_INVALID_ARG;
  if (!all_aligned(q, k_cache, v_cache)) return HTA_ERR_INVALID_ARG;
  const hta::PrefixInputs in = {q, k_cache, v_cache, nullptr, nullptr, nullptr, prefix_len};
  return launch_split(h, in, static_cast<hipStream_t>(stream));
}

int hta_merge_prefix(hta_handle_t h, const int32_t* prefix_len, float* o_prefix, float* lse_prefix,
                     void* stream) {
  if (!h || !prefix_len || !o_prefix || !lse_prefix) return HTA_ERR_INVALID_ARG;
  if (!all_aligned(o_prefix)) return HTA_ERR_INVALID_ARG;
  return check_hip(hta::launch_merge_slots(h->dims, h->pl.tile_tokens, h->pl.nwg, 0, 1, prefix_len, h->slots,
                                           nullptr, o_prefix, false, lse_prefix, h->status,
                                           static_cast<hipStream_t>(stream)));
}

int hta_lse_merge(hta_handle_t h, int32_t n_parts, const float* o_parts, const float* lse_parts,
                  float* out, float* lse, void* stream) {
  if (!h || !o_parts || !lse_parts || !out || !lse) return HTA_ERR_INVALID_ARG;
  if (n_parts < 1 || n_parts > 4096) return HTA_ERR_INVALID_ARG;
  if (!all_aligned(o_parts, out)) return HTA_ERR_INVALID_ARG;
  return check_hip(hta::launch_merge_parts(h->dims, n_parts, o_parts, lse_parts, out, lse,
                                           static_cast<hipStream_t>(stream)));
}

int hta_accept(hta_handle_t h, const void* logits, int32_t vocab, int32_t logits_dtype, const int32_t* parent,
               const int32_t* tree_tokens, int32_t* target_tokens, int32_t* accept_len, int32_t* accept_path,
               int32_t* bonus_token, void* stream) {
  if (!h || !logits || !parent || !tree_tokens || !target_tokens || !accept_len || !accept_path || !bonus_token)
    return HTA_ERR_INVALID_ARG;
  if (vocab < 1 || (logits_dtype != HTA_F32 && logits_dtype != HTA_BF16)) return HTA_ERR_INVALID_ARG;
  return check_hip(hta::launch_accept(h->dims, logits, vocab, logits_dtype == HTA_BF16, parent, tree_tokens,
                                      h->argmax_part, target_tokens, accept_len, accept_path, bonus_token,
                                      h->status, static_cast<hipStream_t>(stream)));
}

int hta_commit(hta_handle_t h, const void* k_tree, const void* v_tree, const int32_t* accept_len,
               const int32_t* accept_path, void* k_cache, void* v_cache, int32_t* prefix_len, void* stream) {
  if (!h || !k_tree || !v_tree || !accept_len || !accept_path || !k_cache || !v_cache || !prefix_len)
    return HTA_ERR_INVALID_ARG;
  if (!all_aligned(k_tree, v_tree, static_cast<const void*>(k_cache), static_cast<const void*>(v_cache)))
    return HTA_ERR_INVALID_ARG;
  return check_hip(hta::launch_commit(h->dims, k_tree, v_tree, accept_len, accept_path, k_cache, v_cache,
                                      prefix_len, h->seq_count, h->status,
                                      static_cast<hipStream_t>(stream)));
}

int hta_get_status(hta_handle_t h, void* stream, int32_t* device_status) {
  if (!h || !device_status) return HTA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t v = 0;
  if (hipMemcpyAsync(&v, h->status, sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess)
    return HTA_ERR_HIP;
  HTA_TRY(check_hip(hta::launch_clear_status(h->status, s)));
  if (hipStreamSynchronize(s) != hipSuccess) return HTA_ERR_HIP;
  // A timed-out fused merge leaves its sync words inconsistent: clear them.
  if ((v & HTA_STATUS_MERGE_TIMEOUT) &&
      hipMemset(h->seg_sync, 0, (size_t)h->dims.B * h->dims.Hkv * h->pl.row_groups * 2 * sizeof(int)) != hipSuccess)
    return HTA_ERR_HIP;
  *device_status = v;
  return HTA_OK;
}

}  // extern "C"
