// Internal interface between the C ABI (hta_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hta.h"

namespace hta {

constexpr int kTileTokens = 64;      // prefix tokens per tile of the split (VALU and DOT paths)
constexpr int kMfmaTileTokens = 32;  // prefix tokens per tile of the split (MFMA path)

// Tiles that hold a segment's T tree tokens when the tree part is fused in.
__host__ __device__ inline int tree_tiles_for(int T, int nk) { return (T + nk - 1) / nk; }
// Split weight of a tree tile on the MFMA path (in prefix tiles): the
// workgroup holding a segment's tree tiles also builds the ancestor words and
// masks them, so each tree tile counts as this many tiles when the tile
// stream is split (the extra ones are empty tiles the kernels skip).
constexpr int kTreeTileWeight = 3;

struct Dims {
  int B, Hq, Hkv, G, T, D, Lcap, M;  // M = G*T query rows per KV head
  bool bf16;
  float scale_log2;                  // softmax scale * log2(e)
};

// Partial results of the split-KV kernels: slot s holds M rows of D values
// (normalised output; bf16 from the MFMA path, float from the VALU path) and
// M log2-domain LSE values (float).
struct Slots {
  void* o;
  float* lse2;
  bool o_bf16;
  size_t o_bytes = 0, lse2_bytes = 0;  // sizes of the two arrays
};

struct PrefixLaunch {
  int path;           // 1 MFMA, 2 VALU, 3 DOT
  int tile_tokens;    // tokens per tile of the split
  int nwg;            // workgroups per row group
  int row_groups;     // grid.y
  int rows_per_group; // multiple of 32 (MFMA) or of 16 (VALU)
  int waves;          // MFMA: waves that compute
  int qb;             // MFMA: q-blocks per wave
};

// Inputs of the split-KV kernels. With k_tree/v_tree/parent set, each
// (sequence, KV head) gets tree_tiles_for(T, tile_tokens) extra tiles of tree
// tokens under the ancestor mask (the fused tree part); with them null only
// the cached part is done.
struct PrefixInputs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const void* k_tree;
  const void* v_tree;
  const int* parent;
  const int* prefix_len;
};

// Split-KV kernels: write one partial per (workgroup, segment piece) to slots.
// With the tree fused in, the workgroup holding the tree tile of (b, KV head 0)
// writes err_b[b] (1 if parent[] of b is malformed) and raises the status bit.
// Fused merge of the MFMA kernel (fuse.out != null): final out / lse written
// by the split-KV launch itself, with per (segment, row group) sync words
// (two ints, zero between launches) and tree-check words.
struct FusedMerge {
  void* out = nullptr;
  float* lse = nullptr;
  int* seg_sync = nullptr;
  int* seg_err = nullptr;
};
hipError_t launch_prefix_mfma(const Dims& d, const PrefixLaunch& pl, const PrefixInputs& in, Slots slots,
                              int* err_b, int* status, hipStream_t s, const FusedMerge& fuse = FusedMerge());
hipError_t launch_prefix_valu(const Dims& d, const PrefixLaunch& pl, const PrefixInputs& in, Slots slots,
                              int* err_b, int* status, hipStream_t s);
// Launch plan of a validated config on a device with `cus` compute units: the
// dims, the kernel path, rows, waves and workgroup count, and the chosen
// kernel's workgroups per CU. Allocates nothing. Returns HTA_OK or an HTA_ERR_*.
int plan_launch(const hta_config_t* cfg, int cus, Dims* d, PrefixLaunch* pl, int* occ);
// The planned split-KV launch (any path) into `slots`; HTA_OK or HTA_ERR_HIP.
int launch_split(const Dims& d, const PrefixLaunch& pl, const PrefixInputs& in, Slots slots, int* err_b,
                 int* status, hipStream_t s);
// Small-M bf16 split-KV kernel (v_dot2 + DPP; D = 128 or 64, at most kDotMaxRows
// query rows per KV head, in dot_row_groups(M) groups of up to 8 on grid.y).
// Float slots, same split and tree fusion.
constexpr int kDotMaxRows = 16;
hipError_t launch_prefix_dot(const Dims& d, const PrefixLaunch& pl, const PrefixInputs& in, Slots slots,
                             int* err_b, int* status, hipStream_t s);
bool prefix_dot_supported(int D, int M, bool bf16);
int dot_row_groups(int M);
int prefix_dot_occupancy(int D, int M);
// The drafter's sliding-window self-attention over a ring of W = Lcap slots
// with T new tokens (window.hip), and the append of the new tokens to the
// ring (count: the B arrival counters shared with the commit).
hipError_t launch_window_attn(const Dims& d, const void* q, const void* k_ring, const void* v_ring,
                              const void* k_new, const void* v_new, const int* pos, void* out, float* lse,
                              int* status, hipStream_t s);
hipError_t launch_window_append(const Dims& d, const void* k_new, const void* v_new, void* k_ring, void* v_ring,
                                int* pos, unsigned* count, int* status, hipStream_t s);
// Draft-tree construction from the last logits (tree_build.hip). part holds
// B * topk_split_for(V) * (kMaxTreeGuesses + 1) keys.
constexpr int kMaxTreeGuesses = 31;
constexpr int kMaxNgram = 8;
constexpr int kMaxTreeSplit = 64;  // vocabulary up to kMaxTreeSplit * 4096 entries
struct TreeParams {
  int k, m, keep_first;
  int keep[kMaxTreeGuesses];
};
int topk_split_for(int V);
// aux: 2 * B * (kMaxTreeGuesses + 1) ints (match ends, x1 + guesses).
hipError_t launch_build_tree(const Dims& d, const void* logits, int V, bool logits_bf16, const int* history,
                             int hist_cap, const int* hist_len, const TreeParams& p, unsigned long long* part,
                             int* aux, int* tokens, int* parent, int* n_nodes, int* status, hipStream_t s);
// Hash index of the m-grams of B histories (tree_build.hip): per sequence
// 2^slots_log2 slots of ngram_slot_ints(m) ints {end position of the key
// occurrence (-1: empty), largest end position, the key's m tokens};
// len[b] = the history length it covers.
struct NgramIndex {
  int* table;
  int* len;
  int B, cap, m, slots_log2;
};
// launch_build_tree with the retrieval through the index (brought up to
// hist_len first).
hipError_t launch_build_tree_indexed(const Dims& d, const void* logits, int V, bool logits_bf16, const int* history,
                                     const int* hist_len, const TreeParams& p, unsigned long long* part,
                                     const NgramIndex& ix, int* tokens, int* parent, int* n_nodes, int* status,
                                     hipStream_t s);
int ngram_slot_ints(int m);
// Empties sequence seq's part of the index (seq < 0: all), with a fill kernel.
hipError_t launch_ngram_reset(const NgramIndex& ix, int seq, hipStream_t s);
// Occupancy (workgroups per CU) of the chosen prefix kernel, for sizing nwg.
int prefix_mfma_occupancy(int D, int waves, int qb);
int prefix_valu_occupancy(int D, bool bf16);
bool prefix_mfma_supported(int D, int waves, int qb);

// Tree part. lse_scale converts the log2-domain LSE on store (1 keeps log2,
// ln 2 gives natural log). err_b (may be null) receives per-sequence bad-tree flags.
hipError_t launch_tree_attn(const Dims& d, const void* q, const void* k_tree, const void* v_tree,
                            const int* parent, float* o_tree, float* lse_tree, float lse_scale,
                            int* err_b, int* status, hipStream_t s);
hipError_t launch_tree_mask(const Dims& d, const int* parent, uint64_t* mask_out, int* status,
                            hipStream_t s);

// Merge of the slots of one split-KV launch (tile_tokens, nwg and
// tree_tiles as in that launch) into out (float or bf16) and natural-log
// lse; err_b (may be null) marks sequences whose rows become NaN.
hipError_t launch_merge_slots(const Dims& d, int tile_tokens, int nwg, int tree_tiles, int tree_weight,
                              const int* prefix_len,
                              Slots slots,
                              const int* err_b, void* out, bool out_bf16, float* lse, int* status,
                              hipStream_t s);
// Merge of n_parts caller-provided partials (natural-log LSE) into float out.
hipError_t launch_merge_parts(const Dims& d, int n_parts, const float* o_parts,
                              const float* lse_parts, float* out, float* lse, hipStream_t s);

hipError_t launch_clear_status(int* status, hipStream_t s);

// Accept / commit of a verified draft tree (accept.hip). The argmax over the
// vocabulary splits each logit row over at most kArgmaxMaxSplit workgroups;
// part holds B*T*kArgmaxMaxSplit keys. count (B arrival counters of the
// commit) must be zero before the first call; each call leaves it zero.
constexpr int kArgmaxMaxSplit = 64;
int argmax_split_for(int V, bool logits_bf16);
hipError_t launch_accept(const Dims& d, const void* logits, int V, bool logits_bf16, const int* parent,
                         const int* tree_tokens, unsigned long long* part, int* target_out, int* accept_len,
                         int* accept_path, int* bonus, int* status, hipStream_t s);
hipError_t launch_commit(const Dims& d, const void* k_tree, const void* v_tree, const int* accept_len,
                         const int* accept_path, void* k_cache, void* v_cache, int* prefix_len, unsigned* count,
                         int* status, hipStream_t s);

}  // namespace hta
