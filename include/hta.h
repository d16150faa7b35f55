/*
 * hta.h -- tree-verification attention (Hybrid Tree Attention) for MI355X (gfx950).
 *
 * What the library computes. A target model verifies a draft tree of T
 * speculative tokens in one pass. In each attention layer every tree token
 * attends to (a) the whole cached KV prefix of its sequence, which needs no
 * mask, and (b) the tree tokens on its own root path (itself and its
 * ancestors), which needs the tree mask. The two parts are computed apart
 * and combined exactly with the log-sum-exp trick.
 *   - LongSpec summary pages, section "Fast Tree Attention" (Hybrid Tree
 *     Attention: cached part without a mask, speculative part with a mask,
 *     aggregation by log-sum-exp that keeps the result exact).
 *   - LogitSpec summary page, section "draft tree construction and
 *     verification" (the tree mask lets the target verify every branch in
 *     parallel).
 *
 * Conventions used by every entry point (readings of points the pages leave
 * open):
 *   B batch, Hq query heads, Hkv KV heads (Hq % Hkv == 0, G = Hq / Hkv),
 *   D head_dim (64 or 128), T tree nodes (1..64), Lcap KV capacity.
 *   Query head h reads KV head h / G.
 *   Tensors are dense, row-major, contiguous device memory:
 *     q        [B, Hq,  T,    D]   dtype
 *     k_cache  [B, Hkv, Lcap, D]   dtype   (positions >= prefix_len[b] are never read)
 *     v_cache  [B, Hkv, Lcap, D]   dtype   (same)
 *     k_tree   [B, Hkv, T,    D]   dtype   (post-RoPE keys of the tree tokens)
 *     v_tree   [B, Hkv, T,    D]   dtype
 *     parent   [B, T] int32: parent[b][0] == -1 and -1 <= parent[b][i] < i
 *              (nodes in topological order; an extra -1 starts another root)
 *     prefix_len [B] int32: 0 <= prefix_len[b] <= Lcap
 *     out      [B, Hq, T, D]   dtype
 *     lse      [B, Hq, T] float32: natural log of sum(exp(scale * q.k)) over
 *              the visible keys (the scaled-score convention).
 *   dtype is HTA_BF16 (bfloat16 storage, float32 arithmetic) or HTA_F32.
 *   The softmax scale defaults to 1/sqrt(D).
 *
 * Float tensors (q, k/v cache, k/v tree, out and the float32 partials) must
 * start on a 16-byte boundary; a misaligned pointer is HTA_ERR_INVALID_ARG.
 *
 * Ownership: the caller allocates and owns every tensor argument. A handle
 * owns only its device workspace (partial results and status words), sized
 * at hta_create. Every pointer argument named as a tensor above is a device
 * pointer; the only host pointers are the handle, config, plan and status
 * out-parameters.
 *
 * Streams: `stream` is a hipStream_t (NULL means the null stream). Calls are
 * asynchronous: they validate on the host, enqueue kernels and return. The
 * workspace is shared by all calls on one handle, so at most one call per
 * handle may be in flight (use one handle per concurrent stream).
 *
 * Errors: functions return HTA_OK (0) or a negative HTA_ERR_* code; nothing
 * throws and the library never prints. Host-side checks (null pointers,
 * unsupported shapes) fail before any kernel is enqueued. Checks that need
 * device data (a parent array that breaks the rule above, a prefix_len
 * outside [0, Lcap]) cannot fail the call; instead the affected sequence's
 * outputs are filled with NaN and a sticky bit is set in the handle's device
 * status word, read (and cleared) by hta_get_status. Enqueue failures map to
 * HTA_ERR_HIP.
 */
#ifndef HTA_H_
#define HTA_H_

#include <stdint.h>

#ifndef HTA_API
#define HTA_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef struct hta_handle_s* hta_handle_t;

enum hta_status_code {
  HTA_OK = 0,
  HTA_ERR_INVALID_ARG = -1, /* null pointer, bad size or an impossible config */
  HTA_ERR_UNSUPPORTED = -2, /* valid but not built: D not in {64,128}, T > 64, ... */
  HTA_ERR_NO_MEMORY = -3,   /* workspace allocation failed */
  HTA_ERR_HIP = -4,         /* a HIP runtime call or kernel enqueue failed */
  HTA_ERR_BAD_TREE = -5,    /* reported through hta_get_status only */
  HTA_ERR_BAD_PREFIX = -6,  /* reported through hta_get_status only */
  HTA_ERR_NO_DEVICE = -7,   /* no usable GPU */
  HTA_ERR_TOO_LARGE = -8    /* hta_verify_attn_noalloc: shape needs more than its scratch memory */
};

enum hta_dtype { HTA_F32 = 0, HTA_BF16 = 1 };

/* Bits of the device status word (see hta_get_status). */
enum hta_device_status {
  HTA_STATUS_BAD_TREE = 1,
  HTA_STATUS_BAD_PREFIX = 2,
  HTA_STATUS_COMMIT_OVERFLOW = 4, /* hta_commit: prefix_len + accept_len would pass kv_capacity */
  HTA_STATUS_BAD_PATH = 8,        /* hta_commit: an accept_path entry outside [0, T) */
  HTA_STATUS_MERGE_TIMEOUT = 16   /* hta_verify_attn: a fused merge gave up waiting (rows NaN) */
};

/* Prefix-kernel implementation (see hta_plan_t.path). MFMA: bf16 with
 * G*T >= 16 query rows per KV head (32-row matrix-core blocks). DOT: bf16,
 * D = 128 or 64, G*T <= 16 (dot products on the vector ALUs, cross-lane
 * reductions, up to 8 rows per workgroup; the drafter's cross-attention
 * shape). VALU: float32, and everything else. */
enum hta_path { HTA_PATH_AUTO = 0, HTA_PATH_MFMA = 1, HTA_PATH_VALU = 2, HTA_PATH_DOT = 3 };

typedef struct {
  int32_t batch;          /* B >= 1 */
  int32_t n_q_heads;      /* Hq >= 1 */
  int32_t n_kv_heads;     /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;       /* D: 64 or 128 */
  int32_t tree_nodes;     /* T: 1..64 */
  int32_t kv_capacity;    /* Lcap >= 1 */
  int32_t dtype;          /* enum hta_dtype */
  float softmax_scale;    /* <= 0 selects 1/sqrt(D) */
  int32_t num_workgroups; /* prefix-kernel workgroups; 0 = sized from the device */
  int32_t force_path;     /* enum hta_path; AUTO picks MFMA for bf16 with G*T >= 16, DOT for
                             bf16 with G*T <= 15, else VALU */
  int32_t qblocks_per_wave; /* MFMA path: 32-row query blocks per wave, 1 or 2; 0 = planned */
  int32_t fuse_merge;       /* MFMA path, hta_verify_attn: 1 = merge inside the split-KV launch
                               (see hta_verify_attn), 0 = separate merge launch (default) */
} hta_config_t;

typedef struct {
  int32_t path;                /* HTA_PATH_MFMA, HTA_PATH_VALU or HTA_PATH_DOT */
  int32_t num_workgroups;      /* workgroups per row group of the prefix kernel */
  int32_t row_groups;          /* prefix-kernel grid.y: row groups per KV head */
  int32_t rows_per_group;      /* query rows (of G*T per KV head) per row group */
  int32_t waves_per_workgroup;
  int32_t qblocks_per_wave;    /* 32-row MFMA blocks per wave (MFMA path) */
  int32_t tile_tokens;         /* prefix tokens per pipeline stage */
  int32_t max_slots;           /* partial-result slots in the workspace */
  int64_t workspace_bytes;
  int32_t device;              /* HIP device the handle was created on */
  int32_t compute_units;
} hta_plan_t;

/* Host-only validation of a config; makes no HIP call. Returns HTA_OK,
 * HTA_ERR_INVALID_ARG or HTA_ERR_UNSUPPORTED. */
HTA_API int hta_validate_config(const hta_config_t* cfg);

/* Validates cfg, plans the launch for the current HIP device and allocates
 * the workspace. On success *out holds a new handle; on failure *out is NULL. */
HTA_API int hta_create(hta_handle_t* out, const hta_config_t* cfg);

/* Frees the workspace and the handle (synchronises the device first).
 * NULL is accepted and ignored. */
HTA_API int hta_destroy(hta_handle_t h);

/* Copies the launch plan chosen at hta_create. Host only. */
HTA_API int hta_get_plan(hta_handle_t h, hta_plan_t* plan);

/* Full verification attention: prefix part (split-KV over all compute units,
 * no mask) + tree part (ancestor mask) + exact log-sum-exp merge.
 * Layouts and rules as in the header comment. out has the handle's dtype;
 * lse is float32 natural log. LongSpec, "Fast Tree Attention".
 * With config.fuse_merge on the MFMA path (and a grid no wider than the
 * device) the merge runs inside the split-KV launch: the workgroups of a
 * (sequence, KV head) wait for each other (bounded; past the bound the rows
 * come out NaN with HTA_STATUS_MERGE_TIMEOUT, which hta_get_status also
 * recovers from), so that launch needs the whole device to itself while it
 * runs. Calls on one handle must not overlap. */
HTA_API int hta_verify_attn(hta_handle_t h, const void* q, const void* k_cache, const void* v_cache,
                    const void* k_tree, const void* v_tree, const int32_t* parent,
                    const int32_t* prefix_len, void* out, float* lse, void* stream);

/* The drafter's cross-attention over the target model's KV cache: every
 * query row attends, with no mask, to the first prefix_len[b] positions of
 * its KV head (LongSpec summary pages, §2.A "memory-efficient architecture":
 * the draft model reads the cache the target keeps anyway). q [B,Hq,T,D]
 * with T = the handle's tree_nodes (draft query tokens per sequence), caches
 * [B,Hkv,Lcap,D]; out [B,Hq,T,D] in the handle's dtype, lse [B,Hq,T] float32
 * natural log. A sequence with prefix_len 0 gets out = 0 and lse = -inf; a
 * prefix_len outside [0, Lcap] gives NaN rows + HTA_STATUS_BAD_PREFIX.
 * bf16 handles with G*T <= 15 run the DOT kernel. Same split-KV kernel and
 * merge as hta_verify_attn, without the tree tile. Pointers as there. */
HTA_API int hta_cross_attn(hta_handle_t h, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* prefix_len, void* out, float* lse, void* stream);

/* The drafter's sliding-window self-attention (LongSpec summary pages, §2.A
 * "memory-efficient architecture": a window of 512 positions keeps the draft
 * model's cache at a fixed size). The handle's kv_capacity is the window W
 * and its tree_nodes the number Tn <= W of new tokens per step. The draft
 * cache is a ring, k_ring/v_ring [B,Hkv,W,D], slot = position mod W; pos[b]
 * (int32, device) counts the positions written before this step, so the ring
 * holds positions max(0, pos-W) .. pos-1 (slots not yet written are never
 * read and may hold anything). k_new/v_new [B,Hkv,Tn,D] are the new tokens
 * at positions pos .. pos+Tn-1; q [B,Hq,Tn,D]. New token j attends to the
 * positions max(0, pos+j-W+1) .. pos+j, its own included. out [B,Hq,Tn,D] in
 * the handle's dtype, lse [B,Hq,Tn] float32 natural log. A negative pos[b]
 * gives NaN rows + HTA_STATUS_BAD_PREFIX. Returns HTA_ERR_UNSUPPORTED when
 * Tn > W. Pointers 16-byte aligned. */
HTA_API int hta_window_attn(hta_handle_t h, const void* q, const void* k_ring, const void* v_ring,
                            const void* k_new, const void* v_new, const int32_t* pos, void* out, float* lse,
                            void* stream);

/* Writes the Tn new tokens into the ring (new token j to slot (pos+j) mod W)
 * and advances pos by Tn, on the stream. A negative pos[b] leaves that
 * sequence unchanged and sets HTA_STATUS_BAD_PREFIX. Calls on one handle must
 * not overlap (they share arrival counters with hta_commit). Tn <= W. */
HTA_API int hta_window_append(hta_handle_t h, const void* k_new, const void* v_new, void* k_ring, void* v_ring,
                              int32_t* pos, void* stream);

/* Draft-tree construction (LogitSpec summary pages, §2 "LogitSpec workflow":
 * next token, top-k next-next guesses without it, dual n-gram retrieval,
 * rank-based pruning). */
#define HTA_MAX_TREE_GUESSES 31
#define HTA_MAX_NGRAM 8
typedef struct {
  int32_t k;          /* next-next guesses: 0 .. HTA_MAX_TREE_GUESSES */
  int32_t m;          /* n-gram length of both queries: 1 .. HTA_MAX_NGRAM */
  int32_t keep_first; /* tokens kept after query 1's match: 0 .. 64 */
  int32_t keep[HTA_MAX_TREE_GUESSES]; /* tokens kept after the match for the guess of rank r: 0 .. 64 */
} hta_tree_params_t;

/* Builds one draft tree per sequence from its last logits and its own tokens.
 * logits [B,V] (the last position's, float32 or bfloat16 per logits_dtype,
 * V = vocab <= 262144 and >= k+1); history [B,history_cap] int32 token ids
 * >= 0 with history_len[b] (0 .. history_cap) valid entries, the last being
 * the current token; params is a host pointer. x1 = the largest logit (lowest
 * index on ties); guesses = the next k in that order. The sequence searched is
 * history followed by x1. Query 1 = its last m tokens; query 2 for guess g =
 * its last m-1 tokens followed by g; a match is the most recent earlier
 * occurrence (query 1 never matches itself) and the tokens after it are
 * retrieved. Output (T = the handle's tree_nodes): node 0 = x1 (parent -1);
 * then up to keep_first tokens retrieved for query 1, a chain under node 0;
 * then for each guess by rank r a node under node 0 and up to keep[r]
 * retrieved tokens chained under it; nodes past T are dropped in that order.
 * tree_tokens [B,T], parent [B,T] (a valid parent array for hta_verify_attn),
 * n_nodes [B] = nodes used; unused slots hold token -1 under node 0. A
 * history_len outside [0, history_cap] gives n_nodes 0, all tokens -1 and
 * HTA_STATUS_BAD_PREFIX. Returns HTA_ERR_INVALID_ARG for parameters outside
 * the ranges above, HTA_ERR_UNSUPPORTED for a larger vocabulary. */
HTA_API int hta_build_tree(hta_handle_t h, const void* logits, int32_t vocab, int32_t logits_dtype,
                           const int32_t* history, int32_t history_cap, const int32_t* history_len,
                           const hta_tree_params_t* params, int32_t* tree_tokens, int32_t* parent,
                           int32_t* n_nodes, void* stream);

/* A hash index of the m-grams of B token histories, so that the retrieval of
 * hta_build_tree_indexed costs a few table probes per query instead of a pass
 * over the whole history (LogitSpec summary pages, §4 "experimental results",
 * overhead: the retrieval is hash-based and adds about 1 % of the wall time).
 * Per sequence it maps each distinct m-gram of history[b][0 .. n) to the
 * largest end position at which it occurs, where n = the history length it
 * has been brought up to (kept on the device). Open addressing with linear
 * probing over 2^s slots, 2^s >= 2 * history_cap; a slot holds the end
 * position of the gram's first inserted occurrence (the key: inserts compare
 * grams token by token through the history, so results never depend on hash
 * collisions), the largest end position seen and a copy of the gram's tokens
 * (what lookups compare). Device memory: B * 2^s * 32 bytes (64 for m >= 7)
 * + 4 B bytes, allocated on the current HIP device. */
typedef struct hta_ngram_index_s* hta_ngram_index_t;

/* Creates an empty index for batch sequences of history_cap tokens and grams
 * of m tokens (1 .. HTA_MAX_NGRAM). On failure *out is NULL; returns
 * HTA_ERR_INVALID_ARG for parameters out of range, HTA_ERR_UNSUPPORTED for
 * history_cap > 2^26, HTA_ERR_NO_MEMORY if the table cannot be allocated. */
HTA_API int hta_ngram_index_create(hta_ngram_index_t* out, int32_t batch, int32_t history_cap, int32_t m);

/* Frees the index (synchronises the device first). NULL is accepted. */
HTA_API int hta_ngram_index_destroy(hta_ngram_index_t idx);

/* Empties sequence seq's part of the index (seq = -1: every sequence), on the
 * stream, with a fill kernel (no memset node: capturable). Required before a
 * batch slot starts a new sequence whose first tokens differ from the old
 * one's. seq outside [-1, batch) gives HTA_ERR_INVALID_ARG. */
HTA_API int hta_ngram_index_reset(hta_ngram_index_t idx, int32_t seq, void* stream);

/* hta_build_tree with the retrieval through idx: the same outputs, the same
 * status rules and the same argument rules (history_cap is the index's; the
 * handle's batch and params->m must equal the index's, else
 * HTA_ERR_INVALID_ARG). First the grams ending at positions [n, history_len[b])
 * are added to sequence b's part of the index; a history_len[b] below n
 * (the sequence was cut back) rebuilds that part from position 0. The tokens
 * history[b][0 .. n) must not have changed since they were added (reset the
 * sequence otherwise). Calls with one index must not overlap. */
HTA_API int hta_build_tree_indexed(hta_handle_t h, hta_ngram_index_t idx, const void* logits, int32_t vocab,
                                   int32_t logits_dtype, const int32_t* history, const int32_t* history_len,
                                   const hta_tree_params_t* params, int32_t* tree_tokens, int32_t* parent,
                                   int32_t* n_nodes, void* stream);

/* The tree mask alone: mask_out[b][i] (uint64, device) has bit j set iff
 * tree node j is node i or one of its ancestors. A sequence whose parent
 * array breaks the rule gets all-zero words and sets HTA_STATUS_BAD_TREE.
 * LogitSpec, "draft tree construction and verification". */
HTA_API int hta_tree_mask(hta_handle_t h, const int32_t* parent, uint64_t* mask_out, void* stream);

/* The speculative (tree) part alone: attention of every tree token over the
 * tree tokens it may see. o_tree [B,Hq,T,D] float32 (normalised), lse_tree
 * [B,Hq,T] float32 natural log. Bad trees give NaN rows + status bit.
 * LongSpec, "Fast Tree Attention" (the masked speculative part). */
HTA_API int hta_tree_attn(hta_handle_t h, const void* q, const void* k_tree, const void* v_tree,
                  const int32_t* parent, float* o_tree, float* lse_tree, void* stream);

/* The cached (prefix) part alone: attention of every tree token over the
 * first prefix_len[b] cache positions, unmasked, computed split-KV and
 * merged. o_prefix [B,Hq,T,D] float32 (normalised), lse_prefix [B,Hq,T]
 * float32 natural log; a sequence with prefix_len 0 gives o = 0 and
 * lse = -inf. A prefix_len outside [0, Lcap] gives NaN rows + status bit.
 * LongSpec, "Fast Tree Attention" (the cached part, no mask needed). */
HTA_API int hta_prefix_attn(hta_handle_t h, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* prefix_len, float* o_prefix, float* lse_prefix, void* stream);

/* The split-KV prefix kernel alone (the first half of hta_prefix_attn): leaves
 * one normalised partial per (workgroup, sequence/KV-head piece) in the
 * handle's workspace, to be combined by hta_merge_prefix. Used to time and
 * test the kernel that streams the KV cache. LongSpec, "Fast Tree Attention"
 * (the cached part, no mask needed). */
HTA_API int hta_prefix_partials(hta_handle_t h, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* prefix_len, void* stream);

/* Merges the partials of the last hta_prefix_partials call on this handle
 * (prefix_len must hold the same values) into o_prefix [B,Hq,T,D] float32
 * and lse_prefix [B,Hq,T] float32 natural log, exactly as hta_prefix_attn. */
HTA_API int hta_merge_prefix(hta_handle_t h, const int32_t* prefix_len, float* o_prefix,
                             float* lse_prefix, void* stream);

/* Exact log-sum-exp merge of n_parts normalised partial attentions over
 * disjoint key sets: o_parts [n_parts][B,Hq,T,D] float32, lse_parts
 * [n_parts][B,Hq,T] float32 natural log (-inf marks an empty part). Writes
 * out [B,Hq,T,D] float32 and lse [B,Hq,T] float32:
 *   lse = ln(sum_k exp(lse_k)),  out = sum_k exp(lse_k - lse) * o_k.
 * Rows where every part is empty get out = 0, lse = -inf. 1 <= n_parts <= 4096.
 * LongSpec, "Fast Tree Attention" (aggregation with the log-sum-exp trick). */
HTA_API int hta_lse_merge(hta_handle_t h, int32_t n_parts, const float* o_parts, const float* lse_parts,
                  float* out, float* lse, void* stream);

/* Accepts the verified draft tree of every sequence (LogitSpec, "draft tree
 * construction and verification": a tree rooted at x_{i+1} whose branches the
 * target checks at once; LongSpec: lossless decoding keeps only what the target
 * itself would produce). Greedy reading:
 *   target_tokens[b][j] = argmax_v logits[b][j][v], the lowest v among equal
 *     maxima, on the exact stored values (finite logits);
 *   from the root (node 0, always accepted) the walk moves to the child whose
 *     tree token equals the target token at its parent, the lowest-numbered
 *     such child, until no child matches;
 *   accept_len[b] = accepted nodes (root included), accept_path[b][k] = the
 *     k-th of them root first (-1 from accept_len[b] on), bonus_token[b] =
 *     target_tokens[b][last accepted node].
 * logits [B,T,vocab] of logits_dtype (HTA_F32 or HTA_BF16, any alignment;
 * 16-byte aligned rows take the vector path); parent, tree_tokens,
 * target_tokens, accept_path [B,T] int32; accept_len, bonus_token [B] int32;
 * all device pointers owned by the caller. A sequence whose parent array
 * breaks -1 <= parent[i] < i gets accept_len 0, an all -1 path, bonus -1
 * and HTA_STATUS_BAD_TREE. Uses the handle's workspace (one call in flight
 * per handle). */
HTA_API int hta_accept(hta_handle_t h, const void* logits, int32_t vocab, int32_t logits_dtype,
                       const int32_t* parent, const int32_t* tree_tokens, int32_t* target_tokens,
                       int32_t* accept_len, int32_t* accept_path, int32_t* bonus_token, void* stream);

/* Commits the accepted nodes of the last verification: for every sequence b
 * with 0 < accept_len[b] and prefix_len[b] + accept_len[b] <= kv_capacity,
 * copies k_tree[b][g][accept_path[b][k]] and v_tree[...] to
 * k_cache[b][g][prefix_len[b] + k] and v_cache[...] for every KV head g and
 * k < accept_len[b], then advances prefix_len[b] (device, in place) by
 * accept_len[b]. Other sequences are left unchanged; one whose prefix_len
 * lies outside [0, kv_capacity] raises HTA_STATUS_BAD_PREFIX, one that would
 * overflow raises HTA_STATUS_COMMIT_OVERFLOW, a path entry outside [0, T) raises
 * HTA_STATUS_BAD_PATH (that row is skipped). k_tree, v_tree [B,Hkv,T,D] and
 * k_cache, v_cache [B,Hkv,Lcap,D] have the handle's dtype and must be 16-byte
 * aligned. The accepted tokens' keys and values join the cached part that
 * the next verification reads unmasked (LongSpec, "Fast Tree Attention"). */
HTA_API int hta_commit(hta_handle_t h, const void* k_tree, const void* v_tree, const int32_t* accept_len,
                       const int32_t* accept_path, void* k_cache, void* v_cache, int32_t* prefix_len,
                       void* stream);

/* Synchronises `stream`, returns in *device_status the OR of the status
 * bits raised since the last call (HTA_STATUS_*), and clears them. */
HTA_API int hta_get_status(hta_handle_t h, void* stream, int32_t* device_status);

/* Bytes of device memory that hta_verify_attn_noalloc holds per GPU. */
#define HTA_NOALLOC_SCRATCH_BYTES (32u << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation, kernels and launch plan as hta_verify_attn on a handle made
 * from *cfg (fuse_merge is ignored: the merge runs as its own launch), with
 * no handle and no allocation. The partial results live in a fixed device
 * array of HTA_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds
 * from the first call on that GPU until the process ends. A shape whose
 * partial results need more returns HTA_ERR_TOO_LARGE (a smaller
 * num_workgroups in *cfg needs less). Calls on one GPU share that array:
 * calls that overlap on one GPU (other streams, other threads) race, so the
 * caller orders them. Tensor arguments, layouts and alignment as for
 * hta_verify_attn, on the current device. status (int32, device) receives
 * the HTA_STATUS_* bits of this call OR-ed into it; the caller clears it.
 * Returns HTA_OK, HTA_ERR_INVALID_ARG, HTA_ERR_UNSUPPORTED,
 * HTA_ERR_TOO_LARGE, HTA_ERR_NO_DEVICE or HTA_ERR_HIP. */
HTA_API int hta_verify_attn_noalloc(const hta_config_t* cfg, const void* q, const void* k_cache,
                                    const void* v_cache, const void* k_tree, const void* v_tree,
                                    const int32_t* parent, const int32_t* prefix_len, void* out, float* lse,
                                    int32_t* status, void* stream);

/* Static English text for a return code. Never NULL. */
HTA_API const char* hta_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* HTA_H_ */
