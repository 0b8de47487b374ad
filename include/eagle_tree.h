/*
 * eagle_tree.h -- C ABI of the MI355X (gfx950) draft-tree verification library.
 *
 * One verification step of EAGLE-2 speculative sampling, as five calls:
 *   eagle_tree_expand     grow the dynamic draft tree by one layer
 *   eagle_tree_rerank     keep the n best nodes of the whole tree
 *   eagle_tree_mask       flatten the kept tree: tokens, parents, positions, ancestor mask
 *   eagle_tree_attention  tree attention of the flattened rows against the KV cache
 *   eagle_verify          lossless acceptance (greedy or sampled) over target logits
 * and three calls around it:
 *   eagle_tree_mask_static  positions and ancestor mask of a caller-given fixed tree
 *                           (the static trees of EAGLE / Medusa), in place of the first three
 *   eagle_tree_rope         rotary position encoding of the tree rows at their positions
 *   eagle_tree_attention_rope  tree attention with that rotary applied inside it
 *   eagle_kv_commit         move the accepted rows' K/V behind the context, as
 *                           autoregressive decoding would have left them
 *   eagle_draft_subtree     rows, masks and positions of the draft model's attention
 *                           at a draft layer (the frontier nodes' root paths)
 *   eagle_kv_gather         copy rows (e.g. tree nodes' draft K/V) behind the context
 *
 * Pages defining the operations (cited by title and passage):
 *   EAGLE-2 page -- news write-up of "EAGLE-2: Faster Inference of Language Models
 *     with Dynamic Draft Trees": the passage on the two stages (node value =
 *     product of confidences on the root path; Expand takes the m best nodes of the
 *     last layer; Rerank keeps the n best of the whole tree, shallower first on equal
 *     values so the kept tree stays connected) and the passage after it
 *     (flattening to 1-D, ancestor-only attention mask -- the It / is / a / has
 *     example -- and positions adjusted to match autoregressive decoding); its
 *     opening paragraph (one target forward verifies the draft).
 *   EAGLE page -- abstract of "EAGLE: Speculative Sampling Requires Rethinking
 *     Feature Uncertainty": output distribution identical to vanilla decoding.
 *   CSDN page -- "论文解读：eagle/eagle2", sections 1.1 and 1.2: verification keeps
 *     the target's distribution, under greedy and under sampled decoding.
 *
 * Conventions for every call:
 *   - All array pointers are DEVICE pointers owned by the caller; struct
 *     arguments (eagle_tree_cfg, eagle_tree_state, eagle_attn_desc) are read on the
 *     host during the call only.  The library never allocates or frees device
 *     memory and keeps no state between calls, except the one file-scope scratch
 *     array (and its per-device address) of eagle_tree_attention_noalloc.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream).
 *   - Arguments are validated on the host first; on any failure the call returns
 *     the status and launches nothing.  After launching, a launch error maps to
 *     EAGLE_ERR_HIP.  Faults inside kernels surface at the caller's next sync.
 *   - Logits containing NaN or Inf give unspecified (but memory-safe) results.
 *   - Calls on distinct streams with distinct buffers are independent.
 */
#ifndef EAGLE_TREE_H
#define EAGLE_TREE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    EAGLE_OK = 0,
    EAGLE_ERR_INVALID_ARG = -1, /* null pointer, out-of-range size, inconsistent shape */
    EAGLE_ERR_UNSUPPORTED = -2, /* valid but outside the library's limits (below) */
    EAGLE_ERR_WORKSPACE = -3,   /* workspace pointer null or smaller than required */
    EAGLE_ERR_HIP = -4          /* the HIP runtime reported a launch error */
} eagle_status;

typedef enum { EAGLE_F32 = 0, EAGLE_BF16 = 1 } eagle_dtype;

/* Limits of the library. */
#define EAGLE_MAX_TREE_ROWS 64     /* T = n + 1: one 64-bit ancestor-mask word per row */
#define EAGLE_MAX_TOPK 32          /* children per expanded node */
#define EAGLE_MAX_LAYER_NODES 1024 /* m * topk: nodes created in one layer */
#define EAGLE_MAX_CAPACITY 4096    /* tree nodes incl. the root after `depth` layers */
#define EAGLE_MAX_BATCH 1024
#define EAGLE_MAX_VOCAB 262144    /* draft and target vocabulary size */

/* Tree parameters, identical for every sequence of the batch.
 *   depth : draft layers below the root (>= 1); at most `depth` tokens are accepted
 *   topk  : children given to each expanded node (its draft row's top-k tokens)
 *   m     : nodes of the last layer expanded at the next layer
 *   n     : nodes kept by Rerank, root excluded (the flattened tree has T = n + 1 rows) */
typedef struct {
    int32_t batch, vocab, depth, topk, m, n;
} eagle_tree_cfg;

/* Device-side tree, [batch][capacity] per array (capacity from eagle_tree_capacity).
 * Node 0 of each sequence is the root (parent -1, depth 0, value 0).  Children are
 * numbered in creation order: layer by layer, frontier order, then draft rank.
 * value = sum of fp32 log-confidences on the root path.
 * frontier [batch][m]: ids of the nodes whose draft rows the next layer consumes,
 * best first (value desc, id asc).  n_nodes [batch]: nodes created so far. */
typedef struct {
    int32_t *token, *parent, *depth;
    float *value;
    int32_t *frontier, *n_nodes;
} eagle_tree_state;

/* Nodes after all `depth` layers: 1 + topk * sum_l F_l, F_1 = 1,
 * F_{l+1} = min(m, F_l * topk).  Returns -1 for an invalid cfg. */
int32_t eagle_tree_capacity(const eagle_tree_cfg* cfg);

/* Draft-logit rows consumed at `layer` (1..depth) per sequence: F_layer.
 * Returns -1 for an invalid cfg or layer. */
int32_t eagle_tree_frontier_rows(const eagle_tree_cfg* cfg, int32_t layer);

/* Expand (EAGLE-2 page, two-stage passage): for every frontier node f of every
 * sequence, take its draft row z (fp32, [batch][F_layer][vocab], row j belongs to
 * frontier[j]; at layer 1 the single row belongs to the root), and append its
 * top-k tokens (logit desc, token id asc) as children with
 *     logq  = (z_t - max z) - lse,   lse = log sum exp(z - max z)
 *     value = value(f) + logq
 * lse is summed in fp64 and rounded to fp32 once; logq and value are fp32
 * subtraction / addition.  Then, when layer < depth, frontier := the
 * min(m, |new layer|) new nodes of highest value (ties: lower id).
 * Layer 1 (re)initialises the tree from root_token [batch] (read only then).
 * Layers must be called in order 1..depth on the same stream.
 * Workspace: eagle_tree_expand_workspace bytes of device memory owned by the
 * caller, needing no initialisation; calls that share it must be stream-ordered.
 * A null or smaller workspace is EAGLE_ERR_WORKSPACE; vocab > EAGLE_MAX_VOCAB is
 * EAGLE_ERR_UNSUPPORTED. */
size_t eagle_tree_expand_workspace(const eagle_tree_cfg* cfg);

int eagle_tree_expand(const eagle_tree_cfg* cfg, int32_t layer, const float* draft_logits,
                      const int32_t* root_token, const eagle_tree_state* state, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/* Rerank (EAGLE-2 page, two-stage passage): per sequence, the n non-root nodes
 * that come first in (value desc, depth asc, id asc), written to kept [batch][n]
 * in ascending id order.  Requires all `depth` layers expanded.  n larger than
 * the number of non-root nodes is EAGLE_ERR_INVALID_ARG. */
int eagle_tree_rerank(const eagle_tree_cfg* cfg, const eagle_tree_state* state, int32_t* kept,
                      hipStream_t stream);

/* Flatten + mask + positions (EAGLE-2 page, passage after the two stages).
 * Row 0 is the root, rows 1..n are the kept nodes in ascending id (a topological
 * order).  Outputs, [batch][T] int32: flat_token, flat_parent (row index, -1 for
 * the root), flat_depth, position = ctx_len[b] + depth; mask [batch][T] uint64:
 * bit j of row i is set iff row j lies on the root-to-i path (i included).
 * ctx_len [batch] int32 device. */
int eagle_tree_mask(const eagle_tree_cfg* cfg, const eagle_tree_state* state,
                    const int32_t* kept, const int32_t* ctx_len, int32_t* flat_token,
                    int32_t* flat_parent, int32_t* flat_depth, int32_t* position,
                    uint64_t* mask, hipStream_t stream);

/* Tree attention (EAGLE-2 page: each flattened token attends to the whole
 * context and to its own ancestors only).  For sequence b, tree row i, query head
 * h and KV head g = h / (n_q_heads / n_kv_heads):
 *     keys  = cache rows kv_row_off[b] + c, c in [0, ctx_len[b])  (the context)
 *             and kv_row_off[b] + ctx_len[b] + j for every j with mask bit j of row i
 *     o     = softmax(scale * q . k) V ,   lse = log sum exp(scale * q . k)
 * Layouts (dtype = storage type of q, k_cache, v_cache, o):
 *     q, o      [batch][T][n_q_heads][head_dim]
 *     k_cache,
 *     v_cache   [n_kv_heads][kv_rows_total][head_dim]; sequence b owns rows
 *               kv_row_off[b] .. kv_row_off[b] + ctx_len[b] + T - 1, its tree rows last,
 *               in flattened order
 *     mask      [batch][T] uint64 from eagle_tree_mask
 *     lse       [batch][T][n_q_heads] fp32 natural log, or NULL
 * BF16: fp32 accumulation, probabilities rounded to bf16 before the PV product,
 * output rounded to nearest even.  F32: fp32 throughout.
 * kv_rows_total must be at least sum_b (ctx_len[b] + T) (not checkable on the
 * host; the call checks kv_rows_total >= batch * T).
 * Supported: BF16 or F32 with head_dim <= 128; T <= 64; batch <= EAGLE_MAX_BATCH;
 * for BF16 with head_dim 128 also, with B = min(batch, 256),
 *     n_kv_heads * ceil(G * T / 64) * (4 * (ceil(kv_rows_total / 64) + B) + 16 * B) < 2^31,
 * G = n_q_heads / n_kv_heads (otherwise EAGLE_ERR_UNSUPPORTED).  BF16 with head_dim
 * 128 runs the streaming MFMA kernels: one main kernel launch per 256 sequences --
 * the (sequence, KV head, row group) units of all of them are split over the GPU's
 * compute units together -- and one merge launch for the units split between
 * workgroups (none when no unit is).  Other head sizes, and F32, run one workgroup
 * per (tree row, query head) in fp32 arithmetic (a BF16 output rounded once to
 * nearest even).  The workspace (eagle_tree_attention_workspace bytes: 8,650,752
 * for BF16 with head_dim 128, none otherwise) holds the split-KV partials; it needs
 * no initialisation, and calls that share one must be ordered on one stream.
 * ctx_len_host / kv_row_off_host: optional host copies of ctx_len and kv_row_off
 * (both or neither; NULL = the kernels read the device arrays).  When given they
 * must hold the same values as the device arrays, and the BF16 kernels take each
 * sequence's context length and first row as launch arguments instead of reading
 * them when they start (one memory round trip less before the first load of each
 * kernel).  The call checks 0 <= ctx_len_host[b], 0 <= kv_row_off_host[b] and
 * kv_row_off_host[b] + ctx_len_host[b] + T <= kv_rows_total for every b
 * (EAGLE_ERR_INVALID_ARG otherwise); the host copies are read during the call
 * only.  F32 always reads the device arrays. */
typedef struct {
    eagle_dtype dtype;
    int32_t batch, T, n_q_heads, n_kv_heads, head_dim;
    const int32_t* ctx_len;    /* [batch] device */
    const int64_t* kv_row_off; /* [batch] device */
    int64_t kv_rows_total;
    float scale; /* 0 => 1/sqrt(head_dim) */
    const int32_t* ctx_len_host;    /* [batch] host, or NULL */
    const int64_t* kv_row_off_host; /* [batch] host, or NULL */
} eagle_attn_desc;

size_t eagle_tree_attention_workspace(const eagle_attn_desc* desc);

int eagle_tree_attention(const eagle_attn_desc* desc, const void* q, const void* k_cache,
                         const void* v_cache, const uint64_t* mask, void* o, float* lse,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Tree attention with rotary position encoding at the tree positions, in the
 * same launches (EAGLE-2 page, passage after the two stages: each flattened
 * token's position is adjusted to match plain autoregressive decoding).  The
 * attention of eagle_tree_attention, with every q row and the K of every tree row
 * rotated at its position (position [batch][T], from eagle_tree_mask or
 * eagle_tree_mask_static) as eagle_tree_rope defines the rotation (half-split
 * pairs, theta = p * base^(-2d / head_dim)); the context rows' K are used as
 * stored (already rotated).  Inside the kernel the rotation takes fp32 cosines and
 * sines of the angle reduced modulo one turn in fp64, so o and lse match
 * eagle_tree_rope followed by eagle_tree_attention within the bf16 tolerance, not
 * bit for bit.  Afterwards the tree rows' K in k_cache are rotated exactly as
 * eagle_tree_rope(q = NULL) leaves them (so eagle_kv_commit applies unchanged);
 * q is not modified, V is not touched.  BF16 with head_dim 128 only (any other
 * shape is EAGLE_ERR_UNSUPPORTED: call eagle_tree_rope, then eagle_tree_attention);
 * base > 0 and finite; other arguments, limits and the workspace as
 * eagle_tree_attention. */
int eagle_tree_attention_rope(const eagle_attn_desc* desc, const int32_t* position, double base, const void* q,
                              void* k_cache, const void* v_cache, const uint64_t* mask, void* o, float* lse,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Tree attention without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same operation, arguments, layouts, kernels and results
 * (bit for bit) as eagle_tree_attention; the split-KV partials live in a
 * file-scope device array of EAGLE_NOALLOC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends (its address is taken once per
 * device, on the first call with that device current; `stream` must belong to the
 * current device).  Nothing in it needs clearing between calls.  The call
 * allocates and frees nothing.  A shape whose eagle_tree_attention_workspace
 * exceeded EAGLE_NOALLOC_SCRATCH_BYTES would get EAGLE_ERR_WORKSPACE (nothing
 * launched; the workspace is at most 8,650,752 bytes for every shape, so none does);
 * other checks as eagle_tree_attention.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (other streams, other threads) race; order them on one stream. */
#define EAGLE_NOALLOC_SCRATCH_BYTES (16u << 20)

int eagle_tree_attention_noalloc(const eagle_attn_desc* desc, const void* q, const void* k_cache,
                                 const void* v_cache, const uint64_t* mask, void* o, float* lse,
                                 hipStream_t stream);

/* Verify (CSDN page 1.1/1.2, EAGLE page: the emitted tokens must follow the
 * target's own distribution).  target_logits [batch][T][vocab] fp32: row i is the
 * target's next-token logits after flattened row i.  The children of a row are
 * the rows whose flat_parent it is, in flattened order; a row may have up to
 * T - 1 of them (static trees), and siblings may carry the same token.
 *   temperature == 0: greedy -- starting at the root row, accept the child whose
 *     token is the row's argmax (lowest id on ties) while one exists; the final
 *     row's argmax is the bonus token.
 *   temperature > 0: sampled -- p = softmax(z / temperature); the children of the
 *     current row are tested in flattened order, child c accepted iff
 *     u < p(tok c) / (mass of the tokens not yet rejected at this row); a rejected
 *     child's token is removed, so a later sibling carrying the same token is
 *     never accepted.  With no acceptance (or no child) the bonus token
 *     is the smallest t whose running residual mass exceeds u * (residual total).
 *     u = top 24 bits / 2^24 of word 0 of Philox4x32-10 (Salmon et al., SC'11) with
 *     key (seed low, seed high) and counter (slot, row, sequence, step low 32
 *     bits); slot = child index, 0xFFFFFFFF for the bonus draw.
 * Outputs: accept_len [batch] (0..depth), accept_path [batch][depth] (flattened
 * rows, -1 padded), out_tokens [batch][depth + 1] (accepted tokens then the bonus,
 * -1 padded).  flat_token / flat_parent from eagle_tree_mask (or the caller's
 * static tree: flat_parent[b][0] = -1, 0 <= flat_parent[b][i] < i otherwise;
 * 0 <= flat_token[b][i] < vocab).
 * Only batch, vocab, depth and n of cfg are read (T = n + 1; topk and m are
 * ignored); n + 1 > EAGLE_MAX_TREE_ROWS, vocab > EAGLE_MAX_VOCAB or depth > 255 is
 * EAGLE_ERR_UNSUPPORTED.  Negative or NaN temperature is EAGLE_ERR_INVALID_ARG.
 * Workspace: eagle_verify_workspace bytes. */
size_t eagle_verify_workspace(const eagle_tree_cfg* cfg);

int eagle_verify(const eagle_tree_cfg* cfg, const float* target_logits, const int32_t* flat_token,
                 const int32_t* flat_parent, float temperature, uint64_t seed, uint64_t step,
                 int32_t* accept_len, int32_t* accept_path, int32_t* out_tokens, void* workspace,
                 size_t workspace_bytes, hipStream_t stream);

/* Static tree (EAGLE-2 page, opening paragraphs: EAGLE and Medusa draft over a
 * fixed tree shape; passage after the two stages: ancestor-only mask and
 * positions of the flattened tree).  In place of expand / rerank / mask, the
 * caller gives the flattened tree itself: flat_parent [batch][T] int32 device,
 * row 0 the root (-1), every other row's parent an earlier row.  Outputs as for
 * eagle_tree_mask: flat_depth and position = ctx_len[b] + depth ([batch][T]
 * int32) and mask [batch][T] uint64 (bit j of row i set iff row j lies on the
 * root-to-i path).  The caller's tokens serve as flat_token for attention and
 * verify unchanged.  A row whose path to the root meets a parent entry that is
 * not an earlier row (or a root entry other than -1) gets depth -1, position -1
 * and mask 0; the other rows are unaffected.  1 <= T <= EAGLE_MAX_TREE_ROWS
 * (otherwise EAGLE_ERR_INVALID_ARG / EAGLE_ERR_UNSUPPORTED). */
int eagle_tree_mask_static(int32_t batch, int32_t T, const int32_t* flat_parent, const int32_t* ctx_len,
                           int32_t* flat_depth, int32_t* position, uint64_t* mask, hipStream_t stream);

/* Rotary position encoding at the tree positions (EAGLE-2 page, passage after
 * the two stages: the flattened tokens' positions are adjusted so each matches
 * its position in plain autoregressive decoding).  In place, for sequence b and
 * tree row i at p = position[b][i] (from eagle_tree_mask or eagle_tree_mask_static):
 * every head of q [batch][T][n_q_heads][head_dim] and every KV head's tree row
 * kv_row_off[b] + ctx_len[b] + i of k_cache [n_kv_heads][kv_rows_total][head_dim].
 * Half-split form (the LLaMA family's): for d < head_dim / 2 the pair
 * (x[d], x[d + head_dim/2]) is rotated by theta = p * base^(-2d / head_dim).
 * Angles, cosines, sines and the rotation are fp64; the result is rounded to
 * fp32 (nearest even) and, for BF16, then to bf16 (nearest even).  Context rows
 * are not touched (the cache holds them already rotated).  desc as for
 * eagle_tree_attention (scale unused); when it carries host copies of ctx_len and
 * kv_row_off and batch <= 32, each sequence's first tree row rides in the launch
 * arguments (the copies must match the device arrays); otherwise the kernel reads
 * the device arrays.  A tree row outside the cache is left alone.  q or k_cache
 * may be NULL to rotate only the other.  head_dim even and <= 256, base > 0 and
 * finite.  Positions are not checked: p < 0 rotates backwards. */
int eagle_tree_rope(const eagle_attn_desc* desc, const int32_t* position, double base, void* q,
                    void* k_cache, hipStream_t stream);

/* KV commit of the accepted path (EAGLE-2 page, passage after the two stages:
 * verified tokens must stand as autoregressive decoding would have left them;
 * CSDN page 1.1: the accepted draft tokens are the output).  For sequence b with
 * accept_len a and accept_path r_1 < ... < r_a (flattened rows, from eagle_verify),
 * in every layer's K and V cache and every KV head, the row at
 * kv_row_off[b] + ctx_len[b] + r_j moves to kv_row_off[b] + ctx_len[b] + j
 * (j = 1..a; every source row is read before any is written).  The root's row
 * (ctx_len[b]) stays; new_ctx_len[b] = ctx_len[b] + 1 + a, the bonus token being
 * the next root.  Other rows are not touched.
 * Layouts: k_layers, v_layers are HOST arrays of n_layers device pointers, each
 * cache [n_kv_heads][kv_rows_total][head_dim] of dtype; accept_len [batch],
 * accept_path [batch][depth] int32 device (entries past accept_len unread);
 * ctx_len [batch] int32, kv_row_off [batch] int64 device; new_ctx_len [batch]
 * int32 device, which must not alias ctx_len.  Each sequence's rows up to
 * ctx_len[b] + T must lie inside the cache (not checkable on the host).
 * A sequence whose accept_len lies outside 0..min(depth, T - 1) or whose path is
 * not strictly increasing inside 1..T - 1 is not moved and gets new_ctx_len -1.
 * Supported: head_dim a multiple of 8 (BF16) or 4 (F32), head_dim <= 256, T <= 64,
 * depth <= 255; the layers are processed 64 to a launch. */
typedef struct {
    eagle_dtype dtype;
    int32_t batch, T, depth, n_kv_heads, head_dim, n_layers;
    const int32_t* ctx_len;    /* [batch] device */
    const int64_t* kv_row_off; /* [batch] device */
    int64_t kv_rows_total;
} eagle_commit_desc;

int eagle_kv_commit(const eagle_commit_desc* desc, const int32_t* accept_len, const int32_t* accept_path,
                    void* const* k_layers, void* const* v_layers, int32_t* new_ctx_len, hipStream_t stream);

/* Draft-side attention rows (EAGLE-2 page, two-stage passage: the m best nodes of
 * the last layer are fed to the draft model; EAGLE page: the draft model is one
 * decoder layer whose tokens, like the target's, see the context and their own
 * history only).  At draft layer `layer` (2..depth) the queries are the frontier
 * nodes -- eagle_tree_frontier_rows(cfg, layer) of them, in state->frontier after
 * eagle_tree_expand of layer - 1 -- and each attends to the context and to its own
 * root path.  Per sequence, the union of those root paths is flattened in
 * ascending node id (a topological order) into T_sub = eagle_draft_subtree_rows
 * (cfg, layer) = 1 + F_layer * (layer - 1) rows:
 *     sub_node   [batch][T_sub] node id, -1 for padding rows
 *     sub_parent [batch][T_sub] parent's row, -1 for the root and padding
 *     position   [batch][T_sub] ctx_len[b] + depth; padding: ctx_len[b]
 *     mask       [batch][T_sub] uint64: bit c of row r iff row c is on the root-to-r
 *                path (r included); a padding row sees only itself
 *     query_row  [batch][m]     the row of frontier[j]; -1 for j >= F_layer
 * The rows' draft K/V go behind the context with eagle_kv_gather (rows = sub_node),
 * and eagle_tree_attention with T = T_sub then gives every row's draft attention;
 * the frontier's are at query_row.  Layer 1's only query is the root (T_sub = 1).
 * T_sub > EAGLE_MAX_TREE_ROWS is EAGLE_ERR_UNSUPPORTED; layer outside 1..depth is
 * EAGLE_ERR_INVALID_ARG.  eagle_draft_subtree_rows returns -1 for an invalid cfg or
 * layer. */
int32_t eagle_draft_subtree_rows(const eagle_tree_cfg* cfg, int32_t layer);

int eagle_draft_subtree(const eagle_tree_cfg* cfg, int32_t layer, const eagle_tree_state* state,
                        const int32_t* ctx_len, int32_t* sub_node, int32_t* sub_parent, int32_t* position,
                        uint64_t* mask, int32_t* query_row, hipStream_t stream);

/* Row gather into the KV cache (the draft K/V of eagle_draft_subtree's rows, or of
 * any per-sequence row list).  For sequence b and row r < desc->T, every KV head's
 * row kv_row_off[b] + ctx_len[b] + r of k_cache / v_cache ([n_kv_heads]
 * [kv_rows_total][head_dim]) receives row b * src_rows_per_seq + x of src_k / src_v
 * ([n_kv_heads][src_rows_total][head_dim]), x = rows[b][r]; an x outside
 * 0..src_rows_per_seq - 1 (padding, -1) reads row x = 0.  desc as for
 * eagle_tree_attention (scale and host copies unused).  Destination rows outside
 * the cache are skipped.  Supported: head_dim a multiple of 8 (BF16) or 4 (F32),
 * <= 256; T <= 64; pointers 16-byte aligned; src_rows_total >= batch *
 * src_rows_per_seq. */
int eagle_kv_gather(const eagle_attn_desc* desc, const int32_t* rows, int64_t src_rows_per_seq,
                    int64_t src_rows_total, const void* src_k, const void* src_v, void* k_cache, void* v_cache,
                    hipStream_t stream);

/* Human-readable name of a status code. */
const char* eagle_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* EAGLE_TREE_H */
