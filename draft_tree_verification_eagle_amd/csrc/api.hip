// C ABI of the tree-verification library: host-side validation, then launches on
// the caller's stream.  See include/eagle_tree.h for the contract of each call.
#include <math.h>
#include <stdint.h>

#include "launchers.hpp"

namespace {

using eagle::attention_max_batch;

bool tree_cfg_ok(const eagle_tree_cfg* c) {
    return c && c->batch >= 0 && c->batch <= EAGLE_MAX_BATCH && c->vocab >= 1 && c->depth >= 1 &&
           c->topk >= 1 && c->m >= 1 && c->n >= 0 && c->topk <= c->vocab;
}

// Tree shape implied by the cfg; false if it exceeds the library's limits.
bool tree_shape(const eagle_tree_cfg* c, int32_t* capacity) {
    int64_t f = 1, cap = 1;
    for (int l = 0; l < c->depth; ++l) {
        cap += f * c->topk;
        if (cap > EAGLE_MAX_CAPACITY) return false;
        f = f * c->topk < c->m ? f * c->topk : c->m;
    }
    *capacity = (int32_t)cap;
    return true;
}

int tree_limits(const eagle_tree_cfg* c, int32_t* cap) {
    if (!tree_cfg_ok(c)) return EAGLE_ERR_INVALID_ARG;
    if (c->topk > EAGLE_MAX_TOPK || c->depth > 255 || (int64_t)c->m * c->topk > EAGLE_MAX_LAYER_NODES ||
        c->vocab > EAGLE_MAX_VOCAB ||
        c->n + 1 > EAGLE_MAX_TREE_ROWS || !tree_shape(c, cap))
        return EAGLE_ERR_UNSUPPORTED;
    if (c->n > *cap - 1) return EAGLE_ERR_INVALID_ARG;
    return EAGLE_OK;
}

// Verification reads batch, vocab, depth and n only (the flattened tree may come
// from a caller-given static tree, whose shape no topk / m describes).
int verify_limits(const eagle_tree_cfg* c) {
    if (!c || c->batch < 0 || c->vocab < 1 || c->depth < 1 || c->n < 0) return EAGLE_ERR_INVALID_ARG;
    if (c->batch > EAGLE_MAX_BATCH || c->vocab > EAGLE_MAX_VOCAB || c->depth > 255 ||
        c->n + 1 > EAGLE_MAX_TREE_ROWS)
        return EAGLE_ERR_UNSUPPORTED;
    return EAGLE_OK;
}

bool state_ok(const eagle_tree_state* s) {
    return s && s->token && s->parent && s->depth && s->value && s->frontier && s->n_nodes;
}

int from_hip(hipError_t e) { return e == hipSuccess ? EAGLE_OK : EAGLE_ERR_HIP; }

}  // namespace

extern "C" {

int32_t eagle_tree_capacity(const eagle_tree_cfg* cfg) {
    int32_t cap = 0;
    if (!tree_cfg_ok(cfg) || !tree_shape(cfg, &cap)) return -1;
    return cap;
}

int32_t eagle_tree_frontier_rows(const eagle_tree_cfg* cfg, int32_t layer) {
    if (!tree_cfg_ok(cfg) || layer < 1 || layer > cfg->depth) return -1;
    int64_t f = 1;
    for (int l = 1; l < layer; ++l) f = f * cfg->topk < cfg->m ? f * cfg->topk : cfg->m;
    return (int32_t)f;
}

size_t eagle_tree_expand_workspace(const eagle_tree_cfg* cfg) {
    int32_t cap = 0;
    if (tree_limits(cfg, &cap) != EAGLE_OK) return 0;
    return eagle::expand_workspace_bytes(*cfg);
}

int eagle_tree_expand(const eagle_tree_cfg* cfg, int32_t layer, const float* draft_logits,
                      const int32_t* root_token, const eagle_tree_state* state, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
    int32_t cap = 0;
    const int st = tree_limits(cfg, &cap);
    if (st != EAGLE_OK) return st;
    if (layer < 1 || layer > cfg->depth || !state_ok(state) || (layer == 1 && !root_token))
        return EAGLE_ERR_INVALID_ARG;
    if (cfg->batch == 0) return EAGLE_OK;
    if (!draft_logits) return EAGLE_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < eagle::expand_workspace_bytes(*cfg)) return EAGLE_ERR_WORKSPACE;
    const int rows = eagle_tree_frontier_rows(cfg, layer);
    return from_hip(eagle::launch_expand(*cfg, layer, rows, cap, draft_logits, root_token, *state,
                                         workspace, stream));
}

int eagle_tree_rerank(const eagle_tree_cfg* cfg, const eagle_tree_state* state, int32_t* kept,
                      hipStream_t stream) {
    int32_t cap = 0;
    const int st = tree_limits(cfg, &cap);
    if (st != EAGLE_OK) return st;
    if (!state_ok(state) || (cfg->n > 0 && !kept)) return EAGLE_ERR_INVALID_ARG;
    if (cfg->batch == 0 || cfg->n == 0) return EAGLE_OK;
    return from_hip(eagle::launch_rerank(*cfg, cap, *state, kept, stream));
}

int eagle_tree_mask(const eagle_tree_cfg* cfg, const eagle_tree_state* state, const int32_t* kept,
                    const int32_t* ctx_len, int32_t* flat_token, int32_t* flat_parent,
                    int32_t* flat_depth, int32_t* position, uint64_t* mask, hipStream_t stream) {
    int32_t cap = 0;
    const int st = tree_limits(cfg, &cap);
    if (st != EAGLE_OK) return st;
    if (!state_ok(state) || (cfg->n > 0 && !kept) || !ctx_len || !flat_token || !flat_parent ||
        !flat_depth || !position || !mask)
        return EAGLE_ERR_INVALID_ARG;
    if (cfg->batch == 0) return EAGLE_OK;
    return from_hip(eagle::launch_mask(*cfg, cap, *state, kept, ctx_len, flat_token, flat_parent,
                                       flat_depth, position, mask, stream));
}

static int attn_desc_check(const eagle_attn_desc* d) {
    if (!d || d->batch < 0 || d->T < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 1 ||
        d->n_q_heads % d->n_kv_heads != 0 || d->kv_rows_total < (int64_t)d->batch * d->T ||
        !(d->scale >= 0.0f) || isinf(d->scale))
        return EAGLE_ERR_INVALID_ARG;
    if (d->dtype != EAGLE_F32 && d->dtype != EAGLE_BF16) return EAGLE_ERR_INVALID_ARG;
    if (d->T > EAGLE_MAX_TREE_ROWS) return EAGLE_ERR_UNSUPPORTED;
    if (d->head_dim > 128) return EAGLE_ERR_UNSUPPORTED;
    if (d->dtype == EAGLE_BF16 && d->head_dim == 128 &&
        (d->batch > attention_max_batch() || !eagle::attention_split_fits(*d)))
        return EAGLE_ERR_UNSUPPORTED;
    if (d->batch > EAGLE_MAX_BATCH) return EAGLE_ERR_UNSUPPORTED;
    if ((d->ctx_len_host == nullptr) != (d->kv_row_off_host == nullptr)) return EAGLE_ERR_INVALID_ARG;
    if (d->ctx_len_host) {
        for (int b = 0; b < d->batch; ++b) {
            const int64_t c = d->ctx_len_host[b], off = d->kv_row_off_host[b];
            if (c < 0 || off < 0 || off > d->kv_rows_total - d->T - c) return EAGLE_ERR_INVALID_ARG;
        }
    }
    return EAGLE_OK;
}

size_t eagle_tree_attention_workspace(const eagle_attn_desc* desc) {
    if (attn_desc_check(desc) != EAGLE_OK) return 0;
    return eagle::attention_workspace_bytes(*desc);
}

int eagle_tree_attention(const eagle_attn_desc* desc, const void* q, const void* k_cache,
                         const void* v_cache, const uint64_t* mask, void* o, float* lse,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const int st = attn_desc_check(desc);
    if (st != EAGLE_OK) return st;
    if (desc->batch == 0) return EAGLE_OK;
    if (!q || !k_cache || !v_cache || !mask || !o || !desc->ctx_len || !desc->kv_row_off)
        return EAGLE_ERR_INVALID_ARG;
    const size_t need = eagle::attention_workspace_bytes(*desc);
    if (need > 0 && (!workspace || workspace_bytes < need)) return EAGLE_ERR_WORKSPACE;
    return from_hip(eagle::launch_attention(*desc, q, k_cache, v_cache, mask, o, lse, workspace, stream));
}

int eagle_tree_attention_rope(const eagle_attn_desc* desc, const int32_t* position, double base, const void* q,
                              void* k_cache, const void* v_cache, const uint64_t* mask, void* o, float* lse,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const int st = attn_desc_check(desc);
    if (st != EAGLE_OK) return st;
    if (desc->dtype != EAGLE_BF16 || desc->head_dim != 128) return EAGLE_ERR_UNSUPPORTED;
    if (!(base > 0.0) || isinf(base)) return EAGLE_ERR_INVALID_ARG;
    if (desc->batch == 0) return EAGLE_OK;
    if (!position || !q || !k_cache || !v_cache || !mask || !o || !desc->ctx_len || !desc->kv_row_off)
        return EAGLE_ERR_INVALID_ARG;
    const size_t need = eagle::attention_workspace_bytes(*desc);
    if (need > 0 && (!workspace || workspace_bytes < need)) return EAGLE_ERR_WORKSPACE;
    return from_hip(eagle::launch_attention(*desc, q, k_cache, v_cache, mask, o, lse, workspace, stream, position,
                                            base));
}

int eagle_tree_attention_noalloc(const eagle_attn_desc* desc, const void* q, const void* k_cache,
                                 const void* v_cache, const uint64_t* mask, void* o, float* lse,
                                 hipStream_t stream) {
    const int st = attn_desc_check(desc);
    if (st != EAGLE_OK) return st;
    if (desc->batch == 0) return EAGLE_OK;
    if (!q || !k_cache || !v_cache || !mask || !o || !desc->ctx_len || !desc->kv_row_off)
        return EAGLE_ERR_INVALID_ARG;
    if (eagle::attention_workspace_bytes(*desc) > (size_t)EAGLE_NOALLOC_SCRATCH_BYTES) return EAGLE_ERR_WORKSPACE;
    return from_hip(eagle::launch_attention_noalloc(*desc, q, k_cache, v_cache, mask, o, lse, stream));
}

size_t eagle_verify_workspace(const eagle_tree_cfg* cfg) {
    if (verify_limits(cfg) != EAGLE_OK) return 0;
    return eagle::verify_workspace_bytes(*cfg);
}

int eagle_verify(const eagle_tree_cfg* cfg, const float* target_logits, const int32_t* flat_token,
                 const int32_t* flat_parent, float temperature, uint64_t seed, uint64_t step,
                 int32_t* accept_len, int32_t* accept_path, int32_t* out_tokens, void* workspace,
                 size_t workspace_bytes, hipStream_t stream) {
    const int st = verify_limits(cfg);
    if (st != EAGLE_OK) return st;
    if (!(temperature >= 0.0f) || isinf(temperature)) return EAGLE_ERR_INVALID_ARG;
    if (cfg->batch == 0) return EAGLE_OK;
    if (!target_logits || !flat_token || !flat_parent || !accept_len || !accept_path || !out_tokens)
        return EAGLE_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < eagle::verify_workspace_bytes(*cfg)) return EAGLE_ERR_WORKSPACE;
    return from_hip(eagle::launch_verify(*cfg, target_logits, flat_token, flat_parent, temperature, seed,
                                         step, accept_len, accept_path, out_tokens, workspace, stream));
}

int eagle_tree_mask_static(int32_t batch, int32_t T, const int32_t* flat_parent, const int32_t* ctx_len,
                           int32_t* flat_depth, int32_t* position, uint64_t* mask, hipStream_t stream) {
    if (batch < 0 || T < 1) return EAGLE_ERR_INVALID_ARG;
    if (batch > EAGLE_MAX_BATCH || T > EAGLE_MAX_TREE_ROWS) return EAGLE_ERR_UNSUPPORTED;
    if (batch == 0) return EAGLE_OK;
    if (!flat_parent || !ctx_len || !flat_depth || !position || !mask) return EAGLE_ERR_INVALID_ARG;
    return from_hip(eagle::launch_mask_static(batch, T, flat_parent, ctx_len, flat_depth, position, mask,
                                              stream));
}

int eagle_tree_rope(const eagle_attn_desc* desc, const int32_t* position, double base, void* q,
                    void* k_cache, hipStream_t stream) {
    const eagle_attn_desc* d = desc;
    if (!d || d->batch < 0 || d->T < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 2 ||
        d->head_dim % 2 != 0 || d->kv_rows_total < 0 || !(base > 0.0) || isinf(base))
        return EAGLE_ERR_INVALID_ARG;
    if (d->dtype != EAGLE_F32 && d->dtype != EAGLE_BF16) return EAGLE_ERR_INVALID_ARG;
    if (d->T > EAGLE_MAX_TREE_ROWS || d->head_dim > 256 || d->batch > EAGLE_MAX_BATCH) return EAGLE_ERR_UNSUPPORTED;
    if (d->batch == 0 || (!q && !k_cache)) return EAGLE_OK;
    if (!position || (k_cache && (!d->ctx_len || !d->kv_row_off))) return EAGLE_ERR_INVALID_ARG;
    return from_hip(eagle::launch_rope(*d, position, base, q, k_cache, stream));
}

int eagle_kv_commit(const eagle_commit_desc* desc, const int32_t* accept_len, const int32_t* accept_path,
                    void* const* k_layers, void* const* v_layers, int32_t* new_ctx_len, hipStream_t stream) {
    const eagle_commit_desc* d = desc;
    if (!d || d->batch < 0 || d->T < 1 || d->depth < 1 || d->n_kv_heads < 1 || d->head_dim < 1 ||
        d->n_layers < 0 || d->kv_rows_total < 0)
        return EAGLE_ERR_INVALID_ARG;
    if (d->dtype != EAGLE_F32 && d->dtype != EAGLE_BF16) return EAGLE_ERR_INVALID_ARG;
    const int align = d->dtype == EAGLE_BF16 ? 8 : 4;
    if (d->T > EAGLE_MAX_TREE_ROWS || d->depth > 255 || d->head_dim > 256 || d->head_dim % align != 0 ||
        d->batch > EAGLE_MAX_BATCH || d->n_kv_heads > 65535)
        return EAGLE_ERR_UNSUPPORTED;
    if (d->batch == 0) return EAGLE_OK;
    if (!accept_len || !accept_path || !new_ctx_len || !d->ctx_len || !d->kv_row_off ||
        (const void*)new_ctx_len == (const void*)d->ctx_len)
        return EAGLE_ERR_INVALID_ARG;
    if (d->n_layers > 0 && (!k_layers || !v_layers)) return EAGLE_ERR_INVALID_ARG;
    for (int l = 0; l < d->n_layers; ++l) {
        if (!k_layers[l] || !v_layers[l] || ((uintptr_t)k_layers[l] & 15) || ((uintptr_t)v_layers[l] & 15))
            return EAGLE_ERR_INVALID_ARG;
    }
    return from_hip(eagle::launch_kv_commit(*d, accept_len, accept_path, k_layers, v_layers, new_ctx_len,
                                            stream));
}

int32_t eagle_draft_subtree_rows(const eagle_tree_cfg* cfg, int32_t layer) {
    const int32_t F = eagle_tree_frontier_rows(cfg, layer);
    if (F < 0) return -1;
    const int64_t t = 1 + (int64_t)F * (layer - 1);
    return t > INT32_MAX ? -1 : (int32_t)t;
}

int eagle_draft_subtree(const eagle_tree_cfg* cfg, int32_t layer, const eagle_tree_state* state,
                        const int32_t* ctx_len, int32_t* sub_node, int32_t* sub_parent, int32_t* position,
                        uint64_t* mask, int32_t* query_row, hipStream_t stream) {
    int32_t cap = 0;
    const int st = tree_limits(cfg, &cap);
    if (st != EAGLE_OK) return st;
    if (layer < 1 || layer > cfg->depth || !state_ok(state)) return EAGLE_ERR_INVALID_ARG;
    const int32_t T_sub = eagle_draft_subtree_rows(cfg, layer);
    if (T_sub < 1) return EAGLE_ERR_INVALID_ARG;
    if (T_sub > EAGLE_MAX_TREE_ROWS) return EAGLE_ERR_UNSUPPORTED;
    if (cfg->batch == 0) return EAGLE_OK;
    if (!ctx_len || !sub_node || !sub_parent || !position || !mask || !query_row) return EAGLE_ERR_INVALID_ARG;
    const int F = eagle_tree_frontier_rows(cfg, layer);
    return from_hip(eagle::launch_draft_subtree(*cfg, layer, cap, F, T_sub, *state, ctx_len, sub_node, sub_parent,
                                                position, mask, query_row, stream));
}

int eagle_kv_gather(const eagle_attn_desc* desc, const int32_t* rows, int64_t src_rows_per_seq,
                    int64_t src_rows_total, const void* src_k, const void* src_v, void* k_cache, void* v_cache,
                    hipStream_t stream) {
    const eagle_attn_desc* d = desc;
    if (!d || d->batch < 0 || d->T < 1 || d->n_kv_heads < 1 || d->head_dim < 1 || d->kv_rows_total < 0 ||
        src_rows_per_seq < 1 || src_rows_total < 0)
        return EAGLE_ERR_INVALID_ARG;
    if (d->dtype != EAGLE_F32 && d->dtype != EAGLE_BF16) return EAGLE_ERR_INVALID_ARG;
    const int align = d->dtype == EAGLE_BF16 ? 8 : 4;
    if (d->T > EAGLE_MAX_TREE_ROWS || d->head_dim > 256 || d->head_dim % align != 0 || d->batch > EAGLE_MAX_BATCH ||
        d->n_kv_heads > 65535)
        return EAGLE_ERR_UNSUPPORTED;
    if (src_rows_total < (int64_t)d->batch * src_rows_per_seq) return EAGLE_ERR_INVALID_ARG;
    if (d->batch == 0) return EAGLE_OK;
    if (!rows || !src_k || !src_v || !k_cache || !v_cache || !d->ctx_len || !d->kv_row_off) return EAGLE_ERR_INVALID_ARG;
    if (((uintptr_t)src_k | (uintptr_t)src_v | (uintptr_t)k_cache | (uintptr_t)v_cache) & 15)
        return EAGLE_ERR_INVALID_ARG;
    return from_hip(eagle::launch_kv_gather(*d, rows, src_rows_per_seq, src_rows_total, src_k, src_v, k_cache,
                                            v_cache, stream));
}

const char* eagle_status_string(int status) {
    switch (status) {
        case EAGLE_OK: return "ok";
        case EAGLE_ERR_INVALID_ARG: return "invalid argument";
        case EAGLE_ERR_UNSUPPORTED: return "unsupported shape or type";
        case EAGLE_ERR_WORKSPACE: return "workspace missing or too small";
        case EAGLE_ERR_HIP: return "HIP launch error";
        default: return "unknown status";
    }
}

}  // extern "C"
