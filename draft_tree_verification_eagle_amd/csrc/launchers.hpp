// Internal host-side launch entry points of the tree-verification library.  The
// C ABI (api.hip) validates arguments and then calls these; they only enqueue
// kernels on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "eagle_tree.h"

namespace eagle {

// Expand: vocabulary chunks per draft row, then a per-sequence merge.
int expand_chunks(int vocab);
size_t expand_workspace_bytes(const eagle_tree_cfg& cfg);
hipError_t launch_expand(const eagle_tree_cfg& cfg, int layer, int rows, int cap,
                         const float* logits, const int32_t* root_token,
                         const eagle_tree_state& st, void* workspace, hipStream_t stream);

hipError_t launch_rerank(const eagle_tree_cfg& cfg, int cap, const eagle_tree_state& st,
                         int32_t* kept, hipStream_t stream);

hipError_t launch_mask(const eagle_tree_cfg& cfg, int cap, const eagle_tree_state& st,
                       const int32_t* kept, const int32_t* ctx_len, int32_t* flat_token,
                       int32_t* flat_parent, int32_t* flat_depth, int32_t* position,
                       uint64_t* mask, hipStream_t stream);

// Tree attention.  Workspace layout and launch shape are decided here.
int attention_max_batch();
size_t attention_workspace_bytes(const eagle_attn_desc& d);
// The bf16 path splits its work on a 31-bit cost line; false if this shape would
// not fit it.
bool attention_split_fits(const eagle_attn_desc& d);
// rope_position non-null: the bf16 attention of q and the tree K rows rotated at
// those positions (rotary with base rope_base), the cache's tree K rows left rotated.
hipError_t launch_attention(const eagle_attn_desc& d, const void* q, const void* k,
                            const void* v, const uint64_t* mask, void* o, float* lse,
                            void* workspace, hipStream_t stream,
                            const int32_t* rope_position = nullptr, double rope_base = 0.0);

// The same launch with the partials in the library's per-device array of
// EAGLE_NOALLOC_SCRATCH_BYTES (no caller workspace); the caller has checked the
// size against the array's.
hipError_t launch_attention_noalloc(const eagle_attn_desc& d, const void* q, const void* k,
                                    const void* v, const uint64_t* mask, void* o, float* lse,
                                    hipStream_t stream);

size_t verify_workspace_bytes(const eagle_tree_cfg& cfg);
hipError_t launch_verify(const eagle_tree_cfg& cfg, const float* target, const int32_t* flat_token,
                         const int32_t* flat_parent, float temperature, uint64_t seed,
                         uint64_t step, int32_t* accept_len, int32_t* accept_path,
                         int32_t* out_tokens, void* workspace, hipStream_t stream);

// Around the step: static-tree mask, rotary at the tree positions, KV commit.
constexpr int kCommitMaxLayers = 64;  // layers per commit launch (their pointers ride in the arguments)
hipError_t launch_mask_static(int batch, int T, const int32_t* flat_parent, const int32_t* ctx_len,
                              int32_t* flat_depth, int32_t* position, uint64_t* mask, hipStream_t stream);
hipError_t launch_rope(const eagle_attn_desc& d, const int32_t* position, double base, void* q, void* k,
                       hipStream_t stream);
hipError_t launch_kv_commit(const eagle_commit_desc& d, const int32_t* accept_len, const int32_t* accept_path,
                            void* const* k_layers, void* const* v_layers, int32_t* new_ctx_len,
                            hipStream_t stream);

// Draft-side attention rows and the row gather into the KV cache.
hipError_t launch_draft_subtree(const eagle_tree_cfg& cfg, int layer, int cap, int F, int T_sub,
                                const eagle_tree_state& st, const int32_t* ctx_len, int32_t* sub_node,
                                int32_t* sub_parent, int32_t* position, uint64_t* mask, int32_t* query_row,
                                hipStream_t stream);
hipError_t launch_kv_gather(const eagle_attn_desc& d, const int32_t* rows, int64_t src_rows_per_seq,
                            int64_t src_rows_total, const void* src_k, const void* src_v, void* k, void* v,
                            hipStream_t stream);

}  // namespace eagle
