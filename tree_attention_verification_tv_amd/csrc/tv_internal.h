// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tv.h"

#define TV_MAX_NODES_DEV 64

namespace tv {

hipError_t launch_build_tree(const int32_t* parents, const int32_t* n_nodes, int B, int n_max,
                             uint64_t* anc, int32_t* depth, int32_t* err, hipStream_t s);

hipError_t launch_accept(const int32_t* cand_tok, const int32_t* tgt, const int32_t* parents,
                         const uint64_t* anc, const int32_t* depth, const int32_t* n_nodes,
                         const int32_t* err, int B, int n_max, int32_t* accept_len,
                         int32_t* path, int32_t* bonus, int32_t* out_tokens, hipStream_t s);

hipError_t launch_accept_typical(const int32_t* cand_tok, const int32_t* tgt_argmax,
                                 const float* p_tok, const float* entropy, float eps, float delta,
                                 const int32_t* parents, const uint64_t* anc, const int32_t* depth,
                                 const int32_t* n_nodes, const int32_t* err, int B, int n_max,
                                 int32_t* accept_len, int32_t* path, int32_t* bonus,
                                 int32_t* out_tokens, hipStream_t s);

hipError_t launch_eagle2_tree(const float* conf, const int32_t* cand, const int32_t* root_tok, int B, int S,
                              int K, int M, int n_max, int32_t* parents, int32_t* tokens, float* values,
                              int32_t* n_nodes, hipStream_t s);

hipError_t launch_speculative_sample(const void* p_logits, const void* q_logits, int elem_bytes, int V,
                                     const int32_t* draft, const float* u_acc, const float* u_res, int B, int L,
                                     float* p_tok, float* q_tok, int32_t* accept_len, int32_t* tokens,
                                     float* stats, hipStream_t s);

hipError_t launch_typical_stats(const void* logits, int elem_bytes, int V, const int32_t* cand_tok,
                                const int32_t* parents, const int32_t* n_nodes, const int32_t* err,
                                int B, int n_max, float* entropy, float* p_tok, int32_t* argmax,
                                hipStream_t s);

hipError_t launch_accept_commit(const int32_t* cand_tok, const int32_t* tgt, const int32_t* parents,
                                const uint64_t* anc, const int32_t* depth, const int32_t* n_nodes,
                                const int32_t* err, int B, int n_max, int32_t* accept_len, int32_t* path,
                                int32_t* bonus, int32_t* out_tokens, void* k_cache, void* v_cache, int Hkv,
                                int cap, int D, int elem_bytes, const int32_t* prefix_len_in,
                                int32_t* prefix_len_out, const tv_paged_kv* pk, hipStream_t s);

// pk: paged cache (nullptr: the dense layout)
// V cache layout conversion (tv_layout.hip): n_blocks 64-slot blocks of D
// dims, rows -> blocked, or blocked -> rows when to_rows.
hipError_t launch_v_layout(const void* src, void* dst, long n_blocks, int D, int elem_bytes, bool to_rows,
                           hipStream_t s);
hipError_t launch_commit(void* k_cache, void* v_cache, int B, int Hkv, int cap, int D,
                         int elem_bytes, const int32_t* prefix_len_in, const int32_t* accept_len,
                         const int32_t* path, int n_max, int32_t* prefix_len_out,
                         const tv_paged_kv* pk, hipStream_t s);

// Launch plan of the bf16 attention: waves per workgroup, row blocks, KV
// splits and the workspace they need.
struct AttnPlan {
  int waves;       // wavefronts per workgroup
  int qt;          // 32-row query tiles per wavefront
  int row_blocks;  // workgroups along the (node, head-in-group) rows
  int splits;      // workgroups along the prefix keys
  int rows_pad;    // row_blocks * waves * 32
  bool fused;      // the splits merge inside the main kernel (no merge kernel)
  bool last_merges;  // (fused) the last split to arrive merges every range
                     // and none waits: for grids that do not run at once
  size_t workspace_bytes;
};

AttnPlan plan_attention_bf16(const tv_attn_args* a);

// pk: paged cache (nullptr: the dense layout); parents (dense only): the
// kernel builds the tree from it and writes a->anc, a->depth and a->err
hipError_t launch_attention_bf16(const tv_attn_args* a, const AttnPlan& plan, const tv_paged_kv* pk,
                                 const int32_t* parents, hipStream_t s);
hipError_t launch_attention_f32(const tv_attn_args* a, hipStream_t s);

// Bytes of the static device scratch behind tv_tree_attention_noalloc (every
// workload of this library needs at most about 35 MB), and its device address
// on the current device (looked up once per device).
constexpr size_t kScratchBytes = size_t(48) << 20;
// largest query-head group Hq / Hkv of the bf16 attention (its index
// arithmetic divides query rows by the group with a bounded multiplier)
constexpr int kMaxGroup = 4096;
hipError_t scratch_workspace(void** ptr);

}  // namespace tv
