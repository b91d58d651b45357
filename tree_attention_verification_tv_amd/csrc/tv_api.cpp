// C ABI of libtv: host-side argument checks, launch planning and dispatch.
// Every check happens before the first HIP call, so invalid arguments are
// reported without touching the device.
#include <hip/hip_runtime.h>

#include "tv.h"
#include "tv_internal.h"

namespace {

bool dtype_ok(int32_t d) { return d == TV_F32 || d == TV_BF16; }
int elem_bytes(int32_t d) { return d == TV_F32 ? 4 : 2; }

tv_status from_hip(hipError_t e) { return e == hipSuccess ? TV_OK : TV_ERR_HIP; }

// Shapes of tv_tree_attention that the kernels accept.
tv_status check_attn_shapes(const tv_attn_args* a) {
  if (a == nullptr) return TV_ERR_INVALID_ARG;
  if (a->B < 0 || a->n_max < 1 || a->n_max > TV_MAX_NODES) return TV_ERR_INVALID_ARG;
  if (a->Hq < 1 || a->Hkv < 1 || a->Hq % a->Hkv != 0) return TV_ERR_INVALID_ARG;
  if (a->cap < a->n_max || a->cap % 64 != 0 || a->D < 1) return TV_ERR_INVALID_ARG;
  if (!dtype_ok(a->dtype)) return TV_ERR_INVALID_ARG;
  if (a->D != 64 && a->D != 128) return TV_ERR_UNSUPPORTED;
  if (a->dtype == TV_BF16 && a->D == 128 && a->Hq / a->Hkv > tv::kMaxGroup) return TV_ERR_UNSUPPORTED;
  return TV_OK;
}

// fp32 inputs, and bf16 at head dim 64, take the vector-ALU kernel (no
// workspace); bf16 at head dim 128 the matrix-core kernels.
bool vector_path(const tv_attn_args* a) { return a->dtype == TV_F32 || a->D != 128; }

}  // namespace

extern "C" {

const char* tv_status_string(tv_status s) {
  switch (s) {
    case TV_OK: return "ok";
    case TV_ERR_INVALID_ARG: return "invalid argument";
    case TV_ERR_BAD_TREE: return "parents array is not a parents-first tree";
    case TV_ERR_CAPACITY: return "prefix plus tree exceeds the cache capacity";
    case TV_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case TV_ERR_HIP: return "HIP runtime or launch error";
    case TV_ERR_BAD_PAGE: return "block table names a page outside the pools";
    case TV_ERR_SCRATCH: return "shapes need more scratch than the allocation-free entry point holds";
  }
  return "unknown status";
}

const char* tv_version(void) { return "tv 0.1.0 (gfx950)"; }

tv_status tv_build_tree(const int32_t* parents, const int32_t* n_nodes, int32_t B, int32_t n_max,
                        uint64_t* anc, int32_t* depth, int32_t* err, hipStream_t stream) {
  if (B < 0 || n_max < 1 || n_max > TV_MAX_NODES) return TV_ERR_INVALID_ARG;
  if (B == 0) return TV_OK;
  if (!parents || !n_nodes || !anc || !depth || !err) return TV_ERR_INVALID_ARG;
  return from_hip(tv::launch_build_tree(parents, n_nodes, B, n_max, anc, depth, err, stream));
}

size_t tv_tree_attention_workspace_size(const tv_attn_args* a) {
  if (check_attn_shapes(a) != TV_OK || a->B == 0) return 0;
  if (vector_path(a)) return 0;
  return tv::plan_attention_bf16(a).workspace_bytes;
}

tv_status tv_tree_attention(const tv_attn_args* a, hipStream_t stream) {
  const tv_status st = check_attn_shapes(a);
  if (st != TV_OK) return st;
  if (a->B == 0) return TV_OK;
  if (!a->q || !a->k_new || !a->v_new || !a->k_cache || !a->v_cache || !a->prefix_len ||
      !a->n_nodes || !a->anc || !a->depth || !a->err || !a->out)
    return TV_ERR_INVALID_ARG;
  if (vector_path(a)) return from_hip(tv::launch_attention_f32(a, stream));
  const tv::AttnPlan plan = tv::plan_attention_bf16(a);
  if (plan.workspace_bytes > 0 && (a->workspace == nullptr || a->workspace_bytes < plan.workspace_bytes))
    return TV_ERR_INVALID_ARG;
  return from_hip(tv::launch_attention_bf16(a, plan, nullptr, nullptr, stream));
}

tv_status tv_tree_attention_noalloc(const tv_attn_args* a, hipStream_t stream) {
  const tv_status st = check_attn_shapes(a);
  if (st != TV_OK) return st;
  if (a->B == 0) return TV_OK;
  if (!a->q || !a->k_new || !a->v_new || !a->k_cache || !a->v_cache || !a->prefix_len ||
      !a->n_nodes || !a->anc || !a->depth || !a->err || !a->out)
    return TV_ERR_INVALID_ARG;
  if (vector_path(a)) return from_hip(tv::launch_attention_f32(a, stream));   // (no workspace)
  const tv::AttnPlan plan = tv::plan_attention_bf16(a);
  if (plan.workspace_bytes > tv::kScratchBytes) return TV_ERR_SCRATCH;
  tv_attn_args b = *a;
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  if (plan.workspace_bytes > 0) {
    if (tv::scratch_workspace(&b.workspace) != hipSuccess) return TV_ERR_HIP;
    b.workspace_bytes = tv::kScratchBytes;
  }
  return from_hip(tv::launch_attention_bf16(&b, plan, nullptr, nullptr, stream));
}

tv_status tv_tree_attention_from_parents(const tv_attn_args* a, const int32_t* parents, uint64_t* anc,
                                         int32_t* depth, hipStream_t stream) {
  const tv_status st = check_attn_shapes(a);
  if (st != TV_OK) return st;
  if (a->B == 0) return TV_OK;
  if (!a->q || !a->k_new || !a->v_new || !a->k_cache || !a->v_cache || !a->prefix_len ||
      !a->n_nodes || !a->err || !a->out || !parents || !anc || !depth)
    return TV_ERR_INVALID_ARG;
  tv_attn_args b = *a;
  b.anc = anc;
  b.depth = depth;
  if (vector_path(a)) {
    // (the vector-ALU kernel reads a built tree: two launches)
    const hipError_t e = tv::launch_build_tree(parents, a->n_nodes, a->B, a->n_max, anc, depth, a->err, stream);
    if (e != hipSuccess) return TV_ERR_HIP;
    return from_hip(tv::launch_attention_f32(&b, stream));
  }
  const tv::AttnPlan plan = tv::plan_attention_bf16(a);
  if (plan.workspace_bytes > 0 && (a->workspace == nullptr || a->workspace_bytes < plan.workspace_bytes))
    return TV_ERR_INVALID_ARG;
  return from_hip(tv::launch_attention_bf16(&b, plan, nullptr, parents, stream));
}

tv_status tv_tree_attention_paged(const tv_attn_args* a, const tv_paged_kv* pk, hipStream_t stream) {
  const tv_status st = check_attn_shapes(a);
  if (st != TV_OK) return st;
  if (pk == nullptr || pk->max_pages < 1 || pk->num_pages < 1) return TV_ERR_INVALID_ARG;
  if (a->cap != 64 * pk->max_pages) return TV_ERR_INVALID_ARG;
  if (a->dtype != TV_BF16 || a->D != 128 || pk->max_pages > TV_MAX_PAGES_PER_SEQ) return TV_ERR_UNSUPPORTED;
  if (a->B == 0) return TV_OK;
  if (!a->q || !a->k_new || !a->v_new || !a->k_cache || !a->v_cache || !a->prefix_len ||
      !a->n_nodes || !a->anc || !a->depth || !a->err || !a->out || !pk->block_table)
    return TV_ERR_INVALID_ARG;
  const tv::AttnPlan plan = tv::plan_attention_bf16(a);
  if (plan.workspace_bytes > 0 && (a->workspace == nullptr || a->workspace_bytes < plan.workspace_bytes))
    return TV_ERR_INVALID_ARG;
  return from_hip(tv::launch_attention_bf16(a, plan, pk, nullptr, stream));
}

tv_status tv_tree_attention_paged_from_parents(const tv_attn_args* a, const tv_paged_kv* pk, const int32_t* parents,
                                               uint64_t* anc, int32_t* depth, hipStream_t stream) {
  const tv_status st = check_attn_shapes(a);
  if (st != TV_OK) return st;
  if (pk == nullptr || pk->max_pages < 1 || pk->num_pages < 1) return TV_ERR_INVALID_ARG;
  if (a->cap != 64 * pk->max_pages) return TV_ERR_INVALID_ARG;
  if (a->dtype != TV_BF16 || a->D != 128 || pk->max_pages > TV_MAX_PAGES_PER_SEQ) return TV_ERR_UNSUPPORTED;
  if (a->B == 0) return TV_OK;
  if (!a->q || !a->k_new || !a->v_new || !a->k_cache || !a->v_cache || !a->prefix_len ||
      !a->n_nodes || !a->err || !a->out || !pk->block_table || !parents || !anc || !depth)
    return TV_ERR_INVALID_ARG;
  const tv::AttnPlan plan = tv::plan_attention_bf16(a);
  if (plan.workspace_bytes > 0 && (a->workspace == nullptr || a->workspace_bytes < plan.workspace_bytes))
    return TV_ERR_INVALID_ARG;
  tv_attn_args b = *a;
  b.anc = anc;
  b.depth = depth;
  return from_hip(tv::launch_attention_bf16(&b, plan, pk, parents, stream));
}

tv_status tv_accept(const int32_t* cand_tok, const int32_t* tgt_argmax, const int32_t* parents,
                    const uint64_t* anc, const int32_t* depth, const int32_t* n_nodes,
                    const int32_t* err, int32_t B, int32_t n_max, int32_t* accept_len,
                    int32_t* path, int32_t* bonus_tok, int32_t* out_tokens, hipStream_t stream) {
  if (B < 0 || n_max < 1 || n_max > TV_MAX_NODES) return TV_ERR_INVALID_ARG;
  if (B == 0) return TV_OK;
  if (!cand_tok || !tgt_argmax || !parents || !anc || !depth || !n_nodes || !accept_len || !path ||
      !bonus_tok)
    return TV_ERR_INVALID_ARG;
  return from_hip(tv::launch_accept(cand_tok, tgt_argmax, parents, anc, depth, n_nodes, err, B,
                                    n_max, accept_len, path, bonus_tok, out_tokens, stream));
}

tv_status tv_accept_commit(const int32_t* cand_tok, const int32_t* tgt_argmax, const int32_t* parents,
                           const uint64_t* anc, const int32_t* depth, const int32_t* n_nodes,
                           const int32_t* err, int32_t B, int32_t n_max, int32_t* accept_len, int32_t* path,
                           int32_t* bonus_tok, int32_t* out_tokens, void* k_cache, void* v_cache, int32_t Hkv,
                           int32_t cap, int32_t D, int32_t dtype, const int32_t* prefix_len_in,
                           int32_t* prefix_len_out, hipStream_t stream) {
  if (B < 0 || n_max < 1 || n_max > TV_MAX_NODES || Hkv < 1 || cap < n_max || cap % 64 != 0)
    return TV_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return TV_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return TV_ERR_UNSUPPORTED;
  if (B == 0) return TV_OK;
  if (!cand_tok || !tgt_argmax || !parents || !anc || !depth || !n_nodes || !accept_len || !path ||
      !bonus_tok || !k_cache || !v_cache || !prefix_len_in || !prefix_len_out)
    return TV_ERR_INVALID_ARG;
  return from_hip(tv::launch_accept_commit(cand_tok, tgt_argmax, parents, anc, depth, n_nodes, err, B, n_max,
                                           accept_len, path, bonus_tok, out_tokens, k_cache, v_cache, Hkv, cap, D,
                                           elem_bytes(dtype), prefix_len_in, prefix_len_out, nullptr, stream));
}

tv_status tv_accept_commit_paged(const int32_t* cand_tok, const int32_t* tgt_argmax, const int32_t* parents,
                                 const uint64_t* anc, const int32_t* depth, const int32_t* n_nodes,
                                 const int32_t* err, int32_t B, int32_t n_max, int32_t* accept_len, int32_t* path,
                                 int32_t* bonus_tok, int32_t* out_tokens, void* k_pool, void* v_pool,
                                 const tv_paged_kv* pk, int32_t Hkv, int32_t D, int32_t dtype,
                                 const int32_t* prefix_len_in, int32_t* prefix_len_out, hipStream_t stream) {
  if (pk == nullptr || pk->max_pages < 1 || pk->num_pages < 1) return TV_ERR_INVALID_ARG;
  if (B < 0 || n_max < 1 || n_max > TV_MAX_NODES || Hkv < 1 || 64 * pk->max_pages < n_max)
    return TV_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return TV_ERR_INVALID_ARG;
  if ((D != 64 && D != 128) || pk->max_pages > TV_MAX_PAGES_PER_SEQ) return TV_ERR_UNSUPPORTED;
  if (B == 0) return TV_OK;
  if (!cand_tok || !tgt_argmax || !parents || !anc || !depth || !n_nodes || !accept_len || !path ||
      !bonus_tok || !k_pool || !v_pool || !pk->block_table || !prefix_len_in || !prefix_len_out)
    return TV_ERR_INVALID_ARG;
  return from_hip(tv::launch_accept_commit(cand_tok, tgt_argmax, parents, anc, depth, n_nodes, err, B, n_max,
                                           accept_len, path, bonus_tok, out_tokens, k_pool, v_pool, Hkv,
                                           64 * pk->max_pages, D, elem_bytes(dtype), prefix_len_in, prefix_len_out,
                                           pk, stream));
}

tv_status tv_eagle2_tree(const float* conf, const int32_t* cand, const int32_t* root_tok, int32_t B,
                         int32_t S, int32_t K, int32_t M, int32_t n_max, int32_t* parents,
                         int32_t* tokens, float* values, int32_t* n_nodes, hipStream_t stream) {
  if (B < 0 || S < 1 || K < 1 || M < 1 || n_max < 1 || n_max > TV_MAX_NODES) return TV_ERR_INVALID_ARG;
  if (static_cast<int64_t>(S) * K * M > TV_MAX_DRAFT_PROPOSALS) return TV_ERR_UNSUPPORTED;
  if (B == 0) return TV_OK;
  if (!conf || !cand || !root_tok || !parents || !tokens || !values || !n_nodes) return TV_ERR_INVALID_ARG;
  return from_hip(tv::launch_eagle2_tree(conf, cand, root_tok, B, S, K, M, n_max, parents, tokens, values,
                                         n_nodes, stream));
}

size_t tv_speculative_sample_workspace_size(int32_t B, int32_t L) {
  if (B < 1 || L < 1 || L > TV_MAX_NODES) return 0;
  return static_cast<size_t>(B) * (2 * L + 1) * 2 * sizeof(float);
}

tv_status tv_speculative_sample(const void* p_logits, const void* q_logits, int32_t dtype, int32_t vocab,
                                const int32_t* draft, const float* u_acc, const float* u_res, int32_t B,
                                int32_t L, float* p_tok, float* q_tok, int32_t* accept_len, int32_t* tokens,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || B > 65535 || L < 1 || L > TV_MAX_NODES || vocab < 1) return TV_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return TV_ERR_INVALID_ARG;
  if (B == 0) return TV_OK;
  if (!p_logits || !q_logits || !draft || !u_acc || !u_res || !p_tok || !q_tok || !accept_len || !tokens ||
      !workspace || workspace_bytes < tv_speculative_sample_workspace_size(B, L))
    return TV_ERR_INVALID_ARG;
  return from_hip(tv::launch_speculative_sample(p_logits, q_logits, elem_bytes(dtype), vocab, draft, u_acc,
                                                u_res, B, L, p_tok, q_tok, accept_len, tokens,
                                                static_cast<float*>(workspace), stream));
}

tv_status tv_accept_typical(const void* logits, int32_t dtype, int32_t vocab,
                            const int32_t* cand_tok, const int32_t* parents, const uint64_t* anc,
                            const int32_t* depth, const int32_t* n_nodes, const int32_t* err,
                            int32_t B, int32_t n_max, float epsilon, float delta, float* entropy,
                            float* p_tok, int32_t* tgt_argmax, int32_t* accept_len, int32_t* path,
                            int32_t* bonus_tok, int32_t* out_tokens, hipStream_t stream) {
  if (B < 0 || B > 65535 || n_max < 1 || n_max > TV_MAX_NODES || vocab < 1)
    return TV_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return TV_ERR_INVALID_ARG;
  // NaN thresholds fail both comparisons; negative ones mean "no floor"
  if (!(epsilon == epsilon) || !(delta == delta)) return TV_ERR_INVALID_ARG;
  if (B == 0) return TV_OK;
  if (!logits || !cand_tok || !parents || !anc || !depth || !n_nodes || !entropy || !p_tok ||
      !tgt_argmax || !accept_len || !path || !bonus_tok)
    return TV_ERR_INVALID_ARG;
  const hipError_t e = tv::launch_typical_stats(logits, elem_bytes(dtype), vocab, cand_tok, parents,
                                                n_nodes, err, B, n_max, entropy, p_tok, tgt_argmax,
                                                stream);
  if (e != hipSuccess) return TV_ERR_HIP;
  return from_hip(tv::launch_accept_typical(cand_tok, tgt_argmax, p_tok, entropy, epsilon, delta,
                                            parents, anc, depth, n_nodes, err, B, n_max,
                                            accept_len, path, bonus_tok, out_tokens, stream));
}

tv_status tv_commit(void* k_cache, void* v_cache, int32_t B, int32_t Hkv, int32_t cap, int32_t D,
                    int32_t dtype, const int32_t* prefix_len_in, const int32_t* accept_len,
                    const int32_t* path, int32_t n_max, int32_t* prefix_len_out,
                    hipStream_t stream) {
  if (B < 0 || Hkv < 1 || n_max < 1 || n_max > TV_MAX_NODES || cap < n_max || cap % 64 != 0)
    return TV_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return TV_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return TV_ERR_UNSUPPORTED;
  if (B == 0) return TV_OK;
  if (!k_cache || !v_cache || !prefix_len_in || !accept_len || !path || !prefix_len_out)
    return TV_ERR_INVALID_ARG;
  return from_hip(tv::launch_commit(k_cache, v_cache, B, Hkv, cap, D, elem_bytes(dtype),
                                    prefix_len_in, accept_len, path, n_max, prefix_len_out, nullptr,
                                    stream));
}

tv_status tv_commit_paged(void* k_pool, void* v_pool, const tv_paged_kv* pk, int32_t B, int32_t Hkv,
                          int32_t D, int32_t dtype, const int32_t* prefix_len_in,
                          const int32_t* accept_len, const int32_t* path, int32_t n_max,
                          int32_t* prefix_len_out, hipStream_t stream) {
  if (pk == nullptr || pk->max_pages < 1 || pk->num_pages < 1) return TV_ERR_INVALID_ARG;
  if (B < 0 || Hkv < 1 || n_max < 1 || n_max > TV_MAX_NODES || 64 * pk->max_pages < n_max)
    return TV_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return TV_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return TV_ERR_UNSUPPORTED;
  if (B == 0) return TV_OK;
  if (!k_pool || !v_pool || !pk->block_table || !prefix_len_in || !accept_len || !path ||
      !prefix_len_out)
    return TV_ERR_INVALID_ARG;
  return from_hip(tv::launch_commit(k_pool, v_pool, B, Hkv, 64 * pk->max_pages, D, elem_bytes(dtype),
                                    prefix_len_in, accept_len, path, n_max, prefix_len_out, pk,
                                    stream));
}

tv_status tv_v_cache_layout(const void* src, void* dst, int64_t n, int32_t cap, int32_t D, int32_t dtype,
                            int32_t to_rows, hipStream_t stream) {
  if (n < 0 || cap < 64 || cap % 64 != 0 || (to_rows != 0 && to_rows != 1)) return TV_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return TV_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return TV_ERR_UNSUPPORTED;
  if (n == 0) return TV_OK;
  if (n > 0x7fffffffll / (cap / 64)) return TV_ERR_UNSUPPORTED;   // (more than 2^31 - 1 blocks)
  const int64_t blocks = n * (cap / 64);
  if (!src || !dst) return TV_ERR_INVALID_ARG;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a % 16 != 0 || b % 16 != 0) return TV_ERR_INVALID_ARG;
  const uintptr_t bytes = static_cast<uintptr_t>(blocks) * 64u * static_cast<uintptr_t>(D) *
                          static_cast<uintptr_t>(elem_bytes(dtype));
  if (a < b + bytes && b < a + bytes) return TV_ERR_INVALID_ARG;   // (out of place only)
  return from_hip(tv::launch_v_layout(src, dst, static_cast<long>(blocks), D, elem_bytes(dtype), to_rows != 0,
                                      stream));
}

}  // extern "C"
