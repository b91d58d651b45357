// EAGLE-2 dynamic draft tree: the draft's proposals -> the parents array that
// verification takes (infra-guide "5.3 Medusa、EAGLE 与 MTP", section 5.2: a
// node's value is the product of the draft's confidences along its path; the
// expansion grows the best nodes of the newest layer, the rerank keeps the
// best nodes of all for verification).
//
// One workgroup per sequence. The proposal table (at most 512 confidences
// and tokens) is staged in LDS with one round trip; the tree of created
// nodes (at most 513 with the root) lives in LDS. Every selection is a rank
// count: a node's rank is the number of nodes ahead of it in (value
// descending, creation ascending) order, so no sort and no atomics, and the
// same total order as the oracle's. Values are float32 products
// v(parent) * clamp(conf, 0, 1), rounded once per node, so both sides rank
// identical numbers. The kept nodes are numbered in creation order (which is
// depth order), so parents come first.
#include "tv_device.h"
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxCreated = 1 + TV_MAX_DRAFT_PROPOSALS;

__global__ __launch_bounds__(kThreads) void eagle2_tree_kernel(
    const float* __restrict__ conf, const int32_t* __restrict__ cand, const int32_t* __restrict__ root_tok,
    int S, int K, int M, int n_max, int32_t* __restrict__ parents, int32_t* __restrict__ tokens,
    float* __restrict__ values, int32_t* __restrict__ n_nodes) {
  __shared__ float s_conf[TV_MAX_DRAFT_PROPOSALS];
  __shared__ int s_cand[TV_MAX_DRAFT_PROPOSALS];
  __shared__ float s_val[kMaxCreated];
  __shared__ int s_par[kMaxCreated];
  __shared__ int s_tok[kMaxCreated];
  __shared__ int s_keep[kMaxCreated];
  __shared__ int s_new[kMaxCreated];

  const int b = blockIdx.x, tid = threadIdx.x;
  const int n_prop = S * K * M;
  const size_t prop = static_cast<size_t>(b) * n_prop;
  for (int e = tid; e < n_prop; e += kThreads) {
    // clamp into [0, 1]; fmaxf returns 0 for a NaN confidence
    s_conf[e] = fminf(fmaxf(conf[prop + e], 0.0f), 1.0f);
    s_cand[e] = cand[prop + e];
  }
  if (tid == 0) {
    s_val[0] = 1.0f;
    s_par[0] = -1;
    s_tok[0] = root_tok[b];
  }
  __syncthreads();

  // expansion: the newest layer is created nodes [f0, f1)
  int f0 = 0, f1 = 1;
  for (int s = 0; s < S; ++s) {
    const int grown = min(K, f1 - f0);
    for (int i = f0 + tid; i < f1; i += kThreads) {
      const float v = s_val[i];
      int r = 0;
      for (int j = f0; j < f1; ++j) {
        const float u = s_val[j];
        r += (u > v) || (u == v && j < i);
      }
      if (r < grown) {
        for (int c = 0; c < M; ++c) {
          const int e = (s * K + r) * M + c;
          const int child = f1 + r * M + c;
          s_val[child] = v * s_conf[e];
          s_par[child] = i;
          s_tok[child] = s_cand[e];
        }
      }
    }
    __syncthreads();
    f0 = f1;
    f1 += grown * M;
  }
  const int T = f1;   // created nodes, the root included

  // rerank: the root and the n_max - 1 best other nodes are kept
  for (int i = tid; i < T; i += kThreads) {
    int keep = 1;
    if (i > 0) {
      const float v = s_val[i];
      int r = 0;
      for (int j = 1; j < T; ++j) {
        const float u = s_val[j];
        r += (u > v) || (u == v && j < i);
      }
      keep = r < n_max - 1;
    }
    s_keep[i] = keep;
  }
  __syncthreads();
  // flattened index of a kept node: kept nodes created before it
  for (int i = tid; i < T; i += kThreads) {
    int idx = 0;
    for (int j = 0; j < i; ++j) idx += s_keep[j];
    s_new[i] = s_keep[i] ? idx : -1;
  }
  __syncthreads();

  const size_t row = static_cast<size_t>(b) * n_max;
  const int kept = min(n_max, T);   // the root and min(n_max - 1, T - 1) others
  for (int i = tid; i < T; i += kThreads) {
    const int ni = s_new[i];
    if (ni < 0) continue;
    parents[row + ni] = i == 0 ? -1 : s_new[s_par[i]];
    tokens[row + ni] = s_tok[i];
    values[row + ni] = s_val[i];
  }
  if (tid == 0) n_nodes[b] = kept;
  for (int i = kept + tid; i < n_max; i += kThreads) {
    parents[row + i] = -1;
    tokens[row + i] = -1;
    values[row + i] = 0.0f;
  }
}

}  // namespace

hipError_t launch_eagle2_tree(const float* conf, const int32_t* cand, const int32_t* root_tok, int B, int S,
                              int K, int M, int n_max, int32_t* parents, int32_t* tokens, float* values,
                              int32_t* n_nodes, hipStream_t s) {
  hipLaunchKernelGGL(eagle2_tree_kernel, dim3(B), dim3(kThreads), 0, s, conf, cand, root_tok, S, K, M, n_max,
                     parents, tokens, values, n_nodes);
  return hipGetLastError();
}

}  // namespace tv
