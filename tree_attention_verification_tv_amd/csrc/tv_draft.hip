// EAGLE-2 dynamic draft tree: the draft's proposals -> the parents array that
// verification takes (infra-guide "5.3 Medusa、EAGLE 与 MTP", section 5.2: a
// node's value is the product of the draft's confidences along its path; the
// expansion grows the best nodes of the newest layer, the rerank keeps the
// best nodes of all for verification).
//
// One workgroup of 1024 threads per sequence. The proposal table (at most
// 512 confidences and tokens) is staged in LDS with one round trip; the tree
// of created nodes (at most 513 with the root) lives in LDS. Every selection
// is a rank count: a node's rank is the number of nodes ahead of it in
// (value descending, creation ascending) order, counted by several lanes at
// once, so no sort and no atomics, and the same total order as the
// oracle's; each child of a step is created by a thread of its own. Values are float32 products
// v(parent) * clamp(conf, 0, 1), rounded once per node, so both sides rank
// identical numbers. The kept nodes are numbered in creation order (which is
// depth order), so parents come first.
#include "tv_device.h"
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kThreads = 1024;
constexpr int kMaxCreated = 1 + TV_MAX_DRAFT_PROPOSALS;
constexpr int kValSlots = (kMaxCreated + 3) & ~3;   // whole four-value runs past the last node

// Number of j in [a, b) with vals[j] >= v (GE) or vals[j] > v: aligned runs
// of four values per LDS access; a ragged first or last run is one aligned
// read with its values outside [a, b) masked (vals holds whole runs).
template <bool GE>
__device__ __forceinline__ int count_from(const float* vals, int a, int b, float v) {
  auto ahead = [&](float u) { return GE ? (u >= v) : (u > v); };
  auto masked_run = [&](int j) {
    const float4 u = *reinterpret_cast<const float4*>(vals + j);
    return (j >= a && j < b && ahead(u.x)) + (j + 1 >= a && j + 1 < b && ahead(u.y)) +
           (j + 2 >= a && j + 2 < b && ahead(u.z)) + (j + 3 >= a && j + 3 < b && ahead(u.w));
  };
  if (a >= b) return 0;
  int r = 0, j = a & ~3;
  if (j < a) {
    r += masked_run(j);
    j += 4;
  }
#pragma unroll 4
  for (; j + 4 <= b; j += 4) {
    const float4 u = *reinterpret_cast<const float4*>(vals + j);
    r += ahead(u.x) + ahead(u.y) + ahead(u.z) + ahead(u.w);
  }
  if (j < b) r += masked_run(j);
  return r;
}

// rank[i - j0] for every node i of [j0, j1) (at most kThreads nodes): the
// nodes of [j0, j1) ahead of i in (value descending, creation ascending)
// order, i.e. the earlier ones worth at least v(i) and the later ones worth
// more. Each node's count is split over `segs` consecutive lanes (a power
// of two dividing 64), summed with shuffles.
__device__ __forceinline__ void rank_all(const float* vals, int j0, int j1, int* rank, int tid) {
  const int L = j1 - j0;
  int segs = 1;
  while (segs < 16 && 2 * segs * L <= kThreads) segs *= 2;
  const int seg_len = ((L + segs - 1) / segs + 3) & ~3;
  const int node = tid / segs, seg = tid % segs;
  int r = 0;
  float v = 0.0f;
  const int i = j0 + node;
  if (node < L) {
    v = vals[i];
    const int a = j0 + seg * seg_len, b = min(j1, a + seg_len);
    r = count_from<true>(vals, a, min(b, i), v) + count_from<false>(vals, max(a, i + 1), b, v);
  }
  for (int off = 1; off < segs; off <<= 1) r += __shfl_xor(r, off);
  if (node < L && seg == 0) rank[node] = r;
}

__global__ __launch_bounds__(kThreads) void eagle2_tree_kernel(
    const float* __restrict__ conf, const int32_t* __restrict__ cand, const int32_t* __restrict__ root_tok,
    int S, int K, int M, int n_max, int32_t* __restrict__ parents, int32_t* __restrict__ tokens,
    float* __restrict__ values, int32_t* __restrict__ n_nodes) {
  __shared__ float s_conf[TV_MAX_DRAFT_PROPOSALS];
  __shared__ int s_cand[TV_MAX_DRAFT_PROPOSALS];
  __shared__ __attribute__((aligned(16))) float s_val[kValSlots];
  __shared__ int s_par[kMaxCreated];
  __shared__ int s_tok[kMaxCreated];
  __shared__ int s_rank[kMaxCreated];
  __shared__ int s_new[kMaxCreated];
  __shared__ int s_grow[TV_MAX_DRAFT_PROPOSALS];   // node of each rank < K in the layer
  __shared__ int s_count[(kMaxCreated + 63) / 64];

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

  // expansion: the newest layer is created nodes [f0, f1); its nodes of rank
  // r < K each get M children, child c of rank r at f1 + r M + c (one thread
  // per child)
  int f0 = 0, f1 = 1;
  for (int s = 0; s < S; ++s) {
    const int grown = min(K, f1 - f0);
    rank_all(s_val, f0, f1, s_rank, tid);
    __syncthreads();
    for (int i = tid; i < f1 - f0; i += kThreads)
      if (s_rank[i] < grown) s_grow[s_rank[i]] = f0 + i;
    __syncthreads();
    for (int t = tid; t < grown * M; t += kThreads) {
      const int r = t / M, e = s * K * M + t, child = f1 + t, p = s_grow[r];
      s_val[child] = s_val[p] * s_conf[e];
      s_par[child] = p;
      s_tok[child] = s_cand[e];
    }
    __syncthreads();
    f0 = f1;
    f1 += grown * M;
  }
  const int T = f1;   // created nodes, the root included

  // rerank: the n_max best of all created nodes are kept; the root (worth
  // 1, the largest value, and created first) is always among them
  rank_all(s_val, 0, T, s_rank, tid);
  __syncthreads();
  // flattened index of a kept node = kept nodes created before it: a ballot
  // per 64 nodes, then the counts of the earlier groups
  const int lane = tid & 63, wave = tid >> 6;
  const int groups = (T + 63) / 64;
  for (int q = wave; q < groups; q += kThreads / 64) {
    const int i = 64 * q + lane;
    const uint64_t bal = __ballot(i < T && s_rank[i] < n_max);
    if (lane == 0) s_count[q] = __popcll(bal);
  }
  __syncthreads();
  for (int q = wave; q < groups; q += kThreads / 64) {
    const int i = 64 * q + lane;
    const bool k = i < T && s_rank[i] < n_max;
    const uint64_t bal = __ballot(k);
    int base = 0;
    for (int qq = 0; qq < q; ++qq) base += s_count[qq];
    if (i < T) s_new[i] = k ? base + __popcll(bal & ((1ull << lane) - 1ull)) : -1;
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
