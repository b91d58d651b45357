// Typical acceptance, first pass: statistics of the target's next-token
// distribution at every tree node.
//
// The rule (vibeengines.com "Medusa, explained", section "Typical
// acceptance"; pofe.ai "Medusa and EAGLE ...", "Typical acceptance";
// infra-guide "5.3 Medusa、EAGLE 与 MTP" section 9.1) keeps a drafted token
// when the target gives it probability above min(eps, delta * exp(-H)), H
// being the entropy of the target's distribution at its parent. This pass
// produces, per node i, H(i) and the target's argmax at i, and for every
// child c of i the probability of c's token under i's distribution; the
// tree scan that follows (tv_tree.hip) applies the rule.
//
// One workgroup of 512 threads per (node, sequence) reads that node's logits
// row once, in 16-byte chunks, eight chunks in flight per thread (a whole
// 32000-entry bf16 row in one round trip). Each thread keeps the largest
// logit and its first index, and, in base-2 units, z = sum 2^u and
// s = sum u * 2^u over u = x * log2(e) - ref for a reference ref that trails
// its maximum; partial statistics combine by moving to the larger reference.
// Then H = ln 2 * (log2 z - s / z) nats and p(t) = 2^(x_t * log2(e) - ref) / z.
// The row is HBM traffic read exactly once. Its first batch goes out before
// the node count is known (so a padding row's first batch may be read and
// dropped), and the candidate tokens' logits are gathered while the row
// streams in: lane t reads node t's token and then row i at that token
// before it is known whether t is a child of i.
#include <climits>

#include "tv_device.h"
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kBatch = 8;   // chunks per thread in flight
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 2^u for u <= 0 by the bare hardware instruction: results below 2^-126
// flush to 0, which changes no sum here (every row's sum is at least 1).
__device__ __forceinline__ float exp2_sum_term(float u) { return __builtin_amdgcn_exp2f(u); }

// The sums are kept relative to a reference ref (log2 units) that trails
// the running maximum: u = x * log2(e) - ref stays below kSlack, and ref is
// raised (the sums rescaled) only when a chunk's maximum would exceed that.
// Any reference gives the same p and H, since both are ratios of the sums.
constexpr float kSlack = 8.0f;

struct RowStat {
  float mx;   // largest logit seen, -inf if none
  int idx;    // lowest index holding mx
  float ref;  // reference of the sums, -inf if none
  float z;    // sum of 2^u, u = x * log2(e) - ref
  float s;    // sum of u * 2^u
};

// Adds a's sums, moved from a.ref to the reference ref >= a.ref.
__device__ __forceinline__ void rescaled(const RowStat& a, float ref, float& z, float& s) {
  if (a.z > 0.f) {
    const float d = a.ref - ref;   // <= 0
    const float f = exp2_sum_term(d);
    z += f * a.z;
    s += f * fmaf(d, a.z, a.s);
  }
}

__device__ __forceinline__ RowStat combine(RowStat a, RowStat b) {
  RowStat r;
  r.mx = fmaxf(a.mx, b.mx);
  const int ia = a.idx, ib = b.idx;
  const bool take_b = (b.mx > a.mx) || (b.mx == a.mx && ib < ia);
  r.idx = take_b ? ib : ia;
  r.ref = fmaxf(a.ref, b.ref);
  r.z = 0.f;
  r.s = 0.f;
  rescaled(a, r.ref, r.z, r.s);
  rescaled(b, r.ref, r.z, r.s);
  return r;
}

// Wave-wide reductions without LDS: DPP moves within each row of 16 lanes
// (swap neighbours, swap pairs, mirror each half-row, mirror the row) leave
// every lane of a row holding the row's result, and the four rows' lanes 0,
// 16, 32 and 48 are then read into scalars and combined; every lane gets the
// wave's result.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float wave_max_f(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum_f(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dpp_i<kDppXor1>(v));
  v = min(v, dpp_i<kDppXor2>(v));
  v = min(v, dpp_i<kDppHalfMirror>(v));
  v = min(v, dpp_i<kDppMirror>(v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// The workgroup's statistics from each wavefront's own: every thread rescales
// its sums to the wave's largest reference, the wave adds them and keeps the
// lowest index holding its maximum; lane 0 of each wave posts that to s_part,
// and after the barrier the caller folds the kWaves partials with
// fold_parts. (Thread statistics carry ref, and the maximum separately: the
// reference may trail the maximum.)
__device__ __forceinline__ void post_wave_stat(const RowStat& st, int tid, RowStat* s_part) {
  const float wref = wave_max_f(st.ref);
  const float wmx = wave_max_f(st.mx);
  float z = 0.f, s = 0.f;
  rescaled(st, wref, z, s);
  z = wave_sum_f(z);
  s = wave_sum_f(s);
  const int widx = wave_min_i(st.mx == wmx ? st.idx : INT_MAX);
  if ((tid & (kWave - 1)) == 0) s_part[tid / kWave] = RowStat{wmx, widx, wref, z, s};
}

// The kWaves partials folded at once: the largest reference and maximum
// first, then every partial's sums moved to that reference (independent
// steps), and the lowest index among the partials holding the maximum.
__device__ __forceinline__ RowStat fold_parts(const RowStat* s_part) {
  RowStat part[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) part[w] = s_part[w];
  RowStat r{part[0].mx, INT_MAX, part[0].ref, 0.f, 0.f};
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    r.mx = fmaxf(r.mx, part[w].mx);
    r.ref = fmaxf(r.ref, part[w].ref);
  }
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    rescaled(part[w], r.ref, r.z, r.s);
    r.idx = part[w].mx == r.mx ? min(r.idx, part[w].idx) : r.idx;
  }
  return r;
}

// A chunk is 16 bytes (8 bf16 or 4 fp32) on the vector path, one element
// otherwise.
template <typename T, int E>
struct ChunkOf {
  using type = uint4;
};
template <typename T>
struct ChunkOf<T, 1> {
  using type = uint32_t;
};

template <typename T, int E>
__device__ __forceinline__ typename ChunkOf<T, E>::type load_chunk(const T* row, int c) {
  if constexpr (E == 1) {
    if constexpr (sizeof(T) == 2) return static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(row)[c]);
    else return reinterpret_cast<const uint32_t*>(row)[c];
  } else {
    return reinterpret_cast<const uint4*>(row)[c];
  }
}

template <typename T, int E>
__device__ __forceinline__ float chunk_elem(const typename ChunkOf<T, E>::type& v, int j) {
  if constexpr (E == 1) {
    return sizeof(T) == 2 ? __uint_as_float(v << 16) : __uint_as_float(v);
  } else if constexpr (sizeof(T) == 2) {
    const uint32_t w = (j >> 1) == 0 ? v.x : (j >> 1) == 1 ? v.y : (j >> 1) == 2 ? v.z : v.w;
    return (j & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
  } else {
    return __uint_as_float(j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w);
  }
}

template <typename T>
__device__ __forceinline__ float load_elem(const T* row, int t) {
  if constexpr (sizeof(T) == 2) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(row)[t]);
  else return reinterpret_cast<const float*>(row)[t];
}

// c ? a : b on values, component by component (a select of whole
// aggregates becomes a select of their addresses and sends them to scratch)
__device__ __forceinline__ uint4 pick(bool c, uint4 a, uint4 b) {
  return make_uint4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}
__device__ __forceinline__ uint32_t pick(bool c, uint32_t a, uint32_t b) { return c ? a : b; }

// Every load is unconditional (indices clamped into the row; out-of-range
// chunks are loaded again and skipped by the arithmetic), so that the wait
// before each chunk's use counts exactly the loads still in flight behind it.
template <typename T, int E>
__device__ __forceinline__ void load_batch(typename ChunkOf<T, E>::type (&v)[kBatch], const T* row, int base,
                                           int nchunks, int tid) {
#pragma unroll
  for (int k = 0; k < kBatch; ++k) v[k] = load_chunk<T, E>(row, min(base + k * kThreads + tid, nchunks - 1));
}

// Folds a batch into the running statistics, chunk by chunk as they land: a
// chunk whose maximum would put u above kSlack first raises the reference
// (rare after the first chunk), and the chunk holding the maximum is kept,
// so that the index is found once at the end (chunks ascend, and only a
// strictly larger maximum replaces it, so the first index wins).
template <typename T, int E>
__device__ __forceinline__ void fold_batch(const typename ChunkOf<T, E>::type (&v)[kBatch], int base, int nchunks,
                                           int tid, RowStat& st, typename ChunkOf<T, E>::type& vmax,
                                           int& cmax_at) {
#pragma unroll
  for (int k = 0; k < kBatch; ++k) {
    const int c = base + k * kThreads + tid;
    if (c < nchunks) {
      float cm = chunk_elem<T, E>(v[k], 0);
#pragma unroll
      for (int j = 1; j < E; ++j) cm = fmaxf(cm, chunk_elem<T, E>(v[k], j));
      const float cref = cm * kLog2e;
      if (cref > st.ref + kSlack) {
        float z = 0.f, s = 0.f;
        rescaled(st, cref, z, s);
        st.ref = cref;
        st.z = z;
        st.s = s;
      }
      const bool raised = cm > st.mx;
      vmax = pick(raised, v[k], vmax);
      cmax_at = raised ? c : cmax_at;
      st.mx = fmaxf(st.mx, cm);
      const float m = st.ref;
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const float u = fmaf(chunk_elem<T, E>(v[k], j), kLog2e, -m);
        const float w = exp2_sum_term(u);
        st.z += w;
        st.s = fmaf(u, w, st.s);
      }
    }
  }
}

// Grid (n_max, B), 512 threads. T is uint16_t (bf16 bits) or float; E the
// elements per chunk (V must be a multiple of E on the vector paths).
template <typename T, int E>
__global__ __launch_bounds__(kThreads) void typical_stats_kernel(
    const T* __restrict__ logits, int V, const int32_t* __restrict__ cand_tok,
    const int32_t* __restrict__ parents, const int32_t* __restrict__ n_nodes,
    const int32_t* __restrict__ err, int n_max, float* __restrict__ entropy,
    float* __restrict__ p_tok, int32_t* __restrict__ argmax) {
  using Chunk = typename ChunkOf<T, E>::type;
  __shared__ RowStat s_part[kWaves];

  const int i = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const size_t seq = static_cast<size_t>(b) * n_max;
  const T* row = logits + (seq + i) * static_cast<size_t>(V);

  // wave 0, lane t = node t: its parent, its token and row i's logit at that
  // token, gathered without waiting for the node count
  const bool lane_node = tid >= 1 && tid < n_max;
  const int node_c = min(tid, n_max - 1);
  const int par = parents[seq + node_c];
  const int tok = cand_tok[seq + node_c];

  // the row's first batch goes out before the node count is known (a padding
  // row's batch is then dropped unread)
  const int nchunks = V / E;
  Chunk v0[kBatch];
  load_batch<T, E>(v0, row, 0, nchunks, tid);
  const bool tok_in = lane_node && tok >= 0 && tok < V;
  const float x_tok = load_elem<T>(row, tok_in ? tok : 0);

  const int n = n_nodes[b];
  const int e_in = err ? err[b] : 0;
  const bool active = (e_in == 0) && (n > 0) && (n <= n_max);
  if (!active || i >= n) {
    // padding node or skipped sequence
    if (tid == 0) {
      entropy[seq + i] = 0.f;
      argmax[seq + i] = -1;
      p_tok[seq + i] = 0.f;
    }
    return;
  }
  const bool child = lane_node && tid < n && par == i;

  RowStat st{-INFINITY, INT_MAX, -INFINITY, 0.f, 0.f};
  Chunk vmax{};
  int cmax_at = -1;
  fold_batch<T, E>(v0, 0, nchunks, tid, st, vmax, cmax_at);
  for (int base = kThreads * kBatch; base < nchunks; base += kThreads * kBatch) {
    Chunk v[kBatch];
    load_batch<T, E>(v, row, base, nchunks, tid);
    fold_batch<T, E>(v, base, nchunks, tid, st, vmax, cmax_at);
  }
  if (cmax_at >= 0) {
#pragma unroll
    for (int j = E - 1; j >= 0; --j)
      if (chunk_elem<T, E>(vmax, j) == st.mx) st.idx = cmax_at * E + j;
  }

  post_wave_stat(st, tid, s_part);
  __syncthreads();
  if (tid >= kWave) return;
  const RowStat r = fold_parts(s_part);

  if (child) p_tok[seq + tid] = tok_in ? exp2f(fmaf(x_tok, kLog2e, -r.ref)) / r.z : 0.f;
  if (tid == 0) {
    entropy[seq + i] = kLn2 * (log2f(r.z) - r.s / r.z);
    argmax[seq + i] = r.idx;
    if (i == 0) p_tok[seq] = 1.f;   // the root is the target's own token
  }
}

// ---------------------------------------------------------------------------
// Chain speculative sampling (robertz.co "Drafters ...", section "Why the
// answer does not change"): drafted token x_i is kept with probability
// min(1, p_i(x_i) / q_i(x_i)), p the target's and q the draft's
// distribution; at the first rejection j the step draws from
// max(0, p_j - q_j) normalised, or from p_L when all L tokens are kept.
// The uniform draws are inputs (keep iff u_i q_i(x_i) < p_i(x_i); the final
// draw by inverse CDF over ascending token ids).
// ---------------------------------------------------------------------------

// (ref, z) of one logits row over the workgroup, z = sum 2^(x log2(e) - ref),
// handed to every thread; s_part is reusable once every thread has it.
template <typename T, int E>
__device__ __forceinline__ void row_ref_z(const T* row, int V, int tid, RowStat* s_part, float& ref, float& z) {
  using Chunk = typename ChunkOf<T, E>::type;
  const int nchunks = V / E;
  RowStat st{-INFINITY, INT_MAX, -INFINITY, 0.f, 0.f};
  for (int base = 0; base < nchunks; base += kThreads * kBatch) {
    Chunk v[kBatch];
    load_batch<T, E>(v, row, base, nchunks, tid);
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int c = base + k * kThreads + tid;
      if (c < nchunks) {
        float cm = chunk_elem<T, E>(v[k], 0);
#pragma unroll
        for (int j = 1; j < E; ++j) cm = fmaxf(cm, chunk_elem<T, E>(v[k], j));
        const float cref = cm * kLog2e;
        if (cref > st.ref + kSlack) {
          float zz = 0.f, ss = 0.f;
          rescaled(st, cref, zz, ss);
          st.ref = cref;
          st.z = zz;
        }
#pragma unroll
        for (int j = 0; j < E; ++j) st.z += exp2_sum_term(fmaf(chunk_elem<T, E>(v[k], j), kLog2e, -st.ref));
      }
    }
  }
  post_wave_stat(st, tid, s_part);
  __syncthreads();
  const RowStat r = fold_parts(s_part);
  ref = r.ref;
  z = r.z;
  __syncthreads();
}

// Grid (2L + 1, B), 512 threads, one logits row each: rows r <= L are the
// target's rows r, rows L + 1 + i the draft's rows i. (ref, z) of each row
// into stats [B][2L + 1][2], and the drafted token's probability under it
// (0 for an id outside [0, V)) into p_tok / q_tok.
template <typename T, int E>
__global__ __launch_bounds__(kThreads) void spec_stats_kernel(
    const T* __restrict__ p_logits, const T* __restrict__ q_logits, int V, int L,
    const int32_t* __restrict__ draft, float* __restrict__ stats, float* __restrict__ p_tok,
    float* __restrict__ q_tok) {
  __shared__ RowStat s_part[kWaves];
  const int r = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const bool target = r <= L;
  const int i = target ? r : r - (L + 1);
  const T* row = target ? p_logits + (static_cast<size_t>(b) * (L + 1) + i) * V
                        : q_logits + (static_cast<size_t>(b) * L + i) * V;
  float ref, z;
  row_ref_z<T, E>(row, V, tid, s_part, ref, z);
  if (tid == 0) {
    float* st = stats + (static_cast<size_t>(b) * (2 * L + 1) + r) * 2;
    st[0] = ref;
    st[1] = z;
    if (i < L) {
      const int x = draft[static_cast<size_t>(b) * L + i];
      const float pr = (x >= 0 && x < V) ? exp2f(fmaf(load_elem<T>(row, x), kLog2e, -ref)) / z : 0.f;
      (target ? p_tok : q_tok)[static_cast<size_t>(b) * L + i] = pr;
    }
  }
}

constexpr int kSampleThreads = 1024;
constexpr int kRun = 32;   // token ids per thread per round

// The weights of one thread's run of kRun token ids from y0 (ids past V
// weigh 0): p(y) or max(0, p(y) - q(y)), p(y) = 2^(x log2(e) - ref) / z.
// Whole runs of a 16-byte-aligned row are read as 16-byte vectors.
template <typename T, int E>
__device__ __forceinline__ void run_weights(const T* prow, const T* qrow, bool resid, int V, int y0, float pref,
                                            float pinv, float qref, float qinv, float (&w)[kRun]) {
  auto one = [&](float xp, float xq) {
    const float a = exp2_sum_term(fmaf(xp, kLog2e, -pref)) * pinv;
    return resid ? fmaxf(a - exp2_sum_term(fmaf(xq, kLog2e, -qref)) * qinv, 0.0f) : a;
  };
  if (E > 1 && y0 + kRun <= V) {
    using Chunk = typename ChunkOf<T, E>::type;
#pragma unroll
    for (int k = 0; k < kRun / E; ++k) {
      const Chunk cp = load_chunk<T, E>(prow, y0 / E + k);
      const Chunk cq = resid ? load_chunk<T, E>(qrow, y0 / E + k) : cp;
#pragma unroll
      for (int e = 0; e < E; ++e) w[k * E + e] = one(chunk_elem<T, E>(cp, e), chunk_elem<T, E>(cq, e));
    }
  } else {
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
      const int y = y0 + k;
      w[k] = y < V ? one(load_elem<T>(prow, y), resid ? load_elem<T>(qrow, y) : 0.0f) : 0.0f;
    }
  }
}

// Grid B, 1024 threads: the keep decisions, then the draw. The row is cut
// into rounds of 1024 runs of kRun ids (round r, thread t: ids from
// (r * 1024 + t) * kRun); in id order a thread sums its run's weights, and a
// block scan of those sums places every run in the running total. A first
// pass over the rounds gives the total W; the second repeats the same sums
// in the same order, so the runs tile [0, W) exactly, and the one thread
// whose run holds u * W finds the token in its run. If rounding leaves
// u * W past every run, the last token of positive weight is drawn.
template <typename T, int E>
__global__ __launch_bounds__(kSampleThreads) void spec_sample_kernel(
    const T* __restrict__ p_logits, const T* __restrict__ q_logits, int V, int L,
    const int32_t* __restrict__ draft, const float* __restrict__ u_acc, const float* __restrict__ u_res,
    const float* __restrict__ stats, const float* __restrict__ p_tok, const float* __restrict__ q_tok,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ tokens) {
  constexpr int kW = kSampleThreads / kWave;
  __shared__ int s_j, s_y;
  __shared__ float s_wsum[kW];
  __shared__ int s_last[kW];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  if (wave == 0) {
    bool rej = false;
    if (lane < L) {
      const size_t e = static_cast<size_t>(b) * L + lane;
      rej = !(u_acc[e] * q_tok[e] < p_tok[e]);
    }
    const uint64_t m = __ballot(rej);
    if (lane == 0) {
      s_j = m ? __ffsll(static_cast<long long>(m)) - 1 : L;
      s_y = -1;
    }
  }
  __syncthreads();
  const int j = s_j;
  const bool resid = j < L;
  const float* st = stats + static_cast<size_t>(b) * (2 * L + 1) * 2;
  const float pref = st[2 * j], pinv = 1.0f / st[2 * j + 1];
  const float qref = resid ? st[2 * (L + 1 + j)] : 0.f, qinv = resid ? 1.0f / st[2 * (L + 1 + j) + 1] : 0.f;
  const T* prow = p_logits + (static_cast<size_t>(b) * (L + 1) + j) * V;
  const T* qrow = q_logits + (static_cast<size_t>(b) * L + (resid ? j : 0)) * V;
  const int rounds = (V + kSampleThreads * kRun - 1) / (kSampleThreads * kRun);

  // Block scan of one value per thread: the running sums before (exc) and
  // after (inc) this thread's value, and the block's total. A thread's exc
  // is bit for bit the previous thread's inc (the same additions in the
  // same order), so the runs' intervals meet exactly.
  auto block_scan = [&](float S, float& exc, float& inc, float& total) {
    float x = S;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const float o = __shfl_up(x, off);
      if (lane >= off) x += o;
    }
    float xe = __shfl_up(x, 1);
    if (lane == 0) xe = 0.f;
    if (lane == kWave - 1) s_wsum[wave] = x;
    __syncthreads();
    float before = 0.f;
    total = 0.f;
    for (int w = 0; w < kW; ++w) {
      if (w < wave) before += s_wsum[w];
      total += s_wsum[w];
    }
    __syncthreads();
    exc = lane == 0 ? before : before + xe;
    inc = before + x;
  };

  float w[kRun];
  float W = 0.f;
  int last = -1;
  for (int pass = 0; pass < 2; ++pass) {
    const float t = pass ? u_res[b] * W : 0.f;
    float base = 0.f;
    for (int r = 0; r < rounds; ++r) {
      const int y0 = (r * kSampleThreads + tid) * kRun;
      if (pass == 0 || rounds > 1) run_weights<T, E>(prow, qrow, resid, V, y0, pref, pinv, qref, qinv, w);
      float S = 0.f;
#pragma unroll
      for (int k = 0; k < kRun; ++k) {
        S += w[k];
        if (pass == 0 && w[k] > 0.f) last = y0 + k;
      }
      float exc, inc, total;
      block_scan(S, exc, inc, total);
      const float lo = base + exc, hi = base + inc;
      if (pass == 1 && S > 0.f && lo <= t && t < hi) {
        float acc = lo;
        int pick = -1;
#pragma unroll
        for (int k = 0; k < kRun; ++k) {
          acc += w[k];
          if (pick < 0 && w[k] > 0.f && acc > t) pick = y0 + k;
        }
        if (pick < 0)
          for (int k = kRun - 1; k >= 0; --k)
            if (w[k] > 0.f) {
              pick = y0 + k;
              break;
            }
        s_y = pick;
      }
      base += total;
    }
    if (pass == 0) W = base;
  }
  int lmax = last;
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) lmax = max(lmax, __shfl_xor(lmax, off));
  if (lane == 0) s_last[wave] = lmax;
  __syncthreads();
  int last_all = -1;
  for (int q = 0; q < kW; ++q) last_all = max(last_all, s_last[q]);
  const int y = s_y >= 0 ? s_y : last_all;
  const size_t row = static_cast<size_t>(b) * (L + 1);
  for (int k = tid; k <= L; k += kSampleThreads)
    tokens[row + k] = k < j ? draft[static_cast<size_t>(b) * L + k] : (k == j ? y : -1);
  if (tid == 0) accept_len[b] = j;
}

}  // namespace

hipError_t launch_typical_stats(const void* logits, int elem_bytes, int V, const int32_t* cand_tok,
                                const int32_t* parents, const int32_t* n_nodes, const int32_t* err,
                                int B, int n_max, float* entropy, float* p_tok, int32_t* argmax,
                                hipStream_t s) {
  const dim3 grid(n_max, B);
  const bool aligned = (reinterpret_cast<uintptr_t>(logits) % 16 == 0) &&
                       ((static_cast<size_t>(V) * elem_bytes) % 16 == 0);
  if (elem_bytes == 2) {
    const auto* p = static_cast<const uint16_t*>(logits);
    if (aligned)
      hipLaunchKernelGGL((typical_stats_kernel<uint16_t, 8>), grid, dim3(kThreads), 0, s, p, V,
                         cand_tok, parents, n_nodes, err, n_max, entropy, p_tok, argmax);
    else
      hipLaunchKernelGGL((typical_stats_kernel<uint16_t, 1>), grid, dim3(kThreads), 0, s, p, V,
                         cand_tok, parents, n_nodes, err, n_max, entropy, p_tok, argmax);
  } else {
    const auto* p = static_cast<const float*>(logits);
    if (aligned)
      hipLaunchKernelGGL((typical_stats_kernel<float, 4>), grid, dim3(kThreads), 0, s, p, V,
                         cand_tok, parents, n_nodes, err, n_max, entropy, p_tok, argmax);
    else
      hipLaunchKernelGGL((typical_stats_kernel<float, 1>), grid, dim3(kThreads), 0, s, p, V,
                         cand_tok, parents, n_nodes, err, n_max, entropy, p_tok, argmax);
  }
  return hipGetLastError();
}

}  // namespace tv

namespace tv {

hipError_t launch_speculative_sample(const void* p_logits, const void* q_logits, int elem_bytes, int V,
                                     const int32_t* draft, const float* u_acc, const float* u_res, int B, int L,
                                     float* p_tok, float* q_tok, int32_t* accept_len, int32_t* tokens,
                                     float* stats, hipStream_t s) {
  const dim3 grid(2 * L + 1, B);
  const bool aligned = (reinterpret_cast<uintptr_t>(p_logits) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(q_logits) % 16 == 0) &&
                       ((static_cast<size_t>(V) * elem_bytes) % 16 == 0);
  if (elem_bytes == 2) {
    const auto* p = static_cast<const uint16_t*>(p_logits);
    const auto* q = static_cast<const uint16_t*>(q_logits);
    if (aligned)
      hipLaunchKernelGGL((spec_stats_kernel<uint16_t, 8>), grid, dim3(kThreads), 0, s, p, q, V, L, draft, stats,
                         p_tok, q_tok);
    else
      hipLaunchKernelGGL((spec_stats_kernel<uint16_t, 1>), grid, dim3(kThreads), 0, s, p, q, V, L, draft, stats,
                         p_tok, q_tok);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (aligned)
      hipLaunchKernelGGL((spec_sample_kernel<uint16_t, 8>), dim3(B), dim3(kSampleThreads), 0, s, p, q, V, L,
                         draft, u_acc, u_res, stats, p_tok, q_tok, accept_len, tokens);
    else
      hipLaunchKernelGGL((spec_sample_kernel<uint16_t, 1>), dim3(B), dim3(kSampleThreads), 0, s, p, q, V, L,
                         draft, u_acc, u_res, stats, p_tok, q_tok, accept_len, tokens);
  } else {
    const auto* p = static_cast<const float*>(p_logits);
    const auto* q = static_cast<const float*>(q_logits);
    if (aligned)
      hipLaunchKernelGGL((spec_stats_kernel<float, 4>), grid, dim3(kThreads), 0, s, p, q, V, L, draft, stats,
                         p_tok, q_tok);
    else
      hipLaunchKernelGGL((spec_stats_kernel<float, 1>), grid, dim3(kThreads), 0, s, p, q, V, L, draft, stats,
                         p_tok, q_tok);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (aligned)
      hipLaunchKernelGGL((spec_sample_kernel<float, 4>), dim3(B), dim3(kSampleThreads), 0, s, p, q, V, L, draft,
                         u_acc, u_res, stats, p_tok, q_tok, accept_len, tokens);
    else
      hipLaunchKernelGGL((spec_sample_kernel<float, 1>), dim3(B), dim3(kSampleThreads), 0, s, p, q, V, L, draft,
                         u_acc, u_res, stats, p_tok, q_tok, accept_len, tokens);
  }
  return hipGetLastError();
}

}  // namespace tv
