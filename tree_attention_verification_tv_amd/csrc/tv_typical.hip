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
// One workgroup of 256 threads per (node, sequence) reads that node's logits
// row once, in 16-byte chunks, eight chunks in flight per thread. Each thread
// keeps, in base-2 units, the largest logit mx, m = mx * log2(e),
// z = sum 2^u and s = sum u * 2^u over u = x * log2(e) - m; partial
// statistics combine by rescaling to the larger maximum. Then
// H = ln 2 * (log2 z - s / z) nats and p(t) = 2^(x_t * log2(e) - m) / z.
// The row is HBM traffic read exactly once; the child tokens' logits are
// fetched after the first batch, while the rest of the row streams in.
#include <climits>

#include "tv_device.h"
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kBatch = 8;   // chunks per thread in flight
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct RowStat {
  float mx;   // largest logit seen, -inf if none
  int idx;    // lowest index holding mx
  float z;    // sum of 2^u, u relative to mx * log2(e)
  float s;    // sum of u * 2^u
};

// Rescales a's sums from its own maximum to the larger maximum mx.
__device__ __forceinline__ void rescaled(const RowStat& a, float m, float& z, float& s) {
  if (a.z > 0.f) {
    const float d = a.mx * kLog2e - m;   // <= 0
    const float f = exp2f(d);
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
  const float m = r.mx * kLog2e;
  r.z = 0.f;
  r.s = 0.f;
  rescaled(a, m, r.z, r.s);
  rescaled(b, m, r.z, r.s);
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

// Grid (n_max, B), 256 threads. T is uint16_t (bf16 bits) or float; E the
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
  const int n = n_nodes[b];
  const int e_in = err ? err[b] : 0;
  const bool active = (e_in == 0) && (n > 0) && (n <= n_max);
  if (!active || i >= n) {
    // padding node or skipped sequence: nothing reads this row
    if (tid == 0) {
      entropy[seq + i] = 0.f;
      argmax[seq + i] = -1;
      p_tok[seq + i] = 0.f;
    }
    return;
  }

  // children of i and their tokens (lanes of wave 0; node t is lane t)
  const bool child = (tid >= 1) && (tid < n) && (parents[seq + tid] == i);
  const int tok = child ? cand_tok[seq + tid] : -1;
  const bool in_vocab = child && tok >= 0 && tok < V;

  const T* row = logits + (seq + i) * static_cast<size_t>(V);
  const int nchunks = V / E;
  RowStat st{-INFINITY, INT_MAX, 0.f, 0.f};
  float x_tok = 0.f;
  for (int base = 0; base < nchunks; base += kThreads * kBatch) {
    Chunk v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int c = base + k * kThreads + tid;
      if (c < nchunks) v[k] = load_chunk<T, E>(row, c);
    }
    // batch maximum; chunks and elements ascend, so ">" keeps the first index
    float bmx = -INFINITY;
    int bidx = INT_MAX;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int c = base + k * kThreads + tid;
      if (c < nchunks) {
#pragma unroll
        for (int j = 0; j < E; ++j) {
          const float x = chunk_elem<T, E>(v[k], j);
          if (x > bmx) {
            bmx = x;
            bidx = c * E + j;
          }
        }
      }
    }
    if (bmx > st.mx) {
      float z = 0.f, s = 0.f;
      rescaled(st, bmx * kLog2e, z, s);
      st = RowStat{bmx, bidx, z, s};
    }
    const float m = st.mx * kLog2e;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int c = base + k * kThreads + tid;
      if (c < nchunks) {
#pragma unroll
        for (int j = 0; j < E; ++j) {
          const float u = fmaf(chunk_elem<T, E>(v[k], j), kLog2e, -m);
          const float w = exp2f(u);
          st.z += w;
          st.s = fmaf(u, w, st.s);
        }
      }
    }
    // the child tokens' logits go out behind the first batch
    if (base == 0 && in_vocab) x_tok = load_elem<T>(row, tok);
  }

  // wave, then workgroup
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) {
    RowStat o;
    o.mx = __shfl_xor(st.mx, off);
    o.idx = __shfl_xor(st.idx, off);
    o.z = __shfl_xor(st.z, off);
    o.s = __shfl_xor(st.s, off);
    st = combine(st, o);
  }
  if ((tid & (kWave - 1)) == 0) s_part[tid / kWave] = st;
  __syncthreads();
  if (tid >= kWave) return;
  RowStat part[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) part[w] = s_part[w];
  RowStat r = part[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = combine(r, part[w]);

  const float m = r.mx * kLog2e;
  if (child) p_tok[seq + tid] = in_vocab ? exp2f(fmaf(x_tok, kLog2e, -m)) / r.z : 0.f;
  if (tid == 0) {
    entropy[seq + i] = kLn2 * (log2f(r.z) - r.s / r.z);
    argmax[seq + i] = r.idx;
    if (i == 0) p_tok[seq] = 1.f;   // the root is the target's own token
  }
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
