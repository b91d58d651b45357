// Tree-verification attention on the vector ALUs, fp32 arithmetic.
//
// Serves fp32 inputs, whose tolerance (1e-5 relative) rules out bf16 matrix
// cores, and bf16 inputs at head dim 64 (the matrix-core kernel is laid out
// for head dim 128): bf16 elements are widened on load, the rotated tree keys
// appended to the cache and the output rows are rounded to bf16 (to nearest
// even) on store. Every tree node attends to the P prefix keys of its KV head and to
// the keys of its ancestors-or-self, selected by the node's ancestor bitmask
// (infra-guide "5.3 Medusa、EAGLE 与 MTP", section 3.1); queries and tree
// keys are rotated at position P + depth (section 3.2).
//
// Caches: K [B][Hkv][cap][D]; V [B][Hkv][cap/64][D][64] (blocks of 64 slots,
// head dim major inside a block).
//
// Grid (ceil(G*n_max/4), Hkv, B), 256 threads. The block first rotates the n
// tree keys of its KV head into LDS (angles in double precision); the block
// with blockIdx.x == 0 also appends them, and the raw tree values, to cache
// slots [P, P+n). Each wavefront then computes one query row (node i, head
// g*G + hh, rows ordered node-major): lane l owns key t0+l of each 64-key
// tile for the scores and dims {l, l+64} of the output.
#include <math.h>

#include "tv_device.h"
#include "tv_internal.h"

namespace tv {

namespace {

// T: float, or uint16_t holding bf16 bits
template <typename T>
struct VecParams {
  const T* q;
  const T* k_new;
  const T* v_new;
  T* k_cache;
  T* v_cache;
  const int32_t* prefix_len;
  const int32_t* n_nodes;
  const uint64_t* anc;
  const int32_t* depth;
  int32_t* err;
  T* out;
  int n_max, Hq, Hkv, G, D, cap;
  float theta, scale;
};

__device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float ld(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }
__device__ __forceinline__ void st(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16_bits(v); }
// a raw copy (values go to the cache unrounded)
__device__ __forceinline__ void cp(float* d, size_t i, const float* s, size_t j) { d[i] = s[j]; }
__device__ __forceinline__ void cp(uint16_t* d, size_t i, const uint16_t* s, size_t j) { d[i] = s[j]; }

__device__ __forceinline__ void rope_cs(int pos, int pair, int D, float theta, float* c, float* s) {
  if (theta == 0.0f) {
    *c = 1.0f;
    *s = 0.0f;
    return;
  }
  const double inv_freq = pow(static_cast<double>(theta), -2.0 * pair / D);
  double sd, cd;
  sincos(static_cast<double>(pos) * inv_freq, &sd, &cd);
  *c = static_cast<float>(cd);
  *s = static_cast<float>(sd);
}

// Element offset of (slot, d) inside one head's V cache, which is stored in
// blocks of 64 slots, head dim major within a block: [cap/64][D][64].
__device__ __forceinline__ size_t v_off(int slot, int d, int D) {
  return (static_cast<size_t>(slot >> 6) * D + d) * 64 + (slot & 63);
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <typename T>
__global__ __launch_bounds__(256) void attn_vec_kernel(VecParams<T> p) {
  __shared__ float ktree[TV_MAX_NODES_DEV][128];
  __shared__ float qrow[4][128];
  const int g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int D = p.D, half = D / 2;
  const int n = p.n_nodes[b];
  const int P = p.prefix_len[b];
  const int e_in = p.err[b];
  const bool cap_bad = (e_in == 0) && (n > 0) && (n <= p.n_max) && (P < 0 || P + n > p.cap);
  const bool skip = (e_in != 0) || (n <= 0) || (n > p.n_max) || cap_bad;
  if (cap_bad && blockIdx.x == 0 && g == 0 && tid == 0) p.err[b] = TV_ERR_CAPACITY;

  if (!skip) {
    // rotated tree keys of head g, and the append into the cache
    for (int idx = tid; idx < n * half; idx += blockDim.x) {
      const int a = idx / half, pr = idx % half;
      const T* kr = p.k_new + ((static_cast<size_t>(b) * p.n_max + a) * p.Hkv + g) * D;
      float c, s;
      rope_cs(P + p.depth[static_cast<size_t>(b) * p.n_max + a], pr, D, p.theta, &c, &s);
      const float lo = ld(kr, pr), hi = ld(kr, pr + half);
      const float rlo = lo * c - hi * s, rhi = hi * c + lo * s;
      const size_t head = (static_cast<size_t>(b) * p.Hkv + g) * p.cap * D;
      const size_t slot = head + static_cast<size_t>(P + a) * D;
      // the tree's keys are used as the cache will hold them (rounded to
      // bf16 for bf16 caches), like the prefix keys
      if (blockIdx.x == 0) {
        st(p.k_cache, slot + pr, rlo);
        st(p.k_cache, slot + pr + half, rhi);
        const T* vr = p.v_new + ((static_cast<size_t>(b) * p.n_max + a) * p.Hkv + g) * D;
        cp(p.v_cache, head + v_off(P + a, pr, D), vr, pr);
        cp(p.v_cache, head + v_off(P + a, pr + half, D), vr, pr + half);
      }
      if constexpr (sizeof(T) == 2) {
        ktree[a][pr] = bf16_bits_to_f32(f32_to_bf16_bits(rlo));
        ktree[a][pr + half] = bf16_bits_to_f32(f32_to_bf16_bits(rhi));
      } else {
        ktree[a][pr] = rlo;
        ktree[a][pr + half] = rhi;
      }
    }
  }
  __syncthreads();

  // No wavefront leaves before the barrier below; rows past the end only
  // skip the work.
  const int r = blockIdx.x * 4 + wave;
  const bool row_exists = r < p.G * p.n_max;
  const int i = row_exists ? r / p.G : 0, head = g * p.G + (row_exists ? r % p.G : 0);
  T* orow = p.out + ((static_cast<size_t>(b) * p.n_max + i) * p.Hq + head) * D;
  const bool live = row_exists && !skip && i < n;
  uint64_t anc_i = 0;
  if (live) {
    anc_i = p.anc[static_cast<size_t>(b) * p.n_max + i];
    const int pos_i = P + p.depth[static_cast<size_t>(b) * p.n_max + i];
    const T* qr = p.q + ((static_cast<size_t>(b) * p.n_max + i) * p.Hq + head) * D;
    if (lane < half) {
      float c, s;
      rope_cs(pos_i, lane, D, p.theta, &c, &s);
      const float lo = ld(qr, lane), hi = ld(qr, lane + half);
      qrow[wave][lane] = lo * c - hi * s;
      qrow[wave][lane + half] = hi * c + lo * s;
    }
  }
  __syncthreads();
  if (!row_exists) return;
  if (!live) {
    for (int d = lane; d < D; d += 64) st(orow, d, 0.0f);
    return;
  }

  const T* kc = p.k_cache + (static_cast<size_t>(b) * p.Hkv + g) * p.cap * D;
  const T* vc = p.v_cache + (static_cast<size_t>(b) * p.Hkv + g) * p.cap * D;
  float m = -INFINITY, l = 0.0f, acc0 = 0.0f, acc1 = 0.0f;
  const int total = P + n;
  for (int t0 = 0; t0 < total; t0 += 64) {
    const int j = t0 + lane;
    float sc = -INFINITY;
    if (j < P) {
      const T* kr = kc + static_cast<size_t>(j) * D;
      float acc = 0.0f;
      for (int d = 0; d < D; ++d) acc = fmaf(qrow[wave][d], ld(kr, d), acc);
      sc = acc * p.scale;
    } else if (j < total && ((anc_i >> (j - P)) & 1ull)) {
      const float* kr = ktree[j - P];
      float acc = 0.0f;
      for (int d = 0; d < D; ++d) acc = fmaf(qrow[wave][d], kr[d], acc);
      sc = acc * p.scale;
    }
    const float mt = wave_max_f32(sc);
    const float m_new = fmaxf(m, mt);
    const float alpha = (m == -INFINITY) ? 0.0f : expf(m - m_new);
    const float pj = (sc == -INFINITY) ? 0.0f : expf(sc - m_new);
    l = l * alpha + wave_sum_f32(pj);
    acc0 *= alpha;
    acc1 *= alpha;
    m = m_new;
    const int kt = min(64, total - t0);
    for (int jj = 0; jj < kt; ++jj) {
      const float w = __shfl(pj, jj);
      if (w == 0.0f) continue;
      const int key = t0 + jj;
      if (key < P) {
        acc0 = fmaf(w, ld(vc, v_off(key, lane, D)), acc0);
        if (D > 64) acc1 = fmaf(w, ld(vc, v_off(key, lane + 64, D)), acc1);
      } else {
        const T* vr = p.v_new + ((static_cast<size_t>(b) * p.n_max + (key - P)) * p.Hkv + g) * D;
        acc0 = fmaf(w, ld(vr, lane), acc0);
        if (D > 64) acc1 = fmaf(w, ld(vr, lane + 64), acc1);
      }
    }
  }
  const float inv = 1.0f / l;
  st(orow, lane, acc0 * inv);
  if (D > 64) st(orow, lane + 64, acc1 * inv);
}

template <typename T>
hipError_t launch_vec(const tv_attn_args* a, hipStream_t s) {
  VecParams<T> p;
  p.q = static_cast<const T*>(a->q);
  p.k_new = static_cast<const T*>(a->k_new);
  p.v_new = static_cast<const T*>(a->v_new);
  p.k_cache = static_cast<T*>(a->k_cache);
  p.v_cache = static_cast<T*>(a->v_cache);
  p.prefix_len = a->prefix_len;
  p.n_nodes = a->n_nodes;
  p.anc = a->anc;
  p.depth = a->depth;
  p.err = a->err;
  p.out = static_cast<T*>(a->out);
  p.n_max = a->n_max;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.G = a->Hq / a->Hkv;
  p.D = a->D;
  p.cap = a->cap;
  p.theta = a->rope_theta;
  p.scale = a->softmax_scale > 0.0f ? a->softmax_scale : 1.0f / sqrtf(static_cast<float>(a->D));
  dim3 grid((p.G * p.n_max + 3) / 4, p.Hkv, a->B);
  hipLaunchKernelGGL(attn_vec_kernel<T>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_f32(const tv_attn_args* a, hipStream_t s) {
  return a->dtype == TV_BF16 ? launch_vec<uint16_t>(a, s) : launch_vec<float>(a, s);
}

}  // namespace tv
