// Tree-verification attention for the shapes the head-dim-128 bf16 kernel
// does not take: fp32 inputs (head dim 64 or 128), whose tolerance (1e-5
// relative) rules out bf16 products, and bf16 inputs at head dim 64.
//
// Every tree node attends to the P prefix keys of its KV head and to the keys
// of its ancestors-or-self, selected by the node's ancestor bitmask
// (infra-guide "5.3 Medusa、EAGLE 与 MTP", section 3.1); queries and tree keys
// are rotated at position P + depth (section 3.2), rotate-half pairs (d,
// d + D/2) at angle pos * theta^(-2d/D).
//
// Caches: K [B][Hkv][cap][D]; V [B][Hkv][cap/64][D][64] (blocks of 64 slots,
// head dim major inside a block).
//
// Two launches:
//  * append_tree_vec_kernel, grid (Hkv, B): rotates the n tree keys of each
//    KV head (angles reduced in double precision) and writes them, rounded to the
//    cache's type, and the raw tree values to cache slots [P, P + n); flags a
//    tree past the cache capacity (TV_ERR_CAPACITY), which skips the sequence.
//  * attn_vec_kernel<T, D>, grid ceil(G n_max / ROWS) Hkv B, ROWS / 32
//    wavefronts of 32 query rows (ROWS = 64; 128 for fp32 at head dim 128)
//    for each of KS key slices (KS = 4 for bf16, 2 for fp32
//    at head dim 64, 1 at 128): streams the slots [0, P + n) of its KV head
//    (the tree's slots now hold its rotated keys) in rounds of KS 64-key
//    tiles, one per slice, double-buffered in LDS (the next round's loads in
//    flight during the current round's products), merges the slices' partial
//    softmax sums through LDS at the end; the scores and the value products
//    run on the matrix cores: S^T = K Q^T and O^T += V^T P^T, 32x32 tiles
//    (v_mfma_f32_32x32x16_bf16 for bf16, v_mfma_f32_32x32x2f32 for fp32:
//    fp32 products, fp32 sums), and an online softmax in log2 units.
//    Lane l of a wavefront holds query row l % 32 in both products (the
//    operand and accumulator layouts of the 32x32 instructions; the keys are
//    permuted within each 32-key half so that a lane's score registers are
//    the probability operand it feeds into the value product), and the half
//    l / 32 selects which keys (scores) and head dims (outputs) it holds.
#include <math.h>

#include "tv_device.h"
#include "tv_internal.h"

namespace tv {

namespace {

constexpr int kVecKeys = 64;                  // keys per tile (= V cache block)
constexpr float kSlack = 8.0f;                // softmax reference slack (log2 units)
// Key slices: tiles a workgroup processes side by side (one per group of
// row wavefronts), as many as two LDS buffers of them allow.
template <typename T, int D>
constexpr int vec_slices() { return sizeof(T) == 2 ? 4 : (D == 64 ? 2 : 1); }
// Wavefronts of 32 query rows per workgroup: two, or four for fp32 at head
// dim 128 (whose tiles are the largest: more threads share their loads, so
// the chunks a thread holds in flight fit its registers).
template <typename T, int D>
constexpr int vec_row_waves() { return sizeof(T) == 4 && D == 128 ? 4 : 2; }
template <typename T, int D>
constexpr int vec_threads() { return vec_row_waves<T, D>() * vec_slices<T, D>() * kWave; }

typedef uint32_t vu32x4 __attribute__((ext_vector_type(4)));

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
  int row_blocks;     // workgroups per (sequence, KV head) in the attention grid
  float theta;        // 0: no rotation
  double log2_theta;
  float scale_log2;   // softmax scale times log2(e)
};

__device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float ld(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }
__device__ __forceinline__ void st(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16_bits(v); }

// Element offset of (slot, d) inside one head's V cache: [cap/64][D][64].
__device__ __forceinline__ size_t v_off(int slot, int d, int D) {
  return (static_cast<size_t>(slot >> 6) * D + d) * 64 + (slot & 63);
}

// cos/sin of pos * 2^(log2_theta * (-2 j / D)): the angle in double precision
// reduced to [-pi, pi], then single-precision sincos.
__device__ __forceinline__ float2 rope_cs_vec(int pos, int j, int D, double log2_theta) {
  const double ang = static_cast<double>(pos) * exp2(log2_theta * (-2.0 * j / D));
  const double red = fma(-6.283185307179586476925286766559, rint(ang * 0.15915494309189533576888376337251), ang);
  float s, c;
  sincosf(static_cast<float>(red), &s, &c);
  return make_float2(c, s);
}

// ---------------------------------------------------------------------------
// The tree append (and the capacity check). Grid (Hkv, B), 256 threads.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void append_tree_vec_kernel(VecParams<T> p) {
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int D = p.D, half = D / 2;
  const int n = p.n_nodes[b];
  const int P = p.prefix_len[b];
  const int e_in = p.err[b];
  const bool cap_bad = (e_in == 0) && (n > 0) && (n <= p.n_max) && (P < 0 || P + n > p.cap);
  if (cap_bad) {
    if (g == 0 && tid == 0) p.err[b] = TV_ERR_CAPACITY;
    return;
  }
  if (e_in != 0 || n <= 0 || n > p.n_max) return;
  const size_t head = (static_cast<size_t>(b) * p.Hkv + g) * p.cap * D;
  // item = (node a, pairs j0 .. j0 + 7): every load of an item goes out
  // before its arithmetic, and most threads take one item
  const int per_node = half / 8;
  for (int it = tid; it < n * per_node; it += blockDim.x) {
    const int a = it / per_node, j0 = 8 * (it - a * per_node);
    const size_t src = ((static_cast<size_t>(b) * p.n_max + a) * p.Hkv + g) * D;
    const int pos = P + p.depth[static_cast<size_t>(b) * p.n_max + a];
    float lo[8], hi[8];
    T vlo[8], vhi[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lo[e] = ld(p.k_new, src + j0 + e);
      hi[e] = ld(p.k_new, src + half + j0 + e);
      vlo[e] = p.v_new[src + j0 + e];
      vhi[e] = p.v_new[src + half + j0 + e];
    }
    const size_t slot = head + static_cast<size_t>(P + a) * D;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float2 cs = p.theta != 0.0f ? rope_cs_vec(pos, j0 + e, D, p.log2_theta) : make_float2(1.0f, 0.0f);
      st(p.k_cache, slot + j0 + e, lo[e] * cs.x - hi[e] * cs.y);
      st(p.k_cache, slot + half + j0 + e, hi[e] * cs.x + lo[e] * cs.y);
      p.v_cache[head + v_off(P + a, j0 + e, D)] = vlo[e];
      p.v_cache[head + v_off(P + a, half + j0 + e, D)] = vhi[e];
    }
  }
}

// Key of accumulator row m (0..31) in a 32-key half: the score registers of
// a lane then hold exactly the keys its probability operand needs, 8
// consecutive keys per 16-key step (bf16), or key 2k + (lane / 32) for step k
// (fp32). Row m = 8a + 4h + c (register 4a + c of a lane in half h).
__device__ __forceinline__ int key_of_row(int m, bool bf) {
  const int a = m >> 3, h = (m >> 2) & 1, c = m & 3;
  return bf ? 16 * (a >> 1) + 8 * h + 4 * (a & 1) + c : 8 * a + 2 * c + h;
}

__device__ __forceinline__ float half_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef float vf32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 vbf16x2 __attribute__((ext_vector_type(2)));
// two floats to bf16, rounded to nearest even (one conversion instruction)
__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
  const vf32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, vbf16x2));
}

// ---------------------------------------------------------------------------
// The attention. Grid ceil(G n_max / ROWS) Hkv B (one workgroup per ROWS
// query rows of a KV head), ROWS / 32 wavefronts per key slice.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__((vec_threads<T, D>())) void attn_vec_kernel(VecParams<T> p) {
  constexpr bool BF = sizeof(T) == 2;
  static_assert(!BF || D == 64, "bf16 at head dim 64 only (head dim 128 has its own kernel)");
  constexpr int KS = vec_slices<T, D>();                   // key slices
  constexpr int NT = vec_threads<T, D>();
  constexpr int EPC = 16 / static_cast<int>(sizeof(T));   // elements per 16-byte chunk
  constexpr int SK = D + EPC;                              // padded LDS row strides (elements)
  constexpr int SV = kVecKeys + EPC;
  constexpr int KCPR = D / EPC, VCPR = kVecKeys / EPC;     // chunks per K row, per V row
  constexpr int TCH = kVecKeys * D / EPC;                  // chunks of a K (or V) tile
  constexpr int CH = KS * TCH / NT;                        // chunks per thread of the KS tiles
  static_assert(TCH % NT == 0, "every chunk slot u of a thread falls in one tile");
  constexpr int BUF = kVecKeys * SK + D * SV;              // one tile (K and V), elements
  constexpr int DT = D / 32;                               // 32-dim output tiles
  constexpr int QK = BF ? D / 16 : D / 2;                  // score steps (and query operands)
  static_assert(2 * KS * BUF * sizeof(T) <= 160 * 1024, "two buffers of KS tiles fit the LDS");
  __shared__ __attribute__((aligned(16))) T smem[2 * KS * BUF];

  // Workgroups go to the eight XCDs round-robin by index: when the (sequence,
  // KV head) pairs come in multiples of eight, the row blocks of one pair get
  // indices eight apart, so they share an L2 and read each key tile from HBM
  // once. (A placement hint only: any bijection is correct.)
  const int R = p.row_blocks, U = gridDim.x / R;
  int rb, u;
  if (U % 8 == 0) {
    const int k = blockIdx.x >> 3;
    rb = k % R;
    u = (k / R) * 8 + (blockIdx.x & 7);
  } else {
    rb = blockIdx.x % R;
    u = blockIdx.x / R;
  }
  const int b = u / p.Hkv, g = u - b * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, col = lane & 31;
  constexpr int RWV = vec_row_waves<T, D>(), ROWS = 32 * RWV;
  const int rw = wave % RWV, ks = wave / RWV;   // row wavefront, key slice
  const int G = p.G, n_max = p.n_max;
  const int n = p.n_nodes[b];
  const int P = p.prefix_len[b];
  const int e_in = p.err[b];
  const bool skip = e_in != 0 || n <= 0 || n > n_max || P < 0 || P + n > p.cap;

  const int rows_all = G * n_max;
  const int r = rb * ROWS + rw * 32 + col;   // this lane's query row
  const bool row_exists = r < rows_all;
  const int node = row_exists ? r / G : 0;
  const int head = g * G + (row_exists ? r - node * G : 0);
  const bool live = row_exists && !skip && node < n;
  T* orow = p.out + ((static_cast<size_t>(b) * n_max + node) * p.Hq + head) * D;

  if (skip) {
    // (uniform over the workgroup) zero rows; lane half h writes half the dims
    if (row_exists)
      for (int d = h * (D / 2); d < (h + 1) * (D / 2); ++d) st(orow, d, 0.0f);
    return;
  }

  // ---- the tile loads (16-byte chunks): K rows [key][D] and the V block
  // [D][64] of slots t0 .. t0 + 63, both contiguous in the cache
  const size_t head_off = (static_cast<size_t>(b) * p.Hkv + g) * p.cap * D;
  const T* kc = p.k_cache + head_off;
  const T* vc = p.v_cache + head_off;
  const int total = P + n;
  const int nt = (total + kVecKeys - 1) / kVecKeys;   // tiles
  const int nit = (nt + KS - 1) / KS;                  // rounds of KS tiles
  // Round it holds tiles it KS + j, j < KS, in LDS slot j of buffer it % 2;
  // thread chunk u of a round belongs to tile j = (u NT + tid) / TCH (the
  // same j for the whole workgroup). A tile past the last one loads the last
  // one again (every load valid and unconditional) and is not used.
  // (chunks are held as four words between their load and their LDS store,
  // so that the compiler does not turn the pair into a copy through memory)
  typedef uint32_t Chunks[CH][4];
  auto load_round = [&](int it, Chunks& kreg, Chunks& vreg) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int c = u * NT + tid, j = c / TCH, rem = c - j * TCH, key = rem / KCPR, part = rem % KCPR;
      const int t0 = min(it * KS + j, nt - 1) * kVecKeys;
      const uint4 x = *reinterpret_cast<const uint4*>(kc + static_cast<size_t>(t0 + key) * D + part * EPC);
      kreg[u][0] = x.x;
      kreg[u][1] = x.y;
      kreg[u][2] = x.z;
      kreg[u][3] = x.w;
    }
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int c = u * NT + tid, j = c / TCH, rem = c - j * TCH, d = rem / VCPR, part = rem % VCPR;
      const int t0 = min(it * KS + j, nt - 1) * kVecKeys;
      const uint4 x = *reinterpret_cast<const uint4*>(vc + static_cast<size_t>(t0) * D + d * kVecKeys + part * EPC);
      vreg[u][0] = x.x;
      vreg[u][1] = x.y;
      vreg[u][2] = x.z;
      vreg[u][3] = x.w;
    }
  };
  // Into buffer `buf`; value elements of slots past P + n are zeroed (their
  // probabilities are 0, but a cache slot past the tree may hold anything).
  auto store_round = [&](int it, int buf, const Chunks& kreg, const Chunks& vreg) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int c = u * NT + tid, j = c / TCH, rem = c - j * TCH, key = rem / KCPR, part = rem % KCPR;
      T* kd = smem + (buf * KS + j) * BUF;
      *reinterpret_cast<uint4*>(kd + key * SK + part * EPC) = make_uint4(kreg[u][0], kreg[u][1], kreg[u][2], kreg[u][3]);
    }
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int c = u * NT + tid, j = c / TCH, rem = c - j * TCH, d = rem / VCPR, part = rem % VCPR;
      T* vd = smem + (buf * KS + j) * BUF + kVecKeys * SK;
      const int t0 = (it * KS + j) * kVecKeys;
      const bool ragged = t0 + kVecKeys > total;   // (uniform)
      uint32_t w[4] = {vreg[u][0], vreg[u][1], vreg[u][2], vreg[u][3]};
      if (ragged) {
        const int k0 = t0 + part * EPC;   // slot of the chunk's first element
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const bool dead = k0 + e >= total;
          if constexpr (BF)
            w[e >> 1] &= dead ? ((e & 1) ? 0x0000FFFFu : 0xFFFF0000u) : 0xFFFFFFFFu;
          else
            w[e] = dead ? 0u : w[e];
        }
      }
      *reinterpret_cast<uint4*>(vd + d * SV + part * EPC) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  };

  // the first round's loads go out before the query work
  Chunks ka, va;
  load_round(0, ka, va);

  // ---- this lane's query row, rotated at P + depth, times scale * log2(e):
  // bf16: dims 16k + 8h .. + 7 for step k (the B operand of the score
  // product), fp32: dim 2k + h for step k. Rows that are not live are zero.
  // The angles come from a table of (cos, sin) at P + d for the depths d < n
  // of the sequence's nodes and every pair j, built by the workgroup in LDS
  // buffer 1 (idle until round 1 is stored, after the first barrier of the
  // loop): each thread takes one pair j (its frequency computed once) and
  // every (NT / (D/2))-th depth.
  uint64_t anc_row = 0;
  int dep = 0;
  const T* qsrc = p.q + ((static_cast<size_t>(b) * n_max + node) * p.Hq + head) * D;
  if (live) {
    anc_row = p.anc[static_cast<size_t>(b) * n_max + node];
    dep = min(max(p.depth[static_cast<size_t>(b) * n_max + node], 0), n - 1);
  }
  constexpr int HALF = D / 2;
  static_assert(NT % HALF == 0 && TV_MAX_NODES_DEV * HALF * sizeof(float2) <= KS * BUF * sizeof(T),
                "the RoPE table fits buffer 1");
  float2* const cs_tab = reinterpret_cast<float2*>(smem + KS * BUF);
  if (p.theta != 0.0f) {
    const int j = tid % HALF;
    const double f = exp2(p.log2_theta * (-2.0 * j / D));
    for (int d = tid / HALF; d < n; d += NT / HALF) {
      const double ang = static_cast<double>(P + d) * f;
      const double red = fma(-6.283185307179586476925286766559, rint(ang * 0.15915494309189533576888376337251), ang);
      float sn, cn;
      sincosf(static_cast<float>(red), &sn, &cn);
      cs_tab[d * HALF + j] = make_float2(cn, sn);
    }
  }
  __syncthreads();
  const float2* const cs_row = cs_tab + dep * HALF;
  auto rope_at = [&](int j) { return p.theta != 0.0f ? cs_row[j] : make_float2(1.0f, 0.0f); };
  bf16x8 qf[BF ? QK : 1];
  float qv[BF ? 1 : QK];
  if constexpr (BF) {
    float x[QK][8];
#pragma unroll
    for (int k = 0; k < QK; ++k) {
      const uint4 w = live ? *reinterpret_cast<const uint4*>(qsrc + 16 * k + 8 * h) : make_uint4(0u, 0u, 0u, 0u);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) x[k][e] = bf16_bits_to_f32(static_cast<uint16_t>(ws[e >> 1] >> (16 * (e & 1))));
    }
    // pairs (d, d + D/2): step k < QK/2 with step k + QK/2
#pragma unroll
    for (int k = 0; k < QK / 2; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 cs = rope_at(16 * k + 8 * h + e);
        const float lo = x[k][e], hi = x[k + QK / 2][e];
        x[k][e] = (lo * cs.x - hi * cs.y) * p.scale_log2;
        x[k + QK / 2][e] = (hi * cs.x + lo * cs.y) * p.scale_log2;
      }
#pragma unroll
    for (int k = 0; k < QK; ++k) {
      const vu32x4 w = {pack_bf16_rne(x[k][0], x[k][1]), pack_bf16_rne(x[k][2], x[k][3]),
                        pack_bf16_rne(x[k][4], x[k][5]), pack_bf16_rne(x[k][6], x[k][7])};
      qf[k] = __builtin_bit_cast(bf16x8, w);
    }
  } else {
#pragma unroll
    for (int k = 0; k < QK; ++k) qv[k] = live ? ld(qsrc, 2 * k + h) : 0.0f;
    // pairs (d, d + D/2): step k < QK/2 with step k + QK/2
#pragma unroll
    for (int k = 0; k < QK / 2; ++k) {
      const float2 cs = rope_at(2 * k + h);
      const float lo = qv[k], hi = qv[k + QK / 2];
      qv[k] = (lo * cs.x - hi * cs.y) * p.scale_log2;
      qv[k + QK / 2] = (hi * cs.x + lo * cs.y) * p.scale_log2;
    }
  }

  // per-lane LDS element offsets of the operands: K row of accumulator row
  // `col` in each 32-key half, V row (head dim) `col` of each output tile
  const int krow = key_of_row(col, BF);

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
  float m = -INFINITY, l = 0.0f;

  // Products of round it (this wavefront's tile, in LDS buffer buf).
  auto compute = [&](int it, int buf) __attribute__((always_inline)) {
    const int t = it * KS + ks;   // this wavefront's tile (uniform over the wavefront)
    if (t < nt) {
    const T* kt = smem + (buf * KS + ks) * BUF;
    const T* vs = kt + kVecKeys * SK;
    const int t0 = t * kVecKeys;

    // scores, S^T = K Q^T: two 32-key halves
    f32x16 s[2];
    bf16x8 vf[BF ? DT : 1][4];
    if constexpr (BF) {
      // every fragment read goes out before the products that use it (one
      // wait for the LDS latency, not one per product); the value fragments
      // go out behind the score products and land during the softmax
      bf16x8 kf[2][QK];
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
        for (int k = 0; k < QK; ++k)
          kf[g2][k] = *reinterpret_cast<const bf16x8*>(kt + (krow + 32 * g2) * SK + 16 * k + 8 * h);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        s[g2] = f32x16{};
#pragma unroll
        for (int k = 0; k < QK; ++k) s[g2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[g2][k], qf[k], s[g2], 0, 0, 0);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          vf[dt][k] = *reinterpret_cast<const bf16x8*>(vs + (32 * dt + col) * SV + 16 * k + 8 * h);
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        s[g2] = f32x16{};
        const T* kr = kt + (krow + 32 * g2) * SK;
#pragma unroll
        for (int k = 0; k < QK; ++k) s[g2] = __builtin_amdgcn_mfma_f32_32x32x2f32(kr[2 * k + h], qv[k], s[g2], 0, 0, 0);
      }
    }
    // visibility: slots below P, and the row's ancestors-or-self among the
    // tree's slots [P, P + n) (only tiles that reach past P need the test)
    if (t0 + kVecKeys > P) {
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = t0 + 32 * g2 + key_of_row(8 * (v >> 2) + 4 * h + (v & 3), BF);
          const bool vis = key < P || (key < total && ((anc_row >> (key - P)) & 1ull));
          if (!vis) s[g2][v] = -INFINITY;
        }
    }
    // softmax of the row (both halves of the wavefront hold it) against the
    // reference m (log2 units; -inf until the first visible key): terms are
    // 2^(s - m), and m is raised only when a tile's max exceeds it by more
    // than kSlack, so every term stays below 2^kSlack and the rescale of the
    // running sums is rare (any m gives the same ratios)
    float tmax = -INFINITY;
#pragma unroll
    for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
      for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, s[g2][v]);
    tmax = half_max(tmax);
    const bool raise = tmax != -INFINITY && (m == -INFINITY || tmax > m + kSlack);
    if (__any(raise)) {
      const float alpha = !raise ? 1.0f : m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - tmax);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
      m = raise ? tmax : m;
    }
    const float ref = m == -INFINITY ? 0.0f : m;   // (no visible key yet: every term is 0)
    float sum = 0.0f;
#pragma unroll
    for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        s[g2][v] = __builtin_amdgcn_exp2f(s[g2][v] - ref);
        sum += s[g2][v];
      }
    l += sum;

    // values, O^T += V^T P^T
    if constexpr (BF) {
      bf16x8 pb[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x16& sv = s[k >> 1];
        const int v0 = 8 * (k & 1);
        const vu32x4 w = {pack_bf16_rne(sv[v0], sv[v0 + 1]), pack_bf16_rne(sv[v0 + 2], sv[v0 + 3]),
                          pack_bf16_rne(sv[v0 + 4], sv[v0 + 5]), pack_bf16_rne(sv[v0 + 6], sv[v0 + 7])};
        pb[k] = __builtin_bit_cast(bf16x8, w);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int k = 0; k < 4; ++k) o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[dt][k], pb[k], o[dt], 0, 0, 0);
    } else {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const T* vr = vs + (32 * dt + col) * SV;
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
          for (int k = 0; k < 16; ++k)
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vr[32 * g2 + 2 * k + h], s[g2][k], o[dt], 0, 0, 0);
      }
    }
    }
  };

  // Rounds it + 1 and it + 2 are in flight in registers while round it
  // computes (two register sets, a and b, alternating; the loop is unrolled
  // by two so that each has fixed registers), or only round it + 1 where two
  // sets would not fit the registers (fp32 at head dim 128). Every load is
  // unconditional (rounds past the last one load the last tile again, from
  // L2), so the compiler's in-order wait for one set never waits for the
  // other. Round r + 1 goes to the buffer round r - 1 used: every wavefront
  // finished reading it before the barrier that ended round r - 1.
  constexpr bool kTwoDeep = 2 * 2 * CH * 4 <= 128;   // registers of two sets
  store_round(0, 0, ka, va);
  if constexpr (kTwoDeep) {
    Chunks kb, vb;
    load_round(1, ka, va);
    load_round(2, kb, vb);
    __syncthreads();
    for (int it = 0; it < nit; it += 2) {
      compute(it, 0);
      if (it + 1 < nit) store_round(it + 1, 1, ka, va);
      __syncthreads();
      load_round(it + 3, ka, va);
      compute(it + 1, 1);   // (nothing to do past the last round)
      if (it + 2 < nit) store_round(it + 2, 0, kb, vb);
      __syncthreads();
      load_round(it + 4, kb, vb);
    }
  } else {
    load_round(1, ka, va);
    __syncthreads();
    for (int it = 0; it < nit; ++it) {
      compute(it, it & 1);
      if (it + 1 < nit) store_round(it + 1, (it + 1) & 1, ka, va);
      __syncthreads();
      load_round(it + 2, ka, va);
    }
  }

  // ---- the key slices of each row wavefront merge through LDS (idle after
  // the last barrier): slice s's (max, sum, outputs) weighted by 2^(m_s - M)
  float lt = half_sum(l);
  if constexpr (KS > 1) {
    constexpr int MW = 2 + 16 * DT;   // floats per lane
    static_assert(NT * MW * sizeof(float) <= 2 * KS * BUF * sizeof(T), "the merge fits the LDS");
    float* mrg = reinterpret_cast<float*>(smem);
    float* mine = mrg + static_cast<size_t>(tid) * MW;
    if (ks != 0) {
      mine[0] = m;
      mine[1] = lt;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) mine[2 + 16 * dt + v] = o[dt][v];
    }
    __syncthreads();
    if (ks != 0) return;
    float M = m;
#pragma unroll
    for (int s2 = 1; s2 < KS; ++s2) M = fmaxf(M, mrg[static_cast<size_t>(s2 * RWV * 64 + tid) * MW]);
    const float w0 = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
    lt *= w0;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= w0;
#pragma unroll
    for (int s2 = 1; s2 < KS; ++s2) {
      const float* other = mrg + static_cast<size_t>(s2 * RWV * 64 + tid) * MW;
      const float ms = other[0];
      const float ws = ms == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
      lt = fmaf(ws, other[1], lt);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[dt][v] = fmaf(ws, other[2 + 16 * dt + v], o[dt][v]);
    }
  }

  // ---- the row: lane half h holds dims 32 dt + 8 a + 4 h + c (register 4a + c)
  if (!row_exists) return;
  const float inv = (live && lt > 0.0f) ? 1.0f / lt : 0.0f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * dt + 8 * a + 4 * h;
      const float y0 = o[dt][4 * a] * inv, y1 = o[dt][4 * a + 1] * inv;
      const float y2 = o[dt][4 * a + 2] * inv, y3 = o[dt][4 * a + 3] * inv;
      if constexpr (BF) {
        *reinterpret_cast<uint2*>(orow + d0) = make_uint2(pack_bf16_rne(y0, y1), pack_bf16_rne(y2, y3));
      } else {
        *reinterpret_cast<float4*>(orow + d0) = make_float4(y0, y1, y2, y3);
      }
    }
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
  p.log2_theta = a->rope_theta != 0.0f ? log2(static_cast<double>(a->rope_theta)) : 0.0;
  const float scale = a->softmax_scale > 0.0f ? a->softmax_scale : 1.0f / sqrtf(static_cast<float>(a->D));
  p.scale_log2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(append_tree_vec_kernel<T>, dim3(p.Hkv, a->B), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = 32 * (sizeof(T) == 4 && a->D == 128 ? vec_row_waves<T, 128>() : vec_row_waves<T, 64>());
  p.row_blocks = (p.G * p.n_max + rows - 1) / rows;
  const dim3 grid(p.row_blocks * p.Hkv * a->B);
  if constexpr (sizeof(T) == 2) {
    if (a->D != 64) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_vec_kernel<T, 64>), grid, dim3(vec_threads<T, 64>()), 0, s, p);
  } else {
    if (a->D == 64)
      hipLaunchKernelGGL((attn_vec_kernel<T, 64>), grid, dim3(vec_threads<T, 64>()), 0, s, p);
    else if (a->D == 128)
      hipLaunchKernelGGL((attn_vec_kernel<T, 128>), grid, dim3(vec_threads<T, 128>()), 0, s, p);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_f32(const tv_attn_args* a, hipStream_t s) {
  return a->dtype == TV_BF16 ? launch_vec<uint16_t>(a, s) : launch_vec<float>(a, s);
}

}  // namespace tv
