// bf16 tree-verification attention on CDNA4 matrix cores (gfx950).
//
// What is computed (infra-guide "5.3 Medusa、EAGLE 与 MTP", sections 3.1 and
// 3.2; pofe.ai "Medusa and EAGLE ...", "Trees"): every node i of a flattened
// draft tree attends to the P prefix keys of its KV head and to the keys of
// its ancestors-or-self, with query and tree keys rotated at position
// P + depth. Siblings and other branches are masked out by the node's
// ancestor bitmask.
//
// How (this file's design, not the pages'):
//   * Workgroup = (sequence b, KV head g, row block rb, KV split s). Its query
//     rows are the G query heads of g for every tree node, node-major
//     (row = node * G + head_in_group); each wavefront owns 32 rows. All rows
//     share one pass over the prefix K/V of (b, g): the prefix is read from
//     HBM once per split, coalesced, and staged in LDS in 64-key tiles
//     (double-buffered; the next tile is loaded into registers while the
//     current one is multiplied).
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: a lane then holds 16 keys of ONE query row,
//     so the row max and row sum are lane-local plus one exchange with the
//     lane 32 away. The output is also transposed, O^T = V^T P^T, so the
//     probabilities leave the score accumulator straight into the B operand
//     (no LDS round trip) and the rescale factor of a row is lane-local.
//   * K is stored row-major in LDS with 16-byte units XOR-swizzled by key;
//     V is stored transposed (d-major) with keys permuted to the order the
//     score accumulator produces them, units swizzled by d.
//   * Online softmax in base 2 with a lazily moved running max: the output is
//     rescaled only when a tile's max exceeds the running max by more than
//     2^8, so most tiles skip the rescale (exact up to rounding: the shared
//     exponent offset cancels in the final division).
//   * The tree tile (n <= 64 nodes) is one more 64-key tile whose keys are the
//     tree nodes, rotated on the fly from k_new; a key j is visible to row r
//     iff bit j of anc[node(r)] is set. The workgroup of the last split with
//     rb == 0 also appends the rotated tree keys and raw values to cache slots
//     [P, P+n).
//   * With several splits, each writes (max, sum, unnormalised output) to the
//     workspace and a merge kernel combines them.
#include <math.h>

#include "tv_device.h"
#include "tv_internal.h"

namespace tv {

namespace {

constexpr int kD = 128;          // head dim (bf16 path)
constexpr int kKT = 64;          // keys per LDS stage
constexpr int kStageElems = kKT * kD;   // bf16 elements of one K (or V) stage
constexpr float kLazyMax = 8.0f;        // log2 headroom before a rescale

struct BfParams {
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_cache;
  uint16_t* v_cache;
  const int32_t* prefix_len;
  const int32_t* n_nodes;
  const uint64_t* anc;
  const int32_t* depth;
  int32_t* err;
  uint16_t* out;
  float* part_o;     // [B][Hkv][S][rows_pad][D]
  float2* part_ml;   // [B][Hkv][S][rows_pad]  (running max in log2 units, sum)
  int n_max, Hq, Hkv, G, cap;
  int splits, row_blocks, rows_pad;
  float theta, scale_log2;
};

// Position of physical key k (0..63) inside a V^T stage row. The score
// accumulator of v_mfma_f32_32x32x16 gives lane half h the keys
// {8i + 4h + j}; the probabilities for the PV product are taken 8 at a time in
// that order, so keys are stored in the same order.
__device__ __forceinline__ int vt_key_slot(int k) {
  const int st = k >> 5, r = k & 31, mf = r >> 4, r2 = r & 15;
  const int hh = (r2 >> 2) & 1, within = ((r2 >> 3) << 2) | (r2 & 3);
  return (st << 5) | (mf << 4) | (hh << 3) | within;
}

__device__ __forceinline__ int ks_index(int key, int unit) {
  return key * kD + ((unit ^ (key & 7)) << 3);
}
__device__ __forceinline__ int vt_index(int d, int unit) {
  return d * kKT + ((unit ^ ((d & 7) ^ ((d >> 3) & 7))) << 3);
}

__device__ __forceinline__ uint16_t u4_elem(const uint4& v, int t) {
  const uint32_t w = (t < 2) ? v.x : (t < 4) ? v.y : (t < 6) ? v.z : v.w;
  return static_cast<uint16_t>((t & 1) ? (w >> 16) : (w & 0xFFFFu));
}

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
  return static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
}

// cos/sin of position pos for rotary pair `pair` (of 64): angle in double
// precision, reduced to [-pi, pi], then single-precision sincos.
__device__ __forceinline__ float2 rope_cs_direct(int pos, int pair, float theta) {
  if (theta == 0.0f) return make_float2(1.0f, 0.0f);
  const double inv_freq = pow(static_cast<double>(theta), -2.0 * pair / kD);
  const double ang = static_cast<double>(pos) * inv_freq;
  const double two_pi = 6.283185307179586476925286766559;
  const double red = ang - two_pi * rint(ang / two_pi);
  float s, c;
  sincosf(static_cast<float>(red), &s, &c);
  return make_float2(c, s);
}

// Writes one 16-byte chunk of V (8 consecutive d of key `key`) transposed.
__device__ __forceinline__ void vt_scatter(uint16_t* vt, int key, int c, const uint4& v) {
  const int slot = vt_key_slot(key);
  const int u = slot >> 3, e = slot & 7;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int d = 8 * c + t;
    vt[vt_index(d, u) + e] = u4_elem(v, t);
  }
}

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void attn_bf16_kernel(BfParams p) {
  constexpr int NT = WAVES * 64;
  constexpr int CPT = (kKT * kD / 8) / NT;   // 16-byte chunks per thread per K (or V) stage
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * kStageElems];  // Ks0 Vt0 Ks1 Vt1
  __shared__ int s_dmax;

  const int s = blockIdx.x % p.splits;
  const int rb = blockIdx.x / p.splits;
  const int g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  const int G = p.G;

  const int n = p.n_nodes[b];
  const int P = p.prefix_len[b];
  const int e_in = p.err[b];
  const bool cap_bad = (e_in == 0) && (n > 0) && (n <= p.n_max) && (P < 0 || P + n > p.cap);
  const bool skip = (e_in != 0) || (n <= 0) || (n > p.n_max) || cap_bad;
  if (cap_bad && blockIdx.x == 0 && g == 0 && tid == 0) p.err[b] = TV_ERR_CAPACITY;

  const int rows_live = skip ? 0 : G * n;
  const int rows_all = G * p.n_max;
  const int rb0 = rb * WAVES * 32;
  const int r0 = rb0 + wave * 32;
  const int my_row = r0 + (lane & 31);

  if (rb0 >= rows_live) {
    // nothing live in this row block: zero rows (single split) and leave
    if (p.splits == 1) {
      for (int r = rb0 + tid / 16; r < min(rb0 + WAVES * 32, rows_all); r += NT / 16) {
        const int i = r / G, head = g * G + r % G;
        uint16_t* orow = p.out + ((static_cast<size_t>(b) * p.n_max + i) * p.Hq + head) * kD;
        reinterpret_cast<uint4*>(orow)[tid % 16] = make_uint4(0, 0, 0, 0);
      }
    }
    return;
  }

  const bool wave_active = r0 < rows_live;
  const bool row_live = my_row < rows_live;
  const int my_node = row_live ? my_row / G : 0;
  const uint64_t my_anc = row_live ? p.anc[static_cast<size_t>(b) * p.n_max + my_node] : 0ull;

  // prefix keys of this split, in whole 64-key tiles
  const int n_tiles_all = (P + kKT - 1) / kKT;
  const int tiles_per_split = (n_tiles_all + p.splits - 1) / p.splits;
  const int k_begin = min(P, s * tiles_per_split * kKT);
  const int k_end = min(P, k_begin + tiles_per_split * kKT);
  const int n_tiles = (k_end - k_begin + kKT - 1) / kKT;
  const bool last_split = (s == p.splits - 1);

  uint16_t* Ks0 = smem;
  uint16_t* Vt0 = smem + kStageElems;
  uint16_t* Ks1 = smem + 2 * kStageElems;
  uint16_t* Vt1 = smem + 3 * kStageElems;
  float2* cs_table = reinterpret_cast<float2*>(Ks1);   // aliases stage 1 in the prologue

  const size_t head_off = (static_cast<size_t>(b) * p.Hkv + g) * p.cap * kD;
  const uint16_t* kc = p.k_cache + head_off;
  const uint16_t* vc = p.v_cache + head_off;

  // ---- 1. start loading prefix tile 0 (latency overlaps the prologue)
  uint4 kreg[CPT], vreg[CPT];
  auto load_tile = [&](int kt0) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int qi = tid + j * NT;
      const int key = qi >> 4, unit = qi & 15;
      const int kidx = kt0 + key;
      if (kidx < k_end) {
        kreg[j] = *reinterpret_cast<const uint4*>(kc + static_cast<size_t>(kidx) * kD + unit * 8);
        vreg[j] = *reinterpret_cast<const uint4*>(vc + static_cast<size_t>(kidx) * kD + unit * 8);
      } else {
        kreg[j] = make_uint4(0, 0, 0, 0);
        vreg[j] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](uint16_t* ks, uint16_t* vt) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int qi = tid + j * NT;
      const int key = qi >> 4, unit = qi & 15;
      *reinterpret_cast<uint4*>(ks + ks_index(key, unit)) = kreg[j];
      vt_scatter(vt, key, unit, vreg[j]);
    }
  };
  if (n_tiles > 0) load_tile(k_begin);

  // ---- 2. deepest node -> size of the cos/sin table
  if (wave == 0) {
    int dv = (lane < n) ? p.depth[static_cast<size_t>(b) * p.n_max + lane] : 0;
    dv = wave_max_i32(dv);
    if (lane == 0) s_dmax = dv;
  }
  __syncthreads();
  const int dmax = s_dmax;
  // one table row (64 pairs) per depth; stage 1 holds 32 rows of float2
  const bool use_table = dmax < (2 * kStageElems * 2) / (64 * 8);
  if (use_table) {
    for (int idx = tid; idx < (dmax + 1) * 64; idx += NT)
      cs_table[idx] = rope_cs_direct(P + (idx >> 6), idx & 63, p.theta);
  }
  __syncthreads();
  auto rope_cs = [&](int dep, int pair) -> float2 {
    return use_table ? cs_table[dep * 64 + pair] : rope_cs_direct(P + dep, pair, p.theta);
  };

  // ---- 3. rotated queries as B operands: qf[ks] = Q[row][16ks + 8h .. +8]
  bf16x8 qf[8];
  {
    uint16_t lo16[4][8], hi16[4][8];
    if (row_live) {
      const int head = g * G + my_row % G;
      const int dep = p.depth[static_cast<size_t>(b) * p.n_max + my_node];
      const uint16_t* qrow = p.q + ((static_cast<size_t>(b) * p.n_max + my_node) * p.Hq + head) * kD;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int d0 = 16 * s4 + 8 * h;
        const uint4 lo = *reinterpret_cast<const uint4*>(qrow + d0);
        const uint4 hi = *reinterpret_cast<const uint4*>(qrow + 64 + d0);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float2 cs = rope_cs(dep, d0 + t);
          const float xl = bf16_bits_to_f32(u4_elem(lo, t));
          const float xh = bf16_bits_to_f32(u4_elem(hi, t));
          lo16[s4][t] = f32_to_bf16_bits(xl * cs.x - xh * cs.y);
          hi16[s4][t] = f32_to_bf16_bits(xh * cs.x + xl * cs.y);
        }
      }
    } else {
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
        for (int t = 0; t < 8; ++t) lo16[s4][t] = hi16[s4][t] = 0;
    }
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      uint4 a = make_uint4(pack2(lo16[s4][0], lo16[s4][1]), pack2(lo16[s4][2], lo16[s4][3]),
                           pack2(lo16[s4][4], lo16[s4][5]), pack2(lo16[s4][6], lo16[s4][7]));
      uint4 c = make_uint4(pack2(hi16[s4][0], hi16[s4][1]), pack2(hi16[s4][2], hi16[s4][3]),
                           pack2(hi16[s4][4], hi16[s4][5]), pack2(hi16[s4][6], hi16[s4][7]));
      qf[s4] = __builtin_bit_cast(bf16x8, a);
      qf[s4 + 4] = __builtin_bit_cast(bf16x8, c);
    }
  }

  // ---- running softmax state (rows = lane & 31; both lane halves agree on m)
  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.0f;
  float m_run = -INFINITY;   // in log2 units (score * scale * log2 e)
  float l_part = 0.0f;       // this lane's share of the row sum

  // Multiplies one staged 64-key tile into the running state.
  // valid_keys: keys >= valid_keys are masked; tree: mask by ancestor bits.
  auto compute_tile = [&](const uint16_t* ks, const uint16_t* vt, int valid_keys, bool tree) {
    float x[2][16];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      f32x16 acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
      const int key = 32 * st + (lane & 31);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + ks_index(key, 2 * kk + h));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], acc, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) x[st][e] = acc[e];
    }
    // masking: accumulator element e of sub-tile st is key 32st + 8(e>>2) + 4h + (e&3)
    if (tree || valid_keys < kKT) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = 32 * st + 8 * (e >> 2) + 4 * h + (e & 3);
          const bool vis = tree ? ((my_anc >> key) & 1ull) != 0ull : key < valid_keys;
          if (!vis) x[st][e] = -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 16; ++e) mt = fmaxf(mt, x[st][e]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mt2 = mt * p.scale_log2;
    if (__any(mt2 > m_run + kLazyMax)) {
      const float m_new = fmaxf(m_run, mt2);
      const float alpha = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - m_new);
      l_part *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
    bf16x8 pf[2][2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      uint16_t pb[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = exp2f(fmaf(x[st][e], p.scale_log2, -m_use));
        l_part += pe;
        pb[e] = f32_to_bf16_bits(pe);
      }
#pragma unroll
      for (int mf = 0; mf < 2; ++mf) {
        uint4 w = make_uint4(pack2(pb[8 * mf + 0], pb[8 * mf + 1]), pack2(pb[8 * mf + 2], pb[8 * mf + 3]),
                             pack2(pb[8 * mf + 4], pb[8 * mf + 5]), pack2(pb[8 * mf + 6], pb[8 * mf + 7]));
        pf[st][mf] = __builtin_bit_cast(bf16x8, w);
      }
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int d = 32 * dt + (lane & 31);
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int mf = 0; mf < 2; ++mf) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + vt_index(d, 4 * st + 2 * mf + h));
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[st][mf], oacc[dt], 0, 0, 0);
        }
    }
  };

  // ---- 4. tree tile (last split only): rotate k_new, stage, append, multiply
  if (last_split) {
    const size_t new_base = static_cast<size_t>(b) * p.n_max;
    uint16_t* kslot = p.k_cache + head_off + static_cast<size_t>(P) * kD;
    uint16_t* vslot = p.v_cache + head_off + static_cast<size_t>(P) * kD;
    const bool append = (rb == 0);
    for (int it = tid; it < 64 * 8; it += NT) {
      const int a = it >> 3, c = it & 7;
      uint4 lo_o = make_uint4(0, 0, 0, 0), hi_o = make_uint4(0, 0, 0, 0);
      if (a < n) {
        const uint16_t* kr = p.k_new + ((new_base + a) * p.Hkv + g) * kD;
        const uint4 lo = *reinterpret_cast<const uint4*>(kr + 8 * c);
        const uint4 hi = *reinterpret_cast<const uint4*>(kr + 64 + 8 * c);
        const int dep = p.depth[new_base + a];
        uint16_t ol[8], oh[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float2 cs = rope_cs(dep, 8 * c + t);
          const float xl = bf16_bits_to_f32(u4_elem(lo, t));
          const float xh = bf16_bits_to_f32(u4_elem(hi, t));
          ol[t] = f32_to_bf16_bits(xl * cs.x - xh * cs.y);
          oh[t] = f32_to_bf16_bits(xh * cs.x + xl * cs.y);
        }
        lo_o = make_uint4(pack2(ol[0], ol[1]), pack2(ol[2], ol[3]), pack2(ol[4], ol[5]), pack2(ol[6], ol[7]));
        hi_o = make_uint4(pack2(oh[0], oh[1]), pack2(oh[2], oh[3]), pack2(oh[4], oh[5]), pack2(oh[6], oh[7]));
        if (append) {
          *reinterpret_cast<uint4*>(kslot + static_cast<size_t>(a) * kD + 8 * c) = lo_o;
          *reinterpret_cast<uint4*>(kslot + static_cast<size_t>(a) * kD + 64 + 8 * c) = hi_o;
        }
      }
      *reinterpret_cast<uint4*>(Ks0 + ks_index(a, c)) = lo_o;
      *reinterpret_cast<uint4*>(Ks0 + ks_index(a, c + 8)) = hi_o;
    }
    for (int it = tid; it < 64 * 16; it += NT) {
      const int a = it >> 4, c = it & 15;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (a < n) {
        v = *reinterpret_cast<const uint4*>(p.v_new + ((new_base + a) * p.Hkv + g) * kD + 8 * c);
        if (append) *reinterpret_cast<uint4*>(vslot + static_cast<size_t>(a) * kD + 8 * c) = v;
      }
      vt_scatter(Vt0, a, c, v);
    }
    __syncthreads();
    if (wave_active) compute_tile(Ks0, Vt0, kKT, true);
    __syncthreads();
  }

  // ---- 5. prefix tiles, double-buffered
  if (n_tiles > 0) {
    store_tile(Ks0, Vt0);
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
      const bool more = (t + 1 < n_tiles);
      if (more) load_tile(k_begin + (t + 1) * kKT);
      const uint16_t* ks = (t & 1) ? Ks1 : Ks0;
      const uint16_t* vt = (t & 1) ? Vt1 : Vt0;
      if (wave_active) compute_tile(ks, vt, min(kKT, k_end - (k_begin + t * kKT)), false);
      if (more) store_tile((t & 1) ? Ks0 : Ks1, (t & 1) ? Vt0 : Vt1);
      __syncthreads();
    }
  }

  // ---- 6. epilogue
  const float l_tot = l_part + __shfl_xor(l_part, 32);
  if (p.splits == 1) {
    if (my_row < min(rows_all, rb0 + WAVES * 32)) {
      const int head = g * G + my_row % G;
      const int node = my_row / G;
      uint16_t* orow = p.out + ((static_cast<size_t>(b) * p.n_max + node) * p.Hq + head) * kD;
      const float inv = (row_live && l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = 32 * dt + 8 * i4 + 4 * h;
          uint2 w;
          w.x = pack2(f32_to_bf16_bits(oacc[dt][4 * i4 + 0] * inv), f32_to_bf16_bits(oacc[dt][4 * i4 + 1] * inv));
          w.y = pack2(f32_to_bf16_bits(oacc[dt][4 * i4 + 2] * inv), f32_to_bf16_bits(oacc[dt][4 * i4 + 3] * inv));
          *reinterpret_cast<uint2*>(orow + d0) = w;
        }
    }
  } else {
    const size_t prow = ((static_cast<size_t>(b) * p.Hkv + g) * p.splits + s) * p.rows_pad + my_row;
    float* po = p.part_o + prow * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = 32 * dt + 8 * i4 + 4 * h;
        *reinterpret_cast<float4*>(po + d0) =
            make_float4(oacc[dt][4 * i4 + 0], oacc[dt][4 * i4 + 1], oacc[dt][4 * i4 + 2], oacc[dt][4 * i4 + 3]);
      }
    if (h == 0) p.part_ml[prow] = make_float2(m_run, l_tot);
  }
}

// Combines the split partials of each row: one wavefront per row, two output
// dims per lane.
__global__ __launch_bounds__(256) void merge_bf16_kernel(BfParams p) {
  const int g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = blockIdx.x * 4 + wave;
  if (r >= p.G * p.n_max) return;
  const int node = r / p.G, head = g * p.G + r % p.G;
  const int n = p.n_nodes[b];
  const int P = p.prefix_len[b];
  const bool skip = (p.err[b] != 0) || (n <= 0) || (n > p.n_max) || (P < 0) || (P + n > p.cap);
  uint16_t* orow = p.out + ((static_cast<size_t>(b) * p.n_max + node) * p.Hq + head) * kD;
  float o0 = 0.0f, o1 = 0.0f;
  if (!skip && node < n) {
    const size_t base = (static_cast<size_t>(b) * p.Hkv + g) * p.splits;
    float M = -INFINITY;
    for (int s = 0; s < p.splits; ++s) M = fmaxf(M, p.part_ml[(base + s) * p.rows_pad + r].x);
    float L = 0.0f;
    for (int s = 0; s < p.splits; ++s) {
      const size_t prow = (base + s) * p.rows_pad + r;
      const float2 ml = p.part_ml[prow];
      const float w = (ml.x == -INFINITY) ? 0.0f : exp2f(ml.x - M);
      L += w * ml.y;
      const float2 o = *reinterpret_cast<const float2*>(p.part_o + prow * kD + 2 * lane);
      o0 += w * o.x;
      o1 += w * o.y;
    }
    const float inv = (L > 0.0f) ? 1.0f / L : 0.0f;
    o0 *= inv;
    o1 *= inv;
  }
  reinterpret_cast<uint32_t*>(orow)[lane] = pack2(f32_to_bf16_bits(o0), f32_to_bf16_bits(o1));
}

}  // namespace

AttnPlan plan_attention_bf16(const tv_attn_args* a) {
  AttnPlan pl;
  const int G = a->Hq / a->Hkv;
  const int rows = G * a->n_max;
  pl.waves = rows <= 64 ? 2 : (rows <= 128 ? 4 : 8);
  pl.row_blocks = (rows + pl.waves * 32 - 1) / (pl.waves * 32);
  const long units = static_cast<long>(a->B) * a->Hkv * pl.row_blocks;
  // Split the prefix until the grid covers the 256 compute units, keeping at
  // least four 64-key tiles per split. The prefix length lives on the device,
  // so the cache capacity bounds it here.
  const int max_tiles = (a->cap + kKT - 1) / kKT;
  int splits = 1;
  while (units * splits < 256 && (max_tiles / (splits * 2)) >= 4) splits *= 2;
  pl.splits = splits;
  pl.rows_pad = pl.row_blocks * pl.waves * 32;
  pl.workspace_bytes = 0;
  if (splits > 1) {
    const size_t rows_total = static_cast<size_t>(a->B) * a->Hkv * splits * pl.rows_pad;
    pl.workspace_bytes = rows_total * kD * sizeof(float) + rows_total * sizeof(float2);
  }
  return pl;
}

hipError_t launch_attention_bf16(const tv_attn_args* a, const AttnPlan& pl, hipStream_t s) {
  BfParams p;
  p.q = static_cast<const uint16_t*>(a->q);
  p.k_new = static_cast<const uint16_t*>(a->k_new);
  p.v_new = static_cast<const uint16_t*>(a->v_new);
  p.k_cache = static_cast<uint16_t*>(a->k_cache);
  p.v_cache = static_cast<uint16_t*>(a->v_cache);
  p.prefix_len = a->prefix_len;
  p.n_nodes = a->n_nodes;
  p.anc = a->anc;
  p.depth = a->depth;
  p.err = a->err;
  p.out = static_cast<uint16_t*>(a->out);
  p.n_max = a->n_max;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.G = a->Hq / a->Hkv;
  p.cap = a->cap;
  p.splits = pl.splits;
  p.row_blocks = pl.row_blocks;
  p.rows_pad = pl.rows_pad;
  p.theta = a->rope_theta;
  const float scale = a->softmax_scale > 0.0f ? a->softmax_scale : 1.0f / sqrtf(static_cast<float>(kD));
  p.scale_log2 = scale * 1.4426950408889634f;
  p.part_o = nullptr;
  p.part_ml = nullptr;
  if (pl.splits > 1) {
    const size_t rows_total = static_cast<size_t>(a->B) * a->Hkv * pl.splits * pl.rows_pad;
    p.part_o = static_cast<float*>(a->workspace);
    p.part_ml = reinterpret_cast<float2*>(static_cast<char*>(a->workspace) + rows_total * kD * sizeof(float));
  }
  dim3 grid(pl.splits * pl.row_blocks, a->Hkv, a->B);
  switch (pl.waves) {
    case 2: hipLaunchKernelGGL(attn_bf16_kernel<2>, grid, dim3(128), 0, s, p); break;
    case 4: hipLaunchKernelGGL(attn_bf16_kernel<4>, grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL(attn_bf16_kernel<8>, grid, dim3(512), 0, s, p); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.splits == 1) return e;
  dim3 mgrid((p.G * p.n_max + 3) / 4, a->Hkv, a->B);
  hipLaunchKernelGGL(merge_bf16_kernel, mgrid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace tv
