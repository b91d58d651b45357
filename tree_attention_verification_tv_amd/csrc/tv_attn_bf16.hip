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
//     (row = node * G + head_in_group); each wavefront owns QT tiles of 32
//     rows, so every K or V fragment read from LDS feeds QT MFMAs. All rows
//     share one pass over the prefix K/V of (b, g): the prefix is read from
//     HBM once per split, coalesced, and copied straight into LDS in 64-key
//     tiles (global_load_lds into a ring of four stages, three tiles in
//     flight), so the copies cost no registers and no LDS write instructions.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: a lane then holds 16 keys of ONE query row,
//     so the row max is lane-local plus one v_permlane32_swap. The output is
//     also transposed, O^T = V^T P^T, so the probabilities go from the score
//     accumulator straight into the B operand, and a row's rescale factor is
//     lane-local.
//   * The queries are pre-scaled by softmax_scale * log2(e) and the score
//     MFMA starts from an accumulator holding -r, where r is the row's score
//     against the tree root (visible to every node), so the accumulator IS
//     the exponent: p = exp2(acc), with no running max and no branch in the
//     tile loop. A row whose later scores rise more than 2^62 above r is
//     caught from its final sum; the workgroup then finds every row's exact
//     max in a scores-only pass and redoes the pass with r = max, where
//     every p <= 1 (exact for any score range).
//     Row sums are dot products of the bf16 probabilities with ones, i.e.
//     exactly the weights the PV product used.
//   * The score MFMA reads K rows in a permuted order (row m of a 32-key block
//     is key perm(m)), so each lane half holds 8 CONSECUTIVE keys per 16-key
//     group: the probabilities then match the V tile in natural key order.
//   * V is cached tile-blocked and d-major ([cap/64][D][64]), so a 64-key V
//     tile is one contiguous 16 KB block whose rows (one per head dim) are
//     exactly the A operand of the PV product. K rows and V rows sit in LDS
//     with 16-byte units XOR-swizzled against bank conflicts.
//   * The tree tile (n <= 64 nodes) is one more 64-key tile, processed first
//     (in the ring's fourth stage, while the first prefix tiles are in
//     flight), whose keys are the tree nodes rotated on the fly from k_new; a
//     key j is visible to row r iff bit j of anc[node(r)] is set. The
//     workgroup of the last split with rb == 0 also appends the rotated tree
//     keys and raw values to cache slots [P, P+n).
//   * RoPE angles: the host passes theta^(-2d/D) in double precision; the
//     kernel forms pos * inv_freq in double, reduces it to [-pi, pi] and
//     takes a single-precision sincos.
//   * With several splits, each writes (reference score, sum, unnormalised
//     output) to the workspace and a merge kernel combines them.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <type_traits>

#include "tv_device.h"
#include "tv_internal.h"

namespace tv {

namespace {

constexpr int kD = 128;                 // head dim (bf16 path)
constexpr int kKT = 64;                 // keys per LDS stage (= V cache block)
constexpr int kStageElems = kKT * kD;   // bf16 elements of one K (or V) stage
constexpr int kStages = 4;              // LDS ring of prefix tiles (3 in flight)
constexpr int kTableDepths = 16;        // cos/sin rows kept in LDS

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct BfParams {
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_cache;     // [B][Hkv][cap][D]
  uint16_t* v_cache;     // [B][Hkv][cap/64][D][64]
  const int32_t* prefix_len;
  const int32_t* n_nodes;
  const uint64_t* anc;
  const int32_t* depth;
  int32_t* err;
  uint16_t* out;
  float* part_o;     // [B][Hkv][S][rows_pad][D]
  float2* part_ml;   // [B][Hkv][S][rows_pad]  (reference max in log2 units, sum)
  int n_max, Hq, Hkv, G, cap;
  int splits, row_blocks, rows_pad;
  int rope;          // 0: no rotation
  float scale_log2;  // softmax scale * log2(e)
  double inv_freq[kD / 2];
};

// Two floats -> packed bf16 pair (hardware round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint16_t u4_elem(const uint4& v, int t) {
  const uint32_t w = (t < 2) ? v.x : (t < 4) ? v.y : (t < 6) ? v.z : v.w;
  return static_cast<uint16_t>((t & 1) ? (w >> 16) : (w & 0xFFFFu));
}

// Row m of a 32-key score block reads key perm(m): then lane half h holds
// keys 16i + 8h + 0..7 of each 16-key group in accumulator order.
__device__ __forceinline__ int key_perm(int m) {
  return ((m >> 4) << 4) | (((m >> 2) & 1) << 3) | (((m >> 3) & 1) << 2) | (m & 3);
}
// 16-byte unit swizzle of K rows; distinct over the keys 8 lanes read.
__device__ __forceinline__ int k_swz(int key) { return (key & 7) ^ (((key >> 3) & 1) << 2); }
// element offsets in LDS
__device__ __forceinline__ int ks_off(int key, int unit) { return key * kD + ((unit ^ k_swz(key)) << 3); }
__device__ __forceinline__ int vs_off(int d, int unit) { return d * kKT + ((unit ^ (d & 7)) << 3); }
// element offset of (slot, d) in one head's blocked V cache
__device__ __forceinline__ size_t v_cache_off(int slot, int d) {
  return (static_cast<size_t>(slot >> 6) * kD + d) * kKT + (slot & 63);
}

// cos/sin of pos * inv_freq: angle in double precision, reduced to [-pi, pi],
// then single-precision sincos.
__device__ __forceinline__ float2 rope_cs(int pos, double inv_freq) {
  const double ang = static_cast<double>(pos) * inv_freq;
  const double red = fma(-6.283185307179586476925286766559, rint(ang * 0.15915494309189533576888376337251), ang);
  float s, c;
  sincosf(static_cast<float>(red), &s, &c);
  return make_float2(c, s);
}

// max / sum of a value and the value of the lane 32 away (the other half of
// the same query row), on the vector ALU
__device__ __forceinline__ float row_max2(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row_sum2(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Running softmax state of one 32-row query tile.
struct RowState {
  f32x16 o[4];      // O^T accumulator: d = 32 dt + 8 (e>>2) + 4 h + (e&3)
  f32x16 negr;      // -r in every element: the score MFMA's starting accumulator
  float r;          // reference score (log2 units): scores are taken relative to it
  float l;          // this lane's share of the row sum
};

// Softmax of one 32-key score block of one query tile. x holds the scores
// minus the row's reference r (fixed for the pass): no max, no branch.
// Returns the probabilities packed as two B operands (keys 16 half + 8 h +
// 0..7).
template <bool MASKED, bool TREE>
__device__ __forceinline__ void block_softmax(RowState& st, f32x16& x, bf16x8 (&pf)[2], int sub, int h,
                                              int valid_keys, uint64_t anc) {
  if (MASKED) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = 32 * sub + 16 * (e >> 3) + 8 * h + (e & 7);
      const bool vis = TREE ? ((anc >> key) & 1ull) != 0ull : key < valid_keys;
      if (!vis) x[e] = -INFINITY;
    }
  }
  float pe[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) pe[e] = __builtin_amdgcn_exp2f(x[e]);
  uint32_t w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = pack_bf16(pe[2 * j], pe[2 * j + 1]);
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3F803F80u);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    st.l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[j]), ones, st.l, false);
  pf[0] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
  pf[1] = __builtin_bit_cast(bf16x8, make_uint4(w[4], w[5], w[6], w[7]));
}

// One staged 64-key tile times the QT query tiles of a wavefront, in two
// 32-key halves. Each K and V fragment read from LDS feeds QT MFMAs. All
// fragment reads are issued up front and the whole tile is one basic block,
// so the scheduler can overlap one half's exponentials with the other half's
// matrix work.
template <int QT, bool MASKED, bool TREE>
__device__ __forceinline__ void tile_product(RowState (&st)[QT], const uint16_t* __restrict__ ks,
                                             const uint16_t* __restrict__ vs, const bf16x8 (&qf)[QT][8],
                                             const int (&k_addr)[8], const int (&v_addr)[4], int h,
                                             int valid_keys, const uint64_t (&anc)[QT]) {
  f32x16 x[2][QT];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    bf16x8 ka[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) ka[kk] = *reinterpret_cast<const bf16x8*>(ks + k_addr[kk] + sub * 32 * kD);
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      x[sub][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], qf[t][0], st[t].negr, 0, 0, 0);
#pragma unroll
      for (int kk = 1; kk < 8; ++kk)
        x[sub][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], qf[t][kk], x[sub][t], 0, 0, 0);
    }
  }
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    bf16x8 va[8];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int half = 0; half < 2; ++half)
        va[2 * dt + half] = *reinterpret_cast<const bf16x8*>(vs + v_addr[2 * sub + half] + dt * 32 * kKT);
    bf16x8 pf[QT][2];
#pragma unroll
    for (int t = 0; t < QT; ++t) block_softmax<MASKED, TREE>(st[t], x[sub][t], pf[t], sub, h, valid_keys, anc[t]);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int t = 0; t < QT; ++t)
          st[t].o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[2 * dt + half], pf[t][half], st[t].o[dt], 0, 0, 0);
  }
}

// Scores only: raises mx[t] to this lane's max visible score (log2 units) of
// one staged tile. Used by the fallback that finds each row's exact max.
template <int QT, bool MASKED, bool TREE>
__device__ __forceinline__ void tile_max(float (&mx)[QT], const uint16_t* __restrict__ ks, const bf16x8 (&qf)[QT][8],
                                         const int (&k_addr)[8], int h, int valid_keys, const uint64_t (&anc)[QT]) {
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    bf16x8 ka[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) ka[kk] = *reinterpret_cast<const bf16x8*>(ks + k_addr[kk] + sub * 32 * kD);
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      f32x16 x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], qf[t][0], f32x16{}, 0, 0, 0);
#pragma unroll
      for (int kk = 1; kk < 8; ++kk) x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], qf[t][kk], x, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = 32 * sub + 16 * (e >> 3) + 8 * h + (e & 7);
        const bool vis = !MASKED || (TREE ? ((anc[t] >> key) & 1ull) != 0ull : key < valid_keys);
        if (vis) mx[t] = fmaxf(mx[t], x[e]);
      }
    }
  }
}

// Direct global -> LDS copy of 16 bytes per lane: lane i of the wavefront
// writes LDS bytes [lds_base + 16 i, +16). lds_base must be wave-uniform.
__device__ __forceinline__ void load_lds16(const uint16_t* gsrc, uint16_t* lds_base) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)gsrc,
                                   (void __attribute__((address_space(3)))*)lds_base, 16, 0, 0);
}
// Waits until at most N vector memory operations of this wavefront are
// outstanding (N must be a compile-time constant).
template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

template <int WAVES, int QT>
__global__ __launch_bounds__(WAVES * 64) void attn_bf16_kernel(BfParams p) {
  constexpr int NT = WAVES * 64;
  constexpr int ROWS = WAVES * 32 * QT;      // query rows of the workgroup
  constexpr int CPT = (kKT * kD / 8) / NT;   // 16-byte chunks per thread per K (or V) stage
  static_assert(2 * CPT * (kStages - 2) <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kStages * kStageElems];  // (K, V) x stages
  __shared__ float2 cs_table[kTableDepths * 64];
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
  const int rb0 = rb * ROWS;
  const int r0 = rb0 + wave * 32 * QT;       // first row of this wavefront

  if (rb0 >= rows_live) {
    // nothing live in this row block: zero rows (single split) and leave
    if (p.splits == 1) {
      for (int r = rb0 + tid / 16; r < min(rb0 + ROWS, rows_all); r += NT / 16) {
        const int i = r / G, head = g * G + r % G;
        uint16_t* orow = p.out + ((static_cast<size_t>(b) * p.n_max + i) * p.Hq + head) * kD;
        reinterpret_cast<uint4*>(orow)[tid % 16] = make_uint4(0, 0, 0, 0);
      }
    }
    return;
  }

  int my_row[QT];
  bool row_live[QT];
  uint64_t my_anc[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    my_row[t] = r0 + 32 * t + (lane & 31);
    row_live[t] = my_row[t] < rows_live;
    my_anc[t] = row_live[t] ? p.anc[static_cast<size_t>(b) * p.n_max + my_row[t] / G] : 0ull;
  }

  // prefix keys of this split, in whole 64-key tiles
  const int n_tiles_all = (P + kKT - 1) / kKT;
  const int tiles_per_split = (n_tiles_all + p.splits - 1) / p.splits;
  const int k_begin = min(P, s * tiles_per_split * kKT);
  const int k_end = min(P, k_begin + tiles_per_split * kKT);
  const int n_tiles = (k_end - k_begin + kKT - 1) / kKT;
  const bool last_split = (s == p.splits - 1);

  // stage buf: K at smem + 2 buf * kStageElems, V right after it
  auto Ks = [&](int buf) { return smem + 2 * buf * kStageElems; };
  auto Vs = [&](int buf) { return smem + (2 * buf + 1) * kStageElems; };

  const size_t head_off = (static_cast<size_t>(b) * p.Hkv + g) * p.cap * kD;
  const uint16_t* kc = p.k_cache + head_off;
  const uint16_t* vc = p.v_cache + head_off;

  // per-lane LDS offsets of the MFMA operands
  int k_addr[8], v_addr[4];
  {
    const int krow = key_perm(lane & 31);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) k_addr[kk] = ks_off(krow, 2 * kk + h);
    const int d = lane & 31;
#pragma unroll
    for (int u = 0; u < 4; ++u) v_addr[u] = vs_off(d, 2 * u + h);
  }

  // Issues the copy of prefix tile [kt0, kt0+64) into stage `buf`. LDS chunk
  // c (16 bytes) of a stage is K row c/16, position c%16 (unit swizzled by
  // key) and V row c/8, position c%8 (unit swizzled by d); the lane that
  // writes chunk c fetches the matching global chunk. Keys past the prefix
  // are still inside the (64-slot aligned) cache; they are masked later.
  auto issue_tile = [&](int kt0, int buf) {
    const uint16_t* ktile = kc + static_cast<size_t>(kt0) * kD;
    const uint16_t* vtile = vc + static_cast<size_t>(kt0) * kD;   // kt0 is a multiple of 64
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = j * NT + tid;
      const int key = c >> 4, kpos = c & 15;
      load_lds16(ktile + key * kD + ((kpos ^ k_swz(key)) << 3), Ks(buf) + (j * NT + wave * 64) * 8);
      const int d = c >> 3, vpos = c & 7;
      load_lds16(vtile + d * kKT + ((vpos ^ (d & 7)) << 3), Vs(buf) + (j * NT + wave * 64) * 8);
    }
  };

  // ---- 1. start copying the first prefix tiles (overlaps the prologue)
#pragma unroll
  for (int t = 0; t < kStages - 1; ++t)
    if (t < n_tiles) issue_tile(k_begin + t * kKT, t);

  // ---- 2. cos/sin table for the tree's depths (positions P + depth)
  if (wave == 0) {
    int dv = (lane < n) ? p.depth[static_cast<size_t>(b) * p.n_max + lane] : 0;
    dv = wave_max_i32(dv);
    if (lane == 0) s_dmax = dv;
  }
  __syncthreads();
  const int table_rows = min(s_dmax, kTableDepths - 1) + 1;
  for (int idx = tid; idx < table_rows * 64; idx += NT)
    cs_table[idx] = p.rope ? rope_cs(P + (idx >> 6), p.inv_freq[idx & 63]) : make_float2(1.0f, 0.0f);
  __syncthreads();
  auto cs_at = [&](int dep, int pair) -> float2 {
    if (dep < kTableDepths) return cs_table[dep * 64 + pair];
    return p.rope ? rope_cs(P + dep, p.inv_freq[pair]) : make_float2(1.0f, 0.0f);
  };

  // ---- 3. rotated, pre-scaled queries as B operands:
  //         qf[t][kk] = Q[row][16kk + 8h .. +8] * scale * log2(e)
  bf16x8 qf[QT][8];
  const float qs = p.scale_log2;
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    if (row_live[t]) {
      const int node = my_row[t] / G;
      const int head = g * G + my_row[t] % G;
      const int dep = p.depth[static_cast<size_t>(b) * p.n_max + node];
      const uint16_t* qrow = p.q + ((static_cast<size_t>(b) * p.n_max + node) * p.Hq + head) * kD;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int d0 = 16 * s4 + 8 * h;
        const uint4 lo = *reinterpret_cast<const uint4*>(qrow + d0);
        const uint4 hi = *reinterpret_cast<const uint4*>(qrow + 64 + d0);
        uint32_t wl[4], wh[4];
#pragma unroll
        for (int u2 = 0; u2 < 8; u2 += 2) {
          float rl[2], rh[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const float2 cs = cs_at(dep, d0 + u2 + u);
            const float xl = bf16_bits_to_f32(u4_elem(lo, u2 + u));
            const float xh = bf16_bits_to_f32(u4_elem(hi, u2 + u));
            rl[u] = (xl * cs.x - xh * cs.y) * qs;
            rh[u] = (xh * cs.x + xl * cs.y) * qs;
          }
          wl[u2 >> 1] = pack_bf16(rl[0], rl[1]);
          wh[u2 >> 1] = pack_bf16(rh[0], rh[1]);
        }
        qf[t][s4] = __builtin_bit_cast(bf16x8, make_uint4(wl[0], wl[1], wl[2], wl[3]));
        qf[t][s4 + 4] = __builtin_bit_cast(bf16x8, make_uint4(wh[0], wh[1], wh[2], wh[3]));
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) qf[t][kk] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    }
  }

  // ---- 4. reference score per row: the row's score against the tree root,
  // which every node sees. Scores are taken relative to it, so on the fast
  // path no running max is needed.
  float r_root[QT];
  {
    const uint16_t* kr = p.k_new + (static_cast<size_t>(b) * p.n_max * p.Hkv + g) * kD;   // node 0
#pragma unroll
    for (int t = 0; t < QT; ++t) r_root[t] = 0.0f;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int d0 = 16 * s4 + 8 * h;
      const uint4 lo = *reinterpret_cast<const uint4*>(kr + d0);
      const uint4 hi = *reinterpret_cast<const uint4*>(kr + 64 + d0);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float2 cs = cs_at(0, d0 + u);
        const float xl = bf16_bits_to_f32(u4_elem(lo, u));
        const float xh = bf16_bits_to_f32(u4_elem(hi, u));
        // the rotated root key as stored (rounded to bf16)
        const float kl = bf16_bits_to_f32(f32_to_bf16_bits(xl * cs.x - xh * cs.y));
        const float kh = bf16_bits_to_f32(f32_to_bf16_bits(xh * cs.x + xl * cs.y));
#pragma unroll
        for (int t = 0; t < QT; ++t) {
          const uint4 ql = __builtin_bit_cast(uint4, qf[t][s4]);
          const uint4 qh = __builtin_bit_cast(uint4, qf[t][s4 + 4]);
          r_root[t] = fmaf(bf16_bits_to_f32(u4_elem(ql, u)), kl, r_root[t]);
          r_root[t] = fmaf(bf16_bits_to_f32(u4_elem(qh, u)), kh, r_root[t]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < QT; ++t) r_root[t] = row_sum2(r_root[t]);
  }

  RowState st[QT];
  auto reset_state = [&]() {
#pragma unroll
    for (int t = 0; t < QT; ++t) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) st[t].o[dt] = f32x16{};
      st[t].r = r_root[t];
      st[t].negr = f32x16{} - r_root[t];
      st[t].l = 0.0f;
    }
  };
  reset_state();

  // One pass over the tree tile and the prefix tiles; the first kStages - 1
  // prefix tiles must already be in flight. MAX_ONLY passes only raise mx to
  // the row maxima of the scores.
  float mx[QT];
  auto run_pass = [&](auto mode_tag) {
    constexpr bool MAX_ONLY = decltype(mode_tag)::value;
    auto product = [&](auto masked_tag, auto tree_tag, const uint16_t* ks_, const uint16_t* vs_, int valid_) {
      constexpr bool M = decltype(masked_tag)::value, T = decltype(tree_tag)::value;
      if constexpr (MAX_ONLY)
        tile_max<QT, M, T>(mx, ks_, qf, k_addr, h, valid_, my_anc);
      else
        tile_product<QT, M, T>(st, ks_, vs_, qf, k_addr, v_addr, h, valid_, my_anc);
    };
    // ---- 4. tree tile (last split only), in the ring's last stage, which no
    // prefix tile occupies before the first loop iteration: rotate k_new,
    // stage, append to the cache, multiply
    if (last_split) {
      uint16_t* ksT = Ks(kStages - 1);
      uint16_t* vsT = Vs(kStages - 1);
      const size_t new_base = static_cast<size_t>(b) * p.n_max;
      const bool append = (rb == 0);
      for (int it = tid; it < 64 * 8; it += NT) {
        const int a = it >> 3, c = it & 7;
        uint4 lo_o = make_uint4(0, 0, 0, 0), hi_o = make_uint4(0, 0, 0, 0);
        if (a < n) {
          const uint16_t* kr = p.k_new + ((new_base + a) * p.Hkv + g) * kD;
          const uint4 lo = *reinterpret_cast<const uint4*>(kr + 8 * c);
          const uint4 hi = *reinterpret_cast<const uint4*>(kr + 64 + 8 * c);
          const int dep = p.depth[new_base + a];
          uint32_t wl[4], wh[4];
  #pragma unroll
          for (int u2 = 0; u2 < 8; u2 += 2) {
            float rl[2], rh[2];
  #pragma unroll
            for (int u = 0; u < 2; ++u) {
              const float2 cs = cs_at(dep, 8 * c + u2 + u);
              const float xl = bf16_bits_to_f32(u4_elem(lo, u2 + u));
              const float xh = bf16_bits_to_f32(u4_elem(hi, u2 + u));
              rl[u] = xl * cs.x - xh * cs.y;
              rh[u] = xh * cs.x + xl * cs.y;
            }
            wl[u2 >> 1] = pack_bf16(rl[0], rl[1]);
            wh[u2 >> 1] = pack_bf16(rh[0], rh[1]);
          }
          lo_o = make_uint4(wl[0], wl[1], wl[2], wl[3]);
          hi_o = make_uint4(wh[0], wh[1], wh[2], wh[3]);
          if (append) {
            uint16_t* kdst = p.k_cache + head_off + static_cast<size_t>(P + a) * kD;
            *reinterpret_cast<uint4*>(kdst + 8 * c) = lo_o;
            *reinterpret_cast<uint4*>(kdst + 64 + 8 * c) = hi_o;
          }
        }
        *reinterpret_cast<uint4*>(ksT + ks_off(a, c)) = lo_o;
        *reinterpret_cast<uint4*>(ksT + ks_off(a, c + 8)) = hi_o;
      }
      // V: lane <-> node, so the appends of one head dim are consecutive slots
      for (int it = tid; it < 64 * 16; it += NT) {
        const int a = it & 63, c = it >> 6;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (a < n) v = *reinterpret_cast<const uint4*>(p.v_new + ((new_base + a) * p.Hkv + g) * kD + 8 * c);
  #pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int d = 8 * c + u;
          const uint16_t e = u4_elem(v, u);
          vsT[vs_off(d, a >> 3) + (a & 7)] = e;
          if (append && a < n) p.v_cache[head_off + v_cache_off(P + a, d)] = e;
        }
      }
      __syncthreads();
      product(std::true_type{}, std::true_type{}, ksT, vsT, kKT);
    }

    // ---- 5. prefix tiles: a ring of kStages LDS stages, kStages - 1 tiles in
    // flight; tile t lives in stage t % kStages. The steady-state loop only sees
    // full tiles with kStages - 2 later tiles outstanding, so it is one straight
    // block; the last kStages - 1 tiles (the drain, and a partial last tile) are
    // peeled off below. Wavefronts whose rows are all padding compute on zero
    // queries rather than branch around the products.
    int t = 0;
    for (; t + kStages - 1 < n_tiles; ++t) {
      const int cur = t % kStages;
      wait_vm<2 * CPT * (kStages - 2)>();
      __syncthreads();   // tile t has landed for every wave; stage (t-1) % kStages is free
      issue_tile(k_begin + (t + kStages - 1) * kKT, (t + kStages - 1) % kStages);
      product(std::false_type{}, std::false_type{}, Ks(cur), Vs(cur), kKT);
    }
    for (; t < n_tiles; ++t) {
      const int cur = t % kStages;
      const int later = n_tiles - 1 - t;
      static_assert(kStages == 4, "drain waits below assume four stages");
      if (later >= 2) wait_vm<2 * CPT * 2>();
      else if (later == 1) wait_vm<2 * CPT>();
      else wait_vm<0>();
      __syncthreads();
      const int valid = min(kKT, k_end - (k_begin + t * kKT));
      if (valid == kKT) {
        product(std::false_type{}, std::false_type{}, Ks(cur), Vs(cur), kKT);
      } else {
        // stale slots past the prefix may hold anything: zero their V
        for (int idx = tid; idx < (kKT - valid) * kD; idx += NT) {
          const int key = valid + idx / kD, d = idx % kD;
          Vs(cur)[vs_off(d, key >> 3) + (key & 7)] = 0;
        }
        __syncthreads();
        product(std::true_type{}, std::false_type{}, Ks(cur), Vs(cur), valid);
      }
    }

  };

  run_pass(std::false_type{});
  // A row whose scores rose far above its root score (p > 2^62) would lose
  // precision or overflow on that reference: find every row's exact max in a
  // scores-only pass, then redo the pass with r = max (all p <= 1).
  int overflow = 0;
#pragma unroll
  for (int t = 0; t < QT; ++t) overflow |= row_live[t] && !(row_sum2(st[t].l) <= 0x1p62f);
  if (__syncthreads_or(overflow)) {
#pragma unroll
    for (int t = 0; t < QT; ++t) mx[t] = -INFINITY;
#pragma unroll
    for (int t = 0; t < kStages - 1; ++t)
      if (t < n_tiles) issue_tile(k_begin + t * kKT, t);
    run_pass(std::true_type{});
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const float m = row_max2(mx[t]);
      r_root[t] = (m == -INFINITY) ? r_root[t] : m;
    }
    reset_state();
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kStages - 1; ++t)
      if (t < n_tiles) issue_tile(k_begin + t * kKT, t);
    run_pass(std::false_type{});
  }

  // ---- 6. epilogue
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const float l_tot = row_sum2(st[t].l);
    const int row = my_row[t];
    if (p.splits == 1) {
      if (row < rows_all) {
        const int head = g * G + row % G;
        const int node = row / G;
        uint16_t* orow = p.out + ((static_cast<size_t>(b) * p.n_max + node) * p.Hq + head) * kD;
        const float inv = (row_live[t] && l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int d0 = 32 * dt + 8 * i4 + 4 * h;
            uint2 w;
            w.x = pack_bf16(st[t].o[dt][4 * i4 + 0] * inv, st[t].o[dt][4 * i4 + 1] * inv);
            w.y = pack_bf16(st[t].o[dt][4 * i4 + 2] * inv, st[t].o[dt][4 * i4 + 3] * inv);
            *reinterpret_cast<uint2*>(orow + d0) = w;
          }
      }
    } else {
      const size_t prow = ((static_cast<size_t>(b) * p.Hkv + g) * p.splits + s) * p.rows_pad + row;
      float* po = p.part_o + prow * kD;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = 32 * dt + 8 * i4 + 4 * h;
          *reinterpret_cast<float4*>(po + d0) = make_float4(st[t].o[dt][4 * i4 + 0], st[t].o[dt][4 * i4 + 1],
                                                            st[t].o[dt][4 * i4 + 2], st[t].o[dt][4 * i4 + 3]);
        }
      if (h == 0) p.part_ml[prow] = make_float2(st[t].r, l_tot);
    }
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
  reinterpret_cast<uint32_t*>(orow)[lane] = pack_bf16(o0, o1);
}

// Optional launch-shape override for tuning sweeps, read once:
// TV_ATTN_TUNE="waves=4,qt=2,splits=4" (any subset; 0 = automatic).
struct Tune { int waves = 0, qt = 0, splits = 0; };
const Tune& tune() {
  static const Tune t = [] {
    Tune r;
    if (const char* e = getenv("TV_ATTN_TUNE")) {
      if (const char* w = strstr(e, "waves=")) sscanf(w, "waves=%d", &r.waves);
      if (const char* q = strstr(e, "qt=")) sscanf(q, "qt=%d", &r.qt);
      if (const char* s = strstr(e, "splits=")) sscanf(s, "splits=%d", &r.splits);
    }
    return r;
  }();
  return t;
}

}  // namespace

AttnPlan plan_attention_bf16(const tv_attn_args* a) {
  AttnPlan pl;
  const int G = a->Hq / a->Hkv;
  const int rows = G * a->n_max;
  // 64 query rows (two 32-row tiles) per wavefront, so each K and V fragment
  // read from LDS feeds two MFMAs, and up to four wavefronts (one per SIMD,
  // 512 registers each) per workgroup; small row counts use 32-row tiles.
  pl.qt = rows > 128 ? 2 : 1;
  pl.waves = (pl.qt == 2 || rows > 64) ? 4 : 2;
  const Tune& tn = tune();
  if (tn.qt == 1 || tn.qt == 2) pl.qt = tn.qt;
  if (tn.waves == 2 || tn.waves == 4) pl.waves = tn.waves;
  if (pl.qt == 2) pl.waves = 4;
  const int wg_rows = pl.waves * 32 * pl.qt;
  pl.row_blocks = (rows + wg_rows - 1) / wg_rows;
  const long units = static_cast<long>(a->B) * a->Hkv * pl.row_blocks;
  // Split the prefix until the grid covers the 256 compute units, keeping at
  // least four 64-key tiles per split. The prefix length lives on the device,
  // so the cache capacity bounds it here.
  const int max_tiles = (a->cap + kKT - 1) / kKT;
  int splits = 1;
  while (units * splits < 256 && (max_tiles / (splits * 2)) >= 4) splits *= 2;
  if (tn.splits > 0) splits = std::min(tn.splits, std::max(1, max_tiles));
  pl.splits = splits;
  pl.rows_pad = pl.row_blocks * wg_rows;
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
  p.rope = a->rope_theta != 0.0f;
  for (int d = 0; d < kD / 2; ++d)
    p.inv_freq[d] = p.rope ? pow(static_cast<double>(a->rope_theta), -2.0 * d / kD) : 0.0;
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
  const int key = pl.waves * 10 + pl.qt;
  switch (key) {
    case 21: hipLaunchKernelGGL((attn_bf16_kernel<2, 1>), grid, dim3(128), 0, s, p); break;
    case 41: hipLaunchKernelGGL((attn_bf16_kernel<4, 1>), grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((attn_bf16_kernel<4, 2>), grid, dim3(256), 0, s, p); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.splits == 1) return e;
  dim3 mgrid((p.G * p.n_max + 3) / 4, a->Hkv, a->B);
  hipLaunchKernelGGL(merge_bf16_kernel, mgrid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace tv
