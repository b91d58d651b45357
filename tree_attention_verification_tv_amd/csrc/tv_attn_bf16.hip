// bf16 tree-verification attention on CDNA4 matrix cores (gfx950).
//
// What is computed (infra-guide "5.3 Medusa、EAGLE 与 MTP", sections 3.1 and
// 3.2; pofe.ai "Medusa and EAGLE ...", "Trees"): every node i of a flattened
// draft tree attends to the P prefix keys of its KV head and to the keys of
// its ancestors-or-self, with query and tree keys rotated at position
// P + depth. Siblings and other branches are masked out by the node's
// ancestor bitmask.
//
// How (this file's design, not the pages'): two kernels on one stream.
//
//   main   workgroup = (row block rb, KV split s) of (sequence b, KV head g).
//          Its query rows are the G query heads of g for every tree node,
//          node-major (row = node * G + head_in_group); each wavefront owns
//          QT tiles of 32 rows, so every K or V fragment read from LDS feeds
//          QT MFMAs. The keys of b are slots [0, P + n) of the cache: the
//          prefix, then the tree, cut into 64-key tiles that the splits share
//          out. Tiles are copied straight into LDS (global_load_lds into a
//          ring of five stages, three tiles in flight), so the copies cost no
//          registers and no LDS writes. The copies are issued from inline
//          assembly: the compiler then does not see an LDS write it cannot
//          tell apart from the fragment reads, and does not drain every copy
//          in flight before each tile; the kernel waits for exactly the tile
//          it needs (s_waitcnt vmcnt) and a barrier. A tile's copy goes out
//          in parts between the MFMAs of the tile product before it.
//
//          While the first tiles are in flight, the workgroup builds a table
//          of RoPE (cos, sin) for the depths 0 .. deepest node in LDS, and
//          each lane rotates its query rows at P + depth, scales them by
//          softmax_scale * log2(e) and rounds them to bf16 in the register
//          order of the score MFMA's B operand. A split takes its tiles in
//          descending order, so the one or two tiles that reach past P come
//          first; there the tree's keys, rotated the same way, and its values
//          are written into the LDS stage straight from k_new / v_new.
//
//          Scores are computed transposed, S^T = K Q^T, with
//          v_mfma_f32_32x32x16_bf16: a lane then holds 16 keys of ONE query
//          row, so row reductions are lane-local plus one v_permlane32_swap.
//          The output is also transposed, O^T = V^T P^T, so probabilities go
//          from the score accumulator straight into the B operand. Softmax
//          is invariant to a per-row shift, and fp32 / bf16 hold 2^s for
//          scores s in log2 units far beyond any usual range, so the fast
//          pass takes p = exp2(s) with no running max, no shift and no
//          branch in the tile loop. A row whose sum left [2^-60, 2^62] is
//          caught at the end; the workgroup then finds every row's exact max
//          in a scores-only pass and redoes the pass with p = exp2(s - max)
//          (exact for any score range). Row sums add up the fp32
//          probabilities (the PV product weights their bf16 roundings).
//
//          The score MFMA reads K rows in a permuted order (row m of a 32-key
//          block is key perm(m)), so each lane half holds 8 CONSECUTIVE keys
//          per 16-key group: the probabilities then match the V tile in
//          natural key order. V is cached tile-blocked and d-major
//          ([cap/64][D][64]), so a 64-key V tile is one contiguous 16 KB block
//          whose rows (one per head dim) are exactly the A operand of the PV
//          product. K rows and V rows sit in LDS with 16-byte units
//          XOR-swizzled against bank conflicts.
//
//          Only the last one or two tiles of b reach past the prefix: there a
//          key j >= P is visible to a row iff bit j - P of its node's
//          ancestor mask is set, and value rows past P + n are zeroed.
//
//   merge  with several splits, each writes (reference, row sum) in fp32
//          and its output divided by the row sum in 16 bits (fp16, or bf16
//          for a row beyond fp16's range) to the workspace in register order;
//          the merge (inside this kernel when the grid runs at once, else a
//          kernel of its own) combines them in split order (deterministic)
//          with fp32 weights and sums and writes the rows.
//   append row block 0 of the split holding the tree tiles appends the tree
//          to cache slots P + i (the keys as rotated for the tiles, the raw
//          values) after its last tile: no workgroup of the call reads those
//          slots back, and stores issued between the tile copies would
//          delay every later wait for a tile.
//
// RoPE angles: a table entry forms pos * 2^(-2j/D log2 theta) in double
// precision, reduces it to [-pi, pi] and takes a single-precision sincos.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "tv_attn_waits.h"
#include "tv_device.h"
#include "tv_internal.h"

namespace tv {

namespace {

constexpr int kD = 128;                 // head dim (bf16 path)
constexpr int kKT = 64;                 // keys per LDS stage (= V cache block)
constexpr int kStageElems = kKT * kD;   // bf16 elements of one K (or V) stage
constexpr int kStages = 5;              // LDS ring of key tiles
constexpr int kAhead = waits::kAhead;   // tiles in flight
static_assert(waits::kKeys == 64 && waits::kDim == 128, "the wait model counts this kernel's tiles");
constexpr int kMaxSplits = 16;          // key splits per row block
constexpr int kCsElems = 64 * 64 * 4;   // bf16 units of the RoPE table: 64 depths x 64 (cos, sin) = one stage

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Division by a launch constant d without the divide sequence (about 25
// instructions): q = umulhi(x, m) with m = ceil(2^32 / d), exact whenever
// x * d <= 2^32 (write x = q d + f: x m / 2^32 = q + f / d + x e / (d 2^32)
// with 0 <= e < d, below q + 1 as long as x e < 2^32). For d = 1, m = 0
// and id = ~0 pass x through (no branch). DivU is used where the operands are
// bounded so (query rows by the group size: the group is at most
// kMaxGroup); DivUs, for the workgroup index, falls back to dividing when
// the host finds the bound broken.
struct DivU {
  uint32_t d, m, id;
  __device__ __forceinline__ uint32_t div(uint32_t x) const { return __umulhi(x, m) | (x & id); }
};
struct DivUs {
  uint32_t d, m, id, slow;
  __device__ __forceinline__ uint32_t div(uint32_t x) const {
    if (slow) return x / d;
    return __umulhi(x, m) | (x & id);
  }
};

struct BfParams {
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_cache;     // [B][Hkv][cap][D]
  uint16_t* v_cache;     // [B][Hkv][cap/64][D][64]
  const int32_t* prefix_len;
  const int32_t* n_nodes;
  uint64_t* anc;   // (outputs when parents is set)
  int32_t* depth;
  int32_t* err;
  const int32_t* parents;   // non-null: the kernel builds the tree itself and writes anc, depth, err
  uint16_t* out;
  uint4* part_o;     // split partials, 16-bit, register order (see the main epilogue)
  float2* part_ml;   // split (reference, row sum) per lane
  int n_max, Hq, Hkv, G, cap;
  int splits, row_blocks;
  DivU gdiv;        // by G (query rows -> node, head)
  DivUs ph_div, rb_div, kv_div;   // by row_blocks * splits, row_blocks, Hkv (the workgroup index)
  float scale_log2;  // softmax scale * log2(e)
  int rope;          // 0: no rotation
  double log2_theta; // log2 of the RoPE base
  // paged cache (block_table non-null): k_cache / v_cache are pools of
  // pages [num_pages][Hkv][64][D] / [num_pages][Hkv][D][64], and 64-slot block
  // j of sequence b is page block_table[b * max_pages + j]; cap = 64 max_pages
  const int32_t* block_table;
  int max_pages, num_pages;
  // fused split merge (see merge_in_kernel): the partials are published with
  // agent-coherent stores and merged by the workgroups themselves; sync holds
  // four words per (sequence, KV head, row block), zero between calls.
  // 0: no fused merge; 1: every split merges its range (waiting, bounded,
  // for the others); 2: the last split to arrive merges every range
  int fused;
  // the bounded wait of the fused merge, in ticks of the 100 MHz real-time
  // clock (the launch-plan override can shorten it, down to one look at the
  // arrival count, so that the path in which a split leaves its range to the
  // last arrival runs)
  uint32_t spin_ticks;
  uint32_t* sync;
  size_t ws_bytes;   // workspace bytes (buffer-resource range of the partials)
};

// Two floats -> packed bf16 pair (hardware round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// Two floats -> packed fp16 pair (round to nearest even), and back.
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}
__device__ __forceinline__ f32x2 unpack_f16(uint32_t w) {
  return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
}

__device__ __forceinline__ uint16_t u4_elem(const uint4& v, int t) {
  const uint32_t w = (t < 2) ? v.x : (t < 4) ? v.y : (t < 6) ? v.z : v.w;
  return static_cast<uint16_t>((t & 1) ? (w >> 16) : (w & 0xFFFFu));
}
__device__ __forceinline__ uint32_t u4_word(const uint4& v, int t) {
  return (t == 0) ? v.x : (t == 1) ? v.y : (t == 2) ? v.z : v.w;
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

// cos/sin of pos * inv_freq: angle in double precision, reduced to [-pi, pi],
// then single-precision sincos.
__device__ __forceinline__ float2 rope_cs(int pos, double inv_freq) {
  const double ang = static_cast<double>(pos) * inv_freq;
  const double red = fma(-6.283185307179586476925286766559, rint(ang * 0.15915494309189533576888376337251), ang);
  float s, c;
  sincosf(static_cast<float>(red), &s, &c);
  return make_float2(c, s);
}

// Depths index the RoPE table; out-of-range values are clamped to its rows.
static_assert(kCsElems == TV_MAX_NODES_DEV * (kD / 2) * 4, "one table row per possible depth");
__device__ __forceinline__ int clamp_depth(int d) { return min(max(d, 0), TV_MAX_NODES_DEV - 1); }

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

// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// Agent-coherent access to the split partials (the sc1 cache policy: the
// store is performed where every compute unit of the device sees it, and the
// load reads from there), through a buffer resource over the workspace. The
// accesses are compiler-tracked (no inline assembly), so the waits for the
// loads are the compiler's.
constexpr int kCoherent = 16;   // cache-policy operand: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(const void* base, size_t bytes) {
  const int n = static_cast<int>(bytes < 0x7fffffffull ? bytes : 0x7fffffffull);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

// Direct global -> LDS copy of 16 bytes per lane: lane i reads base + voff
// and writes LDS bytes [lds + 16 i, +16). base and lds are wave-uniform.
// Issued from assembly, so the compiler neither tracks it (the kernel waits
// for it explicitly) nor treats later LDS reads as dependent on it.
__device__ __forceinline__ void dma16(const uint16_t* base, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}
// Register loads issued from assembly: the compiler neither counts nor waits
// for them (it would otherwise wait for every tile copy issued after them, as
// it does not count those either). The kernel issues them before the tile
// copies, waits for the copies' count (s_waitcnt vmcnt), and then passes each
// value through landed(), which re-defines it after that wait, so no use can
// be scheduled above it.
__device__ __forceinline__ u32x4 ld_b128(const void* a) {
  u32x4 v;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=&v"(v) : "v"(a) : "memory");
  return v;
}
__device__ __forceinline__ uint32_t ld_b32(const void* a) {
  uint32_t v;
  asm volatile("global_load_dword %0, %1, off" : "=&v"(v) : "v"(a) : "memory");
  return v;
}
__device__ __forceinline__ uint64_t ld_b64(const void* a) {
  uint64_t v;
  asm volatile("global_load_dwordx2 %0, %1, off" : "=&v"(v) : "v"(a) : "memory");
  return v;
}
template <typename T>
__device__ __forceinline__ void landed(T& v) { asm volatile("" : "+v"(v)); }
// Waits until at most N vector memory operations of this wavefront are
// outstanding (N must be a compile-time constant).
template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
// Keeps a value's registers allocated (unmodified) up to this point.
__device__ __forceinline__ void keep_live(const bf16x8& v) { asm volatile("" ::"v"(__builtin_bit_cast(u32x4, v))); }
// Forces a loaded value to have arrived here (the compiler inserts the wait).
__device__ __forceinline__ void touch(const bf16x8& v) { asm volatile("" ::"v"(__builtin_bit_cast(u32x4, v))); }
__device__ __forceinline__ void touch(uint64_t v) { asm volatile("" ::"v"(v)); }
__device__ __forceinline__ void touch(float v) { asm volatile("" ::"v"(v)); }

// Sequence status shared by the three kernels: skipped (earlier error, empty
// or oversized tree) or over the cache capacity.
struct SeqState {
  int n, P;
  bool cap_bad, skip;
};
__device__ __forceinline__ SeqState make_seq_state(const BfParams& p, int n, int P, int e_in) {
  SeqState q;
  q.n = n;
  q.P = P;
  q.cap_bad = (e_in == 0) && (q.n > 0) && (q.n <= p.n_max) && (q.P < 0 || q.P + q.n > p.cap);
  q.skip = (e_in != 0) || (q.n <= 0) || (q.n > p.n_max) || q.cap_bad;
  return q;
}
__device__ __forceinline__ SeqState seq_state(const BfParams& p, int b) {
  return make_seq_state(p, p.n_nodes[b], p.prefix_len[b], p.err[b]);
}
// The same, with the three words loaded together by scalar loads and one
// wait (the compiler would otherwise wait between them); b is uniform over
// the workgroup, so the addresses are read from the first lane into scalar
// registers.
__device__ __forceinline__ const int* uniform_ptr(const int* a) {
  const uint64_t v = reinterpret_cast<uint64_t>(a);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const int*>((static_cast<uint64_t>(hi) << 32) | lo);
}
// (node count and prefix length only: a kernel that builds the tree itself
// has no error word to read)
__device__ __forceinline__ SeqState seq_state_scalar_ne(const BfParams& p, int b) {
  int n, P;
  asm volatile(
      "s_load_dword %0, %2, 0x0\n\t"
      "s_load_dword %1, %3, 0x0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(n), "=&s"(P)
      : "s"(uniform_ptr(p.n_nodes + b)), "s"(uniform_ptr(p.prefix_len + b))
      : "memory");
  return make_seq_state(p, n, P, 0);
}
__device__ __forceinline__ SeqState seq_state_scalar(const BfParams& p, int b) {
  int n, P, e;
  asm volatile(
      "s_load_dword %0, %3, 0x0\n\t"
      "s_load_dword %1, %4, 0x0\n\t"
      "s_load_dword %2, %5, 0x0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(n), "=&s"(P), "=&s"(e)
      : "s"(uniform_ptr(p.n_nodes + b)), "s"(uniform_ptr(p.prefix_len + b)), "s"(uniform_ptr(p.err + b))
      : "memory");
  return make_seq_state(p, n, P, e);
}

// Rotate-half RoPE of one dimension pair (x_lo, x_hi) by the angle whose
// (cos, sin) is cs, in one fixed rounding order (the cache append repeats it
// bit for bit).
__device__ __forceinline__ float rope_lo(float xl, float xh, float2 cs) { return fmaf(xl, cs.x, -(xh * cs.y)); }
__device__ __forceinline__ float rope_hi(float xl, float xh, float2 cs) { return fmaf(xh, cs.x, xl * cs.y); }
// RoPE frequency of pair j: theta^(-2j/D), as 2^(-2j/D log2 theta).
__device__ __forceinline__ double rope_freq(double log2_theta, int j) { return exp2(log2_theta * (-2.0 * j / kD)); }

// Rotate-half RoPE of 8 dimension pairs: lo[e] and hi[e] are dims d + e and
// d + 64 + e, cs[e] the (cos, sin) of their angle. Results are multiplied by
// scale and rounded to bf16.
__device__ __forceinline__ void rope8(const uint4& lo, const uint4& hi, const float2* cs, float scale,
                                      uint4& lo_out, uint4& hi_out) {
  uint32_t wl[4], wh[4];
#pragma unroll
  for (int u2 = 0; u2 < 4; ++u2) {
    float rl[2], rh[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float2 cn = cs[2 * u2 + u];
      const float xl = bf16_bits_to_f32(u4_elem(lo, 2 * u2 + u));
      const float xh = bf16_bits_to_f32(u4_elem(hi, 2 * u2 + u));
      rl[u] = rope_lo(xl, xh, cn) * scale;
      rh[u] = rope_hi(xl, xh, cn) * scale;
    }
    wl[u2] = pack_bf16(rl[0], rl[1]);
    wh[u2] = pack_bf16(rh[0], rh[1]);
  }
  lo_out = make_uint4(wl[0], wl[1], wl[2], wl[3]);
  hi_out = make_uint4(wh[0], wh[1], wh[2], wh[3]);
}

// ---------------------------------------------------------------------------
// main: grid (splits * row_blocks * Hkv * B), WAVES * 64 threads
// ---------------------------------------------------------------------------

// Running softmax state of one 32-row query tile.
struct RowState {
  f32x16 o[4];      // O^T accumulator: d = 32 dt + 8 (e>>2) + 4 h + (e&3)
  float r;          // reference score (log2 units): p = exp2(s - r)
  float l;          // this lane's share of the row sum
};

// Key j of a tile is visible to a row iff j < P, or bit j - P of the row's
// ancestor mask is set; rel = j - P.
__device__ __forceinline__ bool key_visible(int rel, uint64_t anc) {
  return rel < 0 || (rel < 64 && ((anc >> rel) & 1ull) != 0ull);
}

// Score MFMAs with the accumulator in vector registers. The accumulation
// registers hold the output (128 per wavefront), so scores that the vector
// ALU must read would otherwise be shuttled between the two register files;
// issuing these from assembly pins the vector-register form. The compiler
// does not see them as MFMAs, so hazard_wait() must separate the last one
// writing a score block from the first vector-ALU read of it.
// The B operand (the queries, constant over the whole kernel) is read from
// accumulation registers, which keeps 16 x QT vector registers free.
__device__ __forceinline__ f32x16 mfma_s_first(const bf16x8& a, const bf16x8& b) {
  f32x16 d;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
               : "=&v"(d)
               : "v"(__builtin_bit_cast(u32x4, a)), "a"(__builtin_bit_cast(u32x4, b)));
  return d;
}
__device__ __forceinline__ void mfma_s_acc(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
               : "+v"(d)
               : "v"(__builtin_bit_cast(u32x4, a)), "a"(__builtin_bit_cast(u32x4, b)));
}
// 12 wait states: the distance the compiler itself keeps between this
// matrix instruction writing vector registers and a vector-ALU read of them.
// The score blocks pass through the statement, so no read of them can be
// scheduled above it.
template <int QT>
__device__ __forceinline__ void hazard_wait(f32x16 (&x)[QT]) {
  if constexpr (QT == 1)
    asm volatile("s_nop 11" : "+v"(x[0]));
  else
    asm volatile("s_nop 11" : "+v"(x[0]), "+v"(x[1]));
}

// Probabilities of elements 2c, 2c+1 of a 32-key score block (masked to 0
// where invisible): exp2 of the score (minus the row's reference r on the
// fallback pass; the fast pass takes r = 0), packed to bf16, and added to the
// lane's row sum.
// (In two halves, so that a pipelined step can put the exponentials behind
// one MFMA and the rest behind the next.)
// vis: the row's visibility bits for the tile's keys, shifted down by the
// lane half's 8-key offset (see tile_visibility), so that the bit of each
// element sits at a constant position.
template <bool MASKED, bool SHIFT>
__device__ __forceinline__ f32x2 prob_exp(const RowState& st, const f32x16& x, int c, int sub, uint64_t vis) {
  float a = SHIFT ? x[2 * c] - st.r : x[2 * c], b = SHIFT ? x[2 * c + 1] - st.r : x[2 * c + 1];
  if (MASKED) {
    const int key = 32 * sub + 16 * ((2 * c) >> 3) + ((2 * c) & 7);   // (+ 8h, folded into vis)
    if (((vis >> key) & 1ull) == 0ull) a = -INFINITY;
    if (((vis >> (key + 1)) & 1ull) == 0ull) b = -INFINITY;
  }
  return f32x2{__builtin_amdgcn_exp2f(a), __builtin_amdgcn_exp2f(b)};
}
// Bit k of the result: is key k of the tile starting at key P + rel0
// visible to the row with ancestor mask anc (key_visible for k = 0 .. 63),
// shifted down by 8h. A tile with tree keys has -64 < rel0 < 64.
__device__ __forceinline__ uint64_t tile_visibility(int rel0, uint64_t anc, int h) {
  const uint64_t v = rel0 >= 0 ? anc >> rel0 : (anc << -rel0) | ((1ull << -rel0) - 1ull);
  return v >> (8 * h);
}
// The row sum adds the fp32 probabilities before their rounding to bf16:
// two adds per pair (the rounded halves would cost two more instructions
// to unpack, and the wavefront's issue, not the matrix cores, bounds the
// pipelined step). The rounding is to nearest, unbiased, so the sum of the
// rounded weights differs from this one by about 2^-9 / sqrt(keys) of it.
__device__ __forceinline__ uint32_t prob_pack(RowState& st, f32x2 e) {
  st.l += e[0] + e[1];
  return pack_bf16(e[0], e[1]);
}
template <bool MASKED, bool SHIFT>
__device__ __forceinline__ uint32_t prob_pair(RowState& st, const f32x16& x, int c, int sub, uint64_t vis) {
  return prob_pack(st, prob_exp<MASKED, SHIFT>(st, x, c, sub, vis));
}

// One staged 64-key tile times the QT query tiles of a wavefront, as 32
// steps of QT MFMAs each, software-pipelined so that the matrix cores always
// have work while the vector ALU computes probabilities:
//   steps  0- 7  S(half 0)
//   steps  8-15  S(half 1)   + softmax of half 0, two elements per step
//   steps 16-23  PV(half 0)  + softmax of half 1
//   steps 24-31  PV(half 1)
// Step i consumes LDS fragment i (K rows, then V rows) and issues the read
// of fragment i + kLook, so few fragments are live at once. Each fragment
// feeds QT MFMAs. sched_barrier pins the order (the scheduler would
// otherwise group like instructions and hoist every read). copy(j), j < 8,
// issues slot j of a later tile's copy; it is called in the even steps that
// carry no vector-ALU work (0-6, 24-30), where its issue overlaps the
// matrix cores.
constexpr int kLook = 4;
struct NoCopy {
  __device__ __forceinline__ void operator()(int) const {}
};
template <int QT, bool MASKED, bool SHIFT, typename Copy>
__device__ __forceinline__ void tile_product(RowState (&st)[QT], const uint16_t* __restrict__ ks,
                                             const uint16_t* __restrict__ vs, const bf16x8 (&qf)[QT][8],
                                             const int (&k_addr)[8], const int (&v_addr)[4], int h, int rel0,
                                             const uint64_t (&anc)[QT], const Copy& copy) {
  auto frag_ptr = [&](int i) -> const bf16x8* {
    if (i < 16) return reinterpret_cast<const bf16x8*>(ks + k_addr[i & 7] + (i >> 3) * 32 * kD);
    const int j = (i - 16) & 7, sub = (i - 16) >> 3;
    return reinterpret_cast<const bf16x8*>(vs + v_addr[2 * sub + (j & 1)] + (j >> 1) * 32 * kKT);
  };
  bf16x8 fr[32];
  f32x16 x[2][QT];
  uint32_t w[2][QT][8];
  uint64_t vis[QT];
  bf16x8 pv_b[QT], pv_prev[QT];   // B operands of this and the previous step's PV MFMAs
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    vis[t] = MASKED ? tile_visibility(rel0, anc[t], h) : 0ull;
    pv_b[t] = pv_prev[t] = bf16x8{};
  }
#pragma unroll
  for (int i = 0; i < kLook; ++i) fr[i] = *frag_ptr(i);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const bool soft = i >= 8 && i < 24;
    const int ssub = (i - 8) >> 3, c = (i - 8) & 7;
    if (soft && c == 0) hazard_wait<QT>(x[ssub]);
    // An in-order wavefront cannot issue past an MFMA that waits for the
    // matrix pipe, so each MFMA is followed by its own share of vector work
    // rather than by the next MFMA.
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      if (i < 16) {
        const int sub = i >> 3, kk = i & 7;
        if (kk == 0)
          x[sub][t] = mfma_s_first(fr[i], qf[t][kk]);
        else
          mfma_s_acc(x[sub][t], fr[i], qf[t][kk]);
      } else {
        const int sub = (i - 16) >> 3, j = (i - 16) & 7, dt = j >> 1, half = j & 1;
        const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(w[sub][t][4 * half], w[sub][t][4 * half + 1],
                                                               w[sub][t][4 * half + 2], w[sub][t][4 * half + 3]));
        st[t].o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i], pf, st[t].o[dt], 0, 0, 0);
        pv_b[t] = pf;
      }
      __builtin_amdgcn_sched_barrier(0);
      if (t == 0 && i + kLook < 32) fr[i + kLook] = *frag_ptr(i + kLook);   // behind the step's first MFMA
      if (soft) w[ssub][t][c] = prob_pair<MASKED, SHIFT>(st[t], x[ssub][t], c, ssub, vis[t]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if ((i & 1) == 0 && (i < 8 || i >= 24)) {
      copy(i < 8 ? i / 2 : 4 + (i - 24) / 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    // operands stay allocated one step past their last read (as in pipe_iter)
    keep_live(fr[i]);
    if (i > 0) keep_live(fr[i - 1]);
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      if (i > 16) keep_live(pv_prev[t]);
      if (i >= 16) pv_prev[t] = pv_b[t];
    }
  }
}

// Cross-tile software pipeline for tiles without masked keys. Iteration t
// issues four blocks of eight steps (QT MFMAs each), each carrying one
// probability pair per step on the vector ALU:
//   A  S half 0 of tile t         probabilities of tile t-1, half 1, pairs 4-7
//   B  PV half 1 of tile t-1      probabilities of tile t,   half 0, pairs 0-3
//   C  S half 1 of tile t         probabilities of tile t,   half 0, pairs 4-7
//   D  PV half 0 of tile t        probabilities of tile t,   half 1, pairs 0-3
// so no step waits on the vector ALU alone; tile t-1's values are read one
// iteration after its keys. Without a previous tile (PREV false) block B has
// no MFMAs and block A no probabilities; pipe_tail finishes the last tile.
// Fragments are read kLook steps ahead, as in tile_product; copy slots go
// out every fourth step.
template <int QT, bool SHIFT, bool PREV, typename Copy>
__device__ __forceinline__ void pipe_iter(RowState (&st)[QT], f32x16 (&x)[2][QT], uint32_t (&w)[2][QT][8],
                                          const uint16_t* __restrict__ ks, const uint16_t* __restrict__ vs,
                                          const uint16_t* __restrict__ vs_prev, const bf16x8 (&qf)[QT][8],
                                          const int (&k_addr)[8], const int (&v_addr)[4], int h, const Copy& copy) {
  auto frag_ptr = [&](int f) -> const bf16x8* {
    const int blk = f >> 3, j = f & 7;
    if (blk == 0) return reinterpret_cast<const bf16x8*>(ks + k_addr[j]);
    if (blk == 2) return reinterpret_cast<const bf16x8*>(ks + k_addr[j] + 32 * kD);
    if (blk == 1) return reinterpret_cast<const bf16x8*>(vs_prev + v_addr[2 + (j & 1)] + (j >> 1) * 32 * kKT);
    return reinterpret_cast<const bf16x8*>(vs + v_addr[j & 1] + (j >> 1) * 32 * kKT);
  };
  auto active = [](int f) { return PREV || (f >> 3) != 1; };
  bf16x8 fr[32];
#pragma unroll
  for (int f = 0; f < kLook; ++f) fr[f] = *frag_ptr(f);
  // One probability pair per step (query tile j % QT; with QT = 1 every
  // other step): its two exponentials go behind the step's first MFMA and its
  // packing and row sum behind the second (with QT = 1, behind the next
  // step's MFMA), so that neither exceeds the MFMA it overlaps.
  f32x2 e_pend = {0.0f, 0.0f};
  bf16x8 pv_b[QT], pv_prev[QT];   // B operands of this and the previous step's PV MFMAs
#pragma unroll
  for (int t = 0; t < QT; ++t) pv_b[t] = pv_prev[t] = bf16x8{};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int blk = i >> 3, j = i & 7;
    const int psub = (blk == 0 || blk == 3) ? 1 : 0;      // score half whose probabilities this block forms
    const bool soft = PREV || blk != 0;
    const int tq = QT == 2 ? (j & 1) : 0;                 // query tile of this step's pair
    const int pc = ((blk == 0 || blk == 2) ? 4 : 0) + (j >> 1);
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      if (blk == 0 || blk == 2) {
        const int sub = blk >> 1;
        if (j == 0)
          x[sub][t] = mfma_s_first(fr[i], qf[t][j]);
        else
          mfma_s_acc(x[sub][t], fr[i], qf[t][j]);
      } else if (blk == 3 || PREV) {
        const int sub = blk == 1 ? 1 : 0, dt = j >> 1, half = j & 1;
        const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(w[sub][t][4 * half], w[sub][t][4 * half + 1],
                                                               w[sub][t][4 * half + 2], w[sub][t][4 * half + 3]));
        st[t].o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i], pf, st[t].o[dt], 0, 0, 0);
        pv_b[t] = pf;
      }
      __builtin_amdgcn_sched_barrier(0);   // the vector work below goes behind this MFMA
      if (t == 0) {
        // the copy slot (every fourth step) and the fragment read go behind
        // the step's first MFMA, with the exponentials; the packing and row
        // sums go behind the second (each group then nearly fits the 32
        // cycles of the MFMA it follows)
        if ((i & 3) == 0) copy(i >> 2);
        if (i + kLook < 32 && active(i + kLook)) fr[i + kLook] = *frag_ptr(i + kLook);
        // the first probabilities read from a score block follow the MFMAs
        // that wrote it by the hazard distance (this step's first MFMA runs
        // meanwhile)
        if (j == 0 && blk == 1) hazard_wait<QT>(x[0]);
        if (j == 0 && blk == 3) hazard_wait<QT>(x[1]);
        if (QT == 1 && soft && (j & 1) == 1) w[psub][0][pc] = prob_pack(st[0], e_pend);
        if (soft && (QT == 2 || (j & 1) == 0)) e_pend = prob_exp<false, SHIFT>(st[tq], x[psub][tq], pc, psub, 0ull);
      } else if (soft) {
        w[psub][tq][pc] = prob_pack(st[tq], e_pend);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // This step's MFMA operands stay allocated through the next step: a
    // register rewritten (by an LDS read or a vector-ALU result) while an
    // MFMA that reads it is still executing stalls the wavefront.
    keep_live(fr[i]);
    if (i > 0) keep_live(fr[i - 1]);
    const bool pv_now = blk == 3 || (blk == 1 && PREV);
    const bool pv_before = i > 0 && (((i - 1) >> 3) == 3 || (((i - 1) >> 3) == 1 && PREV));
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      if (pv_before) keep_live(pv_prev[t]);
      if (pv_now) pv_prev[t] = pv_b[t];
    }
  }
}
// The last tile's remaining work: probabilities of half 1, pairs 4-7, then
// PV half 1.
template <int QT, bool SHIFT>
__device__ __forceinline__ void pipe_tail(RowState (&st)[QT], f32x16 (&x)[2][QT], uint32_t (&w)[2][QT][8],
                                          const uint16_t* __restrict__ vs, const int (&v_addr)[4], int h) {
  bf16x8 fr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    fr[j] = *reinterpret_cast<const bf16x8*>(vs + v_addr[2 + (j & 1)] + (j >> 1) * 32 * kKT);
#pragma unroll
  for (int c = 4; c < 8; ++c)
#pragma unroll
    for (int t = 0; t < QT; ++t) w[1][t][c] = prob_pair<false, SHIFT>(st[t], x[1][t], c, 1, 0ull);
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const int dt = j >> 1, half = j & 1;
      const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(w[1][t][4 * half], w[1][t][4 * half + 1],
                                                             w[1][t][4 * half + 2], w[1][t][4 * half + 3]));
      st[t].o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[j], pf, st[t].o[dt], 0, 0, 0);
    }
}

// Scores only: raises mx[t] to this lane's max visible score (log2 units) of
// one staged tile. Used by the fallback that finds each row's exact max.
template <int QT, bool MASKED>
__device__ __forceinline__ void tile_max(float (&mx)[QT], const uint16_t* __restrict__ ks, const bf16x8 (&qf)[QT][8],
                                         const int (&k_addr)[8], int h, int rel0, const uint64_t (&anc)[QT]) {
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    bf16x8 ka[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) ka[kk] = *reinterpret_cast<const bf16x8*>(ks + k_addr[kk] + sub * 32 * kD);
    f32x16 x[QT];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      x[t] = mfma_s_first(ka[0], qf[t][0]);
#pragma unroll
      for (int kk = 1; kk < 8; ++kk) mfma_s_acc(x[t], ka[kk], qf[t][kk]);
    }
    hazard_wait<QT>(x);
#pragma unroll
    for (int t = 0; t < QT; ++t) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = 32 * sub + 16 * (e >> 3) + 8 * h + (e & 7);
        if (!MASKED || key_visible(rel0 + key, anc[t])) mx[t] = fmaxf(mx[t], x[t][e]);
      }
    }
  }
}

// Writes the 32 outputs of one row and head-dim block that lanes l and
// l + 32 hold as 4-element pieces (lane half h holds elements 8 i4 + 4 h ..
// + 3, i4 = 0..3): the halves swap pieces so that each lane writes 8
// contiguous elements twice, 16 bytes each (elements 8 h .. and 16 + 8 h ..
// from dst, the block's first element). Lanes l and l + 32 must both be
// active (they hold the same row, so they branch alike).
__device__ __forceinline__ void store_row32(uint16_t* dst, const uint32_t (&w)[4][2]) {
  const int h = static_cast<int>(threadIdx.x >> 5) & 1;
  uint32_t a[2][2], c[2][2];
#pragma unroll
  for (int pr = 0; pr < 2; ++pr)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      // lower half: (own piece 2 pr, the upper lane's piece 2 pr); upper
      // half: (the lower lane's piece 2 pr + 1, own piece 2 pr + 1)
      const auto r = __builtin_amdgcn_permlane32_swap(w[2 * pr][k], w[2 * pr + 1][k], false, false);
      a[pr][k] = r[0];
      c[pr][k] = r[1];
    }
#pragma unroll
  for (int pr = 0; pr < 2; ++pr)
    *reinterpret_cast<uint4*>(dst + 16 * pr + 8 * h) = make_uint4(a[pr][0], a[pr][1], c[pr][0], c[pr][1]);
}

// Writes normalised rows of one wavefront (lane: row row0 + 32 t + l%32,
// dims 32 dt + 8 i4 + 4 h + 0..3); dead rows get zeros.
template <int QT>
__device__ __forceinline__ void write_rows(const BfParams& p, int b, int g, int row0, int rows_live, int rows_all,
                                           int lane, const f32x16 (&o)[QT][4], const float (&l)[QT]) {
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int row = row0 + 32 * t + (lane & 31);
    if (row < rows_all) {
      const bool live = row < rows_live;
      const int node = p.gdiv.div(row), head = g * p.G + row - node * p.G;
      uint16_t* orow = p.out + ((static_cast<size_t>(b) * p.n_max + node) * p.Hq + head) * kD;
      const float inv = (live && l[t] > 0.0f) ? 1.0f / l[t] : 0.0f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        uint32_t w[4][2];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          w[i4][0] = live ? pack_bf16(o[t][dt][4 * i4 + 0] * inv, o[t][dt][4 * i4 + 1] * inv) : 0u;
          w[i4][1] = live ? pack_bf16(o[t][dt][4 * i4 + 2] * inv, o[t][dt][4 * i4 + 3] * inv) : 0u;
        }
        store_row32(orow + 32 * dt, w);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// tree append helpers
// ---------------------------------------------------------------------------
// Element offsets of the (at most two) 64-slot blocks that hold a tree's
// slots [P, P + n) for KV head (b, g), n <= 64: the dense cache's blocks, or
// the pages the block table names (clamped into the pools; a sequence with
// a page outside them is flagged and skipped by the attention kernel).
struct TreeBlocks {
  int blk0;
  size_t off0, off1;
  __device__ __forceinline__ size_t of(int slot) const { return (slot >> 6) == blk0 ? off0 : off1; }
};
__device__ __forceinline__ size_t page_off(const BfParams& p, int b, int g, int blk) {
  const int32_t e = p.block_table[static_cast<size_t>(b) * p.max_pages + min(blk, p.max_pages - 1)];
  const int page = min(max(e, 0), p.num_pages - 1);
  return (static_cast<size_t>(page) * p.Hkv + g) * kKT * kD;
}
__device__ __forceinline__ TreeBlocks tree_blocks(const BfParams& p, int b, int g, int P) {
  TreeBlocks t;
  t.blk0 = P >> 6;
  if (p.block_table) {
    t.off0 = page_off(p, b, g, t.blk0);
    t.off1 = page_off(p, b, g, t.blk0 + 1);
  } else {
    t.off0 = ((static_cast<size_t>(b) * p.Hkv + g) * p.cap + static_cast<size_t>(t.blk0) * kKT) * kD;
    t.off1 = t.off0 + kKT * kD;
  }
  return t;
}

// The write half of the value append: vtr holds the tree's value chunks as
// [node][chunk] (chunk c of node i at position c ^ (i % 16)); thread it of
// nthreads takes (chunk, 8-slot unit) pairs and writes the unit's 8 head-dim
// rows as the blocked cache holds them.
__device__ __forceinline__ void write_tree_values(const BfParams& p, int P, int n, const TreeBlocks& tb,
                                                  const uint4* vtr, int tid, int nthreads) {
  const int u0 = P >> 3, n_units = ((P + n + 7) >> 3) - u0;   // 8-slot units touching [P, P + n)
  for (int idx = tid; idx < 16 * n_units; idx += nthreads) {
    const int c = idx & 15, s0 = (u0 + (idx >> 4)) << 3;
    uint4 src[8];
    bool in[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = s0 + j - P;
      in[j] = i >= 0 && i < n;
      src[j] = in[j] ? vtr[i * 16 + (c ^ (i & 15))] : make_uint4(0u, 0u, 0u, 0u);
    }
    const bool full = s0 >= P && s0 + 8 <= P + n;
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      uint16_t* dst = p.v_cache + tb.of(s0) + (8 * c + dd) * kKT + (s0 & 63);   // (8-slot units stay in one block)
      if (full) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = static_cast<uint32_t>(u4_elem(src[2 * e], dd)) | (static_cast<uint32_t>(u4_elem(src[2 * e + 1], dd)) << 16);
        *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (in[j]) dst[j] = u4_elem(src[j], dd);
      }
    }
  }
}


// ---------------------------------------------------------------------------
// Fused split merge. With a few key splits and a grid that fits the device at
// once, the splits of a (sequence, KV head, row block) group merge their
// partials themselves instead of a second kernel:
//   publish  every split stores its partial with agent-coherent stores and
//            waits until they are performed;
//   arrive   one atomic increment of the group's arrival count (word 0);
//   claim    the row block's items are dealt out in `splits` equal ranges;
//            a split that has seen every split arrive claims its own range
//            (atomic OR of its bit into word 1) and merges it if the bit was
//            still clear. The last split to arrive never waits: after its own
//            range it claims every range still unclaimed and merges those.
//            The others wait for the count with a bounded spin (no workgroup
//            ever waits on another without a time limit, so the scheme cannot
//            deadlock whatever the dispatch order; one that gives up leaves
//            its range to the last arrival);
//   reset    each split increments word 2 as its last access to the words;
//            the one that completes the count zeroes all three, so the words
//            are zero between calls (also across graph replays).
// Agent-coherent (sc1) stores are performed where every compute unit sees
// them and sc1 loads read from there, so no cache flush or invalidation is
// needed; the partials may be on another XCD's side.
// ---------------------------------------------------------------------------
constexpr uint32_t kSpinTicks = 20000;   // 200 us of the 100 MHz real-time clock (default)

__device__ __forceinline__ uint32_t* group_words(const BfParams& p, int grp) { return p.sync + 4 * static_cast<size_t>(grp); }

// Thread 0 counts this split in; words[0] gets the count it saw (1 .. splits).
__device__ __forceinline__ void merge_arrive(const BfParams& p, int grp, uint32_t* words) {
  if (threadIdx.x == 0) {
    uint32_t* w = group_words(p, grp);
    words[0] = __hip_atomic_fetch_add(&w[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  }
}

// Combines one item (32-row tile wt, head-dim block dt, lane) of S split
// partials: fp32 weights 2^(r_s - max r) * l_s over the splits that saw a
// key, fp32 sums, one division; writes the row's 16 values (with the other
// lane half's 16: two 16-byte stores per lane, see store_row32).
// Partials of copies ss >= splits have weight 0.
// Every caller gives the 64 lanes of a wavefront the items of one (tile,
// head-dim block), lane = item lane, so lane 0 holds the tile's lowest row,
// which is live whenever any row of the tile is: the 16-bit format of each
// split's partial (one per tile, the sign bit of the stored row sum, -0.0
// included) is read from lane 0 and the conversion branches uniformly.
template <int S>
__device__ __forceinline__ void merge_item(int splits, const float2 (&ml)[S], const uint4 (&o)[S][2], uint16_t* dst) {
  float M = -INFINITY;
#pragma unroll
  for (int ss = 0; ss < S; ++ss) M = fmaxf(M, ml[ss].x);   // (the copies repeat a split's value)
  float L = 0.0f;
  float4 acc[4];
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) acc[i4] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
  for (int ss = 0; ss < S; ++ss) {
    // weight of the split's normalised rows: 2^(r_s - max r) times its row sum
    const float ls = fabsf(ml[ss].y);
    const uint32_t y0 = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(__float_as_uint(ml[ss].y)));
    const bool f16 = (y0 >> 31) == 0u;
    const float w = (ss >= splits || ml[ss].x == -INFINITY) ? 0.0f : exp2f(ml[ss].x - M) * ls;
    L += w;
    auto accumulate = [&](auto f16_tag) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t wd[4] = {o[ss][j].x, o[ss][j].y, o[ss][j].z, o[ss][j].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const f32x2 v = decltype(f16_tag)::value ? unpack_f16(wd[u]) : f32x2{bf16_lo(wd[u]), bf16_hi(wd[u])};
          float4& a4 = acc[2 * j + (u >> 1)];   // elements 8j + 2u, 8j + 2u + 1
          if ((u & 1) == 0) {
            a4.x = fmaf(w, v[0], a4.x);
            a4.y = fmaf(w, v[1], a4.y);
          } else {
            a4.z = fmaf(w, v[0], a4.z);
            a4.w = fmaf(w, v[1], a4.w);
          }
        }
      }
    };
    if (f16)
      accumulate(std::true_type{});
    else
      accumulate(std::false_type{});
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  uint32_t w[4][2];   // piece i4: elements 8 i4 + 4 h .. + 3 of the row's 32, h = lane / 32
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    w[i4][0] = pack_bf16(acc[i4].x * inv, acc[i4].y * inv);
    w[i4][1] = pack_bf16(acc[i4].z * inv, acc[i4].w * inv);
  }
  store_row32(dst, w);
}

// Merges range r of the row block's items (item = (wt, dt, lane) in the
// partials' register order, 256 per 32-row tile), two items per thread with
// all their coherent loads in flight together. S >= splits.
template <int WAVES, int QT, int S>
__device__ __forceinline__ void merge_range(const BfParams& p, int b, int g, int rb, int r, int rows_live,
                                            __amdgpu_buffer_rsrc_t rml, __amdgpu_buffer_rsrc_t ro) {
  constexpr int ROWS = WAVES * 32 * QT, NT = WAVES * 64, ITEMS = ROWS / 32 * 256;
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  // Ranges are whole groups of 64 items (one (tile, head-dim block) each),
  // so every wavefront holds one group with item lane = its own lane, as
  // merge_item and store_row32 need; the last range takes the remainder when
  // the split count does not divide the groups (e.g. three splits from the
  // launch-plan override).
  const int per = ITEMS / 64 / p.splits * 64, lo = r * per, hi = r == p.splits - 1 ? ITEMS : lo + per;
  const int rows_all = p.G * p.n_max;
  const int wg0 = ((b * p.Hkv + g) * p.row_blocks + rb) * p.splits;
  for (int base = lo; base < hi; base += 2 * NT) {
    float2 ml[2][S];
    uint4 o[2][S][2];
    int it[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      it[k] = base + k * NT + static_cast<int>(threadIdx.x);
      const int ic = it[k] < hi ? it[k] : lo;   // (loads without branches)
      const int wt = ic >> 8, dt = (ic >> 6) & 3, lane = ic & 63;
#pragma unroll
      for (int ss = 0; ss < S; ++ss) {
        const int wg = wg0 + min(ss, p.splits - 1);
        ml[k][ss] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(
                                                   rml, (wg * (ROWS * 2) + wt * 64 + lane) * 8, 0, kCoherent));
#pragma unroll
        for (int j = 0; j < 2; ++j)
          o[k][ss][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      ro, (wg * (ROWS * 16) + (wt * 8 + dt * 2 + j) * 64 + lane) * 16, 0,
                                                      kCoherent));
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (it[k] >= hi) continue;
      const int wt = it[k] >> 8, dt = (it[k] >> 6) & 3, lane = it[k] & 63;
      const int row = rb * ROWS + wt * 32 + (lane & 31);
      if (row >= rows_all) continue;
      const int node = p.gdiv.div(row), head = g * p.G + row - node * p.G;
      uint16_t* dst = p.out + ((static_cast<size_t>(b) * p.n_max + node) * p.Hq + head) * kD + 32 * dt;
      if (row >= rows_live) {
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) *reinterpret_cast<uint4*>(dst + 16 * pr + 8 * (lane >> 5)) = make_uint4(0u, 0u, 0u, 0u);
        continue;
      }
      merge_item<S>(p.splits, ml[k], o[k], dst);
    }
  }
}

// Waits (bounded) until every split has arrived, claims and merges this
// split's range; the last arrival also claims and merges every range still
// unclaimed. Then counts this split out (and the last one out zeroes the
// words). words: three LDS words, words[0] = the arrival count this split saw.
template <int WAVES, int QT, int S>
__device__ __forceinline__ void merge_claim_and_run(const BfParams& p, int grp, int s, int b, int g, int rb,
                                                    int rows_live, uint32_t* words, __amdgpu_buffer_rsrc_t rml,
                                                    __amdgpu_buffer_rsrc_t ro) {
  static_assert(S == 4 || S == 8, "the fused merge serves up to four or eight splits");
  const uint32_t splits = static_cast<uint32_t>(p.splits);
  const uint32_t full = (1u << splits) - 1u, mine = 1u << s;
  uint32_t* w = group_words(p, grp);
  const bool last = words[0] == splits;   // (uniform: read after a barrier)
  if (p.fused == 2) {
    // only the last arrival merges, every range; the others leave at once
    if (last) {
      if (threadIdx.x == 0) words[2] = full & ~__hip_atomic_fetch_or(&w[1], full, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      const uint32_t todo = words[2];
      for (int r = 0; r < static_cast<int>(splits); ++r)
        if ((todo >> r) & 1u) merge_range<WAVES, QT, S>(p, b, g, rb, r, rows_live, rml, ro);
    }
  } else {
  if (threadIdx.x == 0) {
    bool all = last;
    if (!all) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (true) {
        if (__hip_atomic_load(&w[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= splits) {
          all = true;
          break;
        }
        if (__builtin_amdgcn_s_memrealtime() - t0 >= p.spin_ticks) break;
        __builtin_amdgcn_s_sleep(2);
      }
    }
    uint32_t got = 0;
    if (all) got = mine & ~__hip_atomic_fetch_or(&w[1], mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    words[1] = got;
  }
  __syncthreads();
  if (words[1] != 0u) merge_range<WAVES, QT, S>(p, b, g, rb, s, rows_live, rml, ro);
  if (last) {
    __syncthreads();
    if (threadIdx.x == 0)
      words[2] = (full & ~mine) & ~__hip_atomic_fetch_or(&w[1], full & ~mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint32_t todo = words[2];
    for (int r = 0; r < static_cast<int>(splits); ++r)
      if ((todo >> r) & 1u) merge_range<WAVES, QT, S>(p, b, g, rb, r, rows_live, rml, ro);
  }
  }
  if (threadIdx.x == 0) {
    if (__hip_atomic_fetch_add(&w[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u == splits) {
      __hip_atomic_store(&w[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&w[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&w[2], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// BUILD: the kernel builds the sequence's tree from p.parents itself (each
// wavefront, by build_tree_lane, from one load of the parent of node `lane`)
// instead of loading depths and ancestor masks, and the workgroup (b, g = 0,
// row block 0, split 0) writes anc, depth and err as tv_build_tree would
// (err also TV_ERR_CAPACITY, and with a paged cache TV_ERR_BAD_PAGE, as the
// attention call after tv_build_tree would set them).
template <int WAVES, int QT, bool PAGED, bool BUILD>
__global__ __launch_bounds__(WAVES * 64) void attn_bf16_kernel(BfParams p) {
  constexpr int NT = WAVES * 64;
  constexpr int ROWS = WAVES * 32 * QT;      // query rows of the workgroup
  constexpr int CPT = (kKT * kD / 8) / NT;   // 16-byte chunks per thread per K (or V) stage
  static_assert(2 * CPT * kAhead <= 63, "vmcnt range");   // (the counter's limit)
  // (K, V) x stages. At the start, stage 2 holds the RoPE table, float2
  // (cos, sin) of angle (P + depth) f_j at [depth][j], until tile 2 goes
  // out, and the raw query rows pass through the last two stages.
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kStages * kStageElems];
  static_assert(kCsElems == 2 * kStageElems, "the table fills one stage");
  static_assert(kStages >= 5 && kAhead == 3, "the table's stage is free until tile 2 goes out");
  float2* const cs_tab = reinterpret_cast<float2*>(smem + 2 * 2 * kStageElems);

  // Workgroups are handed to the eight XCDs round-robin by index. When the
  // (sequence, KV head) pairs come in multiples of eight, all workgroups of
  // one pair get indices eight apart, so they share an L2 and start
  // together: the row blocks of one split (adjacent there) read the same key
  // tiles, and every split reads the same query rows. (A placement hint
  // only: any bijection is correct.)
  const int per_head = p.row_blocks * p.splits, n_heads = p.ph_div.div(gridDim.x);
  int s, rb, hd;
  if (n_heads % 8 == 0) {
    const int L = blockIdx.x, k = L >> 3, kq = p.ph_div.div(k), w = k - kq * per_head;
    hd = kq * 8 + (L & 7);
    s = p.rb_div.div(w);
    rb = w - s * p.row_blocks;
  } else {
    hd = p.ph_div.div(blockIdx.x);
    const int w = blockIdx.x - hd * per_head;
    s = p.rb_div.div(w);
    rb = w - s * p.row_blocks;
  }
  const int b = p.kv_div.div(hd), g = hd - b * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.G;

  const int rb0 = rb * ROWS;
  const int r0 = rb0 + wave * 32 * QT;       // first row of this wavefront
  const uint32_t lds_base = lds_addr(smem);

  // ---- 1. loads that need only the launch indices go out first: the
  // depths of this wavefront's rows' nodes and of node `lane` (for the
  // deepest node of b), then the workgroup's query rows, raw, copied straight
  // into LDS (the last two ring stages, idle until the queries are read):
  // chunk c = row c/16, position c%16, holding the row's 16-byte piece
  // (c%16) ^ (row%16), so that reads in operand order (one piece of 32
  // consecutive rows) hit distinct banks. The sequence's state (three scalar
  // loads) is read while they are in flight. Every address is valid (node
  // indices are clamped to n_max), so nothing branches; dead rows and nodes
  // are dropped once the data has landed.
  // With a paged cache the sequence's page ids go out first: lane l of
  // pg[u] holds block l + 64 u (clamped to the table; at most 256 blocks).
  constexpr int kPageOps = PAGED ? 4 : 0;
  uint32_t pg[4] = {0u, 0u, 0u, 0u};
  if constexpr (PAGED) {
    const int32_t* bt = p.block_table + static_cast<size_t>(b) * p.max_pages;
#pragma unroll
    for (int u = 0; u < 4; ++u) pg[u] = ld_b32(bt + min(lane + 64 * u, p.max_pages - 1));
  }
  int my_row[QT];
  uint32_t qdep[QT];
  uint32_t dep_lane = 0u, par_lane = 0u;
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    my_row[t] = r0 + 32 * t + (lane & 31);
    if constexpr (!BUILD)
      qdep[t] = ld_b32(p.depth + static_cast<size_t>(b) * p.n_max +
                       min(static_cast<int>(p.gdiv.div(my_row[t])), p.n_max - 1));
  }
  if constexpr (BUILD)
    par_lane = ld_b32(p.parents + static_cast<size_t>(b) * p.n_max + min(lane, p.n_max - 1));
  else
    dep_lane = ld_b32(p.depth + static_cast<size_t>(b) * p.n_max + min(lane, p.n_max - 1));
  constexpr int kDepOps = BUILD ? 1 : QT + 1;
  constexpr int QCPT = ROWS * kD / 8 / NT;              // query chunks per thread
  static_assert(ROWS * kD <= 4 * kStageElems, "query rows must fit the last two stages");
  const uint32_t lds_q = lds_base + 2u * kStageElems * 2u * (kStages - 2);
  {
    const uint16_t* qb = p.q + static_cast<size_t>(b) * p.n_max * p.Hq * kD;
#pragma unroll
    for (int j = 0; j < QCPT; ++j) {
      const int c = j * NT + tid, r = c >> 4, piece = (c & 15) ^ (r & 15);
      const int row = rb0 + r, nq = p.gdiv.div(row), node = min(nq, p.n_max - 1);
      const uint32_t voff = static_cast<uint32_t>(((node * p.Hq + g * G + row - nq * G) * kD + 8 * piece) * 2);
      dma16(qb, voff, lds_q + static_cast<uint32_t>(j * NT + wave * 64) * 16u);
    }
  }

  const SeqState sq = BUILD ? seq_state_scalar_ne(p, b) : seq_state_scalar(p, b);
  const int n = sq.n, P = sq.P;
  const int rows_live = sq.skip ? 0 : G * n;
  const int rows_all = G * p.n_max;
  const bool tree_writer = g == 0 && rb == 0 && s == 0;
  if (!BUILD && sq.cap_bad && tree_writer && tid == 0) p.err[b] = TV_ERR_CAPACITY;
  // (every workgroup of b reads err: before or after this store, b is skipped)

  // BUILD: wavefront 0 of the writing workgroup stores the sequence's tree
  // (as tv_build_tree: zeros for padding nodes and invalid trees) and its
  // error word (a bad tree, else a capacity error, else a page outside the
  // pools, else 0: the precedence of the separate calls). Called once all
  // loads have landed and nothing else is in flight.
  auto write_tree = [&](const LaneTree& tr, bool bad_page) __attribute__((always_inline)) {
    if (BUILD && tree_writer && wave == 0) {
      if (lane < p.n_max) {
        p.anc[static_cast<size_t>(b) * p.n_max + lane] = tr.anc;
        p.depth[static_cast<size_t>(b) * p.n_max + lane] = tr.depth;
      }
      if (lane == 0)
        p.err[b] = !tr.ok ? TV_ERR_BAD_TREE : sq.cap_bad ? TV_ERR_CAPACITY : bad_page ? TV_ERR_BAD_PAGE : 0;
    }
  };

  // A workgroup with nothing to compute: its loads land before its LDS is
  // given up; with separate split merging the merge kernel writes the zero
  // rows, else (one split, or the fused merge: split 0) it does.
  auto retire = [&](int first_row, bool bad_page) __attribute__((always_inline)) {
    wait_vm<0>();
    if constexpr (BUILD) {
      landed(par_lane);
      write_tree(build_tree_lane(static_cast<int>(par_lane), n, p.n_max, lane), bad_page);
    }
    if (p.splits == 1 || (p.fused && s == 0)) {
      for (int r = first_row + tid / 16; r < min(rb0 + ROWS, rows_all); r += NT / 16) {
        const int i = p.gdiv.div(r), head = g * G + r - i * G;
        uint16_t* orow = p.out + ((static_cast<size_t>(b) * p.n_max + i) * p.Hq + head) * kD;
        reinterpret_cast<uint4*>(orow)[tid % 16] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  if (rb0 >= rows_live) {
    retire(rb0, false);   // nothing live in this row block
    return;
  }
  bool row_live[QT];
  uint64_t my_anc[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    row_live[t] = my_row[t] < rows_live;
    my_anc[t] = 0;
  }
  // BUILD: the tree from the parents (every wavefront alike), while the query
  // copies are in flight and before anything else goes out; the rows' and
  // the tree items' depths and the rows' ancestor masks come from it by
  // shuffles. A bad tree retires every workgroup of the sequence.
  LaneTree tree{0ull, 0, true};
  if constexpr (BUILD) {
    wait_vm<waits::vm_parents(WAVES, QT)>();   // (only the query copies stay in flight)
    landed(par_lane);
    tree = build_tree_lane(static_cast<int>(par_lane), n, p.n_max, lane);
    if (!tree.ok) {
      retire(rb0, false);
      return;
    }
    dep_lane = static_cast<uint32_t>(tree.depth);
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const int node = min(static_cast<int>(p.gdiv.div(my_row[t])), p.n_max - 1);
      qdep[t] = static_cast<uint32_t>(__shfl(tree.depth, node));
      my_anc[t] = shfl_u64(tree.anc, node);
    }
  }

  // Keys of b: slots [0, P + n), in aligned 64-key tiles shared out over the
  // splits. A split takes its tiles in DESCENDING order, so the at most two
  // tiles that reach past P (they hold the tree) come first: their tree
  // rows are formed in LDS from data loaded with the queries, and no load
  // waits at the end of the kernel.
  const int key_end = P + n;
  const int tiles_all = (key_end + kKT - 1) / kKT;
  const int tiles_per_split = (tiles_all + p.splits - 1) / p.splits;
  const int t_begin = min(tiles_all, s * tiles_per_split);
  const int n_tiles = min(tiles_all, t_begin + tiles_per_split) - t_begin;
  const int k_begin = t_begin * kKT;
  auto tile_k0 = [&](int pos) { return k_begin + (n_tiles - 1 - pos) * kKT; };   // first key at position pos
  int n_masked = 0;
  while (n_masked < n_tiles && tile_k0(n_masked) + kKT > P) ++n_masked;

  // With tree tiles, the tree's keys and values in 16-byte chunks (lane
  // items: node, chunk) with their nodes' depths, and the ancestor masks of
  // this wavefront's rows, also before the tile copies (vector memory
  // operations complete in order, so anything queued behind the copies would
  // wait for all of them).
  constexpr int KI = 8 * 64 / NT, VI = 16 * 64 / NT;   // tree items per thread: K pairs, V chunks
  constexpr int kTreeOps = BUILD ? 2 * KI + VI : 3 * KI + VI + QT;
  // every loop bound above is the one the wait model counts
  static_assert(CPT == waits::tile_chunks(WAVES) && QCPT == waits::query_ops(WAVES, QT) &&
                    kDepOps == waits::depth_ops(QT, BUILD) && kPageOps == waits::page_ops(PAGED) &&
                    KI == waits::tree_k_items(WAVES) && VI == waits::tree_v_items(WAVES) &&
                    kTreeOps == waits::tree_ops(WAVES, QT, BUILD),
                "the hand-counted waits follow tv_attn_waits.h");
  u32x4 tk_lo[KI], tk_hi[KI], tvv[VI];
  uint32_t t_dep[KI];
  auto load_tree = [&](auto asm_tag) __attribute__((always_inline)) {
    constexpr bool ASM = decltype(asm_tag)::value;
#pragma unroll
    for (int u = 0; u < KI; ++u) {
      const int item = tid + NT * u, node = min(item >> 3, n - 1), c = item & 7;
      const uint16_t* ksrc = p.k_new + ((static_cast<size_t>(b) * p.n_max + node) * p.Hkv + g) * kD + 8 * c;
      tk_lo[u] = ASM ? ld_b128(ksrc) : *reinterpret_cast<const u32x4*>(ksrc);
      tk_hi[u] = ASM ? ld_b128(ksrc + 64) : *reinterpret_cast<const u32x4*>(ksrc + 64);
      if constexpr (BUILD) {
        t_dep[u] = static_cast<uint32_t>(__shfl(tree.depth, node));
      } else {
        const uint32_t* dsrc = reinterpret_cast<const uint32_t*>(p.depth) + static_cast<size_t>(b) * p.n_max + node;
        t_dep[u] = ASM ? ld_b32(dsrc) : *dsrc;
      }
    }
#pragma unroll
    for (int u = 0; u < VI; ++u) {
      const int item = tid + NT * u, node = min(item >> 4, n - 1), c = item & 15;
      const uint16_t* vsrc = p.v_new + ((static_cast<size_t>(b) * p.n_max + node) * p.Hkv + g) * kD + 8 * c;
      tvv[u] = ASM ? ld_b128(vsrc) : *reinterpret_cast<const u32x4*>(vsrc);
    }
    if constexpr (!BUILD) {
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        const uint64_t* asrc =
            p.anc + static_cast<size_t>(b) * p.n_max + min(static_cast<int>(p.gdiv.div(my_row[t])), p.n_max - 1);
        my_anc[t] = ASM ? ld_b64(asrc) : *asrc;
      }
    }
  };
  if (n_masked > 0) load_tree(std::true_type{});

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

  // Copies the tile at position pos into stage pos % kStages. LDS chunk c
  // (16 bytes) of a stage is K row c/16, position c%16 (unit swizzled by
  // key) and V row c/8, position c%8 (unit swizzled by d); the lane that
  // writes chunk c fetches the matching global chunk.
  uint32_t k_voff[CPT], v_voff[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int c = j * NT + tid;
    const int key = c >> 4, kpos = c & 15;
    k_voff[j] = static_cast<uint32_t>(key * kD + ((kpos ^ k_swz(key)) << 3)) * 2u;
    const int d = c >> 3, vpos = c & 7;
    v_voff[j] = static_cast<uint32_t>(d * kKT + ((vpos ^ (d & 7)) << 3)) * 2u;
  }
  // A tile's copy in 8 slots (instruction 2j: K chunk j, 2j + 1: V chunk j;
  // slot k holds instructions [2 CPT k / 8, 2 CPT (k + 1) / 8): two, one, or
  // with eight wavefronts one in every other slot), so that a tile product
  // can spread them over its steps.
  static_assert(2 * CPT % 8 == 0 || 8 % (2 * CPT) == 0, "copy slots");
  struct TileCopy {
    const uint16_t* ktile;
    const uint16_t* vtile;
    uint32_t kl, vl;
    const uint32_t* k_voff;
    const uint32_t* v_voff;
    __device__ __forceinline__ void operator()(int slot) const {
#pragma unroll
      for (int part = slot * 2 * CPT / 8; part < (slot + 1) * 2 * CPT / 8; ++part) {
        const int j = part >> 1;
        if (part & 1)
          dma16(vtile, v_voff[j], vl + j * NT * 16);
        else
          dma16(ktile, k_voff[j], kl + j * NT * 16);
      }
    }
  };
  auto tile_copy = [&](int pos) {
    const int kt0 = tile_k0(pos), buf = pos % kStages;
    TileCopy c;
    if constexpr (PAGED) {
      const int blk = kt0 >> 6;   // < 256
      const uint32_t reg = blk < 64 ? pg[0] : blk < 128 ? pg[1] : blk < 192 ? pg[2] : pg[3];
      const size_t off = (static_cast<size_t>(__builtin_amdgcn_readlane(reg, blk & 63)) * p.Hkv + g) * kKT * kD;
      c.ktile = p.k_cache + off;
      c.vtile = p.v_cache + off;
    } else {
      c.ktile = kc + static_cast<size_t>(kt0) * kD;
      c.vtile = vc + static_cast<size_t>(kt0) * kD;   // kt0 is a multiple of 64
    }
    c.kl = lds_base + static_cast<uint32_t>(2 * buf * kStageElems + wave * 64 * 8) * 2u;
    c.vl = c.kl + kStageElems * 2u;
    c.k_voff = k_voff;
    c.v_voff = v_voff;
    return c;
  };
  auto issue_tile = [&](int pos) {
    const TileCopy c = tile_copy(pos);
#pragma unroll
    for (int slot = 0; slot < 8; ++slot) c(slot);
  };

  // The counter of outstanding vector memory operations holds 63: with
  // narrow workgroups (more chunks per thread) the start's operations and
  // a tile's copies could exceed it, so enough of the former land first.
  // Only the first tile goes out with them: at the start every compute unit
  // loads at once, and a wavefront issuing more copies would stall in the
  // issue until most of them have arrived, with its RoPE work still ahead.
  // Tile 1 goes out once the query rows are in registers, tile 2 after the
  // RoPE, so that work overlaps the first tiles' transfer.
  // (every count below comes from the issue-order model in tv_attn_waits.h)
  constexpr bool kGuard = waits::start_guard(WAVES, QT, PAGED, BUILD);
  static_assert(kAhead == 3, "the start issues three tiles");
  if constexpr (kGuard) wait_vm<waits::vm_start_guard(WAVES)>();
  if constexpr (PAGED) {
    // the page ids (the oldest loads) land; every block of slots [0, P + n)
    // must name a page of the pools (all workgroups of b check alike), else
    // b is flagged and skipped
    if (n_masked > 0)
      wait_vm<waits::vm_pages(WAVES, QT, BUILD, true)>();
    else
      wait_vm<waits::vm_pages(WAVES, QT, BUILD, false)>();
    bool bad = false;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      landed(pg[u]);
      const int page = static_cast<int>(pg[u]);
      bad |= lane + 64 * u < tiles_all && (page < 0 || page >= p.num_pages);
    }
    if (__any(bad)) {
      // (building the tree, the writing workgroup stores the error with it)
      if (!BUILD && g == 0 && rb == 0 && s == 0 && tid == 0) p.err[b] = TV_ERR_BAD_PAGE;
      retire(rb0, true);
      return;
    }
  }
  if (n_tiles > 0) issue_tile(0);

  // ---- 2. the RoPE table for depths 0 .. deepest node of b, float2
  // (cos, sin) of angle (P + depth) f_j at [depth][j], is built in stage 2
  // (idle until tile 2 goes out) as soon as the depths have landed, while
  // the queries are still in flight.
  if constexpr (!kGuard) {
    if (n_masked > 0)
      wait_vm<waits::vm_depths(WAVES, QT, BUILD, true, true)>();
    else if (n_tiles > 0)
      wait_vm<waits::vm_depths(WAVES, QT, BUILD, false, true)>();
    else
      wait_vm<waits::vm_depths(WAVES, QT, BUILD, false, false)>();
  } else {
    // (the guard above left an unknown count: wait for all but tile 0)
    if (n_tiles > 0)
      wait_vm<waits::vm_queries(WAVES, true)>();
    else
      wait_vm<waits::vm_queries(WAVES, false)>();
  }
#pragma unroll
  for (int t = 0; t < QT; ++t) landed(qdep[t]);
  landed(dep_lane);
  int n_cs;          // table entries: depths 0 .. deepest node of b
  {
    const int dmax = wave_max_i32(lane < n ? clamp_depth(static_cast<int>(dep_lane)) : 0);
    n_cs = (dmax + 1) * (kD / 2);
  }
  auto build_table = [&]() {
    const double freq = rope_freq(p.log2_theta, tid & 63);   // column tid % 64 of every row
    for (int e = tid; e < n_cs; e += NT)
      cs_tab[e] = p.rope ? rope_cs(P + (e >> 6), freq) : make_float2(1.0f, 0.0f);
  };
  build_table();

  // ---- 3. once only the first tile's copies are outstanding, the queries
  // and the tree's register loads have landed: the raw query rows go to
  // registers, and the queries, rotated at P + depth, times softmax_scale *
  // log2(e), in bf16, become the B operands of the score MFMA; the tree's
  // keys are rotated at P + depth(node) in their registers.
  if (n_tiles > 0)
    wait_vm<waits::vm_queries(WAVES, true)>();
  else
    wait_vm<waits::vm_queries(WAVES, false)>();
#pragma unroll
  for (int t = 0; t < QT; ++t) landed(my_anc[t]);
#pragma unroll
  for (int u = 0; u < KI; ++u) {
    landed(tk_lo[u]);
    landed(tk_hi[u]);
    landed(t_dep[u]);
  }
#pragma unroll
  for (int u = 0; u < VI; ++u) landed(tvv[u]);
  __syncthreads();   // every wavefront's query copies have landed, and the table is complete
  u32x4 qraw[QT][8];   // qraw[t][kk] = raw Q[row][16kk + 8h .. +8]
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const uint16_t* qs = smem + 2 * kStageElems * (kStages - 2);
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const int r = wave * 32 * QT + 32 * t + (lane & 31);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(qs + r * kD + (((2 * kk + h) ^ (r & 15)) << 3));
        qraw[t][kk] = row_live[t] ? v : z;
      }
    }
  }
  if (n_tiles > 1) issue_tile(1);
  bf16x8 qf[QT][8];      // qf[t][kk] = rotated, scaled Q[row][16kk + 8h .. +8]
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const float2* cs = cs_tab + (row_live[t] ? clamp_depth(static_cast<int>(qdep[t])) : 0) * (kD / 2) + 8 * h;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 lo, hi;
      const u32x4 a = qraw[t][kk], c = qraw[t][kk + 4];
      rope8(make_uint4(a[0], a[1], a[2], a[3]), make_uint4(c[0], c[1], c[2], c[3]), cs + 16 * kk, p.scale_log2, lo, hi);
      qf[t][kk] = __builtin_bit_cast(bf16x8, lo);
      qf[t][kk + 4] = __builtin_bit_cast(bf16x8, hi);
    }
    // the operands live in accumulation registers from here on (every score
    // MFMA reads them from there)
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u32x4 v = __builtin_bit_cast(u32x4, qf[t][kk]);
      asm volatile("" : "+a"(v));
      qf[t][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // Tree keys, lane item u: dims 8c.. and 64 + 8c.. of node item / 8, rotated
  // in place (the cache append repeats this rotation bit for bit).
  auto rope_tree = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < KI; ++u) {
      const int c = (tid + NT * u) & 7;
      uint4 lo, hi;
      rope8(make_uint4(tk_lo[u][0], tk_lo[u][1], tk_lo[u][2], tk_lo[u][3]),
            make_uint4(tk_hi[u][0], tk_hi[u][1], tk_hi[u][2], tk_hi[u][3]),
            cs_tab + clamp_depth(static_cast<int>(t_dep[u])) * (kD / 2) + 8 * c, 1.0f, lo, hi);
      tk_lo[u] = u32x4{lo.x, lo.y, lo.z, lo.w};
      tk_hi[u] = u32x4{hi.x, hi.y, hi.z, hi.w};
    }
  };
  if (n_masked > 0) rope_tree();
  __syncthreads();   // every wavefront is done with the table: tile 2 overwrites it
  if (n_tiles > 2) issue_tile(2);

  // Forms the tree part of the staged tile at position pos (< n_masked):
  // slot P + i holds tree node i, whose key (already rotated at P +
  // depth(i)) and value the lane items carry. Slots past P + n are not this call's keys
  // and may hold anything: their scores are masked and their values zeroed
  // (a masked probability is 0, but 0 * NaN is not).
  // The values reach the tree tiles through a transpose in stage 3 (idle
  // here: the query rows have been read, and tile 3 goes out only in the
  // first loop iteration): the lane items are written there as [node][16-byte
  // chunk of 8 dims], chunk c of node i at position c ^ (i % 16) of the row
  // (stage_tree_values, before the barrier that precedes the fill); then a
  // thread takes one chunk c and KPL consecutive keys of the tile and, for
  // each of its 8 dims, writes those keys' 2-byte elements of the dim's V
  // row as one 8- or 16-byte piece: tree nodes from the transpose, keys past
  // the tree zeroed, prefix keys (below P) kept (only a thread whose keys
  // include some reads the old piece first).
  constexpr int KPL = 64 * 16 / NT;   // tile keys per thread in the value fill
  static_assert(KPL == 2 || KPL == 4 || KPL == 8, "value fill in 4-, 8- or 16-byte pieces");
  static_assert(kStages > 3 && 64 * kD * 2 <= 2 * kStageElems * 2, "the value transpose fits stage 3");
  uint4* const vtr = reinterpret_cast<uint4*>(smem + 2 * 3 * kStageElems);   // [node][chunk]
  auto stage_tree_values = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < VI; ++u) {
      const int item = tid + NT * u, node = item >> 4, c = item & 15;
      vtr[node * 16 + (c ^ (node & 15))] = make_uint4(tvv[u][0], tvv[u][1], tvv[u][2], tvv[u][3]);
    }
  };
  // The tree's append to the cache (a2), by row block 0 of the split that
  // holds the tree tiles, once its ring is idle: the rotated keys straight
  // from the lane items, the raw values through the [node][chunk] transpose
  // in stage 3. The slots [P, P + n) it writes are read by no workgroup of
  // this call (the tree tiles take their tree rows from these registers, and
  // whatever their copies read past P is overwritten or zeroed in LDS).
  // Every thread of the workgroup calls it (it holds a barrier).
  const bool appends = n_masked > 0 && !sq.skip && rb == 0;
  auto append_tree = [&]() __attribute__((always_inline)) {
    const TreeBlocks tb = tree_blocks(p, b, g, P);
#pragma unroll
    for (int u = 0; u < KI; ++u) {
      const int item = tid + NT * u, node = item >> 3, c = item & 7;
      if (node < n) {
        const int slot = P + node;
        uint16_t* dst = p.k_cache + tb.of(slot) + static_cast<size_t>(slot & 63) * kD + 8 * c;
        *reinterpret_cast<u32x4*>(dst) = tk_lo[u];
        *reinterpret_cast<u32x4*>(dst + 64) = tk_hi[u];
      }
    }
    stage_tree_values();
    __syncthreads();
    write_tree_values(p, P, n, tb, vtr, tid, NT);
  };
  auto fill_tree = [&](int pos) __attribute__((always_inline)) {
    const int kt0 = tile_k0(pos), off = P - kt0;   // tile key k holds node k - off (k >= off)
    uint16_t* kd = Ks(pos % kStages);
    uint16_t* vd = Vs(pos % kStages);
    {
      const int c = tid / (64 / KPL), k0 = KPL * (tid % (64 / KPL));
      uint4 src[KPL];
      bool tree[KPL], prefix[KPL];
      bool any_prefix = false;
#pragma unroll
      for (int k = 0; k < KPL; ++k) {
        const int node = k0 + k - off;
        prefix[k] = k0 + k < off;
        tree[k] = !prefix[k] && node < n;
        any_prefix |= prefix[k];
        src[k] = tree[k] ? vtr[node * 16 + (c ^ (node & 15))] : make_uint4(0u, 0u, 0u, 0u);
      }
      uint16_t* rows[8];
      uint32_t wo[8][KPL / 2];
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        rows[dd] = vd + vs_off(8 * c + dd, k0 >> 3) + (k0 & 7);   // KPL keys inside one 16-byte unit
#pragma unroll
        for (int k2 = 0; k2 < KPL / 2; ++k2) wo[dd][k2] = 0u;
      }
      if (any_prefix) {
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          if constexpr (KPL == 2) {
            wo[dd][0] = *reinterpret_cast<const uint32_t*>(rows[dd]);
          } else if constexpr (KPL == 4) {
            const uint2 o2 = *reinterpret_cast<const uint2*>(rows[dd]);
            wo[dd][0] = o2.x;
            wo[dd][1] = o2.y;
          } else {
            const uint4 o4 = *reinterpret_cast<const uint4*>(rows[dd]);
            wo[dd][0] = o4.x;
            wo[dd][1] = o4.y;
            wo[dd][2] = o4.z;
            wo[dd][3] = o4.w;
          }
        }
      }
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        uint32_t wv[KPL / 2];
#pragma unroll
        for (int k2 = 0; k2 < KPL / 2; ++k2) {
          uint32_t e[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int k = 2 * k2 + hh;
            const uint32_t old = hh ? (wo[dd][k2] >> 16) : (wo[dd][k2] & 0xFFFFu);
            e[hh] = tree[k] ? u4_elem(src[k], dd) : (prefix[k] ? old : 0u);
          }
          wv[k2] = e[0] | (e[1] << 16);
        }
        if constexpr (KPL == 2)
          *reinterpret_cast<uint32_t*>(rows[dd]) = wv[0];
        else if constexpr (KPL == 4)
          *reinterpret_cast<uint2*>(rows[dd]) = make_uint2(wv[0], wv[1]);
        else
          *reinterpret_cast<uint4*>(rows[dd]) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      }
    }
#pragma unroll
    for (int u = 0; u < KI; ++u) {
      const int item = tid + NT * u, node = item >> 3, c = item & 7;   // dims 8c.. pair with 64 + 8c..
      const int slot = P + node;
      if (node < n && slot >= kt0 && slot < kt0 + kKT) {
        const int key = slot - kt0;
        *reinterpret_cast<u32x4*>(kd + ks_off(key, c)) = tk_lo[u];
        *reinterpret_cast<u32x4*>(kd + ks_off(key, c + 8)) = tk_hi[u];
      }
    }
  };
  RowState st[QT];
  auto reset_state = [&](const float (&r)[QT]) {
#pragma unroll
    for (int t = 0; t < QT; ++t) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) st[t].o[dt] = f32x16{};
      st[t].r = r[t];
      st[t].l = 0.0f;
    }
  };
  float r_ref[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) r_ref[t] = 0.0f;
  reset_state(r_ref);

  // One pass over this split's tiles (the first kAhead already in flight).
  // MODE 0: p = exp2(s) (fast pass); 1: only raise mx to the row maxima of
  // the scores; 2: p = exp2(s - r) with r = the row max.
  float mx[QT];
  auto run_pass = [&](auto mode_tag) {
    constexpr int MODE = decltype(mode_tag)::value;
    constexpr bool SHIFT = MODE == 2;
    auto product = [&](auto masked_tag, int pos, const auto& copy) {
      constexpr bool M = decltype(masked_tag)::value;
      const int buf = pos % kStages, rel0 = tile_k0(pos) - P;
      if constexpr (MODE == 1) {
        tile_max<QT, M>(mx, Ks(buf), qf, k_addr, h, rel0, my_anc);
#pragma unroll
        for (int slot = 0; slot < 8; ++slot) copy(slot);
      } else {
        tile_product<QT, M, SHIFT>(st, Ks(buf), Vs(buf), qf, k_addr, v_addr, h, rel0, my_anc, copy);
      }
    };
    // Waits until a tile has landed, `later` whole tiles having been issued
    // after it (at most kAhead - 1).
    auto wait_tiles_after = [&](int later) {
      static_assert(kAhead == 3, "waits below assume three tiles in flight");
      if (later >= 2) wait_vm<waits::vm_tile(WAVES, 2)>();
      else if (later == 1) wait_vm<waits::vm_tile(WAVES, 1)>();
      else wait_vm<waits::vm_tile(WAVES, 0)>();
    };
    // the tile at position t, at the top of iteration t
    auto wait_tile = [&](int t) { wait_tiles_after(waits::later_tiles(t, n_tiles)); };
    // A ring of kStages LDS stages, kAhead tiles in flight; position t lives
    // in stage t % kStages, and the copy of position t + kAhead goes out
    // during iteration t, into the stage of position t - 2 (the barrier at
    // the top of iteration t has seen every wavefront finish with it). The
    // tree tiles come first (full products, masked); the rest go through the
    // cross-tile pipeline (the scores-only pass through plain products), whose
    // straight steady block sees kAhead - 1 later tiles outstanding.
    // Wavefronts whose rows are all padding compute on their (zero) queries
    // rather than branch around the products.
    int t = 0;
    if (n_masked > 0) {
      // every tree tile is formed before the first product, so the tree's
      // lane items are not live across a product. Only tiles 0 .. kAhead - 1
      // are in flight here (tile kAhead goes out in the first iteration), so
      // after the last tree tile come min(kAhead, n_tiles) - n_masked tiles
      // (one fewer than wait_tile assumes when the tree spans two tiles).
      stage_tree_values();
      wait_tiles_after(waits::after_tree(n_tiles, n_masked));
      __syncthreads();
      for (int m = 0; m < n_masked; ++m) fill_tree(m);
      __syncthreads();
      for (; t < n_masked; ++t) {
        if (t > 0) {
          wait_tile(t);
          __syncthreads();   // every wavefront is done with the stage the next copy takes
        }
        if (t + kAhead < n_tiles) issue_tile(t + kAhead);
        product(std::true_type{}, t, NoCopy{});
      }
    }
    if constexpr (MODE == 1) {
      for (; t + kAhead < n_tiles; ++t) {
        wait_vm<waits::vm_tile(WAVES, kAhead - 1)>();
        __syncthreads();
        product(std::false_type{}, t, tile_copy(t + kAhead));
      }
      for (; t < n_tiles; ++t) {
        wait_tile(t);
        __syncthreads();
        product(std::false_type{}, t, NoCopy{});
      }
    } else if (t < n_tiles) {
      f32x16 x[2][QT];       // score halves
      uint32_t w[2][QT][8];  // their probabilities, bf16 pairs
      auto iter = [&](int pos, int prev_pos, const auto& copy) {
        pipe_iter<QT, SHIFT, true>(st, x, w, Ks(pos % kStages), Vs(pos % kStages), Vs(prev_pos % kStages), qf, k_addr,
                                   v_addr, h, copy);
      };
      // Before the first tile there is no previous tile: its half-1 scores
      // are -inf (block A turns them into probabilities 0, adding nothing to
      // the row sums) and its pairs 0-3, normally formed by block D, are 0,
      // so block B weights the first tile's own values (finite) by 0.
#pragma unroll
      for (int q = 0; q < QT; ++q) {
#pragma unroll
        for (int e = 0; e < 16; ++e) x[1][q][e] = -INFINITY;
#pragma unroll
        for (int c = 0; c < 8; ++c) w[1][q][c] = 0u;
      }
      int prev = t;
      for (; t + kAhead < n_tiles; ++t) {
        wait_tile(t);
        __syncthreads();
        iter(t, prev, tile_copy(t + kAhead));
        prev = t;
      }
      for (; t < n_tiles; ++t) {
        wait_tile(t);
        __syncthreads();
        iter(t, prev, NoCopy{});
        prev = t;
      }
      pipe_tail<QT, SHIFT>(st, x, w, Vs((n_tiles - 1) % kStages), v_addr, h);
    }
  };

  run_pass(std::integral_constant<int, 0>{});

  // The fast pass is exact while a row's probabilities stay inside the
  // float range; a row whose sum left [2^-60, 2^62] (scores far above 62 or
  // all below about -60, in log2 units) is redone: a scores-only pass finds
  // every row's exact max, then the pass is repeated with r = max (all
  // p <= 1, the largest = 1; exact for any score range).
  // (a split without tiles has nothing to redo: its rows stay empty)
  int redo = 0;
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const float l = row_sum2(st[t].l);
    redo |= row_live[t] && n_tiles > 0 && !(l <= 0x1p62f && l >= 0x1p-60f);
  }
  // workgroup-wide OR through the (now idle) ring
  __syncthreads();
  if (tid == 0) reinterpret_cast<int*>(smem)[0] = 0;
  __syncthreads();
  if (redo) reinterpret_cast<int*>(smem)[0] = 1;
  __syncthreads();
  const bool any_redo = reinterpret_cast<const int*>(smem)[0] != 0;
  __syncthreads();
  if (any_redo) {
    // (rare: the tree's rows are loaded again, by ordinary loads, and the
    // RoPE table, overwritten by tiles, is built again)
#pragma unroll
    for (int t = 0; t < QT; ++t) mx[t] = -INFINITY;
    if (n_masked > 0) load_tree(std::false_type{});
    build_table();
    __syncthreads();
    if (n_masked > 0) rope_tree();
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kAhead; ++t)
      if (t < n_tiles) issue_tile(t);
    run_pass(std::integral_constant<int, 1>{});
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const float m = row_max2(mx[t]);
      r_ref[t] = (m == -INFINITY) ? 0.0f : m;
    }
    reset_state(r_ref);
    __syncthreads();
    if (n_masked > 0) load_tree(std::false_type{});
    build_table();
    __syncthreads();
    if (n_masked > 0) rope_tree();
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kAhead; ++t)
      if (t < n_tiles) issue_tile(t);
    run_pass(std::integral_constant<int, 2>{});
  }

  if constexpr (BUILD) write_tree(tree, false);   // (nothing is in flight here)

  // ---- epilogue
  float l_row[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) l_row[t] = row_sum2(st[t].l);
  // Split partial, per row: the output divided by the split's row sum (a
  // convex combination of value rows, so bounded by the largest value
  // element), as 16-bit floats: fp16 when the largest magnitude of every row
  // of the wavefront's 32-row tile is below 2^15, bf16 otherwise (one choice
  // per tile, so the packing does not branch per lane); the sign of each
  // stored row sum tells which.
  // Register order: the 16 bytes of (wave, t, dt, half j) for lane l sit at
  // (((wave * QT + t) * 8 + dt * 2 + j) * 64 + l) within this workgroup's
  // block (elements 8j .. 8j + 7 of the lane's dt accumulator); the (r, +-l)
  // pair of (wave, t) for lane l at ((wave * QT + t) * 64 + l). Blocks are
  // ordered (b, g, rb, s).
  // (rows past the live ones are never read by the merge). For the merge
  // kernel the partials are stored non-temporally: each is read once, by the
  // merge, and keeping them out of the way in L2 shortens the whole call by
  // about 3% on the 8-sequence, 4096-token workload. For the fused merge they
  // are stored agent-coherently: another compute unit, possibly on another
  // XCD, reads them while this kernel runs.
  // The epilogue has one call site of the tree append, whichever way the
  // rows go (a second call site made the compiler keep the tile copies'
  // uniform base addresses in vector registers).
  const bool fused_merge = p.splits > 1 && p.fused;
  const size_t wg_id = ((static_cast<size_t>(b) * p.Hkv + g) * p.row_blocks + rb) * p.splits + s;
  const __amdgpu_buffer_rsrc_t rml = ws_rsrc(p.part_ml, p.ws_bytes), ro = ws_rsrc(p.part_o, p.ws_bytes);
  if (p.splits == 1) {
    f32x16 o[QT][4];
#pragma unroll
    for (int t = 0; t < QT; ++t)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[t][dt] = st[t].o[dt];
    write_rows<QT>(p, b, g, r0, rows_live, rows_all, lane, o, l_row);
  } else {
    uint4* po = p.part_o + wg_id * (ROWS * 16) + wave * (QT * 8 * 64) + lane;
    float2* pm = p.part_ml + wg_id * (ROWS * 2) + wave * (QT * 64) + lane;
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      if (!row_live[t]) continue;
      const float inv = l_row[t] > 0.0f ? 1.0f / l_row[t] : 0.0f;
      float amax = 0.0f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          st[t].o[dt][e] *= inv;
          amax = fmaxf(amax, fabsf(st[t].o[dt][e]));
        }
      const bool use_f16 = __all(row_max2(amax) < 32768.0f);   // (over the tile's live rows)
      auto store16 = [&](auto f16_tag) __attribute__((always_inline)) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            uint32_t w[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float x0 = st[t].o[dt][8 * j + 2 * u], x1 = st[t].o[dt][8 * j + 2 * u + 1];
              w[u] = decltype(f16_tag)::value ? pack_f16(x0, x1) : pack_bf16(x0, x1);
            }
            const u32x4 x = {w[0], w[1], w[2], w[3]};
            uint4* dst = po + (t * 8 + dt * 2 + j) * 64;
            if (p.fused)
              __builtin_amdgcn_raw_buffer_store_b128(x, ro, static_cast<int>((dst - p.part_o) * 16), 0, kCoherent);
            else
              __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(dst));
          }
      };
      if (use_f16)
        store16(std::true_type{});
      else
        store16(std::false_type{});
      // A row that saw no key in this split (an empty split, or one whose
      // keys are all invisible to it) has row sum 0 and stores the reference
      // -inf, so that the merge leaves it out of the largest reference.
      const f32x2 m = {l_row[t] > 0.0f ? st[t].r : -INFINITY, use_f16 ? l_row[t] : -l_row[t]};
      if (p.fused) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, m), rml,
                                              static_cast<int>((pm + t * 64 - p.part_ml) * 8), 0, kCoherent);
      } else {
        __builtin_nontemporal_store(m, reinterpret_cast<f32x2*>(pm + t * 64));
      }
    }
  }
  uint32_t* const words = reinterpret_cast<uint32_t*>(smem);   // (the ring is idle after the barrier)
  const int grp = (b * p.Hkv + g) * p.row_blocks + rb;
  if (fused_merge) {
    // ---- fused merge (merge_in_kernel): publish, arrive, claim, merge; the
    // workgroup holding the tree appends it to the cache in between
    wait_vm<0>();          // this wavefront's partials are performed
    __syncthreads();
    merge_arrive(p, grp, words);
  } else if (appends) {
    __syncthreads();       // every wavefront is done with the ring
  }
  if (appends) append_tree();
  if (!fused_merge) return;   // (with several splits the merge kernel follows)
  __syncthreads();
  if (p.splits <= 4)
    merge_claim_and_run<WAVES, QT, 4>(p, grp, s, b, g, rb, rows_live, words, rml, ro);
  else
    merge_claim_and_run<WAVES, QT, 8>(p, grp, s, b, g, rb, rows_live, words, rml, ro);
}

// ---------------------------------------------------------------------------
// merge: grid (row_blocks * ROWS / 32, Hkv, B), 256 threads; thread = the
// four float4 of one (32-row tile, head-dim block) of one lane's partial
// (same register order as the main kernel).
// S >= splits is the number of partials a thread loads: split min(s,
// splits - 1) for s < S, so the loads need no branches; copies past splits
// get weight 0.
// ---------------------------------------------------------------------------
template <int WAVES, int QT, int S>
__global__ __launch_bounds__(256) void merge_bf16_kernel(BfParams p) {
  constexpr int ROWS = WAVES * 32 * QT;
  const int g = blockIdx.y, b = blockIdx.z;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  // thread = (row block, 32-row tile wt, head-dim block dt, lane): the four
  // float4 of that lane's (wt, dt) block, which share the lane's (r, l)
  const int rb = idx / (ROWS * 8);
  const int rem = idx % (ROWS * 8);
  const int lane = rem & 63, q = rem >> 6;             // q = wt * 4 + dt
  const int wt = q >> 2, dt = q & 3;
  const int row = rb * ROWS + wt * 32 + (lane & 31);   // wave * 32 QT + 32 t = 32 wt
  // The partials are loaded first, for every thread of the grid (the
  // workspace holds all rows_pad rows of each split; rows the attention
  // kernel did not write are dropped below), so that their latency overlaps
  // the sequence state's.
  const size_t wg0 = ((static_cast<size_t>(b) * p.Hkv + g) * p.row_blocks + rb) * p.splits;
  float2 ml[S];
  uint4 o[S][2];
#pragma unroll
  for (int ss = 0; ss < S; ++ss) {
    const size_t wg = wg0 + min(ss, p.splits - 1);
    ml[ss] = p.part_ml[wg * (ROWS * 2) + wt * 64 + lane];
#pragma unroll
    for (int j = 0; j < 2; ++j) o[ss][j] = p.part_o[wg * (ROWS * 16) + (wt * 8 + dt * 2 + j) * 64 + lane];
  }
  asm volatile("" ::: "memory");   // the sequence state is read after these loads go out
  const SeqState sq = seq_state(p, b);
  const int rows_all = p.G * p.n_max;
  if (row >= rows_all) return;
  const int rows_live = sq.skip ? 0 : p.G * sq.n;
  const int node = p.gdiv.div(row), head = g * p.G + row - node * p.G;
  uint16_t* dst = p.out + ((static_cast<size_t>(b) * p.n_max + node) * p.Hq + head) * kD + 32 * dt;
  if (row >= rows_live) {
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) *reinterpret_cast<uint4*>(dst + 16 * pr + 8 * (lane >> 5)) = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  merge_item<S>(p.splits, ml, o, dst);
}

// Optional launch-shape override for tuning sweeps, read once:
// TV_ATTN_TUNE="waves=4,qt=2,splits=4,fused=0" (any subset; 0 = automatic,
// except fused: 0 = the merge kernel, 1 = the fused merge at up to eight
// splits when the grid runs at once, 2 = the last split merges; left out =
// automatic, the fused merge at up to four splits when the grid runs at once;
// spin: the fused merge's bounded wait in 10 ns ticks, 0 = one look at the
// arrival count, so that waiting splits leave their ranges to the last one).
struct Tune { int waves = 0, qt = 0, splits = 0, fused = -1, spin = -1; };
const Tune& tune() {
  static const Tune t = [] {
    Tune r;
    if (const char* e = getenv("TV_ATTN_TUNE")) {
      if (const char* w = strstr(e, "waves=")) sscanf(w, "waves=%d", &r.waves);
      if (const char* q = strstr(e, "qt=")) sscanf(q, "qt=%d", &r.qt);
      if (const char* s = strstr(e, "splits=")) sscanf(s, "splits=%d", &r.splits);
      if (const char* f = strstr(e, "fused=")) sscanf(f, "fused=%d", &r.fused);
      if (const char* f = strstr(e, "spin=")) sscanf(f, "spin=%d", &r.spin);
    }
    return r;
  }();
  return t;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Workspace layout, only with several splits: sync | part_ml | part_o. sync
// holds four 32-bit words per (sequence, KV head, row block) for the fused
// merge, zero between calls. It is one fixed-size region at the start of
// every workspace with splits, whatever the shapes, so that a call with
// other shapes (whose partials start right after it) never writes over the
// words of a later call sharing the workspace.
constexpr size_t kSyncBytes = 16384;
constexpr long kMaxFusedGroups = kSyncBytes / (4 * sizeof(uint32_t));
struct WsLayout {
  size_t sync, part_ml, part_o, total;
};
WsLayout ws_layout(const tv_attn_args* a, const AttnPlan& pl) {
  WsLayout w{0, 0, 0, 0};
  if (pl.splits == 1) return w;
  const size_t heads = static_cast<size_t>(a->B) * a->Hkv;
  const size_t wg_rows = static_cast<size_t>(pl.waves) * 32 * pl.qt;
  const size_t wgs = heads * pl.row_blocks * pl.splits;
  w.part_ml = kSyncBytes;
  w.part_o = w.part_ml + align_up(wgs * wg_rows * 2 * sizeof(float2));
  w.total = w.part_o + wgs * wg_rows * 16 * sizeof(uint4);
  return w;
}

// Compute units of the current device, queried once per device.
int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

}  // namespace

AttnPlan plan_attention_bf16(const tv_attn_args* a) {
  AttnPlan pl;
  const int G = a->Hq / a->Hkv;
  const int rows = G * a->n_max;
  // 64 query rows (two 32-row tiles) per wavefront, so each K and V fragment
  // read from LDS feeds two MFMAs, and four wavefronts (one per SIMD, 512
  // registers each) per workgroup; small row counts use 32-row tiles. With
  // 64 rows or fewer some wavefronts hold no live row but still share the
  // tile copies, which measured faster than two wavefronts (one sequence of
  // 64 nodes, 32 KV heads, 1024-token prefix: 22.5 to 20.2 us).
  pl.qt = rows > 128 ? 2 : 1;
  pl.waves = 4;
  const Tune& tn = tune();
  if (tn.qt == 1 || tn.qt == 2) pl.qt = tn.qt;
  if (tn.waves == 2 || tn.waves == 4 || tn.waves == 8) pl.waves = tn.waves;
  if (pl.waves == 8) pl.qt = 1;   // (two wavefronts per SIMD: one 32-row tile each)
  if (pl.qt == 2) pl.waves = 4;
  const int wg_rows = pl.waves * 32 * pl.qt;
  pl.row_blocks = (rows + wg_rows - 1) / wg_rows;
  const long units = static_cast<long>(a->B) * a->Hkv * pl.row_blocks;
  // Split the keys until the grid covers the 256 compute units, keeping at
  // least four 64-key tiles per split. The prefix length lives on the device,
  // so the cache capacity bounds it here.
  const int max_tiles = (a->cap + kKT - 1) / kKT;
  // A grid that already needs more than one round of workgroups is split
  // once, so that the last round's tail is shorter when the prefixes are
  // ragged (64 sequences of 512 to 4096 tokens: 170.8 to 166.7 us).
  const long cus = device_cus();
  int splits = 1;
  while (units * splits < cus && splits < kMaxSplits && (max_tiles / (splits * 2)) >= 4) splits *= 2;
  if (units > cus && units <= 2 * cus && max_tiles / 2 >= 4) splits = 2;
  if (tn.splits > 0) splits = std::min(std::min(tn.splits, kMaxSplits), std::max(1, max_tiles));
  pl.splits = splits;
  pl.rows_pad = pl.row_blocks * wg_rows;
  // The splits merge in the kernel (no second launch, partials read while
  // still near) when there are at most four and the whole grid runs at once
  // (one workgroup per compute unit); otherwise the merge kernel follows.
  // (Eight splits can merge in the kernel too, on request: measured slower
  // than the merge kernel, 89.4 against 85.0 us on 4 sequences of 16384
  // tokens, 47.6 against 46.6 on 2.)
  // (fused=2 of the override: only the last split to arrive merges, and no
  // split waits, so it also serves grids that do not run at once; measured
  // no faster than the merge kernel there, 161.0 against 160.9 us on 64
  // ragged sequences, and slower at the headline shape, 51.7 against 48.8,
  // where one workgroup then does every group's whole merge)
  const bool at_once = units * splits <= cus;
  const int fuse_max = tn.fused < 0 ? 4 : 8;
  pl.fused = splits > 1 && splits <= fuse_max && units <= kMaxFusedGroups &&
             ((tn.fused != 0 && tn.fused != 2 && at_once) || tn.fused == 2);
  pl.last_merges = pl.fused && tn.fused == 2;
  pl.workspace_bytes = ws_layout(a, pl).total;
  return pl;
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point: the bf16 attention's workspace
// (split partials and the fused merge's synchronisation words) as one
// file-scope device array. Each device the library runs on holds its own
// copy, zero when the module loads (so the synchronisation words start at
// zero; every call leaves them zero), from first use until the process ends.
// Host code never passes the array's name to a kernel (on the host it only
// stands for the symbol); the device address comes from hipGetSymbolAddress
// once per device, with that device current, and is kept per device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_workspace(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// the multiplier of DivUs for divisor d >= 1 and operands up to x_end
static DivUs make_divus(uint32_t d, uint64_t x_end) {
  DivUs r;
  r.d = d;
  r.m = d == 1 ? 0u : static_cast<uint32_t>(((uint64_t{1} << 32) + d - 1) / d);
  r.id = d == 1 ? ~0u : 0u;
  r.slow = x_end * d > (uint64_t{1} << 32) ? 1u : 0u;
  return r;
}

hipError_t launch_attention_bf16(const tv_attn_args* a, const AttnPlan& pl, const tv_paged_kv* pk,
                                 const int32_t* parents, hipStream_t s) {
  BfParams p;
  p.q = static_cast<const uint16_t*>(a->q);
  p.k_new = static_cast<const uint16_t*>(a->k_new);
  p.v_new = static_cast<const uint16_t*>(a->v_new);
  p.k_cache = static_cast<uint16_t*>(a->k_cache);
  p.v_cache = static_cast<uint16_t*>(a->v_cache);
  p.prefix_len = a->prefix_len;
  p.n_nodes = a->n_nodes;
  p.anc = const_cast<uint64_t*>(a->anc);
  p.depth = const_cast<int32_t*>(a->depth);
  p.parents = parents;
  p.err = a->err;
  p.out = static_cast<uint16_t*>(a->out);
  p.n_max = a->n_max;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.G = a->Hq / a->Hkv;
  p.cap = a->cap;
  p.block_table = pk ? pk->block_table : nullptr;
  p.max_pages = pk ? pk->max_pages : 0;
  p.num_pages = pk ? pk->num_pages : 0;
  p.splits = pl.splits;
  p.row_blocks = pl.row_blocks;
  // each divisor with the largest index it divides (x * d <= 2^32 keeps the
  // multiply exact)
  // (query rows stay below G * 64 + 256, so with G <= kMaxGroup every
  // quotient by G is exact)
  const uint64_t n_wg = static_cast<uint64_t>(pl.splits) * pl.row_blocks * a->Hkv * a->B;
  p.gdiv.d = static_cast<uint32_t>(p.G);
  p.gdiv.m = p.G == 1 ? 0u : static_cast<uint32_t>(((uint64_t{1} << 32) + p.G - 1) / p.G);
  p.gdiv.id = p.G == 1 ? ~0u : 0u;
  p.ph_div = make_divus(static_cast<uint32_t>(pl.row_blocks * pl.splits), n_wg);
  p.rb_div = make_divus(static_cast<uint32_t>(pl.row_blocks), static_cast<uint64_t>(pl.row_blocks) * pl.splits);
  p.kv_div = make_divus(static_cast<uint32_t>(a->Hkv), static_cast<uint64_t>(a->Hkv) * a->B);
  p.rope = a->rope_theta != 0.0f;
  p.log2_theta = p.rope ? log2(static_cast<double>(a->rope_theta)) : 0.0;
  const float scale = a->softmax_scale > 0.0f ? a->softmax_scale : 1.0f / sqrtf(static_cast<float>(kD));
  p.scale_log2 = scale * 1.4426950408889634f;
  const WsLayout w = ws_layout(a, pl);
  char* ws = static_cast<char*>(a->workspace);
  p.part_ml = pl.splits > 1 ? reinterpret_cast<float2*>(ws + w.part_ml) : nullptr;
  p.part_o = pl.splits > 1 ? reinterpret_cast<uint4*>(ws + w.part_o) : nullptr;
  p.sync = pl.splits > 1 ? reinterpret_cast<uint32_t*>(ws + w.sync) : nullptr;
  p.fused = !pl.fused ? 0 : pl.last_merges ? 2 : 1;
  p.spin_ticks = tune().spin >= 0 ? static_cast<uint32_t>(tune().spin) : kSpinTicks;
  p.ws_bytes = pl.workspace_bytes;

  dim3 grid(pl.splits * pl.row_blocks * a->Hkv * a->B);
  const int wg_rows = pl.waves * 32 * pl.qt;
  dim3 mgrid(pl.row_blocks * wg_rows / 32, a->Hkv, a->B);
  const int key = pl.waves * 10 + pl.qt;
  switch (key + (pk ? 100 : 0) + (parents ? 200 : 0)) {
    case 21: hipLaunchKernelGGL((attn_bf16_kernel<2, 1, false, false>), grid, dim3(128), 0, s, p); break;
    case 41: hipLaunchKernelGGL((attn_bf16_kernel<4, 1, false, false>), grid, dim3(256), 0, s, p); break;
    case 42: hipLaunchKernelGGL((attn_bf16_kernel<4, 2, false, false>), grid, dim3(256), 0, s, p); break;
    case 121: hipLaunchKernelGGL((attn_bf16_kernel<2, 1, true, false>), grid, dim3(128), 0, s, p); break;
    case 141: hipLaunchKernelGGL((attn_bf16_kernel<4, 1, true, false>), grid, dim3(256), 0, s, p); break;
    case 142: hipLaunchKernelGGL((attn_bf16_kernel<4, 2, true, false>), grid, dim3(256), 0, s, p); break;
    case 221: hipLaunchKernelGGL((attn_bf16_kernel<2, 1, false, true>), grid, dim3(128), 0, s, p); break;
    case 241: hipLaunchKernelGGL((attn_bf16_kernel<4, 1, false, true>), grid, dim3(256), 0, s, p); break;
    case 242: hipLaunchKernelGGL((attn_bf16_kernel<4, 2, false, true>), grid, dim3(256), 0, s, p); break;
    case 81: hipLaunchKernelGGL((attn_bf16_kernel<8, 1, false, false>), grid, dim3(512), 0, s, p); break;
    case 181: hipLaunchKernelGGL((attn_bf16_kernel<8, 1, true, false>), grid, dim3(512), 0, s, p); break;
    case 281: hipLaunchKernelGGL((attn_bf16_kernel<8, 1, false, true>), grid, dim3(512), 0, s, p); break;
    case 321: hipLaunchKernelGGL((attn_bf16_kernel<2, 1, true, true>), grid, dim3(128), 0, s, p); break;
    case 341: hipLaunchKernelGGL((attn_bf16_kernel<4, 1, true, true>), grid, dim3(256), 0, s, p); break;
    case 342: hipLaunchKernelGGL((attn_bf16_kernel<4, 2, true, true>), grid, dim3(256), 0, s, p); break;
    case 381: hipLaunchKernelGGL((attn_bf16_kernel<8, 1, true, true>), grid, dim3(512), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the main kernel appended the tree; with one split, or the splits merged
  // inside it, it is the only kernel
  if (pl.splits == 1 || pl.fused) return hipSuccess;
  const int sk = pl.splits <= 2 ? 2 : pl.splits <= 4 ? 4 : pl.splits <= 8 ? 8 : 16;
  static_assert(kMaxSplits == 16, "merge instances cover up to sixteen splits");
  switch (key * 100 + sk) {
    case 2102: hipLaunchKernelGGL((merge_bf16_kernel<2, 1, 2>), mgrid, dim3(256), 0, s, p); break;
    case 2104: hipLaunchKernelGGL((merge_bf16_kernel<2, 1, 4>), mgrid, dim3(256), 0, s, p); break;
    case 2108: hipLaunchKernelGGL((merge_bf16_kernel<2, 1, 8>), mgrid, dim3(256), 0, s, p); break;
    case 2116: hipLaunchKernelGGL((merge_bf16_kernel<2, 1, 16>), mgrid, dim3(256), 0, s, p); break;
    case 4102: hipLaunchKernelGGL((merge_bf16_kernel<4, 1, 2>), mgrid, dim3(256), 0, s, p); break;
    case 4104: hipLaunchKernelGGL((merge_bf16_kernel<4, 1, 4>), mgrid, dim3(256), 0, s, p); break;
    case 4108: hipLaunchKernelGGL((merge_bf16_kernel<4, 1, 8>), mgrid, dim3(256), 0, s, p); break;
    case 4116: hipLaunchKernelGGL((merge_bf16_kernel<4, 1, 16>), mgrid, dim3(256), 0, s, p); break;
    case 4202: hipLaunchKernelGGL((merge_bf16_kernel<4, 2, 2>), mgrid, dim3(256), 0, s, p); break;
    case 4204: hipLaunchKernelGGL((merge_bf16_kernel<4, 2, 4>), mgrid, dim3(256), 0, s, p); break;
    case 4208: hipLaunchKernelGGL((merge_bf16_kernel<4, 2, 8>), mgrid, dim3(256), 0, s, p); break;
    case 8102: hipLaunchKernelGGL((merge_bf16_kernel<8, 1, 2>), mgrid, dim3(256), 0, s, p); break;
    case 8104: hipLaunchKernelGGL((merge_bf16_kernel<8, 1, 4>), mgrid, dim3(256), 0, s, p); break;
    case 8108: hipLaunchKernelGGL((merge_bf16_kernel<8, 1, 8>), mgrid, dim3(256), 0, s, p); break;
    case 8116: hipLaunchKernelGGL((merge_bf16_kernel<8, 1, 16>), mgrid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((merge_bf16_kernel<4, 2, 16>), mgrid, dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace tv
