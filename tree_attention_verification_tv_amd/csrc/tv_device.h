// Device-side helpers shared by the libtv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bf16 <-> fp32. Values are finite here; the narrowing rounds to nearest even.
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// 64-bit lane shuffle as two 32-bit ones.
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  uint32_t lo = __shfl(static_cast<uint32_t>(v), src);
  uint32_t hi = __shfl(static_cast<uint32_t>(v >> 32), src);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Wave-wide maximum, every lane active: DPP moves within each row of 16
// lanes (swap neighbours, swap pairs, mirror each half-row, mirror the row)
// leave every lane of a row with the row's maximum; the four rows' lanes 0,
// 16, 32 and 48 are then read into scalars. Every lane gets the result.
__device__ __forceinline__ int wave_max_i32(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));    // quad_perm [1, 0, 3, 2]
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));    // quad_perm [2, 3, 0, 1]
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false));   // row_half_mirror
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false));   // row_mirror
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// The tree of one sequence by one wavefront, lane i = node i, every lane
// active (infra-guide "5.3 Medusa、EAGLE 与 MTP", sections 3.1, 3.2 and 8):
// the node's ancestors-or-self bitmask and depth by pointer jumping, and
// whether the sequence's parents array is a parents-first tree. p_in is
// parents[i] (any value for i >= n), n the sequence's node count.
//
// Each lane keeps (J, A): J is an ancestor of node i (initially its parent),
// A the set of nodes from i up to but excluding J. One round replaces J by
// J's own J and merges A, so after round r, J is the 2^r-th ancestor; six
// rounds cover any depth below 64, and the rounds stop once no lane has an
// ancestor left (three for depths up to 7). The depth is then |A| - 1.
// Nodes past n, and every node of an invalid tree, get A = 0 and depth 0.
struct LaneTree {
  uint64_t anc;
  int depth;
  bool ok;   // the whole sequence's tree is valid (uniform)
};
__device__ __forceinline__ LaneTree build_tree_lane(int p_in, int n, int n_max, int i) {
  const bool n_ok = (n >= 0) && (n <= n_max);
  const bool live = n_ok && (i < n);
  const int p = live ? p_in : -1;
  const bool ok_i = !live || (i == 0 ? (p == -1) : (p >= 0 && p < i));
  const bool tree_ok = n_ok && __all(ok_i);
  int J = (live && tree_ok) ? p : -1;
  uint64_t A = live ? (1ull << i) : 0ull;
#pragma unroll
  for (int r = 0; r < 6; ++r) {
    // (a uniform exit, read into a scalar: no lane has an ancestor left)
    if (__builtin_amdgcn_readfirstlane(static_cast<int>(__any(J >= 0))) == 0) break;
    const int src = (J >= 0) ? J : i;
    const uint64_t A_src = shfl_u64(A, src);
    const int J_src = __shfl(J, src);
    if (J >= 0) {
      A |= A_src;
      J = J_src;
    }
  }
  const bool keep = live && tree_ok;
  return LaneTree{keep ? A : 0ull, keep ? static_cast<int>(__popcll(A)) - 1 : 0, tree_ok};
}

}  // namespace tv
