// V cache layout conversion between the row layout a model's KV cache
// usually has, [N][cap][D] (slot s, dim d at s*D + d), and the blocked,
// head-dim-major layout the attention kernels read, [N][cap/64][D][64]
// (slot s, dim d at ((s/64)*D + d)*64 + s%64). In both layouts one 64-slot
// block of one (sequence, KV head) is one contiguous run of 64*D elements,
// so the conversion is a transpose of each block: [64][D] <-> [D][64].
#include <hip/hip_runtime.h>

#include <cstdint>

#include "tv_internal.h"

namespace tv {
namespace {

// One workgroup of 256 threads per block: the block's R x C tile (rows ->
// blocked: R = 64 slots, C = D dims; blocked -> rows: R = D, C = 64) is read
// with 16-byte loads (all of a thread's loads in flight together), staged in
// LDS row by row (rows padded by 16 bytes, so each row stays 16-byte aligned
// and a column's elements fall in different banks), and written transposed
// with 16-byte stores. Bound: HBM, each byte read once and written once.
template <typename T, int R, int C>
__global__ __launch_bounds__(256) void v_layout_kernel(const T* __restrict__ src, T* __restrict__ dst) {
  constexpr int E = 16 / static_cast<int>(sizeof(T));            // elements per 16 bytes
  constexpr int ROWW = C * static_cast<int>(sizeof(T)) / 4 + 4;   // LDS row stride, 4-byte words
  constexpr int CHUNKS = R * C / E;                               // 16-byte chunks per tile
  constexpr int PER = CHUNKS / 256;
  static_assert(CHUNKS % 256 == 0, "whole chunks per thread");
  static_assert(C % E == 0 && R % E == 0, "rows of whole chunks");
  __shared__ __attribute__((aligned(16))) uint32_t lds[R * ROWW];
  const size_t base = static_cast<size_t>(blockIdx.x) * R * C;
  const uint4* s4 = reinterpret_cast<const uint4*>(src + base);
  const int tid = static_cast<int>(threadIdx.x);
  uint4 v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) v[j] = s4[j * 256 + tid];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int c = j * 256 + tid, r = c / (C / E), w0 = (c % (C / E)) * 4;
    *reinterpret_cast<uint4*>(lds + r * ROWW + w0) = v[j];
  }
  __syncthreads();
  uint4* d4 = reinterpret_cast<uint4*>(dst + base);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    // output row oc (a column of the tile), source rows r0 .. r0 + E - 1
    const int c = j * 256 + tid, oc = c / (R / E), r0 = (c % (R / E)) * E;
    uint32_t w[4];
    if constexpr (sizeof(T) == 4) {
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = lds[(r0 + k) * ROWW + oc];
    } else {
      const int shift = (oc & 1) * 16;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t lo = (lds[(r0 + 2 * k) * ROWW + (oc >> 1)] >> shift) & 0xFFFFu;
        const uint32_t hi = (lds[(r0 + 2 * k + 1) * ROWW + (oc >> 1)] >> shift) & 0xFFFFu;
        w[k] = lo | (hi << 16);
      }
    }
    d4[c] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <typename T, int D>
hipError_t launch_typed(const void* src, void* dst, long n_blocks, bool to_rows, hipStream_t s) {
  const T* a = static_cast<const T*>(src);
  T* b = static_cast<T*>(dst);
  const dim3 grid(static_cast<unsigned>(n_blocks));
  if (to_rows)
    v_layout_kernel<T, D, 64><<<grid, 256, 0, s>>>(a, b);
  else
    v_layout_kernel<T, 64, D><<<grid, 256, 0, s>>>(a, b);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_v_layout(const void* src, void* dst, long n_blocks, int D, int elem_bytes, bool to_rows,
                           hipStream_t s) {
  if (n_blocks == 0) return hipSuccess;
  if (elem_bytes == 2)
    return D == 64 ? launch_typed<uint16_t, 64>(src, dst, n_blocks, to_rows, s)
                   : launch_typed<uint16_t, 128>(src, dst, n_blocks, to_rows, s);
  return D == 64 ? launch_typed<uint32_t, 64>(src, dst, n_blocks, to_rows, s)
                 : launch_typed<uint32_t, 128>(src, dst, n_blocks, to_rows, s);
}

}  // namespace tv
