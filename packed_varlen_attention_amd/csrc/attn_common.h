// Device definitions shared by the attention kernels of libh3.so (dense
// varlen attention in attn_fwd.hip, block-sparse attention in vsa.hip):
// operand vector types, the swizzled 64-key K/V tile layout in LDS and
// the exchange between the two lanes that hold one query's S^T column.
#pragma once

#include "h3_internal.h"

namespace h3 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kTileBytes = 64 * 128 * 2;  // one 64-key K or V tile at head dim 128
constexpr float kRescaleLog2 = 8.f;       // lazy rescale threshold (log2 units)
// Buffer descriptor word 3 for raw (unformatted, unswizzled) dword access.
constexpr int kBufferWord3 = 0x00020000;

// K tile: chunk c of row r sits at slot c ^ (r & 15); conflict-free for the
// 32-row b128 reads of the S^T A operand.
__device__ __forceinline__ int swz_k(int row) { return row & 15; }
// V tile: slot c ^ {0, 6, 10, 12}[r & 3]; conflict-free for the transpose reads.
__device__ __forceinline__ int swz_v(int row) { return (0xCA60 >> ((row & 3) << 2)) & 15; }

// Lanes l and l ^ 32 hold the two 16-key halves of one query's S^T column.
__device__ __forceinline__ float swap_halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Segment of tile t from an exclusive prefix of per-segment tile counts.
__device__ __forceinline__ int find_segment(const int32_t* __restrict__ prefix, int n_seg, int t) {
  int lo = 0, hi = n_seg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int N>
struct Int { static constexpr int value = N; };

}  // namespace
}  // namespace h3
