// Device definitions shared by the attention kernels of libh3.so (dense
// varlen attention in attn_fwd.hip, FP8 Q.K attention in attn_fp8.hip,
// block-sparse attention in vsa.hip): operand vector types, the swizzled
// 64-key K/V tile layout in LDS, the exchange between the two lanes that
// hold one query's S^T column, the exponentials and row sums of P, the lazy
// rescale, and the transposed V operand reads of the P.V product.
#pragma once

#include "h3_internal.h"

namespace h3 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
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

// Largest of a lane's 16 scores of one 32-key half.
__device__ __forceinline__ float lane_max16(const f32x16_t& s) {
  float mx = s[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
  return mx;
}

// P = exp2(S) for one 32-key half (S already relative to the reference), as
// the two bf16 B operands of the P.V product; l gains the row sum of the
// fp32 P, in two interleaved chains of plain adds.  (A sum of the bf16 P by
// v_dot2c_f32_bf16 against ones overlaps the matrix cores' work poorly on
// gfx950; the two sums differ by the bf16 rounding of P, far inside the
// tolerances, and every kernel uses this one helper, so they stay identical
// to each other.)
__device__ __forceinline__ void exp2_to_bf16(const f32x16_t& sacc, bf16x8_t (&pk)[2], float& l_run) {
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __builtin_amdgcn_exp2f(sacc[c * 8 + e]);
      pk[c][e] = (__bf16)p;
      if (e & 1) s1 += p;
      else s0 += p;
    }
  }
  l_run += s0 + s1;
}

// The same P, with l gaining the row sum of the bf16 P by v_dot2c_f32_bf16
// against ones (8 instructions instead of 16 adds): for the FP8 kernel, whose
// vector ALU carries more work per MFMA cycle, the fewer instructions win.
__device__ __forceinline__ void exp2_to_bf16_dotsum(const f32x16_t& sacc, bf16x8_t (&pk)[2], float& l_run) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  float lsum = l_run;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) pk[c][e] = (__bf16)__builtin_amdgcn_exp2f(sacc[c * 8 + e]);
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const bf16x2_t pp = {pk[c][e], pk[c][e + 1]};
      lsum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, lsum, false);
    }
  }
  l_run = lsum;
}

// Four O values times 1/l, rounded to bf16 (nearest even) and packed for one
// 8-byte store.  Built as a bf16 vector so that each adjacent pair becomes a
// single v_cvt_pk_bf16_f32 (scalar conversions packed with shifts and ORs
// cost four instructions per pair).
__device__ __forceinline__ uint2 scale_pack4_bf16(const f32x16_t& o, int i0, float inv) {
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  const bf16x4_t b = {(__bf16)(o[i0] * inv), (__bf16)(o[i0 + 1] * inv), (__bf16)(o[i0 + 2] * inv),
                      (__bf16)(o[i0 + 3] * inv)};
  return __builtin_bit_cast(uint2, b);
}

// Rare path of the lazy online softmax of the bf16 kernels.  `sacc` holds a
// 32-key half's scores relative to the reference m (log2 units); when any
// lane's exceed it by more than 2^kRescaleLog2, m moves to the pair's max,
// O and l are rescaled by 2^-delta, and the pending scores and the -m
// accumulator-input block are shifted by -delta (exact: numerator and
// denominator share m).  Otherwise nothing changes (p <= 256).
//
// O is multiplied in place by inline-asm v_mul_f32 so that the accumulators
// keep their registers on both sides of the branch (a plain multiply makes
// the compiler copy all 64 on the common path).  The compiler's hazard
// checks do not see into the asm, so the waits are explicit:
//   * before the multiplies, 24 wait states (3 x s_nop 7): covers the
//     v_exp_f32 result read (transcendental write -> VALU read) and the last
//     PV MFMA's writes of O (a 32x32 bf16 MFMA result -> VALU read/write,
//     the longest such hazard on this part, 18 states);  alpha is routed
//     through that asm so the exponential is issued before the wait;
//   * after them, 8 wait states (s_nop 7): VALU write -> MFMA read of the
//     same VGPRs by the next PV MFMA.
// The empty volatile asm at the branch head keeps the compiler from
// if-converting the rescale into an unconditional one on every step.
__device__ __forceinline__ void lazy_rescale_bf16(f32x16_t& sacc, f32x16_t (&oacc)[4], float& m_run,
                                                  float& l_run, f32x16_t& neg_m) {
  const float mloc = lane_max16(sacc);
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(mloc > kRescaleLog2) != 0, 0)) {
    __asm__ volatile("; rescale" ::: "memory");
    const float mpair = swap_halves_max(mloc);
    const float delta = mpair > kRescaleLog2 ? mpair : 0.f;
    float alpha = __builtin_amdgcn_exp2f(-delta);
    __asm__ volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(alpha) :: "memory");
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = oacc[db][i];
        __asm__ volatile("v_mul_f32 %0, %1, %0" : "+v"(x) : "v"(alpha));
        oacc[db][i] = x;
      }
    __asm__ volatile("s_nop 7" ::: "memory");
    m_run += delta;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sacc[i] -= delta;
      neg_m[i] = -m_run;
    }
  }
}

// Byte offsets, within a swizzled 64-key V tile, of the lane's transposing
// reads: ds_read_b64_tr_b16 at voff[db] (+ 8 rows for the second half of the
// operand) yields the V^T A operand of output block db (d = 32db .. +31).
__device__ __forceinline__ void v_tr_offsets(int lane, int (&voff)[4]) {
  const int g = lane >> 5;
  const int rl = 4 * g + ((lane & 15) >> 2);
  const int sv = swz_v(rl);
  const int cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
  for (int db = 0; db < 4; ++db)
    voff[db] = rl * 256 + ((((4 * db) ^ (sv & 12)) | (cl ^ (sv & 3))) << 4) + (lane & 1) * 8;
}

// The V^T A operand of output block db (d = 32db .. +31) for keys 16c .. +15
// of a 32-key half whose V rows start at vh_l: two transposing reads.
__device__ __forceinline__ bf16x8_t v_operand_tr(const char* vh_l, const int (&voff)[4], int db, int c) {
  const char* vp = vh_l + voff[db] + (16 * c) * 256;
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(vp));
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(vp + 8 * 256));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// O^T += V^T P^T for the 32 keys of one half whose V rows start at vh_l.
__device__ __forceinline__ void pv_half_tr(const char* vh_l, const int (&voff)[4], const bf16x8_t (&pk)[2],
                                           f32x16_t (&oacc)[4]) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int c = 0; c < 2; ++c)
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand_tr(vh_l, voff, db, c), pk[c], oacc[db], 0, 0, 0);
}

}  // namespace
}  // namespace h3
