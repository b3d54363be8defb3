// Varlen attention with FP8 Q and K for gfx950: MX block-scaled E4M3 Q.K on
// the scaled matrix-core instruction, bf16 V and P.V.
//
// [P1] "生产环境下的音视频联合生成：MiniMax-H3 与 vLLM-Omni 架构解析": section 五
// keeps the DiT block being computed in FP8 and section 六 names a SAGE
// attention operator, but no low-precision attention algorithm is given.  The
// reading taken here:
//   * Q is multiplied by softmax_scale * log2(e) in fp32 (so scores come out
//     in base-2 units, as in the bf16 kernel), then Q and K are stored as
//     OCP E4M3 values with one power-of-two (E8M0) scale per 32 consecutive
//     channels of a row (the MXFP8 layout of the OCP Microscaling format,
//     block 32).  The block exponent is the smallest e with
//     amax <= 448 * 2^e, so no element saturates; values are x * 2^-e rounded
//     to nearest, ties to even.
//   * Attention is then the plain definition on the dequantized Q and K.
//
// quantize_mx_kernel: 16 lanes per (row, head) of 128 channels, 8 channels
// per lane; a block of 32 is 4 lanes, its amax a 4-lane reduction; codes by
// v_cvt_pk_fp8_f32 (round to nearest even on in-range values).
//
// attn_fwd_fp8qk_d128_kernel: the bf16 d128 kernel's structure (8 waves x 32
// query rows, 4-stage LDS ring of 64-key tiles with direct loads, S^T = K Q^T
// with -m folded into the first accumulator input, exp2, bf16 P, transposed V
// reads) with the S product on v_mfma_scale_f32_32x32x64_f8f6f4: two
// instructions per 32-key half instead of eight.  Operand layout of that
// instruction (fp8 A and B, established with an in-bounds probe): lane
// i + 32g holds row (A) / column (B) i and 32 bytes of the reduction index,
// bytes 0..15 = k 16g .. 16g+15 and bytes 16..31 = k 32+16g .. 32+16g+15; the
// E8M0 scale of k-block j (k in [32j, 32j+32)) of row i comes from lane
// i + 32j.  With channels d = 64m + k for the m-th instruction, lane i + 32g
// supplies the scale of MX block 2m + g.
#include "attn_common.h"

namespace h3 {
namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));

constexpr int kQuantThreads = 256;

// Smallest e with amax <= 448 * 2^e (amax = f * 2^x, f in [0.5, 1):
// 448 = 0.875 * 2^9), -127 for zero, within the E8M0 range.
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.f)) return -127;
  int x;
  const float f = frexpf(amax, &x);
  const int e = f <= 0.875f ? x - 9 : x - 8;
  return max(-127, min(127, e));
}

// One (row, head) of 128 channels per 16 lanes; blockIdx.y = 0 for Q (scaled
// by qmul first), 1 for K.  Codes [rows][H][128] u8, exponents + 127
// [rows][H][4] u8.
__global__ __launch_bounds__(kQuantThreads) void quantize_mx_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, uint8_t* __restrict__ q8,
    uint8_t* __restrict__ k8, uint8_t* __restrict__ qe, uint8_t* __restrict__ ke, int64_t n_rh, float qmul) {
  const bool is_q = blockIdx.y == 0;
  const uint16_t* src = is_q ? q : k;
  uint8_t* codes = is_q ? q8 : k8;
  uint8_t* exps = is_q ? qe : ke;
  const float mul = is_q ? qmul : 1.f;
  const int lane16 = threadIdx.x & 15;
  const int64_t rh = (int64_t)blockIdx.x * (kQuantThreads / 16) + (threadIdx.x >> 4);
  const bool live = rh < n_rh;
  float x[8];
  if (live) {
    const uint4 u = *reinterpret_cast<const uint4*>(src + rh * 128 + lane16 * 8);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16) * mul;
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u) * mul;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = 0.f;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
  // block of 32 channels = 4 consecutive lanes
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const int e = mx_exponent(amax);
  const float f = ldexpf(1.f, -e);   // exact power of two
  uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] * f, x[1] * f, 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] * f, x[3] * f, lo, true);
  uint32_t hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[4] * f, x[5] * f, 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[6] * f, x[7] * f, hi, true);
  // the four block exponents of the row, gathered at lane 0 of its 16
  const int eb = e + 127;
  const int e1 = __shfl_down(eb, 4, 16), e2 = __shfl_down(eb, 8, 16), e3 = __shfl_down(eb, 12, 16);
  if (live) {
    *reinterpret_cast<uint2*>(codes + rh * 128 + lane16 * 8) = make_uint2(lo, hi);
    if (lane16 == 0)
      *reinterpret_cast<uint32_t*>(exps + rh * 4) =
          (uint32_t)eb | ((uint32_t)e1 << 8) | ((uint32_t)e2 << 16) | ((uint32_t)e3 << 24);
  }
}

// ---------------------------------------------------------------------------
// FP8-Q.K d128 attention.  Work items, tiles, pipeline and softmax as in
// attn_fwd_bf16_d128_kernel.  Per stage: K codes 64 rows x 128 B (8 KB,
// 16-byte chunks swizzled c ^ ((row >> 1) & 7), conflict-free for the
// 32-row b128 operand reads), K exponents 64 x 4 B, V 64 x 256 B as in the
// bf16 kernel.  Loads per wave per tile: one K instruction (8 rows), one
// exponent instruction (8 rows, lanes 0..7), two V instructions.
// ---------------------------------------------------------------------------
constexpr int kBMf = 256;
constexpr int kStagesF = 4;
constexpr int kK8Bytes = 64 * 128;      // fp8 K tile
constexpr int kKeBytes = 64 * 4;        // its exponents

__device__ __forceinline__ int swz_k8(int row) { return (row >> 1) & 7; }

__global__ __launch_bounds__(512, 1) void attn_fwd_fp8qk_d128_kernel(
    const uint8_t* __restrict__ q8, const uint8_t* __restrict__ qe, const uint8_t* __restrict__ k8,
    const uint8_t* __restrict__ ke, const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ prefix, int n_seg, int H, int total_rows) {
  constexpr int D = 128;
  constexpr int NW = 8;
  constexpr int VROWS = 64 / NW;            // V rows per wave per tile
  constexpr int VINSTR = VROWS / 4;         // 4 V rows (1 KB) per instruction
  constexpr int LOADS = 2 + VINSTR;         // K + exponents + V, per wave per tile
  __shared__ __attribute__((aligned(1024))) char lk0[kK8Bytes], lk1[kK8Bytes], lk2[kK8Bytes], lk3[kK8Bytes];
  __shared__ __attribute__((aligned(256))) char ls0[kKeBytes], ls1[kKeBytes], ls2[kKeBytes], ls3[kKeBytes];
  __shared__ __attribute__((aligned(1024))) char lv0[kTileBytes], lv1[kTileBytes], lv2[kTileBytes], lv3[kTileBytes];
  auto k_stage = [&](int st) __attribute__((always_inline)) -> char* {
    return st == 0 ? lk0 : st == 1 ? lk1 : st == 2 ? lk2 : lk3;
  };
  auto s_stage = [&](int st) __attribute__((always_inline)) -> char* {
    return st == 0 ? ls0 : st == 1 ? ls1 : st == 2 ? ls2 : ls3;
  };
  auto v_stage = [&](int st) __attribute__((always_inline)) -> char* {
    return st == 0 ? lv0 : st == 1 ? lv1 : st == 2 ? lv2 : lv3;
  };

  const int T = prefix[n_seg];
  const int64_t W = (int64_t)T * H;
  const int64_t per = (W + 7) >> 3;
  const int64_t jj = blockIdx.x >> 3;
  const int64_t w = (int64_t)(blockIdx.x & 7) * per + jj;
  if (jj >= per || w >= W) return;
  const int h = (int)(w / T), t = (int)(w - (int64_t)h * T);
  const int s = find_segment(prefix, n_seg, t);
  const int seg_start = min(max(cu[s], 0), total_rows);
  const int seg_end = max(min(cu[s + 1], total_rows), seg_start);
  const int L = seg_end - seg_start;
  const int q0 = seg_start + (t - prefix[s]) * kBMf;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r32 = lane & 31;
  const int64_t rs = (int64_t)H * D;            // elements per row (V, O; bytes for fp8 codes)
  const uint32_t vrow_bytes = (uint32_t)(rs * 2);
  const uint32_t krow_bytes = (uint32_t)rs;
  const uint32_t erow_bytes = (uint32_t)H * 4;

  // ---- direct loads.  K: lane i writes slot i of rows 8w + i/8; V: as in
  // the bf16 kernel; exponents: lanes 0..7 one row each.
  const uint8_t* kseg = k8 + (int64_t)seg_start * rs + (int64_t)h * D;
  const uint8_t* eseg = ke + (int64_t)seg_start * H * 4 + (int64_t)h * 4;
  const uint16_t* vseg = v + (int64_t)seg_start * rs + (int64_t)h * D;
  const int krow = VROWS * wave + (lane >> 3);
  const int kch = (lane & 7) ^ swz_k8(krow);
  const uint32_t koff_dma = (uint32_t)krow * krow_bytes + (uint32_t)kch * 16u;
  const int erow = VROWS * wave + (lane & 7);
  const uint32_t eoff_dma = (uint32_t)erow * erow_bytes;
  int vrow[VINSTR], vch[VINSTR];
  uint32_t voff_dma[VINSTR];
#pragma unroll
  for (int tt = 0; tt < VINSTR; ++tt) {
    vrow[tt] = VROWS * wave + 4 * tt + (lane >> 4);
    vch[tt] = (lane & 15) ^ swz_v(vrow[tt]);
    voff_dma[tt] = (uint32_t)vrow[tt] * vrow_bytes + (uint32_t)vch[tt] * 16u;
  }
  auto issue_tile = [&](int tile_rel, int stage) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(kseg + (int64_t)tile_rel * rs), (short)0, (int)(64u * krow_bytes), kBufferWord3);
    const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(eseg + (int64_t)tile_rel * H * 4), (short)0, (int)(64u * erow_bytes), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(vseg + (int64_t)tile_rel * rs), (short)0, (int)(64u * vrow_bytes), kBufferWord3);
    char* kl = k_stage(stage) + VROWS * wave * 128;
    char* el = s_stage(stage) + VROWS * wave * 4;
    char* vl = v_stage(stage);
    if (__builtin_expect(tile_rel + 64 <= L, 1)) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)kl, 16, koff_dma, 0, 0, 0);
      if (lane < 8) __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (lds_void_t*)el, 4, eoff_dma, 0, 0, 0);
#pragma unroll
      for (int tt = 0; tt < VINSTR; ++tt)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(vl + (VROWS * wave + 4 * tt) * 256), 16,
                                                 voff_dma[tt], 0, 0, 0);
    } else {
      // ragged tail: rows past the segment end repeat its last row
      const uint32_t kr = (uint32_t)min(krow, L - 1 - tile_rel);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)kl, 16, kr * krow_bytes + (uint32_t)kch * 16u,
                                               0, 0, 0);
      const uint32_t er = (uint32_t)min(erow, L - 1 - tile_rel);
      if (lane < 8) __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (lds_void_t*)el, 4, er * erow_bytes, 0, 0, 0);
#pragma unroll
      for (int tt = 0; tt < VINSTR; ++tt) {
        const uint32_t vr = (uint32_t)min(vrow[tt], L - 1 - tile_rel);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(vl + (VROWS * wave + 4 * tt) * 256), 16,
                                                 vr * vrow_bytes + (uint32_t)vch[tt] * 16u, 0, 0, 0);
      }
    }
  };
  auto wait_tiles_in_flight = [&](int n) __attribute__((always_inline)) {
    if (n <= 0) __builtin_amdgcn_s_waitcnt(0x0F70);
    else if (n == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | LOADS);
    else __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * LOADS));
  };
  static_assert(kStagesF == 4 && 2 * LOADS <= 15, "vmcnt encoding above assumes <= 15 loads in flight");
  const int ntiles = (L + 63) >> 6;
#pragma unroll
  for (int t0 = 0; t0 < kStagesF - 1; ++t0)
    if (t0 < ntiles) issue_tile(t0 * 64, t0);

  // ---- Q codes (B operand) and the lane's two block scales
  v8i_t qf[2];
  int qs[2];
  {
    const int qrow = q0 + wave * 32 + r32;
    if (qrow < seg_end) {
      const uint8_t* qp = q8 + qrow * rs + (int64_t)h * D;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint4 a = *reinterpret_cast<const uint4*>(qp + 64 * m + 16 * g);
        const uint4 b = *reinterpret_cast<const uint4*>(qp + 64 * m + 32 + 16 * g);
        qf[m] = v8i_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
      }
      const uint32_t ew = *reinterpret_cast<const uint32_t*>(qe + ((int64_t)qrow * H + h) * 4);
#pragma unroll
      for (int m = 0; m < 2; ++m) qs[m] = (int)((ew >> (8 * (2 * m + g))) & 0xffu);
    } else {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        qf[m] = v8i_t{};
        qs[m] = 127;
      }
    }
  }

  // ---- per-lane LDS read offsets: K row r32 (+32 rows per half), chunks
  // 4m + g and 4m + 2 + g; V as in the bf16 kernel
  int koff[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int c = 0; c < 2; ++c) koff[m][c] = r32 * 128 + (((4 * m + 2 * c + g) ^ swz_k8(r32)) << 4);
  int voff[4];
  v_tr_offsets(lane, voff);

  f32x16_t oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16_t{};
  float m_run = 0.f, l_run = 0.f;
  f32x16_t neg_m = f32x16_t{};

  // S^T for one 32-key half: two scaled fp8 instructions
  auto compute_s = [&](int stage, int half, f32x16_t& sacc, bool biased) __attribute__((always_inline)) {
    const char* kl = k_stage(stage) + half * 32 * 128;
    const uint32_t ew = *reinterpret_cast<const uint32_t*>(s_stage(stage) + (half * 32 + r32) * 4);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint4 a = *reinterpret_cast<const uint4*>(kl + koff[m][0]);
      const uint4 b = *reinterpret_cast<const uint4*>(kl + koff[m][1]);
      const v8i_t kf = v8i_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
      const int ks = (int)((ew >> (8 * (2 * m + g))) & 0xffu);
      sacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          kf, qf[m], m == 0 ? (biased ? neg_m : f32x16_t{}) : sacc, 0, 0, 0, ks, 0, qs[m]);
    }
  };
  auto mask_tail = [&](f32x16_t& sacc, int key_rel) __attribute__((always_inline)) {
    if (__builtin_expect(key_rel + 32 > L, 0)) {
      __asm__ volatile("; ragged tail" ::: "memory");
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = key_rel + 8 * (i >> 2) + 4 * g + (i & 3);
        if (key >= L) sacc[i] = -INFINITY;
      }
    }
  };
  // rare: a half tile's scores exceed the reference by more than 2^8
  auto update_max = [&](f32x16_t& sacc) __attribute__((always_inline)) {
    const float mloc = lane_max16(sacc);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(mloc > kRescaleLog2) != 0, 0)) {
      __asm__ volatile("; rescale" ::: "memory");
      const float mpair = swap_halves_max(mloc);
      const float delta = mpair > kRescaleLog2 ? mpair : 0.f;
      const float alpha = __builtin_amdgcn_exp2f(-delta);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
      m_run += delta;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sacc[i] -= delta;
        neg_m[i] = -m_run;
      }
    }
  };
  auto pv_half = [&](int stage, int half, const bf16x8_t (&pk)[2]) __attribute__((always_inline)) {
    pv_half_tr(v_stage(stage) + half * 8192, voff, pk, oacc);
  };

  // ---- prologue: first half of tile 0 sets the reference
  f32x16_t scur;
  wait_tiles_in_flight(min(ntiles - 1, kStagesF - 2));
  __syncthreads();
  compute_s(0, 0, scur, false);
  mask_tail(scur, 0);
  m_run = swap_halves_max(lane_max16(scur));
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    scur[i] -= m_run;
    neg_m[i] = -m_run;
  }

  auto step = [&](int k_st, int k_half, int key_next, int v_st, int v_half, auto ragged)
      __attribute__((always_inline)) {
    bf16x8_t pk[2];
    f32x16_t snxt;
    exp2_to_bf16_dotsum(scur, pk, l_run);
    compute_s(k_st, k_half, snxt, true);
    pv_half(v_st, v_half, pk);
    if constexpr (decltype(ragged)::value != 0) mask_tail(snxt, key_next);
    update_max(snxt);
    scur = snxt;
  };
  auto final_step = [&](int v_st, int v_half) __attribute__((always_inline)) {
    bf16x8_t pk[2];
    exp2_to_bf16_dotsum(scur, pk, l_run);
    pv_half(v_st, v_half, pk);
  };
  auto tile = [&](auto phase, int j, auto steady) __attribute__((always_inline)) {
    constexpr int cur = decltype(phase)::value;
    constexpr int nxt = (cur + 1) % kStagesF;
    constexpr int dma = (cur + kStagesF - 1) % kStagesF;
    constexpr bool is_steady = decltype(steady)::value != 0;
    step(cur, 1, j * 64 + 32, cur, 0, Int<is_steady ? 0 : 1>{});
    if (is_steady || j + 1 < ntiles) {
      wait_tiles_in_flight(min(ntiles - 2 - j, kStagesF - 3));
      __syncthreads();
      if (j + kStagesF - 1 < ntiles) issue_tile((j + kStagesF - 1) * 64, dma);
      step(nxt, 0, (j + 1) * 64, cur, 1, Int<is_steady ? 0 : 1>{});
    } else {
      final_step(cur, 1);
    }
  };
  int j = 0;
  for (; j + kStagesF + 1 < ntiles; j += kStagesF) {
    tile(Int<0>{}, j, Int<1>{});
    tile(Int<1>{}, j + 1, Int<1>{});
    tile(Int<2>{}, j + 2, Int<1>{});
    tile(Int<3>{}, j + 3, Int<1>{});
  }
  tile(Int<0>{}, j, Int<0>{});
  if (j + 1 < ntiles) {
    tile(Int<1>{}, j + 1, Int<0>{});
    if (j + 2 < ntiles) {
      tile(Int<2>{}, j + 2, Int<0>{});
      if (j + 3 < ntiles) {
        tile(Int<3>{}, j + 3, Int<0>{});
        if (j + 4 < ntiles) tile(Int<0>{}, j + 4, Int<0>{});
      }
    }
  }

  // ---- normalise and store through LDS (whole rows per store): after a
  // barrier every V stage is free; wave w uses half (w & 1) of V stage w / 2.
  const float inv = 1.f / swap_halves_sum(l_run);
  __syncthreads();
  {
    char* ot = v_stage(wave >> 1) + (wave & 1) * 8192;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const uint2 st = scale_pack4_bf16(oacc[db], a4 * 4, inv);
        const int chunk = (4 * db + a4) ^ (r32 & 15);
        *reinterpret_cast<uint2*>(ot + r32 * 256 + chunk * 16 + g * 8) = st;
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 4 * i + (lane >> 4), c = lane & 15;
      const uint4 x = *reinterpret_cast<const uint4*>(ot + row * 256 + ((c ^ (row & 15)) << 4));
      const int orow = q0 + wave * 32 + row;
      if (orow < seg_end) *reinterpret_cast<uint4*>(o + orow * rs + (int64_t)h * D + c * 8) = x;
    }
  }
}

}  // namespace

hipError_t launch_quantize_qk_fp8(const void* q, const void* k, int rows, int H, float scale, uint8_t* q8,
                                  uint8_t* k8, uint8_t* qe, uint8_t* ke, hipStream_t stream) {
  const int64_t n_rh = (int64_t)rows * H;
  if (n_rh == 0) return hipSuccess;
  const int64_t blocks = ceil_div(n_rh, kQuantThreads / 16);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const float qmul = (float)((double)scale * 1.4426950408889634);
  quantize_mx_kernel<<<dim3((unsigned)blocks, 2), kQuantThreads, 0, stream>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), q8, k8, qe, ke, n_rh, qmul);
  return hipGetLastError();
}

hipError_t launch_attn_fp8qk(const uint8_t* q8, const uint8_t* qe, const uint8_t* k8, const uint8_t* ke,
                             const void* v, void* o, const int32_t* cu, int n_seg, int total_rows, int H,
                             void* ws, hipStream_t stream) {
  int32_t* prefix = static_cast<int32_t*>(ws);
  hipError_t e = launch_build_tiles(cu, n_seg, total_rows, kBMf, prefix, stream);
  if (e != hipSuccess) return e;
  const int64_t t_max = ceil_div(total_rows, kBMf) + n_seg;
  const int64_t grid = 8 * ceil_div(t_max * H, 8);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  attn_fwd_fp8qk_d128_kernel<<<(unsigned)grid, 512, 0, stream>>>(
      q8, qe, k8, ke, static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), cu, prefix, n_seg, H,
      total_rows);
  return hipGetLastError();
}

}  // namespace h3
