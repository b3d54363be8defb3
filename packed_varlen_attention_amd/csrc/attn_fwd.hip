// Varlen attention forward, bf16 inputs, for gfx950 (CDNA4) matrix cores.
//
// [P1] "生产环境下的音视频联合生成：MiniMax-H3 与 vLLM-Omni 架构解析", section 三:
// cu_seqlens marks sub-sequences; a token's softmax runs only over keys of its
// own sub-sequence (weight zero elsewhere).  Section 六: rows past the
// effective length are trimmed by passing a length, never read.
//
// Common design (FlashAttention-2 style forward, Dao 2023, laid out for CDNA4):
//   * Work item = (head, segment, query tile).  Tiles are relative to the
//     segment start, so no tile crosses cu_seqlens and no masked pair is ever
//     multiplied; only a segment's last K tile masks its ragged tail.
//   * Work order: items are head-major and split into 8 contiguous chunks, one
//     per XCD (workgroups are dispatched round-robin over the 8 XCDs), so the
//     query tiles running on one XCD share a head's K/V through that XCD's L2.
//   * S is computed transposed, S^T = K Q^T with Q in registers as the B
//     operand of v_mfma_f32_32x32x16_bf16: one query per lane column, so the
//     row max / row sum are lane-local plus one exchange with lane ^ 32, and
//     P^T feeds O^T = V^T P^T straight from the accumulator registers.
//   * Online softmax in fp32, exp2 domain: p = exp2(s * scale*log2e - m).
//
// attn_fwd_bf16_d128_kernel (head dim 128, the performance path) is described
// above its definition.  attn_fwd_bf16_kernel<D> is the generic path (used for
// head dim 64): 128-row tiles, 32 rows per wave, two workgroups per CU, K rows
// read in a permuted order so each lane's S^T registers hold 8 consecutive keys
// (the B-operand layout), V transposed into LDS by the loading threads.
#include "attn_common.h"

namespace h3 {
namespace {

constexpr int kBM = 128;     // query rows per workgroup
constexpr int kBN = 64;      // keys per K/V tile
constexpr int kThreads = 256;

// Key held by S^T accumulator row m (0..31) of a 32-key block: rows
// m = 8a + 4g + b read key 16(a/2) + 8g + 4(a%2) + b, so that register
// i = 8c + e of lane group g holds key 16c + 8g + e.
__device__ __forceinline__ int k_row_perm(int m) {
  const int a = m >> 3, g = (m >> 2) & 1, b = m & 3;
  return ((a >> 1) << 4) | (g << 3) | ((a & 1) << 2) | b;
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, const int32_t* __restrict__ cu, const int32_t* __restrict__ prefix,
    int n_seg, int H, int total_rows, float scale_log2) {
  constexpr int KP = D + 8;          // sK row pitch (elements)
  constexpr int VP = kBN + 8;        // sV row pitch (elements)
  constexpr int KC = D / 16;         // k-chunks of QK^T
  constexpr int DB = D / 32;         // 32-row blocks of O^T
  constexpr int KCH = D / 8;         // 16-byte chunks per K row
  constexpr int KLOAD = kBN * KCH / kThreads;            // K chunks per thread
  constexpr int VUNITS = (kBN / 4) * (D / 8);            // 4 keys x 8 d units
  constexpr int VLOAD = (VUNITS + kThreads - 1) / kThreads;
  __shared__ __attribute__((aligned(16))) uint16_t sK[kBN * KP];
  __shared__ __attribute__((aligned(16))) uint16_t sV[D * VP];

  // ---- work item
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
  const int q0 = seg_start + (t - prefix[s]) * kBM;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;
  const int64_t rs = (int64_t)H * D;

  // ---- Q fragment (B operand): lane holds Q[row r32][d = 16kc + 8g .. +8]
  const int qrow = q0 + wave * 32 + r32;
  bf16x8_t qf[KC];
  if (qrow < seg_end) {
    const uint16_t* qp = q + qrow * rs + (int64_t)h * D + g * 8;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) qf[kc] = *reinterpret_cast<const bf16x8_t*>(qp + kc * 16);
  } else {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) qf[kc] = bf16x8_t{};
  }

  // ---- K/V tile staging
  uint4 kreg[KLOAD];
  uint4 vreg[VLOAD][4];
  const uint16_t* kh = k + (int64_t)h * D;
  const uint16_t* vh = v + (int64_t)h * D;
  auto load_tile = [&](int kb) {
#pragma unroll
    for (int r = 0; r < KLOAD; ++r) {
      const int c = tid + r * kThreads;
      const int row = c / KCH, col = c % KCH;
      const int key = kb + row;
      kreg[r] = key < seg_end ? *reinterpret_cast<const uint4*>(kh + key * rs + col * 8)
                              : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < VLOAD; ++r) {
      const int u = tid + r * kThreads;
      const int dc = u % (D / 8), kq = u / (D / 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = kb + kq * 4 + e;
        vreg[r][e] = (u < VUNITS && key < seg_end)
                         ? *reinterpret_cast<const uint4*>(vh + key * rs + dc * 8)
                         : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int r = 0; r < KLOAD; ++r) {
      const int c = tid + r * kThreads;
      const int row = c / KCH, col = c % KCH;
      *reinterpret_cast<uint4*>(sK + row * KP + col * 8) = kreg[r];
    }
#pragma unroll
    for (int r = 0; r < VLOAD; ++r) {
      const int u = tid + r * kThreads;
      if (u < VUNITS) {
        const int dc = u % (D / 8), kq = u / (D / 8);
        const uint32_t* x0 = reinterpret_cast<const uint32_t*>(&vreg[r][0]);
        const uint32_t* x1 = reinterpret_cast<const uint32_t*>(&vreg[r][1]);
        const uint32_t* x2 = reinterpret_cast<const uint32_t*>(&vreg[r][2]);
        const uint32_t* x3 = reinterpret_cast<const uint32_t*>(&vreg[r][3]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          // element i of each key's 8-wide chunk, keys kq*4 .. kq*4+3
          const int wsel = i >> 1;
          const uint32_t sh = (i & 1) ? 16 : 0;
          const uint32_t e0 = (x0[wsel] >> sh) & 0xffff, e1 = (x1[wsel] >> sh) & 0xffff;
          const uint32_t e2 = (x2[wsel] >> sh) & 0xffff, e3 = (x3[wsel] >> sh) & 0xffff;
          uint2 pk;
          pk.x = e0 | (e1 << 16);
          pk.y = e2 | (e3 << 16);
          *reinterpret_cast<uint2*>(sV + (dc * 8 + i) * VP + kq * 4) = pk;
        }
      }
    }
  };

  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;
  const int krow_base = k_row_perm(r32) * KP + g * 8;

  load_tile(seg_start);
  for (int kb = seg_start; kb < seg_end; kb += kBN) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (kb + kBN < seg_end) load_tile(kb + kBN);

    // S^T = K Q^T for 2 blocks of 32 keys
    f32x16_t sacc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      sacc[mb] = f32x16_t{};
      const uint16_t* kp = sK + mb * 32 * KP + krow_base;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kp + kc * 16);
        sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kc], sacc[mb], 0, 0, 0);
      }
    }
    // ragged tail of the segment: keys past seg_end get -inf
    if (kb + kBN > seg_end) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb + mb * 32 + ((i >> 3) << 4) + g * 8 + (i & 7);
          if (key >= seg_end) sacc[mb][i] = -INFINITY;
        }
    }
    // online softmax (exp2 domain)
    float mx = sacc[0][0];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[mb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float lsum = 0.f;
    bf16x8_t pk[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[mb][c * 8 + e], scale_log2, -m_new));
          lsum += p;
          pk[mb][c][e] = (__bf16)p;
        }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const uint16_t* vp = sV + (db * 32 + r32) * VP + g * 8;
#pragma unroll
      for (int kk = 0; kk < kBN / 16; ++kk) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(vp + kk * 16);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[kk >> 1][kk & 1], oacc[db], 0, 0, 0);
      }
    }
  }

  // ---- normalise and store: lane holds O[row r32][d = 32db + 8a + 4g + 0..3]
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.f / l_tot;
  if (qrow < seg_end) {
    uint16_t* op = o + qrow * rs + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const uint2 st = scale_pack4_bf16(oacc[db], a * 4, inv);
        *reinterpret_cast<uint2*>(op + db * 32 + a * 8 + g * 4) = st;
      }
  }
}

// ---------------------------------------------------------------------------
// D = 128 kernel: 8 waves x 32 query rows = 256 rows per workgroup, one
// workgroup per CU (two waves per SIMD).
//   * K and V tiles (64 keys x 256 B each) move HBM -> LDS with gfx950 direct
//     loads (buffer_load_dwordx4 ... lds: no register staging, no vector
//     address arithmetic: a per-tile buffer descriptor in SGPRs plus a
//     constant per-lane offset) into a 4-stage ring; each tile is requested
//     two tiles before it is used, one barrier per tile.  Every ring stage is
//     its own __shared__ array, so the compiler's wait-count pass can tell the
//     stages apart.  Rows are stored as loaded, with an XOR swizzle of the
//     16-byte chunks (one load instruction fills 1 KB contiguously, so rows
//     cannot be padded).
//   * V^T operands come from the row-major V tile through the LDS transpose
//     read (ds_read_b64_tr_b16): V is never transposed by ALU work.
//   * Q is held in registers as the B operand, pre-multiplied by
//     scale * log2(e) (one bf16 rounding of the product), so S arrives in the
//     exp2 domain.  The first MFMA of every S chain takes its accumulator
//     input from a register block holding -m (the running reference max), so
//     the accumulators hold s - m and the exponential needs no subtraction.
//   * Software pipeline over 32-key halves: the exponentials of half h run
//     alongside the S MFMAs of half h+1, and the max check of half h+1
//     alongside the PV MFMAs of half h.
//   * Softmax: the reference m moves only when a half tile's scores exceed it
//     by more than 2^8 (exact: numerator and denominator share m; p stays
//     <= 256 otherwise).  The test is lane-local (each lane's 16 scores
//     against 8), the exchange between the two lanes of a query only on the
//     rare rescale.  Row sums add the fp32 P in two chains of plain adds
//     (a v_dot2c_f32_bf16 sum of the bf16 P overlaps the MFMAs poorly).
// ---------------------------------------------------------------------------
constexpr int kBM2 = 256;                 // query rows per workgroup
constexpr int kStages = 4;                // ring stages (tiles requested kStages-2 ahead)

__global__ __launch_bounds__(512, 1) void attn_fwd_bf16_d128_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, const int32_t* __restrict__ cu, const int32_t* __restrict__ prefix,
    int n_seg, int H, int total_rows, float scale_log2) {
  constexpr int D = 128;
  constexpr int NW = 8;                    // waves per workgroup
  constexpr int DMA_ROWS = 64 / NW;        // tile rows each wave loads per tensor
  constexpr int DMA_INSTR = DMA_ROWS / 4;  // 4 rows (1 KB) per load instruction
  __shared__ __attribute__((aligned(1024))) char lk0[kTileBytes], lk1[kTileBytes], lk2[kTileBytes], lk3[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lv0[kTileBytes], lv1[kTileBytes], lv2[kTileBytes], lv3[kTileBytes];
  // stage is a compile-time constant at every call, so these fold away
  auto k_stage = [&](int stage) __attribute__((always_inline)) -> char* {
    return stage == 0 ? lk0 : stage == 1 ? lk1 : stage == 2 ? lk2 : lk3;
  };
  auto v_stage = [&](int stage) __attribute__((always_inline)) -> char* {
    return stage == 0 ? lv0 : stage == 1 ? lv1 : stage == 2 ? lv2 : lv3;
  };

  // ---- work item (same XCD-aware head-major order as the generic kernel)
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
  const int q0 = seg_start + (t - prefix[s]) * kBM2;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar
  const int g = lane >> 5, r32 = lane & 31;
  const int64_t rs = (int64_t)H * D;

  // ---- direct HBM -> LDS tile loads: wave w fills tile rows
  // DMA_ROWS*w .. +DMA_ROWS-1, four rows (1 KB) per instruction; lane i
  // writes LDS slot i, so it fetches the chunk that the swizzle places there.
  // Byte offsets are relative to the tile's first row (< 64 rows * H*D*2 B,
  // which the host keeps below 2^31).
  const uint16_t* kseg = k + (int64_t)seg_start * rs + (int64_t)h * D;
  const uint16_t* vseg = v + (int64_t)seg_start * rs + (int64_t)h * D;
  const uint32_t row_bytes = (uint32_t)(rs * 2);
  int drow[DMA_INSTR], kch[DMA_INSTR], vch[DMA_INSTR];
  uint32_t koff_dma[DMA_INSTR], voff_dma[DMA_INSTR];
#pragma unroll
  for (int tt = 0; tt < DMA_INSTR; ++tt) {
    drow[tt] = DMA_ROWS * wave + 4 * tt + (lane >> 4);
    kch[tt] = (lane & 15) ^ swz_k(drow[tt]);
    vch[tt] = (lane & 15) ^ swz_v(drow[tt]);
    koff_dma[tt] = (uint32_t)drow[tt] * row_bytes + (uint32_t)kch[tt] * 16u;
    voff_dma[tt] = (uint32_t)drow[tt] * row_bytes + (uint32_t)vch[tt] * 16u;
  }
  auto issue_tile = [&](int tile_rel, int stage) __attribute__((always_inline)) {
    char* kb_l = k_stage(stage);
    char* vb_l = v_stage(stage);
    const int nrec = (int)(64u * row_bytes);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(kseg + (int64_t)tile_rel * rs), (short)0, nrec, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(vseg + (int64_t)tile_rel * rs), (short)0, nrec, kBufferWord3);
    if (__builtin_expect(tile_rel + 64 <= L, 1)) {
#pragma unroll
      for (int tt = 0; tt < DMA_INSTR; ++tt) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(kb_l + (DMA_ROWS * wave + 4 * tt) * 256), 16,
                                                 koff_dma[tt], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(vb_l + (DMA_ROWS * wave + 4 * tt) * 256), 16,
                                                 voff_dma[tt], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int tt = 0; tt < DMA_INSTR; ++tt) {
        const uint32_t row = (uint32_t)min(drow[tt], L - 1 - tile_rel);   // ragged tail: repeat the last row
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(kb_l + (DMA_ROWS * wave + 4 * tt) * 256), 16,
                                                 row * row_bytes + (uint32_t)kch[tt] * 16u, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(vb_l + (DMA_ROWS * wave + 4 * tt) * 256), 16,
                                                 row * row_bytes + (uint32_t)vch[tt] * 16u, 0, 0, 0);
      }
    }
  };

  // s_waitcnt vmcnt(n * loads per tile): all but the newest n tiles landed
  auto wait_tiles_in_flight = [&](int n) __attribute__((always_inline)) {
    if (n <= 0) __builtin_amdgcn_s_waitcnt(0x0F70);
    else if (n == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * DMA_INSTR));
    else __builtin_amdgcn_s_waitcnt(0x0F70 | (4 * DMA_INSTR));
  };
  static_assert(kStages == 4 && 4 * DMA_INSTR <= 15, "vmcnt encoding above assumes <= 15 loads in flight");
  const int ntiles = (L + 63) >> 6;
#pragma unroll
  for (int t0 = 0; t0 < kStages - 1; ++t0)
    if (t0 < ntiles) issue_tile(t0 * 64, t0);

  // ---- Q fragment (B operand), times scale * log2(e): lane holds
  // Q[row r32][d = 16kc + 8g .. +8]
  bf16x8_t qf[8];
  {
    const int qrow = q0 + wave * 32 + r32;
    if (qrow < seg_end) {
      const uint16_t* qp = q + qrow * rs + (int64_t)h * D + g * 8;
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        qf[kc] = *reinterpret_cast<const bf16x8_t*>(qp + kc * 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[kc][e] = (__bf16)((float)qf[kc][e] * scale_log2);
      }
    } else {
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) qf[kc] = bf16x8_t{};
    }
  }

  // ---- per-lane LDS read offsets (bytes within a tile)
  int koff[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) koff[kc] = r32 * 256 + (((2 * kc + g) ^ swz_k(r32)) << 4);
  int voff[4];
  v_tr_offsets(lane, voff);

  f32x16_t oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16_t{};
  float m_run = 0.f, l_run = 0.f;   // reference max (log2 units), row sum
  f32x16_t neg_m = f32x16_t{};      // -m_run in all 16 elements: S accumulator input

  // S^T for one 32-key half (16 fp32 per lane, all of the lane's query),
  // minus m when `biased`
  auto compute_s = [&](const char* kh_l, f32x16_t& sacc, bool biased) __attribute__((always_inline)) {
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kh_l + koff[kc]);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kc], kc == 0 ? (biased ? neg_m : f32x16_t{}) : sacc,
                                                     0, 0, 0);
    }
  };
  // keys past the segment end get -inf (only a segment's last, ragged tile)
  auto mask_tail = [&](f32x16_t& sacc, int key_rel) __attribute__((always_inline)) {
    if (__builtin_expect(key_rel + 32 > L, 0)) {
      __asm__ volatile("; ragged tail" ::: "memory");   // keep it a branch, not selects
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = key_rel + 8 * (i >> 2) + 4 * g + (i & 3);
        if (key >= L) sacc[i] = -INFINITY;
      }
    }
  };
  // rare path of the lazy softmax (attn_common.h)
  auto update_max = [&](f32x16_t& sacc) __attribute__((always_inline)) {
    lazy_rescale_bf16(sacc, oacc, m_run, l_run, neg_m);
  };
  auto k_half = [&](int stage, int half) __attribute__((always_inline)) { return k_stage(stage) + half * 8192; };
  auto v_half = [&](int stage, int half) __attribute__((always_inline)) { return v_stage(stage) + half * 8192; };

  // ---- prologue: first half of tile 0; its max sets the reference
  f32x16_t scur;
  // tile 0 must have landed; tiles 1 .. kStages-2 may still be in flight
  wait_tiles_in_flight(min(ntiles - 1, kStages - 2));
  __syncthreads();
  compute_s(k_half(0, 0), scur, false);
  mask_tail(scur, 0);
  m_run = swap_halves_max(lane_max16(scur));
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    scur[i] -= m_run;
    neg_m[i] = -m_run;
  }

  // One pipeline step: S of the next half on the matrix cores while the
  // vector ALU exponentiates the current half, then O += V P for the current
  // half while the next half's scores are checked against the reference.
  // `ragged` is false where the next half cannot reach past the segment end
  // (the main loop): no test there keeps the step one basic block.
  auto step = [&](const char* k_next, int key_next, const char* v_cur, auto ragged) __attribute__((always_inline)) {
    bf16x8_t pk[2];
    f32x16_t snxt;
    // Scheduling hint: interleave the step's LDS reads with its MFMAs in
    // small groups (measured 0.5 % faster at the 58,758-token step, same bits).
    __builtin_amdgcn_iglp_opt(0);
    exp2_to_bf16(scur, pk, l_run);
    compute_s(k_next, snxt, true);
    pv_half_tr(v_cur, voff, pk, oacc);
    if constexpr (decltype(ragged)::value != 0) mask_tail(snxt, key_next);
    update_max(snxt);
    scur = snxt;
  };
  auto final_step = [&](const char* v_cur) __attribute__((always_inline)) {
    bf16x8_t pk[2];
    exp2_to_bf16(scur, pk, l_run);
    pv_half_tr(v_cur, voff, pk, oacc);
  };
  // Tile j lives in stage j % kStages: its second half, then (after the
  // barrier that frees tile j-1's stage for tile j+kStages-1) the next tile's
  // first half.  `steady`: tile j+1 exists, so no exit paths.
  auto tile = [&](auto phase, int j, auto steady) __attribute__((always_inline)) {
    constexpr int cur = decltype(phase)::value;
    constexpr int nxt = (cur + 1) % kStages;
    constexpr int dma = (cur + kStages - 1) % kStages;
    constexpr bool is_steady = decltype(steady)::value != 0;
    step(k_half(cur, 1), j * 64 + 32, v_half(cur, 0), Int<is_steady ? 0 : 1>{});
    if (is_steady || j + 1 < ntiles) {
      // tile j+1 must have landed; younger tiles may still be in flight
      wait_tiles_in_flight(min(ntiles - 2 - j, kStages - 3));
      __syncthreads();
      if (j + kStages - 1 < ntiles) issue_tile((j + kStages - 1) * 64, dma);
      step(k_half(nxt, 0), (j + 1) * 64, v_half(cur, 1), Int<is_steady ? 0 : 1>{});
    } else {
      final_step(v_half(cur, 1));
    }
  };

  // Main loop: kStages tiles per trip, one back-edge, so the accumulators
  // keep their registers across the unrolled copies.  A steady tile t also
  // computes S for the first half of tile t+1 without the ragged-tail mask, so
  // the loop stops while t+1 is still short of the last tile (t + 2 < ntiles).
  // The last 1..kStages+1 tiles follow as straight-line code from stage 0.
  int j = 0;
  for (; j + kStages + 1 < ntiles; j += kStages) {
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

  // ---- normalise and store: lane holds O[row][d = 32db + 8a + 4g + 0..3].
  // Each wave's 32 x 128 bf16 tile goes through LDS so that the global stores
  // write whole rows (16 bytes per lane, 4 rows per instruction) instead of
  // 16-byte pieces of 32 rows; on short segments, where the store sits on the
  // critical path of every workgroup, this is ~10 % of the kernel.  Free LDS:
  // every ring stage other than those of the last two tiles (all waves have
  // passed the barrier after which nothing reads them, and every issued tile
  // load has been waited for).
  const float inv = 1.f / swap_halves_sum(l_run);
  {
    const int busy0 = (ntiles - 1) & 3, busy1 = ntiles >= 2 ? (ntiles - 2) & 3 : busy0;
    int f0 = 0;
    while (f0 == busy0 || f0 == busy1) ++f0;
    int f1 = f0 + 1;
    while (f1 == busy0 || f1 == busy1) ++f1;
    const int fs = (wave >> 2) ? f1 : f0;
    char* base_l = ((wave >> 1) & 1) ? v_stage(fs) : k_stage(fs);
    char* ot = base_l + (wave & 1) * 8192;      // 32 rows x 256 B, 16-byte chunks swizzled by row
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const uint2 st = scale_pack4_bf16(oacc[db], a4 * 4, inv);
        const int chunk = (4 * db + a4) ^ (r32 & 15);
        *reinterpret_cast<uint2*>(ot + r32 * 256 + chunk * 16 + g * 8) = st;
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the wave's tile is in LDS
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 4 * i + (lane >> 4), c = lane & 15;
      const uint4 x = *reinterpret_cast<const uint4*>(ot + row * 256 + ((c ^ (row & 15)) << 4));
      const int orow = q0 + wave * 32 + row;
      if (orow < seg_end) *reinterpret_cast<uint4*>(o + orow * rs + (int64_t)h * D + c * 8) = x;
    }
  }
}

// ---------------------------------------------------------------------------
// Short-segment variant of the D = 128 kernel (segments of at most
// kShortMaxLen rows, as in 3-D window attention): 4 waves x 32 query rows =
// 128 rows per workgroup, 32-key K/V tiles in a 4-stage ring of 64 KB, so two
// workgroups share a CU and one's prologue (Q and first tiles) and epilogue
// (O store) overlap the other's matrix work.  Per query row the arithmetic is
// the main kernel's, step for step (32-key halves in key order, the same
// reference and rescale points), so the two give identical bits.
// ---------------------------------------------------------------------------
constexpr int kBMs = 128;                 // query rows per workgroup
constexpr int kShortMaxLen = 512;         // longest segment routed to it

__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_d128_short_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, const int32_t* __restrict__ cu, const int32_t* __restrict__ prefix,
    int n_seg, int H, int total_rows, float scale_log2) {
  constexpr int D = 128;
  constexpr int NW = 4;                    // waves per workgroup
  constexpr int DMA_ROWS = 32 / NW;        // tile rows each wave loads per tensor
  constexpr int DMA_INSTR = DMA_ROWS / 4;  // 4 rows (1 KB) per load instruction
  constexpr int kB = kTileBytes / 2;       // one 32-key K or V tile
  __shared__ __attribute__((aligned(1024))) char lk0[kB], lk1[kB], lk2[kB], lk3[kB];
  __shared__ __attribute__((aligned(1024))) char lv0[kB], lv1[kB], lv2[kB], lv3[kB];
  // stage is a compile-time constant at every call, so these fold away
  auto k_stage = [&](int stage) __attribute__((always_inline)) -> char* {
    return stage == 0 ? lk0 : stage == 1 ? lk1 : stage == 2 ? lk2 : lk3;
  };
  auto v_stage = [&](int stage) __attribute__((always_inline)) -> char* {
    return stage == 0 ? lv0 : stage == 1 ? lv1 : stage == 2 ? lv2 : lv3;
  };

  // ---- work item (same XCD-aware head-major order as the generic kernel)
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
  const int q0 = seg_start + (t - prefix[s]) * kBMs;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar
  const int g = lane >> 5, r32 = lane & 31;
  const int64_t rs = (int64_t)H * D;

  // ---- direct HBM -> LDS tile loads: wave w fills tile rows
  // DMA_ROWS*w .. +DMA_ROWS-1, four rows (1 KB) per instruction; lane i
  // writes LDS slot i, so it fetches the chunk that the swizzle places there.
  // Byte offsets are relative to the tile's first row (< 64 rows * H*D*2 B,
  // which the host keeps below 2^31).
  const uint16_t* kseg = k + (int64_t)seg_start * rs + (int64_t)h * D;
  const uint16_t* vseg = v + (int64_t)seg_start * rs + (int64_t)h * D;
  const uint32_t row_bytes = (uint32_t)(rs * 2);
  int drow[DMA_INSTR], kch[DMA_INSTR], vch[DMA_INSTR];
  uint32_t koff_dma[DMA_INSTR], voff_dma[DMA_INSTR];
#pragma unroll
  for (int tt = 0; tt < DMA_INSTR; ++tt) {
    drow[tt] = DMA_ROWS * wave + 4 * tt + (lane >> 4);
    kch[tt] = (lane & 15) ^ swz_k(drow[tt]);
    vch[tt] = (lane & 15) ^ swz_v(drow[tt]);
    koff_dma[tt] = (uint32_t)drow[tt] * row_bytes + (uint32_t)kch[tt] * 16u;
    voff_dma[tt] = (uint32_t)drow[tt] * row_bytes + (uint32_t)vch[tt] * 16u;
  }
  auto issue_tile = [&](int tile_rel, int stage) __attribute__((always_inline)) {
    char* kb_l = k_stage(stage);
    char* vb_l = v_stage(stage);
    const int nrec = (int)(32u * row_bytes);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(kseg + (int64_t)tile_rel * rs), (short)0, nrec, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(vseg + (int64_t)tile_rel * rs), (short)0, nrec, kBufferWord3);
    if (__builtin_expect(tile_rel + 32 <= L, 1)) {
#pragma unroll
      for (int tt = 0; tt < DMA_INSTR; ++tt) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(kb_l + (DMA_ROWS * wave + 4 * tt) * 256), 16,
                                                 koff_dma[tt], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(vb_l + (DMA_ROWS * wave + 4 * tt) * 256), 16,
                                                 voff_dma[tt], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int tt = 0; tt < DMA_INSTR; ++tt) {
        const uint32_t row = (uint32_t)min(drow[tt], L - 1 - tile_rel);   // ragged tail: repeat the last row
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(kb_l + (DMA_ROWS * wave + 4 * tt) * 256), 16,
                                                 row * row_bytes + (uint32_t)kch[tt] * 16u, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(vb_l + (DMA_ROWS * wave + 4 * tt) * 256), 16,
                                                 row * row_bytes + (uint32_t)vch[tt] * 16u, 0, 0, 0);
      }
    }
  };

  // s_waitcnt vmcnt(n * loads per tile): all but the newest n tiles landed
  auto wait_tiles_in_flight = [&](int n) __attribute__((always_inline)) {
    if (n <= 0) __builtin_amdgcn_s_waitcnt(0x0F70);
    else if (n == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * DMA_INSTR));
    else __builtin_amdgcn_s_waitcnt(0x0F70 | (4 * DMA_INSTR));
  };
  static_assert(kStages == 4 && 4 * DMA_INSTR <= 15, "vmcnt encoding above assumes <= 15 loads in flight");
  const int ntiles = (L + 31) >> 5;
#pragma unroll
  for (int t0 = 0; t0 < kStages - 1; ++t0)
    if (t0 < ntiles) issue_tile(t0 * 32, t0);

  // ---- Q fragment (B operand), times scale * log2(e): lane holds
  // Q[row r32][d = 16kc + 8g .. +8]
  bf16x8_t qf[8];
  {
    const int qrow = q0 + wave * 32 + r32;
    if (qrow < seg_end) {
      const uint16_t* qp = q + qrow * rs + (int64_t)h * D + g * 8;
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        qf[kc] = *reinterpret_cast<const bf16x8_t*>(qp + kc * 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[kc][e] = (__bf16)((float)qf[kc][e] * scale_log2);
      }
    } else {
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) qf[kc] = bf16x8_t{};
    }
  }

  // ---- per-lane LDS read offsets (bytes within a tile)
  int koff[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) koff[kc] = r32 * 256 + (((2 * kc + g) ^ swz_k(r32)) << 4);
  int voff[4];
  v_tr_offsets(lane, voff);

  f32x16_t oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16_t{};
  float m_run = 0.f, l_run = 0.f;   // reference max (log2 units), row sum
  f32x16_t neg_m = f32x16_t{};      // -m_run in all 16 elements: S accumulator input

  // S^T for one 32-key half (16 fp32 per lane, all of the lane's query),
  // minus m when `biased`
  auto compute_s = [&](const char* kh_l, f32x16_t& sacc, bool biased) __attribute__((always_inline)) {
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kh_l + koff[kc]);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kc], kc == 0 ? (biased ? neg_m : f32x16_t{}) : sacc,
                                                     0, 0, 0);
    }
  };
  // keys past the segment end get -inf (only a segment's last, ragged tile)
  auto mask_tail = [&](f32x16_t& sacc, int key_rel) __attribute__((always_inline)) {
    if (__builtin_expect(key_rel + 32 > L, 0)) {
      __asm__ volatile("; ragged tail" ::: "memory");   // keep it a branch, not selects
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = key_rel + 8 * (i >> 2) + 4 * g + (i & 3);
        if (key >= L) sacc[i] = -INFINITY;
      }
    }
  };
  // rare path of the lazy softmax (attn_common.h)
  auto update_max = [&](f32x16_t& sacc) __attribute__((always_inline)) {
    lazy_rescale_bf16(sacc, oacc, m_run, l_run, neg_m);
  };

  // ---- prologue: first half of tile 0; its max sets the reference
  f32x16_t scur;
  // tile 0 must have landed; tiles 1 .. kStages-2 may still be in flight
  wait_tiles_in_flight(min(ntiles - 1, kStages - 2));
  __syncthreads();
  compute_s(k_stage(0), scur, false);
  mask_tail(scur, 0);
  m_run = swap_halves_max(lane_max16(scur));
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    scur[i] -= m_run;
    neg_m[i] = -m_run;
  }

  // One pipeline step: S of the next half on the matrix cores while the
  // vector ALU exponentiates the current half, then O += V P for the current
  // half while the next half's scores are checked against the reference.
  // `ragged` is false where the next half cannot reach past the segment end
  // (the main loop): no test there keeps the step one basic block.
  auto step = [&](const char* k_next, int key_next, const char* v_cur, auto ragged) __attribute__((always_inline)) {
    bf16x8_t pk[2];
    f32x16_t snxt;
    // Scheduling hint: interleave the step's LDS reads with its MFMAs in
    // small groups (measured 0.5 % faster at the 58,758-token step, same bits).
    __builtin_amdgcn_iglp_opt(0);
    exp2_to_bf16(scur, pk, l_run);
    compute_s(k_next, snxt, true);
    pv_half_tr(v_cur, voff, pk, oacc);
    if constexpr (decltype(ragged)::value != 0) mask_tail(snxt, key_next);
    update_max(snxt);
    scur = snxt;
  };
  auto final_step = [&](const char* v_cur) __attribute__((always_inline)) {
    bf16x8_t pk[2];
    exp2_to_bf16(scur, pk, l_run);
    pv_half_tr(v_cur, voff, pk, oacc);
  };
  // Tile j (32 keys) lives in stage j % kStages: after the barrier that
  // frees tile j-1's stage for tile j+kStages-1, the step that exponentiates
  // tile j's scores, computes tile j+1's and adds V P of tile j.  `steady`:
  // tile j+1 exists and is not the last one, so no exit paths or tail mask.
  auto tile = [&](auto phase, int j, auto steady) __attribute__((always_inline)) {
    constexpr int cur = decltype(phase)::value;
    constexpr int nxt = (cur + 1) % kStages;
    constexpr int dma = (cur + kStages - 1) % kStages;
    constexpr bool is_steady = decltype(steady)::value != 0;
    if (is_steady || j + 1 < ntiles) {
      // tile j+1 must have landed; younger tiles may still be in flight
      wait_tiles_in_flight(min(ntiles - 2 - j, kStages - 3));
      __syncthreads();
      if (j + kStages - 1 < ntiles) issue_tile((j + kStages - 1) * 32, dma);
      step(k_stage(nxt), (j + 1) * 32, v_stage(cur), Int<is_steady ? 0 : 1>{});
    } else {
      final_step(v_stage(cur));
    }
  };

  // Main loop: kStages tiles per trip, one back-edge, so the accumulators
  // keep their registers across the unrolled copies.  A steady tile t also
  // computes S for the first half of tile t+1 without the ragged-tail mask, so
  // the loop stops while t+1 is still short of the last tile (t + 2 < ntiles).
  // The last 1..kStages+1 tiles follow as straight-line code from stage 0.
  int j = 0;
  for (; j + kStages + 1 < ntiles; j += kStages) {
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

  // ---- normalise and store: lane holds O[row][d = 32db + 8a + 4g + 0..3].
  // Each wave's 32 x 128 bf16 tile goes through LDS so that the global stores
  // write whole rows (16 bytes per lane, 4 rows per instruction) instead of
  // 16-byte pieces of 32 rows; on short segments, where the store sits on the
  // critical path of every workgroup, this is ~10 % of the kernel.  Free LDS:
  // every ring stage other than those of the last two tiles (all waves have
  // passed the barrier after which nothing reads them, and every issued tile
  // load has been waited for).
  const float inv = 1.f / swap_halves_sum(l_run);
  {
    const int busy0 = (ntiles - 1) & 3, busy1 = ntiles >= 2 ? (ntiles - 2) & 3 : busy0;
    int f0 = 0;
    while (f0 == busy0 || f0 == busy1) ++f0;
    int f1 = f0 + 1;
    while (f1 == busy0 || f1 == busy1) ++f1;
    const int fs = (wave >> 1) ? f1 : f0;
    char* ot = (wave & 1) ? v_stage(fs) : k_stage(fs);   // 32 rows x 256 B, 16-byte chunks swizzled by row
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const uint2 st = scale_pack4_bf16(oacc[db], a4 * 4, inv);
        const int chunk = (4 * db + a4) ^ (r32 & 15);
        *reinterpret_cast<uint2*>(ot + r32 * 256 + chunk * 16 + g * 8) = st;
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the wave's tile is in LDS
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 4 * i + (lane >> 4), c = lane & 15;
      const uint4 x = *reinterpret_cast<const uint4*>(ot + row * 256 + ((c ^ (row & 15)) << 4));
      const int orow = q0 + wave * 32 + row;
      if (orow < seg_end) *reinterpret_cast<uint4*>(o + orow * rs + (int64_t)h * D + c * 8) = x;
    }
  }
}

// Several-items-per-workgroup variant for short segments (the same
// 128-row items as the short-segment kernel).  A fixed grid of two
// workgroups per CU walks the XCD-aware item order with a stride, and the
// 32-key K/V tiles of consecutive items flow through one 4-stage ring: the
// tile loads run two tiles ahead of the consumer across item boundaries, and
// the next item's Q is requested as soon as the current item's last scores
// are computed (Q's registers are free from there), so one item's fixed costs
// (Q and first tiles in flight, O normalised and stored) overlap another
// item's matrix work instead of leaving the CU idle.  An item's first tile
// sits in a ring stage set by the lengths of the items before it, so stages
// are addressed at run time; the tile loads are issued as inline asm (the
// compiler's wait-count pass does not see them, which keeps it from draining
// every tile in flight at each barrier), every wait on them is an explicit
// s_waitcnt, and the barriers are bare (lgkmcnt(0); s_barrier).  Per query
// row the arithmetic is the main kernel's, step for step, so the output is
// bit-identical to it.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kMultiItemsPerSlot = 4;    // items per workgroup slot (host bound) that select it
constexpr int kMultiMaxItems = 512;      // items one workgroup can list in its LDS item table

__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_d128_multi_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, const int32_t* __restrict__ cu, const int32_t* __restrict__ prefix,
    int n_seg, int H, int total_rows, float scale_log2) {
  constexpr int D = 128;
  constexpr int NW = 4;                    // waves per workgroup
  constexpr int DMA_ROWS = 32 / NW;        // tile rows each wave loads per tensor
  constexpr int DMA_INSTR = DMA_ROWS / 4;  // 4 rows (1 KB) per load instruction
  constexpr int LOADS = 2 * DMA_INSTR;     // load instructions per tile per lane
  constexpr int kB = kTileBytes / 2;       // one 32-key K or V tile (8 KB)
  constexpr int NST = 4;                   // ring stages; stage s: K at 2s*kB, V at (2s+1)*kB
  __shared__ __attribute__((aligned(1024))) char ring[NST * 2 * kB];
  // (head, segment start, segment length, first query row) of this
  // workgroup's items in visiting order
  __shared__ int4 item_table[kMultiMaxItems];

  // ---- this workgroup's items: w = w_begin, w_begin + stride, ... < w_end
  const int T = prefix[n_seg];             // items per head
  const int W = T * H;                     // the host keeps the item count below 2^31
  const int per = (W + 7) >> 3;
  const int xcd = blockIdx.x & 7;
  const int stride = gridDim.x >> 3;
  const int w_begin = xcd * per + (int)(blockIdx.x >> 3);
  const int w_end = min(xcd * per + per, W);
  if (w_begin >= w_end) return;
  // at most ceil(per / stride) <= kMultiMaxItems: T <= ceil(total_rows / 128) + n_seg,
  // the host's tile bound, from which it chose this kernel
  const int n_items = min((w_end - w_begin + stride - 1) / stride, kMultiMaxItems);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar
  const int g = lane >> 5, r32 = lane & 31;
  const int64_t rs = (int64_t)H * D;
  const uint32_t row_bytes = (uint32_t)(rs * 2);

  // The item table, built once: each lane looks up one item's segment (the
  // searches run in parallel instead of one dependent scalar chain per item
  // on the loop's critical path).  Segment bounds are clamped as the tile
  // counts were.
  for (int kk = tid; kk < n_items; kk += 256) {
    const int w = w_begin + kk * stride;
    const int h = w / T;
    const int t = w - h * T;
    const int s = find_segment(prefix, n_seg, t);
    const int seg_start = min(max(cu[s], 0), total_rows);
    const int seg_end = max(min(cu[s + 1], total_rows), seg_start);
    item_table[kk] = make_int4(h, seg_start, seg_end - seg_start, seg_start + (t - prefix[s]) * kBMs);
  }
  __syncthreads();

  // Item kk of this workgroup: head, segment bounds and first query row (scalar).
  struct Item { int h, seg_start, L, q0; };
  auto item_at = [&](int kk) __attribute__((always_inline)) -> Item {
    const int4 e = item_table[kk];
    Item it;
    it.h = __builtin_amdgcn_readfirstlane(e.x);
    it.seg_start = __builtin_amdgcn_readfirstlane(e.y);
    it.L = __builtin_amdgcn_readfirstlane(e.z);
    it.q0 = __builtin_amdgcn_readfirstlane(e.w);
    return it;
  };

  // ---- tile loads (HBM -> LDS), as in the short-segment kernel: wave w
  // fills tile rows DMA_ROWS*w .. +DMA_ROWS-1, lane i writes LDS slot i.
  int drow[DMA_INSTR], kch[DMA_INSTR], vch[DMA_INSTR];
#pragma unroll
  for (int tt = 0; tt < DMA_INSTR; ++tt) {
    drow[tt] = DMA_ROWS * wave + 4 * tt + (lane >> 4);
    kch[tt] = (lane & 15) ^ swz_k(drow[tt]);
    vch[tt] = (lane & 15) ^ swz_v(drow[tt]);
  }
  // m0 holds the LDS destination of a load-to-LDS instruction.  The compiler
  // reserves m0 (hence the silenced warning) but needs it only for its own
  // LDS-load and message instructions, of which this kernel has none (checked
  // in its gfx950 code: m0 is written only here); the asm sets it before every
  // load, so no value of the compiler's is live in it across the statement.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  auto dma = [&](const u32x4_t& rsrc, const char* lds, uint32_t voffset) __attribute__((always_inline)) {
    const uint32_t m0v = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)lds);
    __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :: "s"(m0v), "v"(voffset), "s"(rsrc) : "memory", "m0");
  };
#pragma clang diagnostic pop
  auto rsrc_of = [&](const uint16_t* base) __attribute__((always_inline)) -> u32x4_t {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return u32x4_t{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu)),
                   32u * row_bytes, (uint32_t)kBufferWord3};
  };
  auto stage_k = [&](int gt) __attribute__((always_inline)) -> char* { return ring + (gt & (NST - 1)) * (2 * kB); };
  auto stage_v = [&](int gt) __attribute__((always_inline)) -> char* { return stage_k(gt) + kB; };

  // Issue cursor: the next tile to load is tile i_tile of item i_k, global
  // tile number g_issue; kt / vt point at that tile's first K / V row (the
  // item's base is formed once per item, each tile adds 32 rows).
  int i_k = 0, i_tile = 0, g_issue = 0;
  Item i_it = item_at(0);
  const uint16_t* kt = k + (int64_t)i_it.seg_start * rs + (int64_t)i_it.h * D;
  const uint16_t* vt = v + (int64_t)i_it.seg_start * rs + (int64_t)i_it.h * D;
  auto issue_next = [&]() __attribute__((always_inline)) {
    if (i_k >= n_items) return;
    const u32x4_t rk = rsrc_of(kt), rv = rsrc_of(vt);
    const char* kl = stage_k(g_issue);
    const char* vl = stage_v(g_issue);
    const int last = i_it.L - 1 - i_tile * 32;   // last valid row of this tile, relative to its first
#pragma unroll
    for (int tt = 0; tt < DMA_INSTR; ++tt) {
      const uint32_t row = (uint32_t)min(drow[tt], last);   // ragged tail: repeat the last row
      dma(rk, kl + (DMA_ROWS * wave + 4 * tt) * 256, row * row_bytes + (uint32_t)kch[tt] * 16u);
      dma(rv, vl + (DMA_ROWS * wave + 4 * tt) * 256, row * row_bytes + (uint32_t)vch[tt] * 16u);
    }
    ++g_issue;
    if (++i_tile == (i_it.L + 31) >> 5) {
      i_tile = 0;
      if (++i_k < n_items) {
        i_it = item_at(i_k);
        kt = k + (int64_t)i_it.seg_start * rs + (int64_t)i_it.h * D;
        vt = v + (int64_t)i_it.seg_start * rs + (int64_t)i_it.h * D;
      }
    } else {
      kt += 32 * rs;
      vt += 32 * rs;
    }
  };
  // s_waitcnt vmcnt: tile gt has landed.  Loads run two tiles ahead (before
  // the scores of tile t, after the barrier, tile t+2 is requested into the
  // stage of tile t-2, whose last reads came before that barrier), so at the
  // wait at most tile gt+1 is younger; other memory operations issued after
  // tile gt only make this wait longer, never shorter.
  auto wait_tile = [&](int gt) __attribute__((always_inline)) {
    if (g_issue - 1 - gt <= 0) __builtin_amdgcn_s_waitcnt(0x0F70);
    else __builtin_amdgcn_s_waitcnt(0x0F70 | LOADS);
  };
  static_assert(LOADS <= 15, "vmcnt encoding above assumes <= 15 loads in flight");
  auto barrier = [&]() __attribute__((always_inline)) {
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  // ---- per-lane LDS read offsets (bytes within a tile)
  int koff[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) koff[kc] = r32 * 256 + (((2 * kc + g) ^ swz_k(r32)) << 4);
  int voff[4];
  v_tr_offsets(lane, voff);

  // Q loads and O stores go through a buffer descriptor that ends at the
  // item's last valid row: rows past the segment end read as zero and their
  // stores are dropped by the range check, so every lane issues the same
  // fixed number of each (kQLoads, kOStores) with no branch, and the waits
  // below can count them.
  constexpr int kOStores = 8;
  auto rows_rsrc = [&](const uint16_t* base, const Item& it) __attribute__((always_inline)) {
    const int nrows = min(it.seg_start + it.L - it.q0, kBMs);   // >= 1
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base + (int64_t)it.q0 * rs + (int64_t)it.h * D),
                                             (short)0, (int)((uint32_t)(nrows - 1) * row_bytes + 256u),
                                             kBufferWord3);
  };
  bf16x8_t qf[8];
  auto load_q = [&](const Item& it) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rq = rows_rsrc(q, it);
    const uint32_t off = (uint32_t)(wave * 32 + r32) * row_bytes + (uint32_t)g * 16u;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc)
      qf[kc] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(off + kc * 32u), 0, 0));
  };
  auto scale_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int kc = 0; kc < 8; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[kc][e] = (__bf16)((float)qf[kc][e] * scale_log2);
  };

  f32x16_t oacc[4];
  float m_run, l_run;               // reference max (log2 units), row sum
  f32x16_t neg_m;                   // -m_run in all 16 elements: S accumulator input
  int L = 0;                        // current item's segment length

  auto compute_s = [&](const char* kh_l, f32x16_t& sacc, bool biased) __attribute__((always_inline)) {
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kh_l + koff[kc]);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kc], kc == 0 ? (biased ? neg_m : f32x16_t{}) : sacc,
                                                     0, 0, 0);
    }
  };
  auto mask_tail = [&](f32x16_t& sacc, int key_rel) __attribute__((always_inline)) {
    if (__builtin_expect(key_rel + 32 > L, 0)) {
      __asm__ volatile("; ragged tail" ::: "memory");   // keep it a branch, not selects
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = key_rel + 8 * (i >> 2) + 4 * g + (i & 3);
        if (key >= L) sacc[i] = -INFINITY;
      }
    }
  };
  // rare path of the lazy softmax (attn_common.h)
  auto update_max = [&](f32x16_t& sacc) __attribute__((always_inline)) {
    lazy_rescale_bf16(sacc, oacc, m_run, l_run, neg_m);
  };

  // ---- prologue: the first two tiles, then the first item's Q
#pragma unroll
  for (int t0 = 0; t0 < NST - 2; ++t0) issue_next();
  Item it = item_at(0);
  load_q(it);
  scale_q();

  int g_cons = 0;                   // global number of the current item's first tile
  for (int kk = 0;;) {
    // Two workgroups share each CU; at equal priority the arbiter favours the
    // older waves, so the first-placed workgroup ran ~20 % faster and the
    // second finished alone.  Alternating every wave's priority by item
    // parity gives neither a lasting preference.
    if (kk & 1) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
    L = it.L;
    const int nt = (L + 31) >> 5;
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] = f32x16_t{};
    l_run = 0.f;

    // First tile: its max sets the reference.  The memory operations issued
    // after this tile's loads are tile g_cons+1's loads, this item's Q loads
    // and the previous item's kOStores O stores, in that order: keep the
    // stores in flight, everything older has landed.
    f32x16_t scur;
    __builtin_amdgcn_s_waitcnt(0x0F70 | kOStores);
    barrier();
    issue_next();
    compute_s(stage_k(g_cons), scur, false);
    mask_tail(scur, 0);
    m_run = swap_halves_max(lane_max16(scur));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      scur[i] -= m_run;
      neg_m[i] = -m_run;
    }
    // S of tile r on the matrix cores while the vector ALU exponentiates
    // tile r-1, then O += V P for tile r-1
    for (int r = 1; r < nt; ++r) {
      const int gt = g_cons + r;
      wait_tile(gt);
      barrier();
      issue_next();
      bf16x8_t pk[2];
      f32x16_t snxt;
      __builtin_amdgcn_iglp_opt(0);
      exp2_to_bf16(scur, pk, l_run);
      compute_s(stage_k(gt), snxt, true);
      pv_half_tr(stage_v(gt - 1), voff, pk, oacc);
      mask_tail(snxt, r * 32);
      update_max(snxt);
      scur = snxt;
    }
    // Q's registers are free: request the next item's rows now
    const int k_next = kk + 1;
    Item nx = it;
    if (k_next < n_items) {
      nx = item_at(k_next);
      load_q(nx);
    }
    const int g_last = g_cons + nt - 1;
    {
      bf16x8_t pk[2];
      exp2_to_bf16(scur, pk, l_run);
      pv_half_tr(stage_v(g_last), voff, pk, oacc);
    }

    // ---- normalise and store through LDS (whole 256-byte rows per store).
    // The stages of tiles g_last-1 and g_last are free once every wave is
    // past this barrier: the loads in flight are for tiles g_last+1 and
    // g_last+2, and the next load (tile g_last+3, into g_last-1's stage)
    // follows the next item's first barrier.
    barrier();
    const float inv = 1.f / swap_halves_sum(l_run);
    {
      const int gs = (wave >> 1) ? g_last : g_last - 1;
      char* ot = (wave & 1) ? stage_v(gs) : stage_k(gs);   // 32 rows x 256 B, 16-byte chunks swizzled by row
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const uint2 st = scale_pack4_bf16(oacc[db], a4 * 4, inv);
          const int chunk = (4 * db + a4) ^ (r32 & 15);
          *reinterpret_cast<uint2*>(ot + r32 * 256 + chunk * 16 + g * 8) = st;
        }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the wave's tile is in LDS
      const __amdgpu_buffer_rsrc_t ro = rows_rsrc(o, it);
      static_assert(kOStores == 8, "one store per 4 rows of the wave's 32");
#pragma unroll
      for (int i = 0; i < kOStores; ++i) {
        const int row = 4 * i + (lane >> 4), c = lane & 15;
        const u32x4_t x = *reinterpret_cast<const u32x4_t*>(ot + row * 256 + ((c ^ (row & 15)) << 4));
        __builtin_amdgcn_raw_buffer_store_b128(x, ro, (int)((uint32_t)(wave * 32 + row) * row_bytes + c * 16u), 0, 0);
      }
    }
    g_cons += nt;
    kk = k_next;
    if (kk >= n_items) break;
    it = nx;
    scale_q();   // waits for the next item's Q only: the O stores above stay in flight
  }
  // every tile load was waited for (the cursor stops at the last item's last
  // tile, which the last item consumed); LDS reads of the staging are done
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Tile counts per segment: prefix[s] = ceil(L_s / bm) (then scanned), with
// segment bounds clamped to [0, total_rows]; prefix[n_seg] = 0 before the scan.
__global__ void tile_counts_kernel(const int32_t* __restrict__ cu, int n_seg, int total_rows, int bm,
                                   int32_t* __restrict__ prefix) {
  for (int s = blockIdx.x * blockDim.x + threadIdx.x; s <= n_seg; s += gridDim.x * blockDim.x) {
    int c = 0;
    if (s < n_seg) {
      const int a = min(max(cu[s], 0), total_rows);
      const int b = max(min(cu[s + 1], total_rows), a);
      c = (b - a + bm - 1) / bm;
    }
    prefix[s] = c;
  }
}

}  // namespace

size_t attn_workspace_bytes(int64_t total_rows, int64_t n_seg) {
  (void)total_rows;
  return align_up((size_t)(n_seg + 1) * 4, 256) + scan_workspace_bytes(n_seg + 1);
}

hipError_t launch_build_tiles(const int32_t* cu, int n_seg, int total_rows, int bm,
                              int32_t* prefix, hipStream_t stream) {
  const unsigned blocks = (unsigned)std::min<int64_t>(1024, ceil_div((int64_t)n_seg + 1, 256));
  tile_counts_kernel<<<blocks, 256, 0, stream>>>(cu, n_seg, total_rows, bm, prefix);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  char* scan_ws = reinterpret_cast<char*>(prefix) + align_up((size_t)(n_seg + 1) * 4, 256);
  return exclusive_scan_i32(prefix, (int64_t)n_seg + 1, nullptr, scan_ws, stream);
}

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* o,
                            const int32_t* cu, int n_seg, int max_seqlen, int total_rows,
                            int H, int D, float scale, void* ws, hipStream_t stream) {
  int32_t* prefix = static_cast<int32_t*>(ws);
  // segments known to be short (host hint) go to the 2-workgroups-per-CU variants
  const bool short_segs = D == 128 && max_seqlen > 0 && max_seqlen <= kShortMaxLen;
  const int bm = (D == 128) ? (short_segs ? kBMs : kBM2) : kBM;
  hipError_t e = launch_build_tiles(cu, n_seg, total_rows, bm, prefix, stream);
  if (e != hipSuccess) return e;
  const int64_t t_max = ceil_div(total_rows, bm) + n_seg;
  const int64_t w_max = t_max * H;
  const int64_t grid = 8 * ceil_div(w_max, 8);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const float scale_log2 = (float)((double)scale * 1.4426950408889634);
  if (short_segs) {
    // Many items per workgroup slot: the several-items-per-workgroup variant,
    // which overlaps one item's fixed costs with another's matrix work; with
    // few, each workgroup takes one item.
    int dev = 0, n_cu = 0;
    hipError_t de = hipGetDevice(&dev);
    if (de == hipSuccess) de = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (de != hipSuccess) return de;
    const int64_t slots = 8 * ceil_div(2 * (int64_t)std::max(n_cu, 8), 8);   // two workgroups per CU
    // items per workgroup: ceil(ceil(W / 8) / (slots / 8)), W <= w_max
    const int64_t items_per_wg = ceil_div(ceil_div(w_max, 8), slots / 8);
    if (w_max >= kMultiItemsPerSlot * slots && w_max <= 0x7fffffff && items_per_wg <= kMultiMaxItems)
      attn_fwd_bf16_d128_multi_kernel<<<(unsigned)slots, 256, 0, stream>>>(
          static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
          static_cast<uint16_t*>(o), cu, prefix, n_seg, H, total_rows, scale_log2);
    else
      attn_fwd_bf16_d128_short_kernel<<<(unsigned)grid, 256, 0, stream>>>(
          static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
          static_cast<uint16_t*>(o), cu, prefix, n_seg, H, total_rows, scale_log2);
  } else if (D == 128)
    attn_fwd_bf16_d128_kernel<<<(unsigned)grid, 512, 0, stream>>>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
        static_cast<uint16_t*>(o), cu, prefix, n_seg, H, total_rows, scale_log2);
  else
    attn_fwd_bf16_kernel<64><<<(unsigned)grid, kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
        static_cast<uint16_t*>(o), cu, prefix, n_seg, H, total_rows, scale_log2);
  return hipGetLastError();
}

}  // namespace h3
