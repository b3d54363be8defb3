// Unpack by modality for gfx950.
//
// [P1] "生产环境下的音视频联合生成：MiniMax-H3 与 vLLM-Omni 架构解析", section 三:
// the 1-D output keeps cu_seqlens and tags, and is sliced by modality into
// the per-modality velocities.  [P3] "突破视频生成大模型的工程瓶颈",
// window-aligned SP: after attention the tokens are put back in their
// original order.
//
//   1. rank pass: per block of 1024 source tokens, each token's rank among the
//      earlier tokens of its modality in the block (wave ballots), and the
//      per-(modality, block) counts;
//   2. exclusive scan of the [3][blocks] count table; subtracting the row
//      start turns it into per-modality offsets;
//   3. move pass: one workgroup per packed row p: source row i = perm[p],
//      modality m = tags[i], rank k -> idx[m][k] = p, out[m][k] = o[p]
//      (16-byte coalesced row copy, no arithmetic on values).  Rows with
//      perm[p] < 0 hold no token; a token without a packed row keeps its slot
//      with idx -1 (written by pass 1) and an unwritten out row.
//
// The Euler epilogue ([P1] section 四, runtime loop stages 5-7: the
// rectified-flow velocity gives x0 = z - sigma v, the eta = 0 Euler step
// moves the state to sigma_next, z' = z + (sigma_next - sigma) v, with video
// and audio on their own sigma schedules, and pinned anchor rows are restored
// afterwards) replaces pass 3 by a pass that, for packed row p of modality m
// and rank k, reads the velocity row o[p] and updates the fp32 state row
// z[m][k] in place, or copies anchor[m][k] into it when the token is pinned.
// Same ranks, same coalesced 16-byte row streaming.
#include "h3_internal.h"

namespace h3 {
namespace {

constexpr int kMoveThreads = 128;

// Index outputs, pre-filled with -1 by the rank pass: a token with no packed
// row (dropped by the pack) keeps -1, every other slot is overwritten by the
// move pass that runs after it.
struct IdxFill {
  int32_t* idx[3];
  int32_t n[3];
};

__global__ __launch_bounds__(kRankBlock) void unpack_rank_kernel(const uint8_t* __restrict__ tags, int n,
                                                                 int nblk, int32_t* __restrict__ table,
                                                                 int32_t* __restrict__ local_rank,
                                                                 IdxFill fill) {
  constexpr int kWaves = kRankBlock / 64;
  __shared__ int32_t wave_cnt[kWaves][3];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = blockIdx.x * kRankBlock + threadIdx.x;
  {
    // slot i of the three index arrays laid end to end (their total is <= n)
    int j = i, mm = 0;
    while (mm < 3 && j >= fill.n[mm]) j -= fill.n[mm++];
    if (mm < 3 && fill.idx[mm]) fill.idx[mm][j] = -1;
  }
  const int m = (i < n) ? (int)tags[i] : 3;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int rank = 0;
#pragma unroll
  for (int mm = 0; mm < 3; ++mm) {
    const uint64_t b = __ballot(m == mm);
    if (m == mm) rank = __popcll(b & lt_mask);
    if (lane == 0) wave_cnt[w][mm] = __popcll(b);
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    int tot = 0;
    for (int ww = 0; ww < kWaves; ++ww) tot += wave_cnt[ww][threadIdx.x];
    table[threadIdx.x * nblk + blockIdx.x] = tot;
  }
  if (m < 3) {
    int before = 0;
    for (int ww = 0; ww < w; ++ww) before += wave_cnt[ww][m];
    local_rank[i] = before + rank;
  }
}

template <int kElemBytes>
__global__ __launch_bounds__(kMoveThreads) void unpack_move_kernel(
    const void* __restrict__ o, const int32_t* __restrict__ perm, const uint8_t* __restrict__ tags,
    int n, int nblk, int64_t row_bytes, const int32_t* __restrict__ table,
    const int32_t* __restrict__ local_rank, UnpackOut outs) {
  const int p = blockIdx.x;
  const int i = perm[p];
  if (i < 0 || i >= n) return;
  const int m = tags[i];
  if (m > 2) return;
  const int b = i / kRankBlock;
  const int kk = table[m * nblk + b] - table[m * nblk] + local_rank[i];
  if (kk < 0 || kk >= outs.n_per_mod[m]) return;
  if (threadIdx.x == 0 && outs.idx[m]) outs.idx[m][kk] = p;
  if (outs.out[m]) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(o) + p * row_bytes);
    uint4* dst = reinterpret_cast<uint4*>(static_cast<char*>(outs.out[m]) + kk * row_bytes);
    const int nch = (int)(row_bytes >> 4);
    for (int c = threadIdx.x; c < nch; c += kMoveThreads) dst[c] = src[c];
  }
}

// Euler epilogue move pass.  A row is H*D elements, walked in groups of 8
// (one 16-byte bf16 load or two fp32 loads of the velocity, two 16-byte fp32
// loads and stores of the state).
template <bool kBF16>
__global__ __launch_bounds__(kMoveThreads) void unpack_euler_kernel(
    const void* __restrict__ o, const int32_t* __restrict__ perm, const uint8_t* __restrict__ tags,
    const uint8_t* __restrict__ pinned, int n, int nblk, int64_t row_elems,
    const int32_t* __restrict__ table, const int32_t* __restrict__ local_rank, EulerOut eo) {
  const int p = blockIdx.x;
  const int i = perm[p];
  if (i < 0 || i >= n) return;
  const int m = tags[i];
  if (m > 2) return;
  const int b = i / kRankBlock;
  const int kk = table[m * nblk + b] - table[m * nblk] + local_rank[i];
  if (kk < 0 || kk >= eo.n_per_mod[m]) return;
  if (threadIdx.x == 0 && eo.idx[m]) eo.idx[m][kk] = p;
  float* z = eo.z[m];
  if (!z) return;
  float4* zr = reinterpret_cast<float4*>(z + kk * row_elems);
  const int ngrp = (int)(row_elems >> 3);
  if (pinned && pinned[i]) {
    // stage 7: re-pin (no anchor given: the row keeps its current value)
    const float* an = eo.anchor[m];
    if (!an) return;
    const float4* ar = reinterpret_cast<const float4*>(an + kk * row_elems);
    for (int c = threadIdx.x; c < ngrp; c += kMoveThreads) {
      zr[2 * c] = ar[2 * c];
      zr[2 * c + 1] = ar[2 * c + 1];
    }
    return;
  }
  const float ds = eo.dsigma[m];
  for (int c = threadIdx.x; c < ngrp; c += kMoveThreads) {
    float vv[8];
    if constexpr (kBF16) {
      const uint4 raw = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(o) + p * row_elems)[c];
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vv[2 * e] = __uint_as_float(w[e] << 16);
        vv[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
    } else {
      const float4* vr = reinterpret_cast<const float4*>(static_cast<const float*>(o) + p * row_elems);
      const float4 a = vr[2 * c], bq = vr[2 * c + 1];
      vv[0] = a.x; vv[1] = a.y; vv[2] = a.z; vv[3] = a.w;
      vv[4] = bq.x; vv[5] = bq.y; vv[6] = bq.z; vv[7] = bq.w;
    }
    float4 z0 = zr[2 * c], z1 = zr[2 * c + 1];
    z0.x = fmaf(ds, vv[0], z0.x); z0.y = fmaf(ds, vv[1], z0.y);
    z0.z = fmaf(ds, vv[2], z0.z); z0.w = fmaf(ds, vv[3], z0.w);
    z1.x = fmaf(ds, vv[4], z1.x); z1.y = fmaf(ds, vv[5], z1.y);
    z1.z = fmaf(ds, vv[6], z1.z); z1.w = fmaf(ds, vv[7], z1.w);
    zr[2 * c] = z0;
    zr[2 * c + 1] = z1;
  }
}

}  // namespace

size_t unpack_workspace_bytes(int64_t n) {
  const int64_t nblk = ceil_div(n > 0 ? n : 1, kRankBlock);
  return align_up((size_t)(3 * nblk) * 4, 256) + align_up((size_t)(n > 0 ? n : 1) * 4, 256) +
         scan_workspace_bytes(3 * nblk);
}

hipError_t launch_unpack(const void* o, const int32_t* perm, const uint8_t* tags, int n,
                         int H, int D, int elem_bytes, const UnpackOut& outs,
                         void* ws, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int nblk = (int)ceil_div(n, kRankBlock);
  char* w = static_cast<char*>(ws);
  int32_t* table = reinterpret_cast<int32_t*>(w);
  w += align_up((size_t)(3 * nblk) * 4, 256);
  int32_t* local_rank = reinterpret_cast<int32_t*>(w);
  w += align_up((size_t)n * 4, 256);
  const IdxFill fill{{outs.idx[0], outs.idx[1], outs.idx[2]},
                     {outs.n_per_mod[0], outs.n_per_mod[1], outs.n_per_mod[2]}};
  unpack_rank_kernel<<<nblk, kRankBlock, 0, stream>>>(tags, n, nblk, table, local_rank, fill);
  hipError_t e = exclusive_scan_i32(table, 3 * (int64_t)nblk, nullptr, w, stream);
  if (e != hipSuccess) return e;
  const int64_t row_bytes = (int64_t)H * D * elem_bytes;
  unpack_move_kernel<16><<<n, kMoveThreads, 0, stream>>>(o, perm, tags, n, nblk, row_bytes, table,
                                                         local_rank, outs);
  return hipGetLastError();
}

hipError_t launch_unpack_euler(const void* o, const int32_t* perm, const uint8_t* tags,
                               const uint8_t* pinned, int n, int H, int D, bool bf16,
                               const EulerOut& eo, void* ws, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int nblk = (int)ceil_div(n, kRankBlock);
  char* w = static_cast<char*>(ws);
  int32_t* table = reinterpret_cast<int32_t*>(w);
  w += align_up((size_t)(3 * nblk) * 4, 256);
  int32_t* local_rank = reinterpret_cast<int32_t*>(w);
  w += align_up((size_t)n * 4, 256);
  const IdxFill fill{{eo.idx[0], eo.idx[1], eo.idx[2]}, {eo.n_per_mod[0], eo.n_per_mod[1], eo.n_per_mod[2]}};
  unpack_rank_kernel<<<nblk, kRankBlock, 0, stream>>>(tags, n, nblk, table, local_rank, fill);
  hipError_t e = exclusive_scan_i32(table, 3 * (int64_t)nblk, nullptr, w, stream);
  if (e != hipSuccess) return e;
  const int64_t row_elems = (int64_t)H * D;
  if (bf16)
    unpack_euler_kernel<true><<<n, kMoveThreads, 0, stream>>>(o, perm, tags, pinned, n, nblk, row_elems,
                                                              table, local_rank, eo);
  else
    unpack_euler_kernel<false><<<n, kMoveThreads, 0, stream>>>(o, perm, tags, pinned, n, nblk, row_elems,
                                                               table, local_rank, eo);
  return hipGetLastError();
}

}  // namespace h3
