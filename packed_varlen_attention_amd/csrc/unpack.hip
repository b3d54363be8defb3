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
//      (16-byte coalesced row copy, no arithmetic on values).
#include "h3_internal.h"

namespace h3 {
namespace {

constexpr int kMoveThreads = 128;

__global__ __launch_bounds__(kRankBlock) void unpack_rank_kernel(const uint8_t* __restrict__ tags, int n,
                                                                 int nblk, int32_t* __restrict__ table,
                                                                 int32_t* __restrict__ local_rank) {
  constexpr int kWaves = kRankBlock / 64;
  __shared__ int32_t wave_cnt[kWaves][3];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = blockIdx.x * kRankBlock + threadIdx.x;
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
  unpack_rank_kernel<<<nblk, kRankBlock, 0, stream>>>(tags, n, nblk, table, local_rank);
  hipError_t e = exclusive_scan_i32(table, 3 * (int64_t)nblk, nullptr, w, stream);
  if (e != hipSuccess) return e;
  const int64_t row_bytes = (int64_t)H * D * elem_bytes;
  unpack_move_kernel<16><<<n, kMoveThreads, 0, stream>>>(o, perm, tags, n, nblk, row_bytes, table,
                                                         local_rank, outs);
  return hipGetLastError();
}

}  // namespace h3
