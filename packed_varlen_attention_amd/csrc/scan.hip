// Exclusive prefix sum of int32 values in device memory, in place.
//
// Three passes for any length: per-chunk sums, a single-block scan of the
// chunk sums, then a per-chunk scan seeded with its chunk offset.  A length
// that fits one chunk takes only the last pass.  Used by the stable counting
// sort of the pack step and by the modality ranks of the unpack step.
#include "h3_internal.h"

namespace h3 {
namespace {

constexpr int kScanThreads = 1024;
constexpr int kPerThread = kScanChunk / kScanThreads;   // 4

// Block-wide exclusive scan of one value per thread; returns the thread's
// exclusive prefix and writes the block total to *block_total.
__device__ int32_t block_exclusive_scan(int32_t x, int32_t* block_total) {
  __shared__ int32_t warp_sums[kScanThreads / 64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  // inclusive scan inside the wave
  int32_t incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int32_t y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) warp_sums[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    int32_t w = lane < kScanThreads / 64 ? warp_sums[lane] : 0;
    int32_t wincl = w;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int32_t y = __shfl_up(wincl, off, 64);
      if (lane >= off) wincl += y;
    }
    if (lane < kScanThreads / 64) warp_sums[lane] = wincl - w;   // exclusive wave offsets
    if (lane == kScanThreads / 64 - 1) *block_total = wincl;
  }
  __syncthreads();
  int32_t r = warp_sums[wid] + incl - x;
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kScanThreads) void chunk_sums_kernel(const int32_t* __restrict__ data,
                                                                  int64_t count,
                                                                  int32_t* __restrict__ sums) {
  const int64_t base = (int64_t)blockIdx.x * kScanChunk;
  int32_t s = 0;
#pragma unroll
  for (int r = 0; r < kPerThread; ++r) {
    int64_t i = base + (int64_t)r * kScanThreads + threadIdx.x;
    if (i < count) s += data[i];
  }
  __shared__ int32_t total;
  block_exclusive_scan(s, &total);
  if (threadIdx.x == 0) sums[blockIdx.x] = total;
}

// One block scans `count` values serially in chunks of kScanChunk (used for
// the chunk sums; their number is count / 4096).
__global__ __launch_bounds__(kScanThreads) void single_block_scan_kernel(int32_t* __restrict__ data,
                                                                         int64_t count,
                                                                         int32_t* __restrict__ total_out) {
  __shared__ int32_t carry_s;
  __shared__ int32_t tot;
  if (threadIdx.x == 0) carry_s = 0;
  __syncthreads();
  for (int64_t base = 0; base < count; base += kScanChunk) {
    int32_t v[kPerThread];
    int32_t s = 0;
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      int64_t i = base + (int64_t)threadIdx.x * kPerThread + r;
      v[r] = i < count ? data[i] : 0;
      s += v[r];
    }
    int32_t ex = block_exclusive_scan(s, &tot);
    int32_t run = carry_s + ex;
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      int64_t i = base + (int64_t)threadIdx.x * kPerThread + r;
      if (i < count) data[i] = run;
      run += v[r];
    }
    __syncthreads();
    if (threadIdx.x == 0) carry_s += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0 && total_out) *total_out = carry_s;
}

// Per-chunk exclusive scan seeded with offsets[blockIdx.x] (or 0).
__global__ __launch_bounds__(kScanThreads) void chunk_scan_kernel(int32_t* __restrict__ data,
                                                                  int64_t count,
                                                                  const int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ total_out,
                                                                  const int32_t* __restrict__ grand_total) {
  const int64_t base = (int64_t)blockIdx.x * kScanChunk;
  int32_t v[kPerThread];
  int32_t s = 0;
#pragma unroll
  for (int r = 0; r < kPerThread; ++r) {
    int64_t i = base + (int64_t)threadIdx.x * kPerThread + r;
    v[r] = i < count ? data[i] : 0;
    s += v[r];
  }
  __shared__ int32_t tot;
  int32_t run = block_exclusive_scan(s, &tot) + (offsets ? offsets[blockIdx.x] : 0);
#pragma unroll
  for (int r = 0; r < kPerThread; ++r) {
    int64_t i = base + (int64_t)threadIdx.x * kPerThread + r;
    if (i < count) data[i] = run;
    run += v[r];
  }
  if (total_out && threadIdx.x == 0 && blockIdx.x == 0) {
    // single-chunk case: the block total is the grand total
    *total_out = grand_total ? *grand_total : tot;
  }
}

}  // namespace

size_t scan_workspace_bytes(int64_t count) {
  int64_t chunks = ceil_div(count > 0 ? count : 1, kScanChunk);
  return align_up((size_t)(chunks + 1) * sizeof(int32_t), 256);
}

hipError_t exclusive_scan_i32(int32_t* data, int64_t count, int32_t* total, void* ws,
                              hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  const int64_t chunks = ceil_div(count, kScanChunk);
  if (chunks == 1) {
    chunk_scan_kernel<<<1, kScanThreads, 0, stream>>>(data, count, nullptr, total, nullptr);
    return hipGetLastError();
  }
  int32_t* sums = static_cast<int32_t*>(ws);          // [chunks]
  int32_t* grand = sums + chunks;                     // [1]
  chunk_sums_kernel<<<(unsigned)chunks, kScanThreads, 0, stream>>>(data, count, sums);
  single_block_scan_kernel<<<1, kScanThreads, 0, stream>>>(sums, chunks, grand);
  chunk_scan_kernel<<<(unsigned)chunks, kScanThreads, 0, stream>>>(data, count, sums, total, grand);
  return hipGetLastError();
}

}  // namespace h3
