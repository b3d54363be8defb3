// Varlen attention forward in fp32 (correctness path for fp32 inputs).
//
// Same definition as the bf16 kernel ([P1] "生产环境下的音视频联合生成：MiniMax-H3 与
// vLLM-Omni 架构解析", section 三: softmax only over keys of the token's own
// sub-sequence), computed with fp32 vector arithmetic: one wave per
// (query row, head); lanes split the head dim, the dot product is a wave
// reduction, and the softmax is the online (running max / running sum) form.
// Rows are grouped 4 per workgroup in tiles relative to the segment start.
#include "h3_internal.h"

namespace h3 {
namespace {

constexpr int kRowsPerBlock = 4;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, const int32_t* __restrict__ cu, const int32_t* __restrict__ prefix,
    int n_seg, int H, int total_rows, float scale) {
  constexpr int E = D / 64;
  const int T = prefix[n_seg];
  const int64_t W = (int64_t)T * H;
  const int64_t w = blockIdx.x;
  if (w >= W) return;
  const int h = (int)(w / T), t = (int)(w - (int64_t)h * T);
  int lo = 0, hi = n_seg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int s = lo;
  const int seg_start = min(max(cu[s], 0), total_rows);
  const int seg_end = max(min(cu[s + 1], total_rows), seg_start);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = seg_start + (t - prefix[s]) * kRowsPerBlock + wave;
  if (row >= seg_end) return;
  const int64_t rs = (int64_t)H * D;
  float qv[E], acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    qv[e] = q[row * rs + (int64_t)h * D + lane + 64 * e];
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int j = seg_start; j < seg_end; ++j) {
    const float* kj = k + j * rs + (int64_t)h * D;
    const float* vj = v + j * rs + (int64_t)h * D;
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) part = fmaf(qv[e], kj[lane + 64 * e], part);
    const float sc = wave_sum(part) * scale;
    const float m_new = fmaxf(m, sc);
    const float alpha = expf(m - m_new);
    const float p = expf(sc - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(p, vj[lane + 64 * e], acc[e] * alpha);
    m = m_new;
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int e = 0; e < E; ++e) o[row * rs + (int64_t)h * D + lane + 64 * e] = acc[e] * inv;
}

}  // namespace

hipError_t launch_attn_f32(const float* q, const float* k, const float* v, float* o,
                           const int32_t* cu, int n_seg, int total_rows,
                           int H, int D, float scale, void* ws, hipStream_t stream) {
  int32_t* prefix = static_cast<int32_t*>(ws);
  hipError_t e = launch_build_tiles(cu, n_seg, total_rows, kRowsPerBlock, prefix, stream);
  if (e != hipSuccess) return e;
  const int64_t t_max = ceil_div(total_rows, kRowsPerBlock) + n_seg;
  const int64_t grid = t_max * H;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (D == 128)
    attn_fwd_f32_kernel<128><<<(unsigned)grid, 256, 0, stream>>>(q, k, v, o, cu, prefix, n_seg, H,
                                                                  total_rows, scale);
  else
    attn_fwd_f32_kernel<64><<<(unsigned)grid, 256, 0, stream>>>(q, k, v, o, cu, prefix, n_seg, H,
                                                                 total_rows, scale);
  return hipGetLastError();
}

}  // namespace h3
