// Diagnostic kernel: sustained v_mfma_f32_32x32x16_bf16 throughput on random
// operands.  Not on the attention path; it measures the ceiling that the
// attention kernel's matrix-core work actually runs against on the device at
// hand.  Operands that change every instruction and carry random bits draw
// far more power than constant ones, and on MI355X the clock then settles
// well below the one behind the published dense bf16 peak.
#include "attn_common.h"

namespace h3 {
namespace {

constexpr int kProbeThreads = 256;   // 4 waves; two workgroups per CU give two waves per SIMD
constexpr int kProbeSets = 8;        // operand sets cycled through

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  // integer finaliser (xor-shift / multiply rounds), used only to scatter bits
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// bf16 operand with a value uniform in [-0.5, 0.5)
__device__ __forceinline__ __bf16 rand_bf16(uint32_t key) {
  const float u = (float)(mix32(key) >> 8) * (1.0f / 16777216.0f);
  return (__bf16)(u - 0.5f);
}

__global__ __launch_bounds__(kProbeThreads, 2) void mfma_probe_kernel(float* __restrict__ out, int iters) {
  const uint32_t gid = blockIdx.x * kProbeThreads + threadIdx.x;
  bf16x8_t a[kProbeSets], b[kProbeSets];
#pragma unroll
  for (int s = 0; s < kProbeSets; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[s][e] = rand_bf16((gid * 16u + (uint32_t)s) * 8u + (uint32_t)e);
      b[s][e] = rand_bf16(0x9e3779b9u ^ ((gid * 16u + (uint32_t)s) * 8u + (uint32_t)e));
    }
  f32x16_t acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      acc[k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[(k + 3) & 7], acc[k & 3], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[j][i];
  out[gid] = s;
}

}  // namespace

hipError_t launch_mfma_probe(int workgroups, int iters, float* out, hipStream_t stream) {
  mfma_probe_kernel<<<(unsigned)workgroups, kProbeThreads, 0, stream>>>(out, iters);
  return hipGetLastError();
}

}  // namespace h3
