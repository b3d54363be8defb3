// Pack + modality RoPE for gfx950.
//
// [P1] "生产环境下的音视频联合生成：MiniMax-H3 与 vLLM-Omni 架构解析", section 三:
// source rows are concatenated into one 1-D sequence whose sub-sequences are
// marked by cu_seqlens; every token's modality tag selects its RoPE
// frequencies.  [P3] "突破视频生成大模型的工程瓶颈", long-video continuation,
// step 3: the time coordinate is shifted by s * 40 / 24 before RoPE.
//
// Packed order is a stable counting sort by segment id:
//   1. rank pass: per block of 1024 source tokens, each token's rank among the
//      earlier tokens of the same segment inside the block, and the count of
//      every (segment, block) pair, written to a [n_seg][blocks] table;
//   2. an exclusive scan of that table in (segment, block) order gives, for
//      every pair, the packed row of its first token; row 0 of each segment
//      is cu_seqlens[segment];
//   3. move pass: one workgroup per source token computes its packed row,
//      records perm (tokens whose segment id is out of range are dropped; perm
//      is -1 on the packed rows past the last segment), computes the token's D/2 rotation angles once (fp64
//      angle and cos/sin) and streams Q, K, V of all heads with 16-byte
//      coalesced loads and stores, rotating Q and K in fp32 and rounding once.
#include "h3_internal.h"

namespace h3 {
namespace {

constexpr int kMoveThreads = 128;

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int64_t count, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// Pass 1.  Inside a wave, tokens are grouped by segment with ballots (usually
// one or two groups per wave, since segments come in runs); each wave lists
// its (segment, count) groups in LDS and a token's block-local rank is its rank
// inside the wave plus the counts of its segment in earlier waves.
__global__ __launch_bounds__(kRankBlock) void pack_rank_kernel(const int32_t* __restrict__ seg,
                                                               int n, int n_seg, int nblk,
                                                               int32_t* __restrict__ table,
                                                               int32_t* __restrict__ local_rank) {
  constexpr int kWaves = kRankBlock / 64;
  __shared__ int32_t list_seg[kWaves][64];
  __shared__ int32_t list_cnt[kWaves][64];
  __shared__ int32_t list_len[kWaves];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = blockIdx.x * kRankBlock + threadIdx.x;
  int my = -1;
  if (i < n) {
    my = seg[i];
    if (my < 0 || my >= n_seg) my = -1;
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint64_t remaining = __ballot(my >= 0);
  int rank_in_wave = 0, ngroups = 0;
  while (remaining) {
    const int leader = __ffsll((unsigned long long)remaining) - 1;
    const int lseg = __shfl(my, leader, 64);
    const uint64_t m = __ballot(my == lseg);
    if (my == lseg) rank_in_wave = __popcll(m & lt_mask);
    if (lane == 0) {
      list_seg[w][ngroups] = lseg;
      list_cnt[w][ngroups] = __popcll(m);
    }
    ++ngroups;
    remaining &= ~m;
  }
  if (lane == 0) list_len[w] = ngroups;
  __syncthreads();
  if (my < 0) return;
  int before = rank_in_wave, total = 0;
  for (int ww = 0; ww < kWaves; ++ww) {
    const int len = list_len[ww];
    for (int g = 0; g < len; ++g) {
      const int c = (list_seg[ww][g] == my) ? list_cnt[ww][g] : 0;
      total += c;
      if (ww < w) before += c;
    }
  }
  local_rank[i] = before;
  if (before == total - 1) table[(int64_t)my * nblk + blockIdx.x] = total;
}

// cu_seqlens from the scanned table.  Packed rows from cu[n_seg] to n hold no
// token (their tokens' segment ids were out of range): perm = -1 there.
__global__ void write_cu_kernel(const int32_t* __restrict__ table, int n_seg, int nblk,
                                const int32_t* __restrict__ total, int32_t* __restrict__ cu,
                                int32_t* __restrict__ perm, int n) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x, stride = gridDim.x * blockDim.x;
  const int packed = min(max(*total, 0), n);
  for (int s = tid; s <= n_seg; s += stride) cu[s] = (s == n_seg) ? packed : table[(int64_t)s * nblk];
  for (int p = packed + tid; p < n; p += stride) perm[p] = -1;
}

__device__ inline float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ inline uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = (__bf16)x;  // hardware round-to-nearest-even on gfx950
  return __builtin_bit_cast(uint16_t, h);
}

// Pass 3.
template <bool kBF16>
__global__ __launch_bounds__(kMoveThreads) void pack_move_kernel(
    const void* __restrict__ q_src, const void* __restrict__ k_src, const void* __restrict__ v_src,
    const uint8_t* __restrict__ tags, const int32_t* __restrict__ pos, const int32_t* __restrict__ seg,
    int n_seg, int nblk, int H, int D, RopeDev rope,
    const int32_t* __restrict__ table, const int32_t* __restrict__ local_rank,
    void* __restrict__ q_out, void* __restrict__ k_out, void* __restrict__ v_out,
    int32_t* __restrict__ perm) {
  __shared__ float s_cos[64];
  __shared__ float s_sin[64];
  const int i = blockIdx.x;
  const int s = seg[i];
  if (s < 0 || s >= n_seg) return;
  const int p = table[(int64_t)s * nblk + i / kRankBlock] + local_rank[i];
  if (threadIdx.x == 0) perm[p] = i;

  const int half = D >> 1;
  if ((int)threadIdx.x < half) {
    const int j = threadIdx.x;
    const int m = tags[i];
    float c = 1.f, sn = 0.f;
    if (m <= 2) {
      const int pt = rope.d_t[m] >> 1, ph = rope.d_h[m] >> 1;
      double coord;
      int jj, d;
      if (j < pt) {
        coord = (double)pos[3 * (int64_t)i] * rope.tau_scale[m] + rope.tau_shift[m];
        jj = j; d = rope.d_t[m];
      } else if (j < pt + ph) {
        coord = (double)pos[3 * (int64_t)i + 1];
        jj = j - pt; d = rope.d_h[m];
      } else {
        coord = (double)pos[3 * (int64_t)i + 2];
        jj = j - pt - ph; d = rope.d_w[m];
      }
      const double theta = coord * pow(rope.base[m], -2.0 * (double)jj / (double)d);
      double sd, cd;
      sincos(theta, &sd, &cd);
      c = (float)cd;
      sn = (float)sd;
    }
    s_cos[j] = c;
    s_sin[j] = sn;
  }
  __syncthreads();

  const int64_t row = (int64_t)H * D;
  if constexpr (kBF16) {
    // 16-byte chunk = 8 bf16 = 4 channel pairs
    const int nch = (int)(row >> 3);
    const uint4* qs = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q_src) + i * row);
    const uint4* ks = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(k_src) + i * row);
    uint4* qd = reinterpret_cast<uint4*>(static_cast<uint16_t*>(q_out) + p * row);
    uint4* kd = reinterpret_cast<uint4*>(static_cast<uint16_t*>(k_out) + p * row);
    for (int c = threadIdx.x; c < nch; c += kMoveThreads) {
      const int pair0 = ((c << 3) % D) >> 1;
      uint4 xq = qs[c], xk = ks[c];
      uint32_t* wq = reinterpret_cast<uint32_t*>(&xq);
      uint32_t* wk = reinterpret_cast<uint32_t*>(&xk);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float cs = s_cos[pair0 + e], sn = s_sin[pair0 + e];
        {
          const float x0 = bf16_bits_to_f32((uint16_t)(wq[e] & 0xffff));
          const float x1 = bf16_bits_to_f32((uint16_t)(wq[e] >> 16));
          const float y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
          wq[e] = (uint32_t)f32_to_bf16_bits(y0) | ((uint32_t)f32_to_bf16_bits(y1) << 16);
        }
        {
          const float x0 = bf16_bits_to_f32((uint16_t)(wk[e] & 0xffff));
          const float x1 = bf16_bits_to_f32((uint16_t)(wk[e] >> 16));
          const float y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
          wk[e] = (uint32_t)f32_to_bf16_bits(y0) | ((uint32_t)f32_to_bf16_bits(y1) << 16);
        }
      }
      qd[c] = xq;
      kd[c] = xk;
    }
    if (v_out) {
      const uint4* vs = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(v_src) + i * row);
      uint4* vd = reinterpret_cast<uint4*>(static_cast<uint16_t*>(v_out) + p * row);
      for (int c = threadIdx.x; c < nch; c += kMoveThreads) vd[c] = vs[c];
    }
  } else {
    // 16-byte chunk = 4 floats = 2 channel pairs
    const int nch = (int)(row >> 2);
    const float4* qs = reinterpret_cast<const float4*>(static_cast<const float*>(q_src) + i * row);
    const float4* ks = reinterpret_cast<const float4*>(static_cast<const float*>(k_src) + i * row);
    float4* qd = reinterpret_cast<float4*>(static_cast<float*>(q_out) + p * row);
    float4* kd = reinterpret_cast<float4*>(static_cast<float*>(k_out) + p * row);
    for (int c = threadIdx.x; c < nch; c += kMoveThreads) {
      const int pair0 = ((c << 2) % D) >> 1;
      const float c0 = s_cos[pair0], s0 = s_sin[pair0], c1 = s_cos[pair0 + 1], s1 = s_sin[pair0 + 1];
      float4 a = qs[c], b = ks[c];
      float4 ra, rb;
      ra.x = a.x * c0 - a.y * s0; ra.y = a.x * s0 + a.y * c0;
      ra.z = a.z * c1 - a.w * s1; ra.w = a.z * s1 + a.w * c1;
      rb.x = b.x * c0 - b.y * s0; rb.y = b.x * s0 + b.y * c0;
      rb.z = b.z * c1 - b.w * s1; rb.w = b.z * s1 + b.w * c1;
      qd[c] = ra;
      kd[c] = rb;
    }
    if (v_out) {
      const float4* vs = reinterpret_cast<const float4*>(static_cast<const float*>(v_src) + i * row);
      float4* vd = reinterpret_cast<float4*>(static_cast<float*>(v_out) + p * row);
      for (int c = threadIdx.x; c < nch; c += kMoveThreads) vd[c] = vs[c];
    }
  }
}

}  // namespace

size_t pack_workspace_bytes(int64_t n, int64_t n_seg) {
  const int64_t nblk = ceil_div(n > 0 ? n : 1, kRankBlock);
  const int64_t table = n_seg * nblk;
  size_t b = 0;
  b += align_up((size_t)(table > 0 ? table : 1) * 4, 256);   // table
  b += align_up((size_t)(n > 0 ? n : 1) * 4, 256);           // local ranks
  b += 256;                                                  // total
  b += scan_workspace_bytes(table);
  return b;
}

hipError_t launch_pack_rope(const void* q_src, const void* k_src, const void* v_src,
                            const uint8_t* tags, const int32_t* pos, const int32_t* seg,
                            int n, int n_seg, int H, int D, bool bf16, const RopeDev& rope,
                            void* q_out, void* k_out, void* v_out,
                            int32_t* cu, int32_t* perm, void* ws, hipStream_t stream) {
  if (n == 0) {
    fill_i32_kernel<<<1, 256, 0, stream>>>(cu, (int64_t)n_seg + 1, 0);
    return hipGetLastError();
  }
  const int nblk = (int)ceil_div(n, kRankBlock);
  const int64_t table_n = (int64_t)n_seg * nblk;
  char* w = static_cast<char*>(ws);
  int32_t* table = reinterpret_cast<int32_t*>(w);
  w += align_up((size_t)(table_n > 0 ? table_n : 1) * 4, 256);
  int32_t* local_rank = reinterpret_cast<int32_t*>(w);
  w += align_up((size_t)n * 4, 256);
  int32_t* total = reinterpret_cast<int32_t*>(w);
  w += 256;
  void* scan_ws = w;

  const unsigned fill_blocks = (unsigned)std::min<int64_t>(4096, ceil_div(table_n + 1, 256));
  fill_i32_kernel<<<fill_blocks, 256, 0, stream>>>(table, table_n, 0);
  fill_i32_kernel<<<1, 64, 0, stream>>>(total, 1, 0);
  pack_rank_kernel<<<nblk, kRankBlock, 0, stream>>>(seg, n, n_seg, nblk, table, local_rank);
  hipError_t e = exclusive_scan_i32(table, table_n, total, scan_ws, stream);
  if (e != hipSuccess) return e;
  const unsigned cu_blocks = (unsigned)std::min<int64_t>(1024, ceil_div((int64_t)n_seg + 1, 256));
  write_cu_kernel<<<cu_blocks, 256, 0, stream>>>(table, n_seg, nblk, total, cu, perm, n);
  if (bf16)
    pack_move_kernel<true><<<n, kMoveThreads, 0, stream>>>(q_src, k_src, v_src, tags, pos, seg, n_seg,
                                                          nblk, H, D, rope, table, local_rank,
                                                          q_out, k_out, v_out, perm);
  else
    pack_move_kernel<false><<<n, kMoveThreads, 0, stream>>>(q_src, k_src, v_src, tags, pos, seg, n_seg,
                                                           nblk, H, D, rope, table, local_rank,
                                                           q_out, k_out, v_out, perm);
  return hipGetLastError();
}

}  // namespace h3
