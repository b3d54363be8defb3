// VSA-style block-sparse varlen attention for gfx950, head dim 128.
//
// [P3] "突破视频生成大模型的工程瓶颈", sparse-attention section (VSA, block-level
// sparse attention): the video tensor is cut into 4 x 4 x 4 = 64-token
// blocks; a gate scores every block's relevance to the current query; only
// the top-k blocks take part; standard attention runs among the kept blocks.
// The pages give neither the gate nor the top-k share.  Here:
//   * a block is 64 consecutive packed rows of one segment (the caller lays
//     the video grid out cube by cube); a segment's last block may be short;
//   * the gate is the scaled dot product of block means,
//     score(b, c) = mean(Q_b) . mean(K_c) * scale, per head;
//   * every (head, query block) keeps the top-k key blocks of its segment,
//     larger score first, equal scores by lower block index.
//
// Kernels:
//   1. vsa_pool_kernel: fp32 means of the Q and K rows of every block
//      (one pass over Q and K, HBM-bound);
//   2. selection: scores of every key block of the segment against each
//      query block, then the top-k with a 4-pass 8-bit radix select on
//      order-preserving keys and an ordered compaction, so each list comes
//      out in increasing block order.  vsa_select_group_kernel serves 8
//      query blocks per workgroup (the key means pass through LDS once per
//      group, the next chunk prefetched into registers);
//      vsa_select_kernel, one workgroup per query block, serves segments too
//      long for the grouped kernel's LDS.  Both sum each score in the same
//      order, so their selections are identical;
//   3. vsa_attn_kernel: one workgroup of 2 waves per (head, query block),
//      32 query rows per wave; every kept block's K and V (64 keys x 256 B)
//      goes HBM -> LDS by direct loads (inline asm, explicit waits), in two
//      32-key halves double-buffered in 32 KB, and is consumed with the
//      dense kernel's operand layout (Q pre-scaled by scale * log2 e in
//      registers, S^T = K Q^T on 32x32x16 bf16 MFMA with -m folded into the
//      accumulator input, transposed V reads, bf16 P).  Four workgroups share
//      a CU (LDS 32 KB each, at most 256 VGPRs per wave).  Each item walks
//      its kept blocks from a start position that keeps the workgroups
//      resident on one XCD on neighbouring key blocks, so the XCD's L2
//      serves most of them (described above the kernel).
#include "attn_common.h"

namespace h3 {
namespace {

constexpr int kVsaBlock = 64;
constexpr int kPoolThreads = 256;
constexpr int kSelThreads = 256;

// ---------------------------------------------------------------------------
// 1. block means.  Grid: nb_cap workgroups (an upper bound of the block
// count); workgroup j handles block j if j < bprefix[n_seg].
// qmean, kmean: fp32 [nb_cap][H][D].
// ---------------------------------------------------------------------------
template <bool kBF16>
__global__ __launch_bounds__(kPoolThreads) void vsa_pool_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ bprefix, int n_seg, int total_rows, int H, int D,
    float* __restrict__ qmean, float* __restrict__ kmean) {
  const int j = blockIdx.x;
  if (j >= bprefix[n_seg]) return;
  const int s = find_segment(bprefix, n_seg, j);
  const int seg_start = min(max(cu[s], 0), total_rows);
  const int seg_end = max(min(cu[s + 1], total_rows), seg_start);
  const int r0 = seg_start + (j - bprefix[s]) * kVsaBlock;
  const int r1 = min(r0 + kVsaBlock, seg_end);
  const float inv = 1.f / (float)(r1 - r0);
  const int64_t rs = (int64_t)H * D;
  const int nch = (int)(rs >> 3);   // 8-element chunks per row
  float4* qm = reinterpret_cast<float4*>(qmean + (int64_t)j * rs);
  float4* km = reinterpret_cast<float4*>(kmean + (int64_t)j * rs);
  for (int c = threadIdx.x; c < nch; c += kPoolThreads) {
    float aq[8], ak[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) aq[e] = ak[e] = 0.f;
    for (int r = r0; r < r1; ++r) {
      if constexpr (kBF16) {
        const uint4 xq = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q) + r * rs)[c];
        const uint4 xk = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(k) + r * rs)[c];
        const uint32_t wq[4] = {xq.x, xq.y, xq.z, xq.w}, wk[4] = {xk.x, xk.y, xk.z, xk.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          aq[2 * e] += __uint_as_float(wq[e] << 16);
          aq[2 * e + 1] += __uint_as_float(wq[e] & 0xffff0000u);
          ak[2 * e] += __uint_as_float(wk[e] << 16);
          ak[2 * e + 1] += __uint_as_float(wk[e] & 0xffff0000u);
        }
      } else {
        const float4* pq = reinterpret_cast<const float4*>(static_cast<const float*>(q) + r * rs);
        const float4* pk = reinterpret_cast<const float4*>(static_cast<const float*>(k) + r * rs);
        const float4 q0 = pq[2 * c], q1 = pq[2 * c + 1], k0 = pk[2 * c], k1 = pk[2 * c + 1];
        aq[0] += q0.x; aq[1] += q0.y; aq[2] += q0.z; aq[3] += q0.w;
        aq[4] += q1.x; aq[5] += q1.y; aq[6] += q1.z; aq[7] += q1.w;
        ak[0] += k0.x; ak[1] += k0.y; ak[2] += k0.z; ak[3] += k0.w;
        ak[4] += k1.x; ak[5] += k1.y; ak[6] += k1.z; ak[7] += k1.w;
      }
    }
    qm[2 * c] = make_float4(aq[0] * inv, aq[1] * inv, aq[2] * inv, aq[3] * inv);
    qm[2 * c + 1] = make_float4(aq[4] * inv, aq[5] * inv, aq[6] * inv, aq[7] * inv);
    km[2 * c] = make_float4(ak[0] * inv, ak[1] * inv, ak[2] * inv, ak[3] * inv);
    km[2 * c + 1] = make_float4(ak[4] * inv, ak[5] * inv, ak[6] * inv, ak[7] * inv);
  }
}

// ---------------------------------------------------------------------------
// 2. scores and top-k.  Grid: H * nb_cap workgroups, (h, b) = (w / nb_cap,
// w % nb_cap), exiting when b >= bprefix[n_seg].  Segments with more than
// max_blocks key blocks (the host bound from max_seqlen) score only their
// first max_blocks blocks.
// sel: int32 [H][nb_cap][topk], global block numbers in increasing order,
// -1 past the segment's block count.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Block-wide exclusive scan of one int per thread (kSelThreads threads);
// returns the prefix and writes the total to *total.  Each wave scans its 64
// values with lane shifts, the wave totals meet in `buf` (one int per wave
// of LDS): two barriers in all; ends with a barrier.
__device__ int block_excl_scan(int x, int* buf, int* total) {
  constexpr int kWaves = kSelThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) buf[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int v = buf[w];
    before += w < wave ? v : 0;
    tot += v;
  }
  *total = tot;
  __syncthreads();   // buf may be rewritten by the next scan
  return before + incl - x;
}

// Top-k of one query block's keys (order_key of its scores, one per key
// block of its segment; key_at(c) returns key c): writes the kept global block
// numbers cb0 + c in increasing order to out[0 .. min(topk, n_kb)) and -1 to
// the rest.  Keys larger than the k-th largest are all kept; among keys equal
// to it, the lowest block indices.  Called by all kSelThreads threads; ends
// with the writes (callers that reuse the LDS afterwards put a barrier first).
template <class KeyAt>
__device__ __forceinline__ void select_topk(const KeyAt& key_at, int n_kb, int topk, int cb0, int32_t* out,
                                            int* s_hist, int* s_scan, uint32_t& s_prefix, int& s_need) {
  const int tid = threadIdx.x;
  if (tid == 0) { s_prefix = 0u; s_need = min(topk, n_kb); }
  __syncthreads();

  const int need_total = min(topk, n_kb);
  uint32_t thresh = 0u;     // keys >= thresh are candidates; > thresh all kept
  int need_eq = 0;          // how many keys equal to thresh are kept (lowest index first)
  if (n_kb > topk) {
    // radix select of the topk-th largest key, 8 bits per pass from the top
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
      for (int i = tid; i < 256; i += kSelThreads) s_hist[i] = 0;
      __syncthreads();
      const uint32_t pre = s_prefix;
      for (int c = tid; c < n_kb; c += kSelThreads) {
        const uint32_t key = key_at(c);
        if ((key & hi_mask) == pre) atomicAdd(&s_hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      // wave 0: lane l owns digits 255-4l .. 252-4l (descending); find the
      // digit where the count of larger-or-equal keys reaches s_need
      if (tid < 64) {
        const int lane = tid;
        int cnt[4];
        int sum = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) { cnt[e] = s_hist[255 - 4 * lane - e]; sum += cnt[e]; }
        int incl = sum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int y = __shfl_up(incl, off, 64);
          if (lane >= off) incl += y;
        }
        const int excl = incl - sum;
        const int need = s_need;
        if (excl < need && incl >= need) {
          int run = excl;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (run + cnt[e] >= need) {
              const uint32_t digit = (uint32_t)(255 - 4 * lane - e);
              s_prefix = pre | (digit << shift);
              s_need = need - run;
              break;
            }
            run += cnt[e];
          }
        }
      }
      __syncthreads();
    }
    thresh = s_prefix;
    need_eq = s_need;
  }

  // ordered compaction over contiguous per-thread chunks: keys > thresh all
  // kept, keys == thresh kept for the first need_eq of them in index order
  const int chunk = (n_kb + kSelThreads - 1) / kSelThreads;
  const int c_lo = min(tid * chunk, n_kb), c_hi = min(c_lo + chunk, n_kb);
  int n_eq = 0;
  if (n_kb > topk)
    for (int c = c_lo; c < c_hi; ++c) n_eq += key_at(c) == thresh;
  int tot;
  const int eq_before = block_excl_scan(n_eq, s_scan, &tot);
  // count kept per thread (equal keys: by their rank among equal keys)
  int n_keep = 0;
  {
    int eq_rank = eq_before;
    for (int c = c_lo; c < c_hi; ++c) {
      const uint32_t key = key_at(c);
      bool keep;
      if (n_kb <= topk) keep = true;
      else if (key > thresh) keep = true;
      else if (key == thresh) keep = eq_rank++ < need_eq;
      else keep = false;
      n_keep += keep;
    }
  }
  const int keep_before = block_excl_scan(n_keep, s_scan, &tot);
  {
    int eq_rank = eq_before, pos = keep_before;
    for (int c = c_lo; c < c_hi; ++c) {
      const uint32_t key = key_at(c);
      bool keep;
      if (n_kb <= topk) keep = true;
      else if (key > thresh) keep = true;
      else if (key == thresh) keep = eq_rank++ < need_eq;
      else keep = false;
      if (keep && pos < topk) out[pos++] = cb0 + c;
    }
  }
  for (int i = need_total + tid; i < topk; i += kSelThreads) out[i] = -1;
}

// The score of a key-block mean against a scaled query mean: four partial
// sums of fmaf, one per dimension class d mod 4 (each a chain of 32 rather
// than one chain of 128, which bounded the scoring by its latency),
// combined as (s0 + s1) + (s2 + s3).  Every scoring site uses this order,
// so all of them give identical keys.
struct Score4 {
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  __device__ __forceinline__ void add(const float4 x, const float4 y) {
    s0 = fmaf(x.x, y.x, s0);
    s1 = fmaf(x.y, y.y, s1);
    s2 = fmaf(x.z, y.z, s2);
    s3 = fmaf(x.w, y.w, s3);
  }
  __device__ __forceinline__ float sum() const { return (s0 + s1) + (s2 + s3); }
};

// Keys already scored into LDS.
struct LdsKeys {
  const uint32_t* keys;
  __device__ uint32_t operator()(int c) const { return keys[c]; }
};

// Keys scored on demand, for a segment whose key blocks do not fit the LDS
// the launch sized from the max_seqlen hint: key c is the score of key block
// cb0 + c against the scaled query mean sq (in LDS, 16-byte aligned), with
// the summation order of the LDS path (Score4), so both give identical keys
// (the radix select reads every key five times, each time recomputed).
struct ScoredKeys {
  const float* kmean;
  int64_t cb0;
  int H, h;
  const float* sq;
  __device__ uint32_t operator()(int c) const {
    const float4* km = reinterpret_cast<const float4*>(kmean + ((cb0 + c) * H + h) * 128);
    const float4* q4 = reinterpret_cast<const float4*>(sq);
    Score4 sc;
#pragma unroll 8
    for (int d4 = 0; d4 < 32; ++d4) sc.add(km[d4], q4[d4]);
    return order_key(sc.sum());
  }
};

__global__ __launch_bounds__(kSelThreads) void vsa_select_kernel(
    const float* __restrict__ qmean, const float* __restrict__ kmean, const int32_t* __restrict__ bprefix,
    int n_seg, int H, int nb_cap, int max_blocks, int topk, float scale, int32_t* __restrict__ sel) {
  constexpr int D = 128;
  extern __shared__ float lds_f[];   // scores [max_blocks] then keys as uint32 (aliased)
  __shared__ __attribute__((aligned(16))) float s_q[D];
  __shared__ int s_hist[256];
  __shared__ int s_scan[kSelThreads];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;

  const int64_t w = blockIdx.x;
  const int h = (int)(w / nb_cap), b = (int)(w - (int64_t)h * nb_cap);
  const int nb = bprefix[n_seg];
  if (h >= H || b >= nb) return;
  const int s = find_segment(bprefix, n_seg, b);
  const int cb0 = bprefix[s];
  const int n_kb = bprefix[s + 1] - cb0;
  const int tid = threadIdx.x;
  int32_t* out = sel + ((int64_t)h * nb_cap + b) * topk;

  if (tid < D) s_q[tid] = qmean[((int64_t)b * H + h) * D + tid] * scale;
  __syncthreads();
  if (n_kb > max_blocks) {   // longer than the hint: scores recomputed on demand
    select_topk(ScoredKeys{kmean, cb0, H, h, s_q}, n_kb, topk, cb0, out, s_hist, s_scan, s_prefix, s_need);
    return;
  }

  // scores: one thread per key block, the query mean broadcast from LDS
  uint32_t* keys = reinterpret_cast<uint32_t*>(lds_f);
  for (int c = tid; c < n_kb; c += kSelThreads) {
    const float4* km = reinterpret_cast<const float4*>(kmean + ((int64_t)(cb0 + c) * H + h) * D);
    const float4* q4 = reinterpret_cast<const float4*>(s_q);
    Score4 sc;
#pragma unroll 8
    for (int d4 = 0; d4 < D / 4; ++d4) sc.add(km[d4], q4[d4]);
    keys[c] = order_key(sc.sum());
  }
  select_topk(LdsKeys{keys}, n_kb, topk, cb0, out, s_hist, s_scan, s_prefix, s_need);
}

// ---------------------------------------------------------------------------
// 2'. the same scores and top-k for kSelGroup query blocks of one segment and
// head per workgroup, so that the segment's key means are read once per
// group rather than once per query block (they are the kernel's whole memory
// traffic).  Grid: H * ng_cap workgroups, (h, g) = (w / ng_cap, w % ng_cap),
// g indexing groups of kSelGroup consecutive query blocks of a segment
// (gprefix: exclusive prefix of ceil(blocks / kSelGroup) per segment);
// workgroups past gprefix[n_seg] exit.  Key means go through LDS 32 rows at a
// time with coalesced loads; each score is summed in the same order as in
// vsa_select_kernel (Score4), so scores and selections are bit-identical to it.
// Dynamic LDS: kSelGroup * max_blocks keys.
// ---------------------------------------------------------------------------
constexpr int kSelGroup = 8;       // query blocks per workgroup
constexpr int kSelChunk = 32;      // key-mean rows per LDS chunk
constexpr int kSelPitch = 132;     // floats per LDS key-mean row (16-byte aligned, conflict-free b128 reads)

__global__ __launch_bounds__(kSelThreads) void vsa_select_group_kernel(
    const float* __restrict__ qmean, const float* __restrict__ kmean, const int32_t* __restrict__ bprefix,
    const int32_t* __restrict__ gprefix, int n_seg, int H, int nb_cap, int ng_cap, int max_blocks, int topk,
    float scale, int32_t* __restrict__ sel) {
  constexpr int D = 128;
  static_assert(kSelThreads == kSelGroup * kSelChunk, "one score per thread per chunk");
  extern __shared__ float lds_f[];   // keys [kSelGroup][max_blocks] as uint32
  __shared__ __attribute__((aligned(16))) float s_q[kSelGroup][D];
  __shared__ __attribute__((aligned(16))) float s_k[kSelChunk][kSelPitch];
  __shared__ int s_hist[256];
  __shared__ int s_scan[kSelThreads];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;

  const int64_t w = blockIdx.x;
  const int h = (int)(w / ng_cap), g = (int)(w - (int64_t)h * ng_cap);
  if (h >= H || g >= gprefix[n_seg]) return;
  const int s = find_segment(gprefix, n_seg, g);
  const int cb0 = bprefix[s];
  const int nb_s = bprefix[s + 1] - cb0;
  const int n_kb = nb_s;
  const bool fits = n_kb <= max_blocks;   // else: longer than the hint, scores recomputed on demand
  const int qb0 = (g - gprefix[s]) * kSelGroup;            // first query block, relative to the segment
  const int nq = min(kSelGroup, nb_s - qb0);
  const int tid = threadIdx.x;
  uint32_t* keys = reinterpret_cast<uint32_t*>(lds_f);

  // scaled query means of the group (rows past the group's end: zero, unused)
  for (int i = tid; i < kSelGroup * D; i += kSelThreads) {
    const int j = i / D, d = i - j * D;
    s_q[j][d] = j < nq ? qmean[((int64_t)(cb0 + qb0 + j) * H + h) * D + d] * scale : 0.f;
  }
  // thread -> (query j, key row r of the chunk)
  const int j = tid / kSelChunk, r = tid - j * kSelChunk;
  // Key-mean chunks: 32 rows x 128 floats, 32 lanes per row (512 contiguous
  // bytes per row), PER float4 per thread; the next chunk is loaded into
  // registers while the current one is scored.
  constexpr int PER = kSelChunk * (D / 4) / kSelThreads;
  static_assert(PER * kSelThreads == kSelChunk * (D / 4), "whole float4 per thread");
  float4 pf[PER];
  auto load_chunk = [&](int c0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * kSelThreads;
      const int rr = i / (D / 4), d4 = i - rr * (D / 4);
      pf[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c0 + rr < n_kb) pf[u] = reinterpret_cast<const float4*>(kmean + ((int64_t)(cb0 + c0 + rr) * H + h) * D)[d4];
    }
  };
  if (fits) load_chunk(0);
  for (int c0 = 0; c0 < (fits ? n_kb : 0); c0 += kSelChunk) {
    __syncthreads();   // s_q written / previous chunk consumed
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * kSelThreads;
      const int rr = i / (D / 4), d4 = i - rr * (D / 4);
      *reinterpret_cast<float4*>(&s_k[rr][4 * d4]) = pf[u];
    }
    __syncthreads();
    if (c0 + kSelChunk < n_kb) load_chunk(c0 + kSelChunk);
    if (j < nq && c0 + r < n_kb) {
      Score4 sc;
#pragma unroll 8
      for (int d4 = 0; d4 < D / 4; ++d4)
        sc.add(*reinterpret_cast<const float4*>(&s_k[r][4 * d4]), *reinterpret_cast<const float4*>(&s_q[j][4 * d4]));
      keys[j * max_blocks + c0 + r] = order_key(sc.sum());
    }
  }
  for (int jj = 0; jj < nq; ++jj) {
    __syncthreads();   // keys complete / previous selection's LDS use finished
    int32_t* out = sel + ((int64_t)h * nb_cap + cb0 + qb0 + jj) * topk;
    if (fits)
      select_topk(LdsKeys{keys + jj * max_blocks}, n_kb, topk, cb0, out, s_hist, s_scan, s_prefix, s_need);
    else
      select_topk(ScoredKeys{kmean, cb0, H, h, s_q[jj]}, n_kb, topk, cb0, out, s_hist, s_scan, s_prefix, s_need);
  }
}

// ---------------------------------------------------------------------------
// 3. block-sparse attention.  Grid: 8 * ceil(H * nb_cap / 8) workgroups of
// 128 threads, head-major and cut into 8 contiguous chunks (one per XCD) like
// the dense kernel; item w = (h, b) = (w / nb_cap, w % nb_cap).
//
// Key-block order (L2 locality).  A head's K/V (tens of MB) is far larger
// than an XCD's L2, and with unrelated selections the workgroups resident on
// one XCD, all of one head, would each sweep their kept blocks from the
// first, at different phases, through the whole of it.  Instead each item
// starts its (increasing) list at the first kept block at or after position
// ((item index on the XCD) mod R) / R of the segment and wraps around, R
// being the number of workgroups resident per XCD: items start in that order
// one R-th of an item's run time apart, so at any moment the resident
// workgroups sweep a common neighbourhood of key blocks, which the L2 then
// holds.  The order depends only on the item, so results are deterministic;
// softmax does not depend on the order up to rounding.
//
// Pipeline: the 64-key block is loaded in two 32-key halves, each into its
// own K and V arrays; while one half is consumed, the other half's arrays
// receive the next half (this block's second, the next block's first).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128, 2) void vsa_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, const int32_t* __restrict__ cu, const int32_t* __restrict__ bprefix,
    const int32_t* __restrict__ sel, int n_seg, int H, int total_rows, int nb_cap, int topk, int resident,
    float scale_log2) {
  constexpr int D = 128;
  constexpr int NW = 2;                    // waves per workgroup
  constexpr int HALF_ROWS = 32 / NW;       // rows of a 32-key half each wave loads per tensor
  constexpr int DMA_INSTR = HALF_ROWS / 4; // 4 rows (1 KB) per load instruction
  // one array per half and tensor
  __shared__ __attribute__((aligned(1024))) char lk0[kTileBytes / 2], lk1[kTileBytes / 2];
  __shared__ __attribute__((aligned(1024))) char lv0[kTileBytes / 2], lv1[kTileBytes / 2];

  const int64_t W = (int64_t)H * nb_cap;
  const int64_t per = (W + 7) >> 3;
  const int64_t jj = blockIdx.x >> 3;
  const int64_t w = (int64_t)(blockIdx.x & 7) * per + jj;
  if (jj >= per || w >= W) return;
  const int h = (int)(w / nb_cap), b = (int)(w - (int64_t)h * nb_cap);
  if (b >= bprefix[n_seg]) return;
  const int s = find_segment(bprefix, n_seg, b);
  const int seg_start = min(max(cu[s], 0), total_rows);
  const int seg_end = max(min(cu[s + 1], total_rows), seg_start);
  const int cb0 = bprefix[s];
  const int r0 = seg_start + (b - cb0) * kVsaBlock;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r32 = lane & 31;
  const int64_t rs = (int64_t)H * D;
  const uint32_t row_bytes = (uint32_t)(rs * 2);

  // ---- direct HBM -> LDS loads of one 32-key half: wave w fills rows
  // 16w .. 16w+15 of the half, four rows (1 KB) per instruction; lane i
  // writes LDS slot i, so it fetches the chunk that the swizzle places there.
  // Full block: the lane's offset (its row among the instruction's four, its
  // swizzled chunk) in a VGPR, the instruction's first row as the scalar
  // offset.  The K swizzle depends on the row mod 16 (one VGPR per
  // instruction), the V swizzle on the row mod 4 (one VGPR).
  const int lrow = lane >> 4;
  uint32_t koff_dma[DMA_INSTR];
#pragma unroll
  for (int tt = 0; tt < DMA_INSTR; ++tt)
    koff_dma[tt] = (uint32_t)lrow * row_bytes + (uint32_t)(((lane & 15) ^ swz_k(4 * tt + lrow)) << 4);
  const uint32_t voff_dma = (uint32_t)lrow * row_bytes + (uint32_t)(((lane & 15) ^ swz_v(lrow)) << 4);
  const uint16_t* kh = k + (int64_t)h * D;
  const uint16_t* vh = v + (int64_t)h * D;
  // The loads are inline asm: the compiler's wait-count pass does not see
  // them, so it cannot add waits for them (it cannot tell the two halves'
  // arrays apart across the walk's back-edge and would wait for the other
  // half's loads before reading this half); every wait on them is explicit.
  // m0 holds the LDS destination of a load-to-LDS instruction; the asm sets it
  // before every load and nothing else in this kernel uses m0.
  typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));
  auto rsrc_of = [&](const uint16_t* base) __attribute__((always_inline)) -> u32x4v_t {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return u32x4v_t{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu)),
                    64u * row_bytes, (uint32_t)kBufferWord3};
  };
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  auto dma = [&](const u32x4v_t& rsrc, const char* lds, uint32_t voffset, uint32_t soffset) __attribute__((always_inline)) {
    const uint32_t m0v = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)lds);
    __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     :: "s"(m0v), "v"(voffset), "s"(rsrc), "s"(soffset) : "memory", "m0");
  };
#pragma clang diagnostic pop
  auto issue_half = [&](int kr0, int len, auto half_c) __attribute__((always_inline)) {
    constexpr int half = decltype(half_c)::value;
    char* dk = half ? lk1 : lk0;
    char* dv = half ? lv1 : lv0;
    const u32x4v_t rk = rsrc_of(kh + (int64_t)kr0 * rs);
    const u32x4v_t rv = rsrc_of(vh + (int64_t)kr0 * rs);
    if (__builtin_expect(len == kVsaBlock, 1)) {
#pragma unroll
      for (int tt = 0; tt < DMA_INSTR; ++tt) {
        const int row0 = 32 * half + HALF_ROWS * wave + 4 * tt;
        const uint32_t so = (uint32_t)__builtin_amdgcn_readfirstlane((int)(row0 * row_bytes));
        dma(rk, dk + (HALF_ROWS * wave + 4 * tt) * 256, koff_dma[tt], so);
        dma(rv, dv + (HALF_ROWS * wave + 4 * tt) * 256, voff_dma, so);
      }
    } else {
#pragma unroll
      for (int tt = 0; tt < DMA_INSTR; ++tt) {
        // ragged block: rows past its end repeat its last row
        const uint32_t row = (uint32_t)min(32 * half + HALF_ROWS * wave + 4 * tt + lrow, len - 1);
        const uint32_t kc = (uint32_t)(((lane & 15) ^ swz_k(4 * tt + lrow)) << 4);
        const uint32_t vc = (uint32_t)(((lane & 15) ^ swz_v(lrow)) << 4);
        dma(rk, dk + (HALF_ROWS * wave + 4 * tt) * 256, row * row_bytes + kc, 0u);
        dma(rv, dv + (HALF_ROWS * wave + 4 * tt) * 256, row * row_bytes + vc, 0u);
      }
    }
  };

  // ---- kept-block list: its length (entries before the first negative)
  // and the rotated start (entries below the start position), wave-uniform
  const int32_t* my_sel = sel + ((int64_t)h * nb_cap + b) * topk;
  const int seg_blocks = bprefix[s + 1] - cb0;
  int n_list = topk, t0 = 0;
  {
    const int start = (int)(((int64_t)(jj % resident) * seg_blocks) / resident);
    for (int base = 0; base < topk; base += 64) {
      const int t = base + lane;
      const int c = t < topk ? my_sel[t] : -1;
      const uint64_t neg = __builtin_amdgcn_ballot_w64(c < 0);
      const uint64_t below = __builtin_amdgcn_ballot_w64(c >= 0 && c - cb0 < start);
      if (neg != 0) {
        const int lim = __builtin_ctzll(neg);
        n_list = base + lim;
        t0 += __builtin_popcountll(below & ((1ull << lim) - 1));
        break;
      }
      t0 += __builtin_popcountll(below);
    }
    n_list = __builtin_amdgcn_readfirstlane(n_list);
    t0 = __builtin_amdgcn_readfirstlane(t0);
    if (t0 >= n_list) t0 = 0;
  }
  // local block of the i-th entry in rotated order, -1 outside the segment
  auto entry_block = [&](int i) __attribute__((always_inline)) -> int {
    int t = t0 + i;
    if (t >= n_list) t -= n_list;
    const int cl = my_sel[__builtin_amdgcn_readfirstlane(t)] - cb0;
    return (cl >= 0 && cl < seg_blocks) ? cl : -1;
  };

  // The first valid entry sets the softmax reference.  Every later entry
  // outside the segment (possible only in a caller's list) is walked as a
  // block with no keys: it reads the first valid block's rows, all its
  // scores are masked, its P is exactly zero and O and l are unchanged.  The
  // walk then has no inner loops, which would split the accumulators' live
  // ranges and copy them on every block.
  int i = 0, cl = -1;
  while (i < n_list && (cl = entry_block(i)) < 0) ++i;
  const bool any = i < n_list;
  const int kr_first = seg_start + max(cl, 0) * kVsaBlock;
  const int len_first = min(kVsaBlock, seg_end - kr_first);
  int len = len_first;              // keys of the block being consumed (0: none)
  // entry j (j > i): first row and row count to load, keys it contributes
  auto entry_rows = [&](int j, int* kr, int* ln_load, int* ln_keys) __attribute__((always_inline)) {
    const int c = entry_block(j);
    *kr = c >= 0 ? seg_start + c * kVsaBlock : kr_first;
    *ln_load = c >= 0 ? min(kVsaBlock, seg_end - *kr) : len_first;
    *ln_keys = c >= 0 ? *ln_load : 0;
  };
  if (any) {
    issue_half(kr_first, len_first, Int<0>{});
    issue_half(kr_first, len_first, Int<1>{});
  }

  // ---- Q fragment (B operand) times scale * log2(e)
  bf16x8_t qf[8];
  const int qrow = r0 + wave * 32 + r32;
  const int q_end = min(r0 + kVsaBlock, seg_end);
  if (qrow < q_end) {
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

  int koff[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) koff[kc] = r32 * 256 + (((2 * kc + g) ^ swz_k(r32)) << 4);
  int voff[4];
  v_tr_offsets(lane, voff);

  f32x16_t oacc[4];
  float m_run = 0.f, l_run = 0.f;
  f32x16_t neg_m;

  // keys past the block's end (a segment's last, ragged block, or a block
  // without keys) get -inf; a branch, so full blocks pay no compare-and-select
  // per score
  auto mask_tail = [&](f32x16_t& sacc, int key_rel) __attribute__((always_inline)) {
    if (__builtin_expect(key_rel + 32 > len, 0)) {
      __asm__ volatile("; ragged or key-less block" ::: "memory");   // keep it a branch, not selects
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = key_rel + 8 * (e >> 2) + 4 * g + (e & 3);
        if (key >= len) sacc[e] = -INFINITY;
      }
    }
  };
  // one 32-key half: S, reference (first half) or lazy rescale test, P,
  // O += V P (O = V P for the first half)
  auto half_step = [&](const char* kl, const char* vl, int key_rel, auto first) __attribute__((always_inline)) {
    constexpr bool kFirst = decltype(first)::value != 0;
    // scheduling hint: LDS reads interleaved with the MFMAs in small groups
    __builtin_amdgcn_iglp_opt(0);
    f32x16_t sacc;
    // all K operands of the half are requested before its S MFMAs, and all V
    // operands before its exponentials: the tile loads into the other half's
    // arrays share the LDS, and these reads then have the most time to return
    // (2.3 % faster than reading each two MFMAs ahead, same bits)
    bf16x8_t kf[8];
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) kf[kc] = *reinterpret_cast<const bf16x8_t*>(kl + koff[kc]);
#pragma unroll
    for (int kc = 0; kc < 8; ++kc)
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          kf[kc], qf[kc], kc == 0 ? (kFirst ? f32x16_t{} : neg_m) : sacc, 0, 0, 0);
    bf16x8_t vf[8];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int c = 0; c < 2; ++c) vf[db * 2 + c] = v_operand_tr(vl, voff, db, c);
    mask_tail(sacc, key_rel);
    if constexpr (kFirst) {
      // the first half of the first kept block sets the reference
      m_run = swap_halves_max(lane_max16(sacc));
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sacc[e] -= m_run;
        neg_m[e] = -m_run;
      }
    } else {
      lazy_rescale_bf16(sacc, oacc, m_run, l_run, neg_m);
    }
    bf16x8_t pk[2];
    exp2_to_bf16(sacc, pk, l_run);
    // O^T += V^T P^T; the first half starts O from the MFMA's zero
    // accumulator input instead of 64 zeroed registers (same bits: the
    // products are added to +0 either way)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db * 2 + c], pk[c], (kFirst && c == 0) ? f32x16_t{} : oacc[db],
                                                           0, 0, 0);
  };
  // Barrier without the workgroup fence of __syncthreads, which would wait
  // for every tile load in flight: this wave's LDS reads complete first; the
  // tile loads are waited for explicitly (vmcnt: this wave's) before it and
  // by it (the other wave's).
  auto bar = [&]() __attribute__((always_inline)) {
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  // one kept block (entry i): its two halves, with the next entry's halves
  // requested as the arrays free up
  auto block = [&](auto first) __attribute__((always_inline)) {
    const bool more = i + 1 < n_list;
    int kr0n = kr_first, loadn = len_first, lenn = 0;
    if (more) entry_rows(i + 1, &kr0n, &loadn, &lenn);
    __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * DMA_INSTR));   // half 0 landed; half 1 may be in flight
    bar();
    half_step(lk0, lv0, 0, first);
    bar();                                                  // half 0's arrays are free
    if (more) {
      issue_half(kr0n, loadn, Int<0>{});
      __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * DMA_INSTR)); // half 1 landed; the next half 0 may be in flight
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    bar();
    half_step(lk1, lv1, 32, Int<0>{});
    bar();                                                  // half 1's arrays are free
    if (more) issue_half(kr0n, loadn, Int<1>{});
    ++i;
    len = lenn;
  };
  if (any) {
    block(Int<1>{});
    while (i < n_list) block(Int<0>{});
  }

  if (qrow < q_end && any) {
    const float inv = 1.f / swap_halves_sum(l_run);
    uint16_t* op = o + qrow * rs + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const uint2 st = scale_pack4_bf16(oacc[db], a4 * 4, inv);
        *reinterpret_cast<uint2*>(op + db * 32 + a4 * 8 + g * 4) = st;
      }
  }
}

}  // namespace

int64_t vsa_num_blocks_bound(int64_t total_rows, int64_t n_seg) {
  return ceil_div(total_rows, kVsaBlock) + n_seg;
}

size_t vsa_workspace_bytes(int64_t total_rows, int64_t n_seg, int64_t H) {
  const int64_t nb_cap = vsa_num_blocks_bound(total_rows, n_seg);
  const size_t prefix = align_up((size_t)(n_seg + 1) * 4, 256) + align_up(scan_workspace_bytes(n_seg + 1), 256);
  return 2 * prefix + 2 * align_up((size_t)(nb_cap > 0 ? nb_cap : 1) * H * 128 * 4, 256);
}

namespace {
struct VsaWs {
  int32_t* bprefix;   // query/key blocks per segment, scanned
  float* qmean;
  float* kmean;
  int32_t* gprefix;   // groups of kSelGroup blocks per segment, scanned
};
VsaWs carve(void* ws, int64_t total_rows, int64_t n_seg, int64_t H) {
  const int64_t nb_cap = vsa_num_blocks_bound(total_rows, n_seg);
  const size_t prefix = align_up((size_t)(n_seg + 1) * 4, 256) + align_up(scan_workspace_bytes(n_seg + 1), 256);
  const size_t means = align_up((size_t)(nb_cap > 0 ? nb_cap : 1) * H * 128 * 4, 256);
  char* w = static_cast<char*>(ws);
  VsaWs r;
  r.bprefix = reinterpret_cast<int32_t*>(w);
  w += prefix;
  r.qmean = reinterpret_cast<float*>(w);
  w += means;
  r.kmean = reinterpret_cast<float*>(w);
  w += means;
  r.gprefix = reinterpret_cast<int32_t*>(w);
  return r;
}
}  // namespace

// Largest per-segment key-block count for the grouped selection: its keys
// (kSelGroup * max_blocks * 4 bytes) and staging stay within 64 KB of LDS.
constexpr int kSelGroupMaxBlocks = 1280;
// Key blocks the one-query-block selection keeps in LDS: 60 KB of keys, so
// that with its static LDS (2.5 KB) the workgroup stays within 64 KB.
constexpr int kSelMaxBlocks = 15360;

hipError_t launch_vsa_select(const void* q, const void* k, const int32_t* cu, int n_seg, int max_seqlen,
                             int total_rows, int H, bool bf16, int topk, float scale, int32_t* sel,
                             float* qmean_out, float* kmean_out, void* ws, hipStream_t stream) {
  const VsaWs w = carve(ws, total_rows, n_seg, H);
  // block prefix (the dense kernel's tile-count scan with 64-row tiles)
  hipError_t e = launch_build_tiles(cu, n_seg, total_rows, kVsaBlock, w.bprefix, stream);
  if (e != hipSuccess) return e;
  const int64_t nb_cap = vsa_num_blocks_bound(total_rows, n_seg);
  if (nb_cap * H > 0x7fffffff) return hipErrorInvalidValue;   // one workgroup per (head, block)
  float* qm = qmean_out ? qmean_out : w.qmean;
  float* km = kmean_out ? kmean_out : w.kmean;
  if (bf16)
    vsa_pool_kernel<true><<<(unsigned)nb_cap, kPoolThreads, 0, stream>>>(q, k, cu, w.bprefix, n_seg, total_rows,
                                                                         H, 128, qm, km);
  else
    vsa_pool_kernel<false><<<(unsigned)nb_cap, kPoolThreads, 0, stream>>>(q, k, cu, w.bprefix, n_seg, total_rows,
                                                                          H, 128, qm, km);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // LDS for the scores, sized from the hint (0: bounded by total_rows); a
  // longer segment takes the on-demand path, so results do not depend on it
  const int64_t hint = max_seqlen > 0 ? max_seqlen : std::max(total_rows, 1);
  const int max_blocks = (int)std::min<int64_t>(std::min<int64_t>(ceil_div(hint, kVsaBlock), nb_cap),
                                                kSelMaxBlocks);
  if (max_blocks <= kSelGroupMaxBlocks) {
    // groups of kSelGroup query blocks per segment (ceil(L / (64 * kSelGroup)) of them)
    e = launch_build_tiles(cu, n_seg, total_rows, kVsaBlock * kSelGroup, w.gprefix, stream);
    if (e != hipSuccess) return e;
    const int64_t ng_cap = ceil_div(total_rows, kVsaBlock * kSelGroup) + n_seg;
    if (ng_cap * H > 0x7fffffff) return hipErrorInvalidValue;
    const size_t lds = (size_t)kSelGroup * max_blocks * 4;
    vsa_select_group_kernel<<<(unsigned)(ng_cap * H), kSelThreads, lds, stream>>>(
        qm, km, w.bprefix, w.gprefix, n_seg, H, (int)nb_cap, (int)ng_cap, max_blocks, topk, scale, sel);
    return hipGetLastError();
  }
  const size_t lds = (size_t)max_blocks * 4;
  vsa_select_kernel<<<(unsigned)(nb_cap * H), kSelThreads, lds, stream>>>(qm, km, w.bprefix, n_seg, H, (int)nb_cap,
                                                                         max_blocks, topk, scale, sel);
  return hipGetLastError();
}

hipError_t launch_vsa_attn(const void* q, const void* k, const void* v, void* o, const int32_t* cu, int n_seg,
                           int total_rows, int H, int topk, float scale, const int32_t* sel, void* ws,
                           hipStream_t stream) {
  const VsaWs w = carve(ws, total_rows, n_seg, H);
  hipError_t e = launch_build_tiles(cu, n_seg, total_rows, kVsaBlock, w.bprefix, stream);
  if (e != hipSuccess) return e;
  const int64_t nb_cap = vsa_num_blocks_bound(total_rows, n_seg);
  const int64_t grid = 8 * ceil_div(nb_cap * H, 8);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const float scale_log2 = (float)((double)scale * 1.4426950408889634);
  // workgroups resident per XCD: four per CU (32 KB of LDS and 2 waves of
  // 256 VGPRs each), CUs spread evenly over the 8 XCDs
  int dev = 0, n_cu = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int resident = std::max(1, n_cu / 8) * 4;
  vsa_attn_kernel<<<(unsigned)grid, 128, 0, stream>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
      static_cast<uint16_t*>(o), cu, w.bprefix, sel, n_seg, H, total_rows, (int)nb_cap, topk, resident,
      scale_log2);
  return hipGetLastError();
}

}  // namespace h3
