// Internal declarations shared by the host API and the kernel launchers of
// libh3.so.  Not part of the public ABI (include/h3.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/h3.h"

namespace h3 {

// Tokens per block of the counting passes (pack ranks, unpack ranks).
constexpr int kRankBlock = 1024;
// Elements per block of the multi-block exclusive scan.
constexpr int kScanChunk = 4096;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---- device exclusive scan of int32 in place (scan.hip) -------------------
// Workspace: scan_workspace_bytes(count).  Writes the grand total to *total.
size_t scan_workspace_bytes(int64_t count);
hipError_t exclusive_scan_i32(int32_t* data, int64_t count, int32_t* total,
                              void* ws, hipStream_t stream);

// ---- pack + RoPE (pack_rope.hip) ------------------------------------------
struct RopeDev {            // per-modality RoPE, as passed to the kernel
  double base[3];
  double tau_scale[3];
  double tau_shift[3];      // already s * 40 / 24 or 0
  int d_t[3], d_h[3], d_w[3];
};

size_t pack_workspace_bytes(int64_t n, int64_t n_seg);
hipError_t launch_pack_rope(const void* q_src, const void* k_src, const void* v_src,
                            const uint8_t* tags, const int32_t* pos, const int32_t* seg,
                            int n, int n_seg, int H, int D, bool bf16, const RopeDev& rope,
                            void* q_out, void* k_out, void* v_out,
                            int32_t* cu, int32_t* perm, void* ws, hipStream_t stream);

// ---- attention (attn_fwd.hip, attn_f32.hip) ------------------------------
size_t attn_workspace_bytes(int64_t total_rows, int64_t n_seg);
hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* o,
                            const int32_t* cu, int n_seg, int max_seqlen, int total_rows,
                            int H, int D, float scale, void* ws, hipStream_t stream);
hipError_t launch_attn_f32(const float* q, const float* k, const float* v, float* o,
                           const int32_t* cu, int n_seg, int total_rows,
                           int H, int D, float scale, void* ws, hipStream_t stream);
// Tile list: tile_prefix[s] = number of BM-row query tiles of segments < s.
hipError_t launch_build_tiles(const int32_t* cu, int n_seg, int total_rows, int bm,
                              int32_t* tile_prefix, hipStream_t stream);

// ---- VSA block-sparse attention (vsa.hip) ----------------------------------
// Blocks are 64 consecutive rows of a segment; vsa_num_blocks_bound bounds
// their count (the row count of the selection array).
int64_t vsa_num_blocks_bound(int64_t total_rows, int64_t n_seg);
size_t vsa_workspace_bytes(int64_t total_rows, int64_t n_seg, int64_t H);
hipError_t launch_vsa_select(const void* q, const void* k, const int32_t* cu, int n_seg, int max_seqlen,
                             int total_rows, int H, bool bf16, int topk, float scale, int32_t* sel,
                             float* qmean_out, float* kmean_out, void* ws, hipStream_t stream);
hipError_t launch_vsa_attn(const void* q, const void* k, const void* v, void* o, const int32_t* cu, int n_seg,
                           int total_rows, int H, int topk, float scale, const int32_t* sel, void* ws,
                           hipStream_t stream);

// ---- unpack (unpack.hip) ---------------------------------------------------
size_t unpack_workspace_bytes(int64_t n);
struct UnpackOut {
  void* out[3];
  int32_t* idx[3];
  int32_t n_per_mod[3];
};
hipError_t launch_unpack(const void* o, const int32_t* perm, const uint8_t* tags, int n,
                         int H, int D, int elem_bytes, const UnpackOut& outs,
                         void* ws, hipStream_t stream);
struct EulerOut {
  float* z[3];              // per-modality fp32 state [n_m][H][D], updated in place (NULL: skip)
  const float* anchor[3];   // per-modality anchor values (NULL: pinned rows keep z)
  int32_t* idx[3];
  float dsigma[3];          // sigma_next - sigma per modality
  int32_t n_per_mod[3];
};
hipError_t launch_unpack_euler(const void* o, const int32_t* perm, const uint8_t* tags,
                               const uint8_t* pinned, int n, int H, int D, bool bf16,
                               const EulerOut& eo, void* ws, hipStream_t stream);

// FP8 Q.K attention (attn_fp8.hip)
hipError_t launch_quantize_qk_fp8(const void* q, const void* k, int rows, int H, float scale, uint8_t* q8,
                                  uint8_t* k8, uint8_t* qe, uint8_t* ke, hipStream_t stream);
hipError_t launch_attn_fp8qk(const uint8_t* q8, const uint8_t* qe, const uint8_t* k8, const uint8_t* ke,
                             const void* v, void* o, const int32_t* cu, int n_seg, int total_rows, int H,
                             void* ws, hipStream_t stream);

}  // namespace h3
