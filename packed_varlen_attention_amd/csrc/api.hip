// C ABI of libh3.so: argument validation, workspace layout and dispatch to
// the gfx950 kernels.  Every host-visible error is returned before anything
// is launched; the library allocates no device memory and keeps no state.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "h3_internal.h"

// Scratch of h3_varlen_attn_fwd_noalloc: one copy per GPU, resident until the
// process ends.  In host code `scratch` names a host-side stand-in, not device
// memory: host code only ever uses the address hipGetSymbolAddress returns
// for the current device (noalloc_scratch below).
static __device__ __align__(256) char scratch[H3_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int32_t kMaxRows = 1 << 30;
// Heads per row: keeps one 64-row tile of a head (64 * H * D * 2 bytes) below
// 2^31, the reach of the attention kernels' 32-bit tile offsets.
constexpr int32_t kMaxHeads = 4096;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A C caller may pass any int as h3_dtype; loading a value outside the
// enumerators' range as the enum type is undefined in C++, so the argument's
// bits are checked in its slot before the enum value is used anywhere.
bool dtype_valid(const h3_dtype& dt) {
  int32_t v;
  static_assert(sizeof(dt) == sizeof(v), "h3_dtype is int-sized");
  memcpy(&v, &dt, sizeof v);
  return v == H3_BF16 || v == H3_F32;
}

h3_status check_dims(int32_t H, int32_t D, const h3_dtype& dt) {
  if (!dtype_valid(dt)) return H3_ERR_DTYPE;
  if (H <= 0 || H > kMaxHeads) return H3_ERR_SHAPE;
  if (D != 64 && D != 128) return H3_ERR_UNSUPPORTED;
  return H3_OK;
}

h3_status from_hip(hipError_t e) { return e == hipSuccess ? H3_OK : H3_ERR_HIP; }

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

h3_status noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return H3_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return H3_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return H3_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return H3_OK;
}

// Host checks of the attention call that do not involve the workspace.
// Returns H3_OK with *nothing = true for an empty problem.
h3_status attn_checks(const void* q, const void* k, const void* v, const int32_t* cu_seqlens, int32_t n_seg,
                      int32_t max_seqlen, int32_t total_rows, int32_t H, int32_t D, const h3_dtype& dt,
                      float softmax_scale, const void* o, bool* nothing) {
  *nothing = false;
  h3_status st = check_dims(H, D, dt);
  if (st != H3_OK) return st;
  if (n_seg < 0 || total_rows < 0 || max_seqlen < 0 || total_rows > kMaxRows) return H3_ERR_SHAPE;
  if (!(softmax_scale >= 0.f) || !isfinite(softmax_scale)) return H3_ERR_UNSUPPORTED;
  if (total_rows == 0 || n_seg == 0) {
    *nothing = true;
    return H3_OK;
  }
  if (!q || !k || !v || !o || !cu_seqlens) return H3_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return H3_ERR_ALIGN;
  return H3_OK;
}

h3_status attn_dispatch(const void* q, const void* k, const void* v, const int32_t* cu_seqlens, int32_t n_seg,
                        int32_t max_seqlen, int32_t total_rows, int32_t H, int32_t D, h3_dtype dt,
                        float softmax_scale, void* o, void* workspace, hipStream_t stream) {
  const float scale = softmax_scale > 0.f ? softmax_scale : (float)(1.0 / sqrt((double)D));
  if (dt == H3_BF16)
    return from_hip(h3::launch_attn_bf16(q, k, v, o, cu_seqlens, n_seg, max_seqlen, total_rows, H, D,
                                         scale, workspace, stream));
  return from_hip(h3::launch_attn_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                      static_cast<const float*>(v), static_cast<float*>(o), cu_seqlens,
                                      n_seg, total_rows, H, D, scale, workspace, stream));
}

}  // namespace

extern "C" {

const char* h3_status_string(h3_status s) {
  // A C caller may pass any int: read the bits as int, since loading a value
  // outside the enumerators' range as h3_status is undefined in C++.
  int32_t v;
  static_assert(sizeof(s) == sizeof(v), "h3_status is int-sized");
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case H3_OK: return "ok";
    case H3_ERR_NULL: return "a required pointer is NULL";
    case H3_ERR_DTYPE: return "unknown dtype";
    case H3_ERR_SHAPE: return "invalid sizes (n, n_seg, H, D or rows)";
    case H3_ERR_SEQLENS: return "cu_seqlens is not a non-decreasing array starting at 0";
    case H3_ERR_CAPACITY: return "rows do not fit the buffer capacity";
    case H3_ERR_UNSUPPORTED: return "unsupported head dim, RoPE split or softmax scale";
    case H3_ERR_HIP: return "HIP launch or runtime error";
    case H3_ERR_WORKSPACE: return "workspace missing or too small";
    case H3_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
    case H3_ERR_TOO_LARGE: return "problem exceeds the fixed scratch of the no-allocation entry point";
  }
  return "unknown status";
}

const char* h3_version(void) { return "h3 0.1.0 gfx950"; }

size_t h3_pack_workspace_bytes(int32_t n, int32_t n_seg) {
  if (n < 0 || n_seg < 0) return 0;
  return h3::pack_workspace_bytes(n, n_seg);
}

h3_status h3_pack_rope(const void* q_src, const void* k_src, const void* v_src,
                       const uint8_t* tags, const int32_t* pos_thw, const int32_t* seg_id,
                       int32_t n, int32_t n_seg, int32_t H, int32_t D, h3_dtype dt,
                       const h3_rope_cfg* rope, double time_offset_frames,
                       void* q_out, void* k_out, void* v_out, int32_t capacity,
                       int32_t* cu_seqlens, int32_t* perm,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  h3_status st = check_dims(H, D, dt);
  if (st != H3_OK) return st;
  if (n < 0 || n_seg < 0 || capacity < 0 || n > kMaxRows) return H3_ERR_SHAPE;
  if (n > capacity) return H3_ERR_CAPACITY;
  if (!rope || !cu_seqlens) return H3_ERR_NULL;
  if (!isfinite(time_offset_frames)) return H3_ERR_UNSUPPORTED;
  h3::RopeDev rd;
  for (int m = 0; m < 3; ++m) {
    const h3_rope_modality& r = rope->m[m];
    if (r.d_t < 0 || r.d_h < 0 || r.d_w < 0 || (r.d_t | r.d_h | r.d_w) & 1 ||
        r.d_t + r.d_h + r.d_w != D || !(r.base > 0.0) || !isfinite(r.base) || !isfinite(r.time_scale))
      return H3_ERR_UNSUPPORTED;
    rd.base[m] = r.base;
    rd.tau_scale[m] = r.time_scale;
    rd.tau_shift[m] = r.shift_time ? time_offset_frames * 40.0 / 24.0 : 0.0;
    rd.d_t[m] = r.d_t;
    rd.d_h[m] = r.d_h;
    rd.d_w[m] = r.d_w;
  }
  if (n > 0) {
    if (!q_src || !k_src || !tags || !pos_thw || !seg_id || !q_out || !k_out || !perm) return H3_ERR_NULL;
    if (v_out && !v_src) return H3_ERR_NULL;
    if (!aligned16(q_src) || !aligned16(k_src) || !aligned16(q_out) || !aligned16(k_out) ||
        (v_out && (!aligned16(v_src) || !aligned16(v_out))))
      return H3_ERR_ALIGN;
    if (!workspace || workspace_bytes < h3::pack_workspace_bytes(n, n_seg)) return H3_ERR_WORKSPACE;
  }
  return from_hip(h3::launch_pack_rope(q_src, k_src, v_src, tags, pos_thw, seg_id, n, n_seg, H, D,
                                       dt == H3_BF16, rd, q_out, k_out, v_out, cu_seqlens, perm,
                                       workspace, stream));
}

size_t h3_attn_workspace_bytes(int32_t total_rows, int32_t n_seg) {
  if (total_rows < 0 || n_seg < 0) return 0;
  return h3::attn_workspace_bytes(total_rows, n_seg);
}

h3_status h3_varlen_attn_fwd(const void* q, const void* k, const void* v,
                             const int32_t* cu_seqlens, int32_t n_seg, int32_t max_seqlen,
                             int32_t total_rows, int32_t H, int32_t D, h3_dtype dt,
                             float softmax_scale, void* o,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  bool nothing = false;
  h3_status st = attn_checks(q, k, v, cu_seqlens, n_seg, max_seqlen, total_rows, H, D, dt, softmax_scale, o,
                             &nothing);
  if (st != H3_OK || nothing) return st;
  if (!workspace || workspace_bytes < h3::attn_workspace_bytes(total_rows, n_seg))
    return H3_ERR_WORKSPACE;
  return attn_dispatch(q, k, v, cu_seqlens, n_seg, max_seqlen, total_rows, H, D, dt, softmax_scale, o, workspace,
                       stream);
}

h3_status h3_varlen_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                                     const int32_t* cu_seqlens, int32_t n_seg, int32_t max_seqlen,
                                     int32_t total_rows, int32_t H, int32_t D, h3_dtype dt,
                                     float softmax_scale, void* o, hipStream_t stream) {
  bool nothing = false;
  h3_status st = attn_checks(q, k, v, cu_seqlens, n_seg, max_seqlen, total_rows, H, D, dt, softmax_scale, o,
                             &nothing);
  if (st != H3_OK || nothing) return st;
  if (h3::attn_workspace_bytes(total_rows, n_seg) > (size_t)H3_NOALLOC_SCRATCH_BYTES) return H3_ERR_TOO_LARGE;
  void* ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != H3_OK) return st;
  // The tile list and the scan partials in the scratch are fully rewritten
  // by every call before they are read: nothing needs clearing.
  return attn_dispatch(q, k, v, cu_seqlens, n_seg, max_seqlen, total_rows, H, D, dt, softmax_scale, o, ws,
                       stream);
}

h3_status h3_quantize_qk_fp8(const void* q, const void* k, int32_t rows, int32_t H, int32_t D, h3_dtype dt,
                             float softmax_scale, uint8_t* q8, uint8_t* qe, uint8_t* k8, uint8_t* ke,
                             hipStream_t stream) {
  if (!dtype_valid(dt)) return H3_ERR_DTYPE;
  if (dt != H3_BF16 || D != 128) return H3_ERR_UNSUPPORTED;
  if (H <= 0 || H > kMaxHeads || rows < 0 || rows > kMaxRows) return H3_ERR_SHAPE;
  if (!(softmax_scale >= 0.f) || !isfinite(softmax_scale)) return H3_ERR_UNSUPPORTED;
  if (rows == 0) return H3_OK;
  if (!q || !k || !q8 || !qe || !k8 || !ke) return H3_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(q8) || !aligned16(k8) ||
      (reinterpret_cast<uintptr_t>(qe) & 3u) || (reinterpret_cast<uintptr_t>(ke) & 3u))
    return H3_ERR_ALIGN;
  const float scale = softmax_scale > 0.f ? softmax_scale : (float)(1.0 / sqrt((double)D));
  return from_hip(h3::launch_quantize_qk_fp8(q, k, rows, H, scale, q8, k8, qe, ke, stream));
}

h3_status h3_varlen_attn_fwd_fp8qk(const uint8_t* q8, const uint8_t* qe, const uint8_t* k8, const uint8_t* ke,
                                   const void* v, const int32_t* cu_seqlens, int32_t n_seg, int32_t max_seqlen,
                                   int32_t total_rows, int32_t H, int32_t D, h3_dtype dt, void* o,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!dtype_valid(dt)) return H3_ERR_DTYPE;
  if (dt != H3_BF16 || D != 128) return H3_ERR_UNSUPPORTED;
  if (H <= 0 || H > kMaxHeads) return H3_ERR_SHAPE;
  if (n_seg < 0 || total_rows < 0 || max_seqlen < 0 || total_rows > kMaxRows) return H3_ERR_SHAPE;
  if (total_rows == 0 || n_seg == 0) return H3_OK;
  if (!q8 || !qe || !k8 || !ke || !v || !o || !cu_seqlens) return H3_ERR_NULL;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v) || !aligned16(o) ||
      (reinterpret_cast<uintptr_t>(qe) & 3u) || (reinterpret_cast<uintptr_t>(ke) & 3u))
    return H3_ERR_ALIGN;
  if (!workspace || workspace_bytes < h3::attn_workspace_bytes(total_rows, n_seg)) return H3_ERR_WORKSPACE;
  return from_hip(h3::launch_attn_fp8qk(q8, qe, k8, ke, v, o, cu_seqlens, n_seg, total_rows, H, workspace,
                                        stream));
}

size_t h3_unpack_workspace_bytes(int32_t n) {
  if (n < 0) return 0;
  return h3::unpack_workspace_bytes(n);
}

h3_status h3_unpack_by_modality(const void* o, const int32_t* perm, const uint8_t* tags_src,
                                int32_t n, int32_t H, int32_t D, h3_dtype dt,
                                void* const out[3], int32_t* const idx[3],
                                const int32_t n_per_mod[3],
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  h3_status st = check_dims(H, D, dt);
  if (st != H3_OK) return st;
  if (n < 0 || n > kMaxRows) return H3_ERR_SHAPE;
  if (!out || !idx || !n_per_mod) return H3_ERR_NULL;
  h3::UnpackOut uo;
  int64_t sum = 0;
  for (int m = 0; m < 3; ++m) {
    if (n_per_mod[m] < 0) return H3_ERR_SHAPE;
    sum += n_per_mod[m];
    uo.out[m] = out[m];
    uo.idx[m] = idx[m];
    uo.n_per_mod[m] = n_per_mod[m];
    if (out[m] && !aligned16(out[m])) return H3_ERR_ALIGN;
  }
  if (sum > n) return H3_ERR_SHAPE;
  if (n == 0) return H3_OK;
  if (!o || !perm || !tags_src) return H3_ERR_NULL;
  if (!aligned16(o)) return H3_ERR_ALIGN;
  if (!workspace || workspace_bytes < h3::unpack_workspace_bytes(n)) return H3_ERR_WORKSPACE;
  return from_hip(h3::launch_unpack(o, perm, tags_src, n, H, D, dt == H3_BF16 ? 2 : 4, uo, workspace,
                                    stream));
}

h3_status h3_unpack_euler(const void* o, const int32_t* perm, const uint8_t* tags_src,
                          const uint8_t* pinned_src, int32_t n, int32_t H, int32_t D, h3_dtype dt,
                          float* const z[3], const float* const anchor[3],
                          const double sigma[3], const double sigma_next[3],
                          int32_t* const idx[3], const int32_t n_per_mod[3],
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  h3_status st = check_dims(H, D, dt);
  if (st != H3_OK) return st;
  if (n < 0 || n > kMaxRows) return H3_ERR_SHAPE;
  if (!z || !anchor || !sigma || !sigma_next || !idx || !n_per_mod) return H3_ERR_NULL;
  h3::EulerOut eo;
  int64_t sum = 0;
  for (int m = 0; m < 3; ++m) {
    if (n_per_mod[m] < 0) return H3_ERR_SHAPE;
    sum += n_per_mod[m];
    if (z[m] && (!isfinite(sigma[m]) || !isfinite(sigma_next[m]))) return H3_ERR_UNSUPPORTED;
    if ((z[m] && !aligned16(z[m])) || (anchor[m] && !aligned16(anchor[m]))) return H3_ERR_ALIGN;
    eo.z[m] = z[m];
    eo.anchor[m] = anchor[m];
    eo.idx[m] = idx[m];
    eo.dsigma[m] = z[m] ? (float)(sigma_next[m] - sigma[m]) : 0.f;
    eo.n_per_mod[m] = n_per_mod[m];
  }
  if (sum > n) return H3_ERR_SHAPE;
  if (n == 0) return H3_OK;
  if (!o || !perm || !tags_src) return H3_ERR_NULL;
  if (!aligned16(o)) return H3_ERR_ALIGN;
  if (!workspace || workspace_bytes < h3::unpack_workspace_bytes(n)) return H3_ERR_WORKSPACE;
  return from_hip(h3::launch_unpack_euler(o, perm, tags_src, pinned_src, n, H, D, dt == H3_BF16, eo,
                                          workspace, stream));
}

h3_status h3_sigma_schedule(int32_t n_steps, double shift, double* out) {
  if (n_steps < 1) return H3_ERR_SHAPE;
  if (!out) return H3_ERR_NULL;
  if (!(shift > 0.0) || !isfinite(shift)) return H3_ERR_UNSUPPORTED;
  for (int32_t i = 0; i < n_steps; ++i) {
    const double u = 1.0 - (double)i / (double)n_steps;
    out[i] = shift * u / (1.0 + (shift - 1.0) * u);
  }
  out[n_steps] = 0.0;
  return H3_OK;
}

int32_t h3_vsa_blocks_bound(int32_t total_rows, int32_t n_seg) {
  if (total_rows < 0 || n_seg < 0) return 0;
  return (int32_t)h3::vsa_num_blocks_bound(total_rows, n_seg);
}

size_t h3_vsa_workspace_bytes(int32_t total_rows, int32_t n_seg, int32_t H) {
  if (total_rows < 0 || n_seg < 0 || H <= 0) return 0;
  return h3::vsa_workspace_bytes(total_rows, n_seg, H);
}

namespace {
h3_status vsa_common_checks(int32_t n_seg, int32_t total_rows, int32_t H, int32_t D, const h3_dtype& dt, float scale,
                            int32_t topk) {
  h3_status st = check_dims(H, D, dt);
  if (st != H3_OK) return st;
  if (D != 128) return H3_ERR_UNSUPPORTED;
  if (n_seg < 0 || total_rows < 0 || total_rows > kMaxRows || topk < 1) return H3_ERR_SHAPE;
  if (!(scale >= 0.f) || !isfinite(scale)) return H3_ERR_UNSUPPORTED;
  return H3_OK;
}
}  // namespace

h3_status h3_vsa_select(const void* q, const void* k, const int32_t* cu_seqlens, int32_t n_seg,
                        int32_t max_seqlen, int32_t total_rows, int32_t H, int32_t D, h3_dtype dt,
                        float softmax_scale, int32_t topk, int32_t* sel, float* qmean, float* kmean,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  h3_status st = vsa_common_checks(n_seg, total_rows, H, D, dt, softmax_scale, topk);
  if (st != H3_OK) return st;
  if (max_seqlen < 0) return H3_ERR_SHAPE;
  if (total_rows == 0 || n_seg == 0) return H3_OK;
  if (!q || !k || !cu_seqlens || !sel) return H3_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || (qmean && !aligned16(qmean)) || (kmean && !aligned16(kmean)))
    return H3_ERR_ALIGN;
  if (!workspace || workspace_bytes < h3::vsa_workspace_bytes(total_rows, n_seg, H)) return H3_ERR_WORKSPACE;
  const float scale = softmax_scale > 0.f ? softmax_scale : (float)(1.0 / sqrt((double)D));
  return from_hip(h3::launch_vsa_select(q, k, cu_seqlens, n_seg, max_seqlen, total_rows, H, dt == H3_BF16, topk,
                                        scale, sel, qmean, kmean, workspace, stream));
}

h3_status h3_vsa_attn_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens, int32_t n_seg,
                          int32_t total_rows, int32_t H, int32_t D, h3_dtype dt, float softmax_scale,
                          const int32_t* sel, int32_t topk, void* o, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  h3_status st = vsa_common_checks(n_seg, total_rows, H, D, dt, softmax_scale, topk);
  if (st != H3_OK) return st;
  if (dt != H3_BF16) return H3_ERR_UNSUPPORTED;
  if (total_rows == 0 || n_seg == 0) return H3_OK;
  if (!q || !k || !v || !cu_seqlens || !sel || !o) return H3_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return H3_ERR_ALIGN;
  if (!workspace || workspace_bytes < h3::vsa_workspace_bytes(total_rows, n_seg, H)) return H3_ERR_WORKSPACE;
  const float scale = softmax_scale > 0.f ? softmax_scale : (float)(1.0 / sqrt((double)D));
  return from_hip(h3::launch_vsa_attn(q, k, v, o, cu_seqlens, n_seg, total_rows, H, topk, scale, sel, workspace,
                                      stream));
}

h3_status h3_validate_seqlens(const int32_t* cu_seqlens, int32_t n_seg, int32_t capacity,
                              hipStream_t stream) {
  if (n_seg < 0 || capacity < 0) return H3_ERR_SHAPE;
  if (!cu_seqlens) return H3_ERR_NULL;
  std::vector<int32_t> h((size_t)n_seg + 1);
  if (hipMemcpyAsync(h.data(), cu_seqlens, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream) !=
      hipSuccess)
    return H3_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return H3_ERR_HIP;
  if (h[0] != 0) return H3_ERR_SEQLENS;
  for (int32_t s = 0; s < n_seg; ++s)
    if (h[s + 1] < h[s]) return H3_ERR_SEQLENS;
  if (h[n_seg] > capacity) return H3_ERR_CAPACITY;
  return H3_OK;
}

}  // extern "C"
