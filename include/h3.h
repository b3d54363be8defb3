/*
 * h3.h — C ABI of the packed varlen modality-RoPE attention library (libh3.so).
 *
 * The path: text, video-latent and audio-latent token rows are packed into one
 * 1-D sequence split into mutually invisible sub-sequences by cu_seqlens; RoPE
 * with modality-selected frequencies is applied to Q and K; attention runs
 * inside each sub-sequence; the output is sliced back per modality.
 *
 * Pages cited below:
 *   [P1] "生产环境下的音视频联合生成：MiniMax-H3 与 vLLM-Omni 架构解析"
 *   [P2] "vLLM-Omni 实战：基于分布式逐层卸载（DLO）在 RTX 5090 上部署 MiniMax-H3 视频音频生成服务"
 *   [P3] "突破视频生成大模型的工程瓶颈"
 *
 * Conventions shared by every call:
 *   - Device buffers are owned and allocated by the caller.  The library never
 *     allocates, keeps no state between calls and is re-entrant.  Calls that
 *     need scratch memory take a caller workspace whose size the matching
 *     h3_*_workspace_bytes() function returns; its contents need not be
 *     initialised and are meaningless after the call.  The one exception is
 *     h3_varlen_attn_fwd_noalloc, which uses a fixed library-held buffer per
 *     GPU instead (see there).
 *   - Tensors are contiguous, token-major [rows][H][D], 16-byte aligned.
 *     Element type is given by h3_dtype (bf16 = IEEE bfloat16, f32 = float).
 *   - Work is enqueued on `stream` and the call returns without waiting,
 *     except h3_validate_seqlens, which synchronises.
 *   - Errors that the host can see (NULL pointers, sizes, dtype, alignment,
 *     workspace size) return a non-zero h3_status before anything is
 *     launched.  A failed launch returns H3_ERR_HIP.  Device-side data
 *     (cu_seqlens, segment ids, tags) is checked by h3_validate_seqlens, not
 *     by the hot calls; malformed device data gives unspecified values but no
 *     access outside the buffers described here.
 */
#ifndef H3_H
#define H3_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  H3_OK = 0,
  H3_ERR_NULL = 1,         /* a required pointer is NULL */
  H3_ERR_DTYPE = 2,        /* unknown h3_dtype */
  H3_ERR_SHAPE = 3,        /* negative or inconsistent n / n_seg / H / D / rows;
                              H > 4096 */
  H3_ERR_SEQLENS = 4,      /* cu_seqlens not monotone, cu[0] != 0 (validate only) */
  H3_ERR_CAPACITY = 5,     /* rows do not fit the output capacity */
  H3_ERR_UNSUPPORTED = 6,  /* D not in {64, 128}, RoPE split invalid, bad scale */
  H3_ERR_HIP = 7,          /* a HIP launch or runtime call failed */
  H3_ERR_WORKSPACE = 8,    /* workspace NULL or smaller than required */
  H3_ERR_ALIGN = 9,        /* a tensor pointer is not 16-byte aligned */
  H3_ERR_TOO_LARGE = 10    /* the problem exceeds the fixed scratch of a
                              no-allocation entry point */
} h3_status;

/* Modality tags, one uint8 per token ([P1] section 三: discrete text / video /
 * audio label on every token, selecting the RoPE frequencies). */
typedef enum { H3_TEXT = 0, H3_VIDEO = 1, H3_AUDIO = 2 } h3_modality;

typedef enum { H3_BF16 = 0, H3_F32 = 1 } h3_dtype;

/* RoPE of one modality.  A token with position (t, h, w) has time coordinate
 *   tau = t * time_scale + (shift_time ? s * 40 / 24 : 0)
 * ([P3] long-video continuation, step 3: t_global = t_local + s * 40 / 24,
 * 40 Hz audio latents over 24 FPS video, fraction kept; time axis only).
 * The head dim is cut into consecutive slices of widths d_t, d_h, d_w
 * (d_t + d_h + d_w = D, each even) for tau, h and w.  Inside a slice of width
 * d, channels (2j, 2j+1) are rotated by theta = coord * base^(-2j/d):
 *   (x0, x1) -> (x0 cos theta - x1 sin theta, x0 sin theta + x1 cos theta). */
typedef struct {
  double base;
  double time_scale;
  int32_t shift_time;
  int32_t d_t, d_h, d_w;
} h3_rope_modality;

typedef struct { h3_rope_modality m[3]; } h3_rope_cfg;   /* indexed by h3_modality */

/* ------------------------------------------------------------------------ */
/* Pack + modality RoPE ([P1] section 三: source rows -> packed 1-D sequence
 * with cu_seqlens; modality tags select RoPE; [P3] continuation time shift).
 *
 *   q_src, k_src, v_src : [n][H][D] in source order (device, read only)
 *   tags                : uint8 [n], h3_modality per token (device).  A tag
 *                         outside 0..2 leaves that row unrotated.
 *   pos_thw             : int32 [n][3], (t, h, w) per token (device)
 *   seg_id              : int32 [n], sub-sequence of each token, 0..n_seg-1
 *                         (device).  A token with an id outside that range
 *                         belongs to no sub-sequence and gets no packed row
 *                         (then cu_seqlens[n_seg] < n).
 *   rope                : host struct; time_offset_frames = s of the shift.
 *   q_out, k_out        : [capacity][H][D] packed, Q and K rotated (device)
 *   v_out               : [capacity][H][D] packed V, or NULL to skip V
 *   cu_seqlens          : int32 [n_seg+1] out: cu[0] = 0, segment k occupies
 *                         packed rows [cu[k], cu[k+1])
 *   perm                : int32 [n] out: perm[p] = source row at packed row p
 *                         for p < cu_seqlens[n_seg], -1 from there to n
 * Packed order is the stable order by segment id: rows of one segment keep
 * their source order.  Rows [cu[n_seg], capacity) are not written.
 * Requires n <= capacity; n = 0 is a no-op apart from cu_seqlens = 0.
 * Rotation: fp64 angle and cos/sin, fp32 rotation, one RNE rounding on store. */
size_t h3_pack_workspace_bytes(int32_t n, int32_t n_seg);
h3_status h3_pack_rope(const void* q_src, const void* k_src, const void* v_src,
                       const uint8_t* tags, const int32_t* pos_thw, const int32_t* seg_id,
                       int32_t n, int32_t n_seg, int32_t H, int32_t D, h3_dtype dt,
                       const h3_rope_cfg* rope, double time_offset_frames,
                       void* q_out, void* k_out, void* v_out, int32_t capacity,
                       int32_t* cu_seqlens, int32_t* perm,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Varlen attention forward ([P1] section 三: a token attends only to keys of
 * its own sub-sequence, softmax normalised inside it, weight zero outside;
 * bidirectional.  [P1] section 六: rows past the effective length are
 * trimmed by a length, not a copy).
 *
 *   q, k, v      : packed [>= total_rows][H][D] (device)
 *   cu_seqlens   : int32 [n_seg+1] (device), non-decreasing, cu[0] = 0
 *   max_seqlen   : host hint, >= every segment length (selects tile shapes;
 *                  results do not depend on it)
 *   total_rows   : host, = cu_seqlens[n_seg]; rows >= total_rows are neither
 *                  read nor written, whatever they hold (pad rows may be NaN)
 *   softmax_scale: 0 -> 1/sqrt(D)
 *   o            : packed [>= total_rows][H][D] out, rows < total_rows written
 * O[i,h] = sum_{j in seg(i)} softmax_j(scale * Q[i,h].K[j,h]) V[j,h].
 * bf16: bf16 MFMA with fp32 accumulation and fp32 online softmax in the
 * exp2 domain; at D = 128 each Q element is multiplied by
 * softmax_scale * log2(e) and rounded to bf16 once before the QK^T product;
 * P is rounded to bf16 for the PV product; one RNE rounding of O.
 * f32: fp32 throughout.
 * Supported D: 64 and 128.  Tiles never cross a cu_seqlens boundary, so no
 * FLOP is spent on masked pairs and each segment's output is bit-identical
 * to that segment computed alone. */
size_t h3_attn_workspace_bytes(int32_t total_rows, int32_t n_seg);
h3_status h3_varlen_attn_fwd(const void* q, const void* k, const void* v,
                             const int32_t* cu_seqlens, int32_t n_seg, int32_t max_seqlen,
                             int32_t total_rows, int32_t H, int32_t D, h3_dtype dt,
                             float softmax_scale, void* o,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Attention without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, results and errors as
 * h3_varlen_attn_fwd (bit-identical output), but the attention's scratch (the
 * per-segment tile list and its scan partials) lives in a buffer of
 * H3_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on,
 * from the first call on that GPU until the process ends.  The call uses the
 * copy of the current device (the stream must belong to it) and allocates
 * nothing.  Returns H3_ERR_TOO_LARGE when h3_attn_workspace_bytes(total_rows,
 * n_seg) exceeds H3_NOALLOC_SCRATCH_BYTES (more than 65,471 segments).
 * Every call on one GPU shares that GPU's buffer: calls whose execution
 * overlaps on one GPU (on two streams, or from two threads without ordering)
 * race and give unspecified results; calls ordered on one stream are safe. */
#define H3_NOALLOC_SCRATCH_BYTES 262144
h3_status h3_varlen_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                                     const int32_t* cu_seqlens, int32_t n_seg, int32_t max_seqlen,
                                     int32_t total_rows, int32_t H, int32_t D, h3_dtype dt,
                                     float softmax_scale, void* o, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Attention with FP8 Q and K.  [P1] section 五 keeps the DiT block being
 * computed in FP8 and section 六 names a SAGE attention operator; the pages
 * give no low-precision attention algorithm.  This pair implements one
 * reading: Q (times softmax_scale * log2 e) and K stored as OCP E4M3 values
 * with one power-of-two scale per 32 consecutive channels of a row (the
 * MXFP8 layout of the OCP Microscaling format), V and P.V in bf16, and
 * attention the plain definition on the dequantized Q and K (the same
 * segment rules as h3_varlen_attn_fwd).  It trades accuracy for speed:
 * against unquantized attention the output differs by ~1e-2 relative RMS on
 * N(0, 0.25) inputs (E4M3 keeps 3 mantissa bits), against attention on the
 * dequantized values by bf16 rounding only.
 *
 * h3_quantize_qk_fp8: for every row r < rows, head h and block j of 32
 * channels, with x = Q * float32(float32(scale) * log2 e) (products in fp32)
 * or x = K: e = the smallest integer with max|x| <= 448 * 2^e (-127 for an
 * all-zero block, clamped to [-127, 127]), exponent byte e + 127, and each
 * code the E4M3 value nearest to x * 2^-e, ties to even mantissa, sign bit
 * from x.  softmax_scale 0 means 1/sqrt(D).  Q and K must be finite (an infinite or
 * NaN element makes its block's exponent and codes meaningless).
 *
 *   q, k     : packed bf16 [>= rows][H][128] (device, 16-byte aligned)
 *   q8, k8   : uint8 codes [rows][H][128] out (16-byte aligned)
 *   qe, ke   : uint8 exponent bytes [rows][H][4] out (4-byte aligned)
 *
 * h3_varlen_attn_fwd_fp8qk: O as h3_varlen_attn_fwd with scores
 * dequant(q8, qe) . dequant(k8, ke) in base-2 units (exp2), V bf16
 * [>= total_rows][H][128], O bf16 out; the workspace is the dense call's
 * (h3_attn_workspace_bytes).  Only bf16 and D = 128 (H3_ERR_UNSUPPORTED
 * otherwise). */
h3_status h3_quantize_qk_fp8(const void* q, const void* k, int32_t rows, int32_t H, int32_t D, h3_dtype dt,
                             float softmax_scale, uint8_t* q8, uint8_t* qe, uint8_t* k8, uint8_t* ke,
                             hipStream_t stream);
h3_status h3_varlen_attn_fwd_fp8qk(const uint8_t* q8, const uint8_t* qe, const uint8_t* k8, const uint8_t* ke,
                                   const void* v, const int32_t* cu_seqlens, int32_t n_seg, int32_t max_seqlen,
                                   int32_t total_rows, int32_t H, int32_t D, h3_dtype dt, void* o,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Unpack by modality ([P1] section 三: the output sequence is sliced by
 * modality into per-modality velocities; [P3] window-aligned SP: token order
 * restored after attention).
 *
 *   o          : packed [>= n][H][D] (device)
 *   perm       : int32 [n] from h3_pack_rope (device)
 *   tags_src   : uint8 [n] in source order (device)
 *   out[m]     : [n_per_mod[m]][H][D] out, or NULL to skip the copy
 *   idx[m]     : int32 [n_per_mod[m]] out (packed row of each token), or NULL
 *   n_per_mod  : host int32[3], number of tokens with tag m
 * For modality m, token k (k-th token of tag m in source order) gets
 * idx[m][k] = packed row p with perm[p] = its source row, and out[m][k] = o[p].
 * A token that no perm entry names (the pack gave it no packed row; entries
 * < 0 name no token) keeps its slot: idx[m][k] = -1, out[m][k] not written.
 * Exact copy: no arithmetic on values. */
size_t h3_unpack_workspace_bytes(int32_t n);
h3_status h3_unpack_by_modality(const void* o, const int32_t* perm, const uint8_t* tags_src,
                                int32_t n, int32_t H, int32_t D, h3_dtype dt,
                                void* const out[3], int32_t* const idx[3],
                                const int32_t n_per_mod[3],
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* VSA-style block-sparse attention ([P3] sparse-attention section, VSA: the
 * video tensor is cut into 4 x 4 x 4 = 64-token blocks; a gate scores each
 * block's relevance to the current query; only the top-k blocks are kept and
 * standard attention runs among them.  The pages give neither the gate nor
 * the top-k share.)
 *
 * Blocks: every segment's rows [cu[s], cu[s+1]) are cut into consecutive
 * blocks of 64 rows, the last one possibly shorter; lay the video grid out
 * cube by cube before packing so a block is a cube.  Blocks are numbered
 * globally in packed order; h3_vsa_blocks_bound(total_rows, n_seg) bounds
 * their count and is the row count nb_cap of the selection array.
 *
 * h3_vsa_select: gate score(b, c) = mean(Q rows of b) . mean(K rows of c) *
 * scale (fp32, per head) for blocks b, c of one segment; for every head h and
 * query block b writes sel[h][b][0..topk) = the topk highest-scoring key
 * blocks of b's segment (equal scores: lower block first), in increasing block
 * order, -1 where the segment has fewer blocks.  Rows of sel past the real
 * block count are not written.  qmean, kmean (optional, fp32
 * [nb_cap][H][D]) receive the block means.  max_seqlen (host) is a hint of
 * the longest segment (0 = unknown) that sizes the scores' on-chip buffer;
 * results do not depend on it (a longer segment is scored by a slower path
 * that gives the same selection).
 *
 * h3_vsa_attn_fwd: every row of query block b, head h, attends to the keys of
 * the blocks listed in sel[h][b] (entries < 0 end the list; blocks outside
 * b's segment are ignored; a block listed twice counts twice): softmax over
 * those keys only.  The list may be in any order; the kernel visits it from a
 * start that depends on the item's position in the launch (for L2
 * locality), so results are deterministic for a given device.  A query block
 * whose list keeps no block of its own segment has no keys: its rows of o
 * are not written.  bf16, D = 128:
 * the dense kernel's numerics (Q * scale * log2 e rounded to bf16 once, fp32
 * accumulation and softmax, bf16 P, one RNE rounding of O).  Rows
 * >= total_rows are neither read nor written.
 *
 *   q, k, v, o   : packed [>= total_rows][H][128]
 *   sel          : int32 [H][nb_cap][topk] (device)
 *   topk         : >= 1 */
int32_t h3_vsa_blocks_bound(int32_t total_rows, int32_t n_seg);
size_t h3_vsa_workspace_bytes(int32_t total_rows, int32_t n_seg, int32_t H);
h3_status h3_vsa_select(const void* q, const void* k, const int32_t* cu_seqlens, int32_t n_seg,
                        int32_t max_seqlen, int32_t total_rows, int32_t H, int32_t D, h3_dtype dt,
                        float softmax_scale, int32_t topk, int32_t* sel, float* qmean, float* kmean,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);
h3_status h3_vsa_attn_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                          int32_t n_seg, int32_t total_rows, int32_t H, int32_t D, h3_dtype dt,
                          float softmax_scale, const int32_t* sel, int32_t topk, void* o,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Unpack + denoising-step epilogue ([P1] section 四, runtime loop stages 5-7:
 * the rectified-flow velocity v gives the clean estimate x0 = z - sigma v; the
 * deterministic Euler solver (eta = 0) moves the state to the next noise
 * level, z' = x0 + sigma_next v = z + (sigma_next - sigma) v, with video and
 * audio on their own sigma schedules; then the pinned anchor rows are
 * restored to their original values).
 *
 *   o, perm, tags_src, n, H, D, dt, idx, n_per_mod: as h3_unpack_by_modality
 *                (o is the velocity, packed; idx[m] may be NULL)
 *   pinned_src : uint8 [n] in source order, non-zero = anchor row, or NULL
 *   z[m]       : fp32 state [n_per_mod[m]][H][D] of modality m in source
 *                order, updated in place; NULL = modality not stepped
 *   anchor[m]  : fp32 [n_per_mod[m]][H][D] anchor values; pinned rows of
 *                modality m are set to them (NULL: pinned rows keep z)
 *   sigma[m], sigma_next[m] : host, this step's noise levels of modality m
 * Non-pinned rows: z += (float)(sigma_next - sigma) * v, one fp32 fma per
 * element.  A token without a packed row (see h3_unpack_by_modality) has no
 * velocity: its state row is left as it is and its idx is -1.
 * Workspace: h3_unpack_workspace_bytes(n). */
h3_status h3_unpack_euler(const void* o, const int32_t* perm, const uint8_t* tags_src,
                          const uint8_t* pinned_src, int32_t n, int32_t H, int32_t D, h3_dtype dt,
                          float* const z[3], const float* const anchor[3],
                          const double sigma[3], const double sigma_next[3],
                          int32_t* const idx[3], const int32_t n_per_mod[3],
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Noise levels of one modality's schedule, host only ([P2] "vLLM-Omni 实战：
 * 基于分布式逐层卸载（DLO）在 RTX 5090 上部署 MiniMax-H3 视频音频生成服务",
 * section 服务与调用: 50 sigma points, flow shift 12 for video and 3 for
 * audio; the schedule itself is not printed).  Writes n_steps + 1 values to
 * out: sigma_i = shift u / (1 + (shift - 1) u) with u = 1 - i / n_steps for
 * i < n_steps, then 0.  shift > 0. */
h3_status h3_sigma_schedule(int32_t n_steps, double shift, double* out);

/* ------------------------------------------------------------------------ */
/* Checks cu_seqlens on the device: cu[0] == 0, non-decreasing,
 * cu[n_seg] <= capacity.  Synchronises `stream`.  Returns H3_OK,
 * H3_ERR_SEQLENS or H3_ERR_CAPACITY. */
h3_status h3_validate_seqlens(const int32_t* cu_seqlens, int32_t n_seg, int32_t capacity,
                              hipStream_t stream);

const char* h3_status_string(h3_status s);
const char* h3_version(void);

#ifdef __cplusplus
}
#endif
#endif /* H3_H */
