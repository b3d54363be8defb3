"""Packed varlen modality-RoPE attention for AMD MI355X (gfx950).

The three calls of the path, each a thin wrapper over the C ABI of libh3.so
(include/h3.h) whose work runs in hand-written HIP kernels:

  pack_rope(q, k, v, tags, pos, seg, n_seg, rope, s)  -> packed Q', K', V, cu_seqlens, perm
  varlen_attn_fwd(q, k, v, cu_seqlens, total_rows)   -> O
  varlen_attn_fwd_noalloc(...)                       -> the same O, library-held scratch, no allocation
  unpack_by_modality(o, perm, tags, n_per_mod)       -> per-modality outputs and row indices

and the denoising-step epilogue that can take unpack's place:

  unpack_euler(o, perm, tags, n_per_mod, z, sigma, sigma_next, pinned=, anchors=)
                                                     -> per-modality fp32 states stepped in place
  sigma_schedule(n_steps, shift)                     -> noise levels (host only)

and VSA-style block-sparse attention over 64-row blocks:

  vsa_select(q, k, cu_seqlens, total_rows, topk, max_seqlen) -> top-k key blocks per query block
  vsa_attn_fwd(q, k, v, cu_seqlens, total_rows, sel, topk)    -> O over the kept blocks

Build the library in-tree first: ``python -m packed_varlen_attention_amd.build``.
"""
from ._lib import (H3Error, H3_BF16, H3_F32, TEXT, VIDEO, AUDIO, LIB_PATH, SIGNATURES, load,
                   status_string, version, pack_rope, varlen_attn_fwd, varlen_attn_fwd_noalloc, unpack_by_modality,
                   unpack_euler, sigma_schedule, vsa_blocks_bound, vsa_select, vsa_attn_fwd,
                   validate_seqlens, pack_workspace_bytes, attn_workspace_bytes,
                   unpack_workspace_bytes, workspace, rope_cfg, quantize_qk_fp8,
                   varlen_attn_fwd_fp8qk)

__all__ = ["H3Error", "H3_BF16", "H3_F32", "TEXT", "VIDEO", "AUDIO", "LIB_PATH", "SIGNATURES",
           "load", "status_string", "version", "pack_rope", "varlen_attn_fwd", "varlen_attn_fwd_noalloc",
           "unpack_by_modality", "unpack_euler", "sigma_schedule", "vsa_blocks_bound", "vsa_select",
           "vsa_attn_fwd", "validate_seqlens", "pack_workspace_bytes",
           "attn_workspace_bytes", "unpack_workspace_bytes", "workspace", "rope_cfg",
           "quantize_qk_fp8", "varlen_attn_fwd_fp8qk"]
