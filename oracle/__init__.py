"""Plain CPU float64 oracle for packed varlen modality-RoPE attention.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this package.  The HIP library never
calls it and shares no code with it.

Every function is the plain definition of one step, written in float64 with
NumPy.  Citations name the page and its section:
  [P1] "生产环境下的音视频联合生成：MiniMax-H3 与 vLLM-Omni 架构解析"
  [P3] "突破视频生成大模型的工程瓶颈"

Steps and the passages they follow:
  pack            [P1] section 三 (packed sequence, cu_seqlens, its worked example)
  time_shift      [P3] long-video continuation, step 3 (RoPE global time alignment)
  rope_angles,
  apply_rope      [P1] section 三 (modality tags select RoPE frequencies) with
                  RoFormer's adjacent-pair rotation (Su et al., 2021)
  attention       [P1] section 三 (softmax normalised inside one sub-sequence,
                  out-of-segment weight zero) and section 六 (rows past the
                  last cu_seqlens entry take no part)
  unpack          [P1] section 三 (output sliced by modality) and [P3]
                  window-aligned SP (token order restored)
  block_layout,
  block_means,
  vsa_scores,
  vsa_select,
  vsa_attention,
  vsa_attention_blocks
                  [P3] sparse-attention section, VSA (64-token blocks, block
                  relevance score, top-k blocks kept, attention among the kept
                  blocks); the gate is a stand-in (block-mean dot product)
  sigma_schedule,
  x0_from_velocity,
  euler_step,
  unpack_euler    [P1] section 四 (runtime loop stages 5-7: rectified-flow
                  velocity to clean estimate, eta = 0 Euler step with separate
                  video / audio sigma schedules, re-pin of anchor rows); the
                  deployment page's 50 sigma points and flow shifts 12 / 3
  e4m3_value,
  e4m3_round,
  mx_exponent,
  quantize_mx_e4m3,
  dequantize_mx_e4m3,
  fp8qk_inputs,
  attention_base2,
  attention_base2_rows,
  attention_fp8qk [P1] section 五 keeps the active DiT block in FP8 and section
                  六 names a SAGE attention operator, with no algorithm for
                  low-precision attention: the reading taken is
                  MX block-scaled E4M3 Q and K (OCP 8-bit floating point and
                  Microscaling format definitions), the plain attention on the
                  dequantized values

Pinning (tests/test_oracle.py): the page's cu_seqlens example and exact zeros,
brute force in pure Python, torch's float64 scaled_dot_product_attention per
segment, closed forms (L = 1, Q = 0, constant V, identical keys), the complex
form of RoPE, the relative-position identity, time-shift invariance, and
key-permutation invariance; for the epilogue, the straight rectified-flow
path (one Euler step of the exact velocity lands on the path), the schedule's
closed-form values and end points, telescoping over a whole schedule, and
the re-pin rule; for VSA, keeping every block reduces to the pinned dense
attention, torch's float64 SDPA with an explicit block mask, brute-force
block means and a brute-force top-k on tiny inputs, and invariance under
permuting keys inside a kept block.  No function here is "parity unpinned".

cache.py stores oracle results on disk (off unless H3_ORACLE_CACHE names a
directory), keyed by the exact input bytes and the oracle's source, so long
float64 references resume across test runs; it computes nothing itself.
"""
from .reference import (TEXT, VIDEO, AUDIO, pack, time_shift, rope_angles, apply_rope,
                        attention, attention_rows, attention_weights, unpack, run,
                        rope_qk, sigma_schedule, x0_from_velocity, euler_step, unpack_euler,
                        block_layout, block_means, vsa_scores, vsa_select, vsa_attention, vsa_attention_blocks,
                        E4M3_MAX, e4m3_value, e4m3_round, mx_exponent, quantize_mx_e4m3,
                        dequantize_mx_e4m3, fp8qk_inputs, attention_base2, attention_base2_rows,
                        attention_fp8qk)

__all__ = ["TEXT", "VIDEO", "AUDIO", "pack", "time_shift", "rope_angles", "apply_rope",
           "attention", "attention_rows", "attention_weights", "unpack", "run", "rope_qk",
           "sigma_schedule", "x0_from_velocity", "euler_step", "unpack_euler",
           "block_layout", "block_means", "vsa_scores", "vsa_select", "vsa_attention", "vsa_attention_blocks",
           "E4M3_MAX", "e4m3_value", "e4m3_round", "mx_exponent", "quantize_mx_e4m3",
           "dequantize_mx_e4m3", "fp8qk_inputs", "attention_base2", "attention_base2_rows",
           "attention_fp8qk"]
