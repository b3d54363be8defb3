"""GPU parity of the FP8 Q.K path (h3_quantize_qk_fp8, h3_varlen_attn_fwd_fp8qk
through the C ABI) against the CPU oracle.

The quantization decides integers (E4M3 codes, block exponents) from
floating-point values; both sides form the scaled values in float32 and round
once, so codes and exponents must be bit-identical.  Attention is then
compared with the oracle's attention on the dequantized operands (base-2
exponentials) at the bf16 tolerances, since from there on the arithmetic is
the bf16 kernel's (fp32 scores and softmax, bf16 P, one rounding of O).  The
accuracy of the method itself (against unquantized attention) is a measured
property, checked against the bound E4M3's 3 mantissa bits give."""
import numpy as np
import pytest
import torch

import oracle
import packed_varlen_attention_amd as h3
import workloads as W
from gpu_common import assert_close, errors

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _packed(rows, H, seed, cap=None, spread=0.0):
    """Packed bf16 Q, K, V [cap, H, 128] ~ N(0, 0.25); with `spread`, every
    (row, head) of Q and K is scaled by exp(uniform(-spread, spread))."""
    cap = cap or rows
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q, k, v = ((torch.randn((cap, H, 128), generator=g) * 0.5) for _ in range(3))
    if spread:
        for t in (q, k):
            t.mul_(torch.exp((torch.rand((cap, H, 1), generator=g) * 2 - 1) * spread))
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def _f32(t):
    return t.float().numpy()


def _check_codes(got, q, k, rows, scale=None):
    qc, qe, kc, ke = oracle.fp8qk_inputs(_f32(q[:rows]), _f32(k[:rows]), scale)
    q8, qe8, k8, ke8 = (t[:rows].cpu().numpy() for t in got)
    assert np.array_equal(q8, qc) and np.array_equal(k8, kc)
    assert np.array_equal(qe8.astype(np.int32) - 127, qe) and np.array_equal(ke8.astype(np.int32) - 127, ke)
    return qc, qe, kc, ke


def test_fp8_quantization_bit_exact():
    rows, H = 700, 3
    q, k, _ = _packed(rows, H, seed=41, spread=20.0)     # block exponents over a wide range
    q[5, 1, 32:64] = 0.0                                  # an all-zero block
    k[7, 0, :] = 0.0
    q[9, 2, :8] = -0.0                                    # negative zeros keep their sign bit
    k[11, 1, 96:] = torch.tensor([1e-30, -1e-30] * 16, dtype=torch.bfloat16)
    k[12, 2, :32] = (torch.linspace(-1.0, 1.0, 32) * 3e38).to(torch.bfloat16)   # near the bf16 maximum
    dq, dk = q.cuda(), k.cuda()
    for scale in (None, 0.1):
        got = h3.quantize_qk_fp8(dq, dk, rows, softmax_scale=scale or 0.0)
        torch.cuda.synchronize()
        _check_codes(got, q, k, rows, scale)


@pytest.mark.parametrize("lengths", [[1, 63, 64, 65, 300, 0, 1100, 257], [2048 + 17]])
def test_fp8_attention_matches_oracle_on_dequantized_operands(lengths):
    rows, H = int(sum(lengths)), 3
    cap = rows + 40
    q, k, v = _packed(rows, H, seed=42, cap=cap, spread=1.0)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    q8, qe, k8, ke = h3.quantize_qk_fp8(dq, dk, cap)
    # pad rows of the codes hold NaN codes and V pad rows NaN: never read
    q8[rows:] = 0x7F
    k8[rows:] = 0x7F
    dv[rows:] = float("nan")
    o = torch.full_like(dv, -7.0)
    h3.varlen_attn_fwd_fp8qk(q8, qe, k8, ke, dv, torch.from_numpy(cu).cuda(), rows, max(lengths), o=o)
    torch.cuda.synchronize()
    qc, qx, kc, kx = _check_codes((q8, qe, k8, ke), q, k, rows)
    ref = oracle.attention_base2(oracle.dequantize_mx_e4m3(qc, qx), oracle.dequantize_mx_e4m3(kc, kx),
                                 _f32(v[:rows]).astype(np.float64), cu)
    assert_close(o[:rows], ref, "bf16", "fp8 Q.K attention %s" % lengths)
    assert (o[rows:] == -7.0).all()


def test_fp8_attention_h3_step_full_size_sampled():
    # the 58,758-token step's segments (256 text + 58,502 joint), 40 heads
    lengths, H = [256, 58502], 40
    rows = sum(lengths)
    q, k, v = _packed(rows, H, seed=43)
    cu = np.array([0, 256, rows], np.int32)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    q8, qe, k8, ke = h3.quantize_qk_fp8(dq, dk, rows)
    o = h3.varlen_attn_fwd_fp8qk(q8, qe, k8, ke, dv, torch.from_numpy(cu).cuda(), rows, max(lengths))
    torch.cuda.synchronize()
    heads = [0, 17, 39]
    sample = np.unique(np.concatenate([[0, 1, 255, 256, 257, 511, 512, rows - 1, rows - 64],
                                       np.random.default_rng(3).choice(rows, 48, replace=False)]))
    qs, ks, vs = _f32(q[:, heads]), _f32(k[:, heads]), _f32(v[:, heads]).astype(np.float64)
    qc, qx, kc, kx = oracle.fp8qk_inputs(qs, ks)
    assert np.array_equal(k8[:, heads].cpu().numpy(), kc) and np.array_equal(ke[:, heads].cpu().numpy().astype(np.int32) - 127, kx)
    assert np.array_equal(q8[:, heads].cpu().numpy(), qc)
    ref = oracle.attention_base2_rows(oracle.dequantize_mx_e4m3(qc, qx), oracle.dequantize_mx_e4m3(kc, kx), vs,
                                      cu, sample)
    got = o[torch.from_numpy(sample).cuda()][:, heads]
    assert_close(got, ref, "bf16", "fp8 Q.K attention, 58,758 tokens, sampled rows")


def test_fp8_attention_accuracy_against_exact_attention():
    lengths, H = [1500, 700], 4
    rows = sum(lengths)
    q, k, v = _packed(rows, H, seed=44)
    cu = np.array([0, 1500, rows], np.int32)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    q8, qe, k8, ke = h3.quantize_qk_fp8(dq, dk, rows)
    o = h3.varlen_attn_fwd_fp8qk(q8, qe, k8, ke, dv, torch.from_numpy(cu).cuda(), rows, 1500)
    torch.cuda.synchronize()
    exact = oracle.attention(*(W.to_f64(t) for t in (q, k, v)), cu)
    max_abs, rel = errors(o, exact)
    # 3 mantissa bits: ~1 % relative RMS on these N(0, 0.25) rows; a wrong
    # scale or exponent base would be off by orders of magnitude
    assert 1e-3 < rel < 3e-2, rel


@pytest.mark.parametrize("rate", [0.3, 0.04])
def test_fp8_attention_rescales_along_the_sequence(rate):
    """Logits that climb along each segment by `rate` (log2 units) per key, so
    the reference max moves every one (0.3) or every few (0.04) 32-key halves
    deep inside the main loop, including on consecutive halves: the kernel
    scales O one step after it finds the move (P.V runs one half behind the
    exponentials).  Every row checked against the oracle on the dequantized
    operands."""
    lengths, H = [3000, 1500, 200], 2
    rows = sum(lengths)
    q, k, v = _packed(rows, H, seed=45)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    amp = 4.0
    qf, kf = q.float() * 0.1, k.float() * 0.1
    qf[:, :, 0] += amp
    ramp = rate / (128 ** -0.5 * np.log2(np.e) * amp)
    for a, b in zip(cu[:-1], cu[1:]):
        kf[a:b, :, 0] += (torch.arange(b - a, dtype=torch.float32) * ramp)[:, None]
    q, k = qf.to(torch.bfloat16), kf.to(torch.bfloat16)
    q8, qe, k8, ke = h3.quantize_qk_fp8(q.cuda(), k.cuda(), rows)
    o = h3.varlen_attn_fwd_fp8qk(q8, qe, k8, ke, v.cuda(), torch.from_numpy(cu).cuda(), rows, max(lengths))
    torch.cuda.synchronize()
    qc, qx, kc, kx = _check_codes((q8, qe, k8, ke), q, k, rows)
    ref = oracle.attention_base2(oracle.dequantize_mx_e4m3(qc, qx), oracle.dequantize_mx_e4m3(kc, kx),
                                 _f32(v).astype(np.float64), cu)
    assert_close(o[:rows], ref, "bf16", "fp8 O rescale rate %g" % rate)


def test_fp8_and_vsa_attention_repeat_bit_identical():
    """Both kernels order their work by item index only (the VSA kernel's
    rotated key-block walk included), so repeated calls give identical bits."""
    lengths, H = [1300, 700, 65], 3
    rows = sum(lengths)
    q, k, v = (t.cuda() for t in _packed(rows, H, seed=46))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)).cuda()
    q8, qe, k8, ke = h3.quantize_qk_fp8(q, k, rows)
    sel = h3.vsa_select(q, k, cu, rows, 7, max_seqlen=max(lengths))
    runs = []
    for _ in range(3):
        a = h3.varlen_attn_fwd_fp8qk(q8, qe, k8, ke, v, cu, rows, max(lengths))
        b = h3.vsa_attn_fwd(q, k, v, cu, rows, sel, 7)
        torch.cuda.synchronize()
        runs.append((a.clone(), b.clone()))
    for a, b in runs[1:]:
        assert torch.equal(a, runs[0][0]) and torch.equal(b, runs[0][1])
