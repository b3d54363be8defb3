"""C-ABI tests that need no GPU: the library loads, exports every function the
header declares, and host-side validation returns its status before any launch.

Calls here never reach a kernel launch: each one fails a host check first
(pointers passed are never dereferenced on those paths)."""
import ctypes
import os
import re

import pytest

import packed_varlen_attention_amd as h3
from packed_varlen_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "h3.h")

OK, NULL, DTYPE, SHAPE, SEQLENS, CAPACITY, UNSUPPORTED, HIP, WORKSPACE, ALIGN, TOO_LARGE = range(11)


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(h3_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(h3.LIB_PATH):
        pytest.fail("libh3.so not built; run python -m packed_varlen_attention_amd.build")
    return h3.load()


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert len(names) == 18
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(_lib.SIGNATURES) == names      # the binding declares the same set


def test_version_and_status_strings(lib):
    assert "gfx950" in h3.version()
    seen = set()
    for s in range(11):
        msg = h3.status_string(s)
        assert msg and msg != "unknown status"
        seen.add(msg)
    assert len(seen) == 11
    assert h3.status_string(99) == "unknown status"


def test_workspace_sizes(lib):
    assert lib.h3_pack_workspace_bytes(-1, 3) == 0
    a = lib.h3_pack_workspace_bytes(58758, 2)
    b = lib.h3_pack_workspace_bytes(114688, 675)
    assert a > 58758 * 4 and b > 114688 * 4 + 675 * 112 * 4
    assert lib.h3_attn_workspace_bytes(58758, 2) >= 3 * 4
    assert lib.h3_unpack_workspace_bytes(153735) >= 153735 * 4


def _rope(D=128):
    import workloads as W
    return _lib.rope_cfg(W.default_rope(D))


P = ctypes.c_void_p(4096)       # aligned, never dereferenced on the paths below
MIS = ctypes.c_void_p(4100)     # misaligned


def _attn(lib, q=P, k=P, v=P, cu=P, n_seg=2, max_seqlen=64, rows=100, H=4, D=128, dt=0, scale=0.0,
          o=P, ws=P, wsb=1 << 20):
    return lib.h3_varlen_attn_fwd(q, k, v, cu, n_seg, max_seqlen, rows, H, D, dt, scale, o, ws, wsb, None)


def test_attn_host_validation(lib):
    assert _attn(lib, D=96) == UNSUPPORTED
    assert _attn(lib, dt=7) == DTYPE
    assert _attn(lib, H=0) == SHAPE
    assert _attn(lib, rows=-1) == SHAPE
    assert _attn(lib, scale=-1.0) == UNSUPPORTED
    assert _attn(lib, scale=float("nan")) == UNSUPPORTED
    assert _attn(lib, q=None) == NULL
    assert _attn(lib, cu=None) == NULL
    assert _attn(lib, o=MIS) == ALIGN
    assert _attn(lib, ws=None) == WORKSPACE
    assert _attn(lib, wsb=1) == WORKSPACE
    # empty problems are a no-op success, nothing launched
    assert _attn(lib, rows=0, q=None, k=None, v=None, o=None) == OK
    assert _attn(lib, n_seg=0, q=None, k=None, v=None, o=None) == OK


def _attn_na(lib, q=P, k=P, v=P, cu=P, n_seg=2, max_seqlen=64, rows=100, H=4, D=128, dt=0, scale=0.0, o=P):
    return lib.h3_varlen_attn_fwd_noalloc(q, k, v, cu, n_seg, max_seqlen, rows, H, D, dt, scale, o, None)


def test_attn_noalloc_host_validation(lib):
    """The no-allocation entry point makes the same host checks, and rejects a
    segment count whose tile list does not fit its fixed scratch, before it
    touches any device (these calls run without a GPU)."""
    assert _attn_na(lib, D=96) == UNSUPPORTED
    assert _attn_na(lib, dt=7) == DTYPE
    assert _attn_na(lib, H=0) == SHAPE
    assert _attn_na(lib, rows=-1) == SHAPE
    assert _attn_na(lib, scale=float("nan")) == UNSUPPORTED
    assert _attn_na(lib, v=None) == NULL
    assert _attn_na(lib, q=MIS) == ALIGN
    assert _attn_na(lib, rows=0, q=None, k=None, v=None, o=None) == OK
    limit = 262144
    assert lib.h3_attn_workspace_bytes(1 << 20, 65471) <= limit < lib.h3_attn_workspace_bytes(1 << 20, 65472)
    assert _attn_na(lib, n_seg=65472, rows=1 << 20) == TOO_LARGE
    assert _attn_na(lib, n_seg=1 << 20, rows=1 << 20) == TOO_LARGE
    assert "no-allocation" in h3.status_string(TOO_LARGE)


def _pack(lib, n=10, n_seg=2, H=2, D=128, dt=0, cap=16, rope="default", s=0.0, qs=P, qo=P, vo=P,
          ws=P, wsb=1 << 20, cu=P):
    cfg = _rope(D) if rope == "default" else rope
    return lib.h3_pack_rope(qs, P, P, P, P, P, n, n_seg, H, D, dt,
                            ctypes.byref(cfg) if cfg is not None else None, s,
                            qo, P, vo, cap, cu, P, ws, wsb, None)


def test_pack_host_validation(lib):
    assert _pack(lib, cap=5) == CAPACITY
    assert _pack(lib, n=-1) == SHAPE
    assert _pack(lib, D=80) == UNSUPPORTED
    assert _pack(lib, rope=None) == NULL
    assert _pack(lib, cu=None) == NULL
    assert _pack(lib, qs=None) == NULL
    assert _pack(lib, qo=MIS) == ALIGN
    assert _pack(lib, ws=None) == WORKSPACE
    assert _pack(lib, s=float("inf")) == UNSUPPORTED
    bad = _rope(128)
    bad.m[1].d_t = 30          # split no longer sums to D
    assert _pack(lib, rope=bad) == UNSUPPORTED
    bad = _rope(128)
    bad.m[2].base = 0.0
    assert _pack(lib, rope=bad) == UNSUPPORTED
    bad = _rope(128)
    bad.m[1].d_t, bad.m[1].d_h = 31, 49   # odd slice widths
    assert _pack(lib, rope=bad) == UNSUPPORTED


def test_host_checks_reject_nan_arguments(lib):
    """Every floating-point argument the host validates rejects NaN (the
    device-only -fno-honor-nans must not reach these host checks)."""
    nan = float("nan")
    assert _pack(lib, s=nan) == UNSUPPORTED                       # time offset s
    assert _pack(lib, s=float("-inf")) == UNSUPPORTED
    for m in range(3):
        bad = _rope(128)
        bad.m[m].base = nan
        assert _pack(lib, rope=bad) == UNSUPPORTED
        bad = _rope(128)
        bad.m[m].time_scale = nan
        assert _pack(lib, rope=bad) == UNSUPPORTED
        bad = _rope(128)
        bad.m[m].base = float("inf")
        assert _pack(lib, rope=bad) == UNSUPPORTED
    assert _attn(lib, scale=nan) == UNSUPPORTED
    assert _attn(lib, scale=float("inf")) == UNSUPPORTED
    assert _attn_na(lib, scale=nan) == UNSUPPORTED
    for i in range(3):
        sig = [0.9, 0.9, 0.9]
        sig[i] = nan
        assert _euler(lib, sig=tuple(sig)) == UNSUPPORTED
        nxt = [0.8, 0.8, 0.8]
        nxt[i] = nan
        assert _euler(lib, nxt=tuple(nxt)) == UNSUPPORTED
    out = (ctypes.c_double * 2)()
    assert lib.h3_sigma_schedule(1, nan, out) == UNSUPPORTED
    assert lib.h3_quantize_qk_fp8(P, P, 300, 4, 128, 0, nan, P, P, P, P, None) == UNSUPPORTED
    assert lib.h3_vsa_select(P, P, P, 2, 256, 300, 4, 128, 0, nan, 4, P, None, None, P, 1 << 30, None) \
        == UNSUPPORTED
    assert lib.h3_vsa_attn_fwd(P, P, P, P, 2, 300, 4, 128, 0, nan, P, 4, P, P, 1 << 30, None) == UNSUPPORTED


def test_unpack_host_validation(lib):
    out = (ctypes.c_void_p * 3)(P, P, P)
    idx = (ctypes.c_void_p * 3)(P, P, P)
    cnt = (ctypes.c_int32 * 3)(3, 3, 3)
    f = lib.h3_unpack_by_modality
    assert f(P, P, P, 8, 2, 128, 0, out, idx, cnt, P, 1 << 20, None) == SHAPE      # 9 > 8 tokens
    cnt = (ctypes.c_int32 * 3)(3, 3, 2)
    assert f(P, P, P, 8, 2, 128, 0, None, idx, cnt, P, 1 << 20, None) == NULL
    assert f(None, P, P, 8, 2, 128, 0, out, idx, cnt, P, 1 << 20, None) == NULL
    assert f(P, P, P, 8, 2, 128, 0, out, idx, cnt, P, 1, None) == WORKSPACE
    out2 = (ctypes.c_void_p * 3)(P, MIS, P)
    assert f(P, P, P, 8, 2, 128, 0, out2, idx, cnt, P, 1 << 20, None) == ALIGN
    assert f(P, P, P, 8, 2, 96, 0, out, idx, cnt, P, 1 << 20, None) == UNSUPPORTED


def test_validate_seqlens_host_checks(lib):
    assert lib.h3_validate_seqlens(None, 2, 10, None) == NULL
    assert lib.h3_validate_seqlens(P, -1, 10, None) == SHAPE


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_LIB", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _lib.load()


def _euler(lib, o=P, n=8, D=128, dt=0, z=(P, P, P), an=(None, None, None), sig=(0.0, 0.9, 0.8),
           nxt=(0.0, 0.8, 0.7), cnt=(3, 3, 2), ws=P, wsb=1 << 20):
    zz = (ctypes.c_void_p * 3)(*z)
    aa = (ctypes.c_void_p * 3)(*an)
    ii = (ctypes.c_void_p * 3)(P, P, P)
    return lib.h3_unpack_euler(o, P, P, None, n, 2, D, dt, zz, aa, (ctypes.c_double * 3)(*sig),
                               (ctypes.c_double * 3)(*nxt), ii, (ctypes.c_int32 * 3)(*cnt), ws, wsb,
                               None)


def test_unpack_euler_host_validation(lib):
    assert _euler(lib, cnt=(3, 3, 3)) == SHAPE              # 9 > 8 tokens
    assert _euler(lib, D=96) == UNSUPPORTED
    assert _euler(lib, sig=(0.0, float("nan"), 0.8)) == UNSUPPORTED
    assert _euler(lib, z=(P, MIS, P)) == ALIGN
    assert _euler(lib, an=(None, None, MIS)) == ALIGN
    assert _euler(lib, o=None) == NULL
    assert _euler(lib, wsb=1) == WORKSPACE
    # nothing to do: n = 0 succeeds without touching any pointer
    assert _euler(lib, o=None, n=0, cnt=(0, 0, 0)) == OK


def test_sigma_schedule_host_matches_oracle(lib):
    import numpy as np
    import oracle
    for n, shift in ((50, 12.0), (50, 3.0), (3, 3.0), (7, 1.0)):
        got = h3.sigma_schedule(n, shift)
        want = oracle.sigma_schedule(n, shift)
        assert np.allclose(got, want, atol=1e-15, rtol=0)
    out = (ctypes.c_double * 2)()
    assert lib.h3_sigma_schedule(0, 3.0, out) == SHAPE
    assert lib.h3_sigma_schedule(1, 0.0, out) == UNSUPPORTED
    assert lib.h3_sigma_schedule(1, 3.0, None) == NULL


def test_vsa_host_validation(lib):
    sel = P
    sel_f = lib.h3_vsa_select
    a = lib.h3_vsa_attn_fwd
    ok = dict(n_seg=2, rows=300, H=4, D=128, dt=0, scale=0.0, topk=4)
    def S(q=P, k=P, cu=P, n_seg=2, max_seqlen=256, rows=300, H=4, D=128, dt=0, scale=0.0, topk=4, sel=P,
          ws=P, wsb=1 << 30):
        return sel_f(q, k, cu, n_seg, max_seqlen, rows, H, D, dt, scale, topk, sel, None, None, ws, wsb, None)
    def A(q=P, cu=P, n_seg=2, rows=300, H=4, D=128, dt=0, scale=0.0, sel=P, topk=4, o=P, ws=P, wsb=1 << 30):
        return a(q, P, P, cu, n_seg, rows, H, D, dt, scale, sel, topk, o, ws, wsb, None)
    assert S(D=64) == UNSUPPORTED and A(D=64) == UNSUPPORTED
    assert S(topk=0) == SHAPE and A(topk=0) == SHAPE
    assert S(max_seqlen=-1) == SHAPE
    assert A(dt=1) == UNSUPPORTED                    # the sparse kernel is bf16 only
    assert S(scale=-1.0) == UNSUPPORTED
    assert S(q=None) == NULL and A(sel=None) == NULL
    assert S(q=MIS) == ALIGN and A(o=MIS) == ALIGN
    assert S(wsb=1) == WORKSPACE and A(ws=None) == WORKSPACE
    assert S(rows=0, q=None, k=None) == OK and A(n_seg=0, q=None, o=None) == OK
    assert lib.h3_vsa_blocks_bound(300, 2) == 5 + 2
    assert lib.h3_vsa_workspace_bytes(300, 2, 4) >= 2 * 7 * 4 * 128 * 4


def test_fp8qk_host_validation(lib):
    qz = lib.h3_quantize_qk_fp8
    at = lib.h3_varlen_attn_fwd_fp8qk
    def Q(q=P, k=P, rows=300, H=4, D=128, dt=0, scale=0.0, q8=P, qe=P, k8=P, ke=P):
        return qz(q, k, rows, H, D, dt, scale, q8, qe, k8, ke, None)
    def A(q8=P, qe=P, k8=P, ke=P, v=P, cu=P, n_seg=2, max_seqlen=256, rows=300, H=4, D=128, dt=0, o=P,
          ws=P, wsb=1 << 30):
        return at(q8, qe, k8, ke, v, cu, n_seg, max_seqlen, rows, H, D, dt, o, ws, wsb, None)
    assert Q(dt=7) == DTYPE and A(dt=7) == DTYPE
    assert Q(dt=1) == UNSUPPORTED and A(dt=1) == UNSUPPORTED      # bf16 only
    assert Q(D=64) == UNSUPPORTED and A(D=64) == UNSUPPORTED      # head dim 128 only
    assert Q(H=0) == SHAPE and A(H=0) == SHAPE and Q(rows=-1) == SHAPE and A(rows=-1) == SHAPE
    assert Q(scale=-1.0) == UNSUPPORTED and Q(scale=float("nan")) == UNSUPPORTED
    assert Q(q=None) == NULL and Q(ke=None) == NULL and A(v=None) == NULL and A(ke=None) == NULL
    assert Q(q8=MIS) == ALIGN and Q(qe=ctypes.c_void_p(4098)) == ALIGN and A(o=MIS) == ALIGN and A(ke=ctypes.c_void_p(4097)) == ALIGN
    assert A(ws=None) == WORKSPACE and A(wsb=1) == WORKSPACE
    assert Q(rows=0, q=None, k=None) == OK and A(n_seg=0, v=None) == OK and A(rows=0, o=None) == OK


def test_fp8_binding_checks_before_any_call():
    """The binding rejects inconsistent tensors itself, before a library call
    (CPU tensors here are never passed to a kernel)."""
    import torch
    q = torch.zeros((10, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        h3.quantize_qk_fp8(q, torch.zeros((10, 3, 128), dtype=torch.bfloat16), 10)     # K heads differ
    with pytest.raises(ValueError):
        h3.quantize_qk_fp8(q, q, 11)                                                    # rows past the tensors
    with pytest.raises(TypeError):
        h3.quantize_qk_fp8(q, q, 10, q8=torch.zeros((10, 2, 128), dtype=torch.int8))  # codes must be uint8
    with pytest.raises(ValueError):
        h3.quantize_qk_fp8(q, q, 10, qe=torch.zeros((9, 2, 4), dtype=torch.uint8))   # exponents too small
    u8 = lambda *s: torch.zeros(s, dtype=torch.uint8)
    cu = torch.tensor([0, 10], dtype=torch.int32)
    with pytest.raises(TypeError):
        h3.varlen_attn_fwd_fp8qk(u8(10, 2, 128), u8(10, 2, 4), u8(10, 2, 128), u8(10, 2, 4), q,
                                 cu.to(torch.int64), 10)
    with pytest.raises(ValueError):
        h3.varlen_attn_fwd_fp8qk(u8(10, 2, 128), u8(10, 2, 4), u8(10, 2, 128), u8(10, 2, 4), q, cu, 11)
    with pytest.raises(ValueError):
        h3.varlen_attn_fwd_fp8qk(u8(10, 2, 128), u8(10, 2, 2), u8(10, 2, 128), u8(10, 2, 4), q, cu, 10)
