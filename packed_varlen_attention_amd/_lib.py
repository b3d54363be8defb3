"""ctypes binding over libh3.so (include/h3.h).

Argument marshalling only: shapes and dtypes of torch tensors are checked,
pointers and the current HIP stream are passed to the C ABI, and a non-zero
status raises H3Error.  Every step of the path runs in the library's HIP
kernels; there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# H3_LIBRARY selects another build of the same library (e.g. the host
# sanitizer build, `python -m packed_varlen_attention_amd.build --sanitize`).
LIB_PATH = os.environ.get("H3_LIBRARY") or os.path.join(PKG_DIR, "libh3.so")

H3_BF16, H3_F32 = 0, 1
TEXT, VIDEO, AUDIO = 0, 1, 2

# Every function include/h3.h declares, with (restype, argtypes).
_c = ctypes
_vp, _i32, _f32, _f64, _sz = _c.c_void_p, _c.c_int32, _c.c_float, _c.c_double, _c.c_size_t


class h3_rope_modality(_c.Structure):
    _fields_ = [("base", _f64), ("time_scale", _f64), ("shift_time", _i32),
                ("d_t", _i32), ("d_h", _i32), ("d_w", _i32)]


class h3_rope_cfg(_c.Structure):
    _fields_ = [("m", h3_rope_modality * 3)]


SIGNATURES = {
    "h3_pack_workspace_bytes": (_sz, [_i32, _i32]),
    "h3_pack_rope": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _c.c_int,
                                _c.POINTER(h3_rope_cfg), _f64, _vp, _vp, _vp, _i32, _vp, _vp,
                                _vp, _sz, _vp]),
    "h3_attn_workspace_bytes": (_sz, [_i32, _i32]),
    "h3_varlen_attn_fwd": (_c.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _c.c_int,
                                      _f32, _vp, _vp, _sz, _vp]),
    "h3_varlen_attn_fwd_noalloc": (_c.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _c.c_int,
                                              _f32, _vp, _vp]),
    "h3_unpack_workspace_bytes": (_sz, [_i32]),
    "h3_unpack_by_modality": (_c.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _c.c_int,
                                         _c.POINTER(_vp), _c.POINTER(_vp), _c.POINTER(_i32),
                                         _vp, _sz, _vp]),
    "h3_unpack_euler": (_c.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _c.c_int,
                                   _c.POINTER(_vp), _c.POINTER(_vp), _c.POINTER(_f64), _c.POINTER(_f64),
                                   _c.POINTER(_vp), _c.POINTER(_i32), _vp, _sz, _vp]),
    "h3_sigma_schedule": (_c.c_int, [_i32, _f64, _c.POINTER(_f64)]),
    "h3_vsa_blocks_bound": (_i32, [_i32, _i32]),
    "h3_vsa_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "h3_vsa_select": (_c.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _c.c_int, _f32, _i32,
                                 _vp, _vp, _vp, _vp, _sz, _vp]),
    "h3_vsa_attn_fwd": (_c.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _c.c_int, _f32, _vp, _i32,
                                   _vp, _vp, _sz, _vp]),
    "h3_quantize_qk_fp8": (_c.c_int, [_vp, _vp, _i32, _i32, _i32, _c.c_int, _f32, _vp, _vp, _vp, _vp, _vp]),
    "h3_varlen_attn_fwd_fp8qk": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                            _c.c_int, _vp, _vp, _sz, _vp]),
    "h3_validate_seqlens": (_c.c_int, [_vp, _i32, _i32, _vp]),
    "h3_status_string": (_c.c_char_p, [_c.c_int]),
    "h3_version": (_c.c_char_p, []),
}

_LIB = None


class H3Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))


def load() -> ctypes.CDLL:
    """Load the in-tree libh3.so; fails loudly if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libh3.so is not built (%s); run `python -m packed_varlen_attention_amd.build`"
                              % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _LIB = lib
    return _LIB


def status_string(status: int) -> str:
    return load().h3_status_string(int(status)).decode()


def version() -> str:
    return load().h3_version().decode()


def _check(status: int, where: str):
    if status != 0:
        raise H3Error(status, where)


# --------------------------------------------------------------------- helpers
def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return H3_BF16
    if t.dtype == torch.float32:
        return H3_F32
    raise TypeError("tensor dtype must be bfloat16 or float32, got %s" % t.dtype)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def rope_cfg(rope: Sequence) -> h3_rope_cfg:
    """Build the C struct from three objects with base, time_scale,
    shift_time, d_t, d_h, d_w attributes (text, video, audio)."""
    cfg = h3_rope_cfg()
    for m in range(3):
        r = rope[m]
        cfg.m[m] = h3_rope_modality(float(r.base), float(r.time_scale), int(r.shift_time),
                                    int(r.d_t), int(r.d_h), int(r.d_w))
    return cfg


def workspace(nbytes: int, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ the calls
def pack_workspace_bytes(n: int, n_seg: int) -> int:
    return int(load().h3_pack_workspace_bytes(n, n_seg))


def attn_workspace_bytes(total_rows: int, n_seg: int) -> int:
    return int(load().h3_attn_workspace_bytes(total_rows, n_seg))


def unpack_workspace_bytes(n: int) -> int:
    return int(load().h3_unpack_workspace_bytes(n))


def pack_rope(q_src, k_src, v_src, tags, pos, seg, n_seg: int, rope, time_offset: float = 0.0,
              capacity: Optional[int] = None, *, q_out=None, k_out=None, v_out=None, cu=None,
              perm=None, ws=None, pack_v: bool = True, stream=None):
    """h3_pack_rope.  Returns (q_out, k_out, v_out or None, cu_seqlens, perm)."""
    torch = _torch()
    lib = load()
    n, H, D = q_src.shape
    dev = q_src.device
    cap = n if capacity is None else int(capacity)
    if tags.dtype != torch.uint8 or pos.dtype != torch.int32 or seg.dtype != torch.int32:
        raise TypeError("tags must be uint8, pos and seg int32")
    if tuple(pos.shape) != (n, 3) or tags.shape[0] != n or seg.shape[0] != n:
        raise ValueError("tags [n], pos [n,3] and seg [n] must match q_src rows")
    if k_src.shape != q_src.shape or (v_src is not None and v_src.shape != q_src.shape):
        raise ValueError("q_src, k_src, v_src shapes differ")
    if q_out is None:
        q_out = torch.empty((cap, H, D), dtype=q_src.dtype, device=dev)
    if k_out is None:
        k_out = torch.empty((cap, H, D), dtype=q_src.dtype, device=dev)
    if pack_v and v_out is None:
        v_out = torch.empty((cap, H, D), dtype=q_src.dtype, device=dev)
    if not pack_v:
        v_out = None
    for t in (q_out, k_out) + ((v_out,) if v_out is not None else ()):
        if t.shape[0] < cap or tuple(t.shape[1:]) != (H, D) or t.dtype != q_src.dtype:
            raise ValueError("output buffers must be [capacity, H, D] of the input dtype")
    if cu is None:
        cu = torch.empty(n_seg + 1, dtype=torch.int32, device=dev)
    if perm is None:
        perm = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(lib.h3_pack_workspace_bytes(n, n_seg), dev)
    cfg = rope_cfg(rope)
    st = lib.h3_pack_rope(_ptr(q_src), _ptr(k_src), _ptr(v_src) if v_out is not None else None,
                          _ptr(tags), _ptr(pos), _ptr(seg), n, int(n_seg), H, D, _dt(q_src),
                          ctypes.byref(cfg), float(time_offset), _ptr(q_out), _ptr(k_out),
                          _ptr(v_out), cap, _ptr(cu), _ptr(perm), _ptr(ws), ws.numel(),
                          _stream(stream))
    _check(st, "h3_pack_rope")
    return q_out, k_out, v_out, cu, perm


def varlen_attn_fwd(q, k, v, cu_seqlens, total_rows: int, max_seqlen: int = 0,
                    softmax_scale: float = 0.0, *, o=None, ws=None, stream=None):
    """h3_varlen_attn_fwd on packed [rows, H, D] tensors.  Returns o."""
    torch = _torch()
    lib = load()
    rows, H, D = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape and dtype")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if total_rows > rows:
        raise ValueError("total_rows exceeds the tensors' rows")
    n_seg = cu_seqlens.shape[0] - 1
    if o is None:
        o = torch.empty_like(q)
    if ws is None:
        ws = workspace(lib.h3_attn_workspace_bytes(total_rows, n_seg), q.device)
    st = lib.h3_varlen_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), n_seg, int(max_seqlen),
                                int(total_rows), H, D, _dt(q), float(softmax_scale), _ptr(o),
                                _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "h3_varlen_attn_fwd")
    return o


def varlen_attn_fwd_noalloc(q, k, v, cu_seqlens, total_rows: int, max_seqlen: int = 0,
                            softmax_scale: float = 0.0, *, o=None, stream=None):
    """h3_varlen_attn_fwd_noalloc: the same attention with the library's fixed
    per-GPU scratch instead of a workspace (the library allocates nothing;
    calls that overlap on one GPU race).  Returns o."""
    torch = _torch()
    lib = load()
    rows, H, D = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape and dtype")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if total_rows > rows:
        raise ValueError("total_rows exceeds the tensors' rows")
    n_seg = cu_seqlens.shape[0] - 1
    if o is None:
        o = torch.empty_like(q)
    st = lib.h3_varlen_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), n_seg, int(max_seqlen),
                                        int(total_rows), H, D, _dt(q), float(softmax_scale), _ptr(o),
                                        _stream(stream))
    _check(st, "h3_varlen_attn_fwd_noalloc")
    return o


def quantize_qk_fp8(q, k, rows: int, softmax_scale: float = 0.0, *, q8=None, qe=None, k8=None, ke=None,
                    stream=None):
    """h3_quantize_qk_fp8 on packed bf16 [>= rows, H, 128] Q and K.  Returns
    (q8, qe, k8, ke): uint8 codes [rows, H, 128] and exponent bytes
    [rows, H, 4]."""
    torch = _torch()
    lib = load()
    _, H, D = q.shape
    if k.shape != q.shape or k.dtype != q.dtype:
        raise ValueError("q and k must share shape and dtype")
    if rows > q.shape[0]:
        raise ValueError("rows exceeds the tensors' rows")
    mk = lambda n: torch.empty((max(rows, 1), H, n), dtype=torch.uint8, device=q.device)
    q8 = mk(D) if q8 is None else q8
    k8 = mk(D) if k8 is None else k8
    qe = mk(D // 32) if qe is None else qe
    ke = mk(D // 32) if ke is None else ke
    for t in (q8, k8, qe, ke):
        if t.dtype != torch.uint8 or not t.is_contiguous():
            raise TypeError("codes and exponents must be contiguous uint8")
    if q8.numel() < rows * H * D or k8.numel() < rows * H * D or qe.numel() < rows * H * (D // 32) \
            or ke.numel() < rows * H * (D // 32):
        raise ValueError("output buffers too small")
    st = lib.h3_quantize_qk_fp8(_ptr(q), _ptr(k), int(rows), H, D, _dt(q), float(softmax_scale), _ptr(q8),
                                _ptr(qe), _ptr(k8), _ptr(ke), _stream(stream))
    _check(st, "h3_quantize_qk_fp8")
    return q8, qe, k8, ke


def varlen_attn_fwd_fp8qk(q8, qe, k8, ke, v, cu_seqlens, total_rows: int, max_seqlen: int = 0, *, o=None,
                          ws=None, stream=None):
    """h3_varlen_attn_fwd_fp8qk: attention on MX-E4M3 Q and K (from
    quantize_qk_fp8) with bf16 V [>= total_rows, H, 128].  Returns o."""
    torch = _torch()
    lib = load()
    rows, H, D = v.shape
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if total_rows > rows or q8.shape[0] < total_rows or k8.shape[0] < total_rows:
        raise ValueError("total_rows exceeds the tensors' rows")
    if tuple(q8.shape[1:]) != (H, D) or tuple(k8.shape[1:]) != (H, D) or tuple(qe.shape[1:]) != (H, D // 32) \
            or tuple(ke.shape[1:]) != (H, D // 32):
        raise ValueError("codes [rows, H, D] and exponents [rows, H, D/32] must match V's heads")
    n_seg = cu_seqlens.shape[0] - 1
    if o is None:
        o = torch.empty_like(v)
    if ws is None:
        ws = workspace(lib.h3_attn_workspace_bytes(total_rows, n_seg), v.device)
    st = lib.h3_varlen_attn_fwd_fp8qk(_ptr(q8), _ptr(qe), _ptr(k8), _ptr(ke), _ptr(v), _ptr(cu_seqlens), n_seg,
                                      int(max_seqlen), int(total_rows), H, D, _dt(v), _ptr(o), _ptr(ws),
                                      ws.numel(), _stream(stream))
    _check(st, "h3_varlen_attn_fwd_fp8qk")
    return o


def unpack_by_modality(o, perm, tags_src, n_per_mod: Sequence[int], *, outs=None, idxs=None,
                       ws=None, copy_values: bool = True, stream=None):
    """h3_unpack_by_modality.  Returns (outs[3], idxs[3])."""
    torch = _torch()
    lib = load()
    n = tags_src.shape[0]
    _, H, D = o.shape
    dev = o.device
    if tags_src.dtype != torch.uint8 or perm.dtype != torch.int32:
        raise TypeError("tags_src must be uint8 and perm int32")
    if outs is None:
        outs = [torch.empty((int(c), H, D), dtype=o.dtype, device=dev) if copy_values else None
                for c in n_per_mod]
    if idxs is None:
        idxs = [torch.empty(int(c), dtype=torch.int32, device=dev) for c in n_per_mod]
    if ws is None:
        ws = workspace(lib.h3_unpack_workspace_bytes(n), dev)
    out_arr = (_vp * 3)(*[_ptr(x) if (x is not None and x.numel()) else None for x in outs])
    idx_arr = (_vp * 3)(*[_ptr(x) if (x is not None and x.numel()) else None for x in idxs])
    cnt_arr = (_i32 * 3)(*[int(c) for c in n_per_mod])
    st = lib.h3_unpack_by_modality(_ptr(o), _ptr(perm), _ptr(tags_src), n, H, D, _dt(o),
                                   out_arr, idx_arr, cnt_arr, _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "h3_unpack_by_modality")
    return outs, idxs


def unpack_euler(o, perm, tags_src, n_per_mod: Sequence[int], z, sigma, sigma_next, *,
                 pinned=None, anchors=None, idxs=None, ws=None, stream=None):
    """h3_unpack_euler: one eta = 0 Euler step of the per-modality fp32 states
    z[m] (updated in place; None = not stepped) with velocity o, then re-pin.
    Returns idxs[3]."""
    torch = _torch()
    lib = load()
    n = tags_src.shape[0]
    _, H, D = o.shape
    dev = o.device
    if tags_src.dtype != torch.uint8 or perm.dtype != torch.int32:
        raise TypeError("tags_src must be uint8 and perm int32")
    if pinned is not None and (pinned.dtype != torch.uint8 or pinned.shape[0] != n):
        raise TypeError("pinned must be uint8 [n] in source order")
    anchors = anchors if anchors is not None else [None, None, None]
    for m in range(3):
        for t in (z[m], anchors[m]):
            if t is None:
                continue
            if t.dtype != torch.float32 or tuple(t.shape) != (int(n_per_mod[m]), H, D):
                raise ValueError("z[m] and anchors[m] must be float32 [n_per_mod[m], H, D]")
    if idxs is None:
        idxs = [torch.empty(int(c), dtype=torch.int32, device=dev) for c in n_per_mod]
    if ws is None:
        ws = workspace(lib.h3_unpack_workspace_bytes(n), dev)
    ptrs = lambda xs: (_vp * 3)(*[_ptr(x) if (x is not None and x.numel()) else None for x in xs])
    st = lib.h3_unpack_euler(_ptr(o), _ptr(perm), _ptr(tags_src), _ptr(pinned), n, H, D, _dt(o),
                             ptrs(z), ptrs(anchors), (_f64 * 3)(*[float(x) for x in sigma]),
                             (_f64 * 3)(*[float(x) for x in sigma_next]), ptrs(idxs),
                             (_i32 * 3)(*[int(c) for c in n_per_mod]), _ptr(ws), ws.numel(),
                             _stream(stream))
    _check(st, "h3_unpack_euler")
    return idxs


def sigma_schedule(n_steps: int, shift: float):
    """h3_sigma_schedule (host only): n_steps + 1 noise levels ending at 0."""
    out = (_f64 * (int(n_steps) + 1))() if n_steps >= 0 else (_f64 * 1)()
    _check(load().h3_sigma_schedule(int(n_steps), float(shift), out), "h3_sigma_schedule")
    return [float(x) for x in out]


def vsa_blocks_bound(total_rows: int, n_seg: int) -> int:
    """Upper bound of the number of 64-row blocks (rows of the selection)."""
    return int(load().h3_vsa_blocks_bound(int(total_rows), int(n_seg)))


def vsa_select(q, k, cu_seqlens, total_rows: int, topk: int, max_seqlen: int, softmax_scale: float = 0.0,
               *, sel=None, means: bool = False, ws=None, stream=None):
    """h3_vsa_select: top-k key blocks per (head, query block).  Returns sel
    int32 [H, nb_cap, topk], or (sel, qmean, kmean) with means=True."""
    torch = _torch()
    lib = load()
    rows, H, D = q.shape
    if k.shape != q.shape or k.dtype != q.dtype:
        raise ValueError("q and k must share shape and dtype")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if total_rows > rows:
        raise ValueError("total_rows exceeds the tensors' rows")
    n_seg = cu_seqlens.shape[0] - 1
    nb_cap = vsa_blocks_bound(total_rows, n_seg)
    if sel is None:
        sel = torch.full((H, max(nb_cap, 1), int(topk)), -1, dtype=torch.int32, device=q.device)
    qm = km = None
    if means:
        qm = torch.zeros((max(nb_cap, 1), H, D), dtype=torch.float32, device=q.device)
        km = torch.zeros_like(qm)
    if ws is None:
        ws = workspace(lib.h3_vsa_workspace_bytes(total_rows, n_seg, H), q.device)
    st = lib.h3_vsa_select(_ptr(q), _ptr(k), _ptr(cu_seqlens), n_seg, int(max_seqlen), int(total_rows), H, D,
                           _dt(q), float(softmax_scale), int(topk), _ptr(sel), _ptr(qm), _ptr(km), _ptr(ws),
                           ws.numel(), _stream(stream))
    _check(st, "h3_vsa_select")
    return (sel, qm, km) if means else sel


def vsa_attn_fwd(q, k, v, cu_seqlens, total_rows: int, sel, topk: int, softmax_scale: float = 0.0, *, o=None,
                 ws=None, stream=None):
    """h3_vsa_attn_fwd: block-sparse attention over the blocks listed in sel."""
    torch = _torch()
    lib = load()
    rows, H, D = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape and dtype")
    if cu_seqlens.dtype != torch.int32 or sel.dtype != torch.int32:
        raise TypeError("cu_seqlens and sel must be int32")
    n_seg = cu_seqlens.shape[0] - 1
    nb_cap = vsa_blocks_bound(total_rows, n_seg)
    if tuple(sel.shape) != (H, max(nb_cap, 1), int(topk)):
        raise ValueError("sel must be [H, vsa_blocks_bound, topk]")
    if o is None:
        o = torch.empty_like(q)
    if ws is None:
        ws = workspace(lib.h3_vsa_workspace_bytes(total_rows, n_seg, H), q.device)
    st = lib.h3_vsa_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), n_seg, int(total_rows), H, D, _dt(q),
                             float(softmax_scale), _ptr(sel), int(topk), _ptr(o), _ptr(ws), ws.numel(),
                             _stream(stream))
    _check(st, "h3_vsa_attn_fwd")
    return o


def validate_seqlens(cu_seqlens, capacity: int, stream=None) -> int:
    """h3_validate_seqlens: returns the status code (0 = valid)."""
    lib = load()
    return int(lib.h3_validate_seqlens(_ptr(cu_seqlens), cu_seqlens.shape[0] - 1, int(capacity),
                                       _stream(stream)))
