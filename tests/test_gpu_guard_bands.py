"""Guard bands around every buffer the library writes.

Each output and workspace buffer is carved out of a larger allocation whose
first and last 4 KiB hold a canary byte pattern; after each call (pack,
every attention kernel the host can choose, the no-allocation entry, FP8
quantization and attention, unpack, the Euler epilogue, VSA selection and
attention) both bands must be unchanged.  A kernel that stores past either
end of a buffer (a wrong row bound, a ragged tail, a negative index) changes
a band.  Reads outside a buffer are not detected this way; the parity tests
and the descriptor range checks cover those."""
import numpy as np
import pytest
import torch

import packed_varlen_attention_amd as h3
import workloads as W

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

GUARD = 4096
CANARY = 0xA5


class Guarded:
    """A buffer of `nbytes` between two canary bands of GUARD bytes."""

    def __init__(self, nbytes: int):
        self.n = max(int(nbytes), 1)
        self.raw = torch.full((GUARD + self.n + GUARD,), CANARY, dtype=torch.uint8, device="cuda")

    def view(self, shape, dtype):
        elem = torch.empty((), dtype=dtype).element_size()
        count = int(np.prod(shape)) if len(shape) else 1
        assert count * elem <= self.n
        return self.raw[GUARD:GUARD + count * elem].view(dtype).view(shape)

    def bytes(self):
        return self.raw[GUARD:GUARD + self.n]

    def intact(self) -> bool:
        torch.cuda.synchronize()
        return bool((self.raw[:GUARD] == CANARY).all()) and bool((self.raw[GUARD + self.n:] == CANARY).all())


def gbuf(shape, dtype, fill=None):
    elem = torch.empty((), dtype=dtype).element_size()
    g = Guarded(int(np.prod(shape)) * elem)
    t = g.view(shape, dtype)
    if fill is not None:
        t.fill_(fill)
    return g, t


def gws(nbytes):
    g = Guarded(nbytes)
    return g, g.bytes()


def check(*guards, what=""):
    for i, g in enumerate(guards):
        assert g.intact(), "%s: guard band of buffer %d changed" % (what, i)


def _segments(lengths, H, D, dtype, seed):
    rows = int(sum(lengths))
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    t = [(torch.randn((rows, H, D), generator=gen) * 0.5).to(dtype).cuda() for _ in range(3)]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32), device="cuda")
    return t, cu, rows


@pytest.mark.parametrize("case", ["main", "short", "multi", "d64", "f32", "noalloc"])
def test_attention_kernels_write_inside_their_buffers(case):
    rng = np.random.default_rng(3)
    if case == "multi":          # >= 4 items per workgroup slot: several-items kernel
        lengths, H, D, dtype, hint = list(rng.integers(1, 257, size=128)), 10, 128, torch.bfloat16, 256
    elif case == "short":        # few short segments: one item per workgroup
        lengths, H, D, dtype, hint = [130, 7, 256, 64, 33], 2, 128, torch.bfloat16, 256
    elif case == "d64":
        lengths, H, D, dtype, hint = [300, 5, 129], 3, 64, torch.bfloat16, 0
    elif case == "f32":
        lengths, H, D, dtype, hint = [200, 3, 77], 2, 128, torch.float32, 0
    else:                        # main kernel (no hint) and the no-allocation entry
        lengths, H, D, dtype, hint = [1000, 1, 257, 64], 3, 128, torch.bfloat16, 0
    (q, k, v), cu, rows = _segments([int(x) for x in lengths], H, D, dtype, seed=9)
    go, o = gbuf((rows, H, D), dtype, fill=float("nan"))
    if case == "noalloc":
        h3.varlen_attn_fwd_noalloc(q, k, v, cu, rows, max_seqlen=hint, o=o)
        check(go, what=case)
    else:
        gw, ws = gws(h3.attn_workspace_bytes(rows, len(lengths)))
        h3.varlen_attn_fwd(q, k, v, cu, rows, max_seqlen=hint, o=o, ws=ws)
        check(go, gw, what=case)
    assert torch.isfinite(o.float()).all()


@pytest.mark.parametrize("which", ["f32", "bf16"])
def test_pack_unpack_and_epilogue_write_inside_their_buffers(which):
    wl = W.make_workload(0) if which == "f32" else W.make_custom([5, 130, 64, 257], H=4, D=128, time_offset=238.0)
    q, k, v = W.make_qkv_on_device(wl, "cuda")
    d = lambda a: torch.from_numpy(a).cuda()
    cap, H, D = wl.capacity, wl.H, wl.D
    gq, qo = gbuf((cap, H, D), q.dtype, fill=float("nan"))
    gk, ko = gbuf((cap, H, D), q.dtype, fill=float("nan"))
    gv, vo = gbuf((cap, H, D), q.dtype, fill=float("nan"))
    gc, cu = gbuf((wl.n_seg + 1,), torch.int32)
    gp, perm = gbuf((max(wl.n, 1),), torch.int32)
    gw, ws = gws(h3.pack_workspace_bytes(wl.n, wl.n_seg))
    h3.pack_rope(q, k, v, d(wl.tags), d(wl.pos), d(wl.seg), wl.n_seg, wl.rope, wl.time_offset, capacity=cap,
                 q_out=qo, k_out=ko, v_out=vo, cu=cu, perm=perm, ws=ws)
    check(gq, gk, gv, gc, gp, gw, what="pack_rope")

    o = h3.varlen_attn_fwd(qo, ko, vo, cu, wl.n)
    npm = [int((wl.tags == m).sum()) for m in range(3)]
    outs_g = [gbuf((c, H, D), q.dtype, fill=0.0) for c in npm]
    idx_g = [gbuf((c,), torch.int32) for c in npm]
    gu, wsu = gws(h3.unpack_workspace_bytes(wl.n))
    h3.unpack_by_modality(o, perm, d(wl.tags), npm, outs=[t for _, t in outs_g], idxs=[t for _, t in idx_g],
                          ws=wsu)
    check(*[g for g, _ in outs_g], *[g for g, _ in idx_g], gu, what="unpack_by_modality")

    z_g = [gbuf((c, H, D), torch.float32, fill=0.5) for c in npm]
    a_g = [gbuf((c, H, D), torch.float32, fill=0.25) for c in npm]
    pinned = torch.from_numpy((np.arange(wl.n) % 5 == 0).astype(np.uint8)).cuda()
    idx2_g = [gbuf((c,), torch.int32) for c in npm]
    ge, wse = gws(h3.unpack_workspace_bytes(wl.n))
    h3.unpack_euler(o, perm, d(wl.tags), npm, [t for _, t in z_g], [1.0, 0.9, 0.0], [0.8, 0.7, 0.0],
                    pinned=pinned, anchors=[t for _, t in a_g], idxs=[t for _, t in idx2_g], ws=wse)
    check(*[g for g, _ in z_g], *[g for g, _ in a_g], *[g for g, _ in idx2_g], ge, what="unpack_euler")


def test_fp8_path_writes_inside_its_buffers():
    lengths, H, D = [300, 1, 190, 64], 3, 128
    (q, k, v), cu, rows = _segments(lengths, H, D, torch.bfloat16, seed=21)
    g8q, q8 = gbuf((rows, H, D), torch.uint8)
    geq, qe = gbuf((rows, H, D // 32), torch.uint8)
    g8k, k8 = gbuf((rows, H, D), torch.uint8)
    gek, ke = gbuf((rows, H, D // 32), torch.uint8)
    h3.quantize_qk_fp8(q, k, rows, q8=q8, qe=qe, k8=k8, ke=ke)
    check(g8q, geq, g8k, gek, what="quantize_qk_fp8")
    go, o = gbuf((rows, H, D), torch.bfloat16, fill=float("nan"))
    gw, ws = gws(h3.attn_workspace_bytes(rows, len(lengths)))
    h3.varlen_attn_fwd_fp8qk(q8, qe, k8, ke, v, cu, rows, o=o, ws=ws)
    check(go, gw, what="varlen_attn_fwd_fp8qk")
    assert torch.isfinite(o.float()).all()


@pytest.mark.parametrize("hint", [0, 1000])
def test_vsa_writes_inside_its_buffers(hint):
    lengths, H, D, topk = [700, 64, 5, 300], 3, 128, 4
    (q, k, v), cu, rows = _segments(lengths, H, D, torch.bfloat16, seed=33)
    nb_cap = h3.vsa_blocks_bound(rows, len(lengths))
    gs, sel = gbuf((H, nb_cap, topk), torch.int32, fill=-1)
    gqm, qm = gbuf((nb_cap, H, D), torch.float32, fill=0.0)
    gkm, km = gbuf((nb_cap, H, D), torch.float32, fill=0.0)
    lib = h3.load()
    vsa_ws = lambda: gws(int(lib.h3_vsa_workspace_bytes(rows, len(lengths), H)))
    gw, ws = vsa_ws()
    st = lib.h3_vsa_select(q.data_ptr(), k.data_ptr(), cu.data_ptr(), len(lengths), hint, rows, H, D, h3.H3_BF16, 0.0,
                           topk, sel.data_ptr(), qm.data_ptr(), km.data_ptr(), ws.data_ptr(), ws.numel(),
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0
    check(gs, gqm, gkm, gw, what="vsa_select")
    go, o = gbuf((rows, H, D), torch.bfloat16, fill=float("nan"))
    gw2, ws2 = vsa_ws()
    h3.vsa_attn_fwd(q, k, v, cu, rows, sel, topk, o=o, ws=ws2)
    check(go, gw2, what="vsa_attn_fwd")
    assert torch.isfinite(o.float()).all()
