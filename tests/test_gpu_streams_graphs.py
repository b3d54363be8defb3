"""The library keeps no state and launches only kernels on the caller's
stream, so (1) two calls in flight on two streams give the results that the
same calls give one after the other, and (2) the whole step (pack -> attention
-> unpack) can be captured into a HIP graph whose replays recompute it
exactly, including after the inputs change.  Results are compared bit for bit
with eager runs, whose agreement with the oracle the parity tests establish."""
import pytest
import torch

import packed_varlen_attention_amd as h3
import workloads as W
from gpu_common import device_inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


class Step:
    """Preallocated buffers and workspaces for one workload; run() enqueues
    pack -> attention -> unpack on the current stream."""

    def __init__(self, wl, seed):
        q, k, v = W.make_qkv(wl, seed=seed)
        self.wl = wl
        self.d = device_inputs(wl, q, k, v)
        cap, H, D, dt = wl.capacity, wl.H, wl.D, self.d["q"].dtype
        mk = lambda: torch.full((cap, H, D), float("nan"), dtype=dt, device="cuda")
        self.qo, self.ko, self.vo, self.o = mk(), mk(), mk(), mk()
        self.cu = torch.empty(wl.n_seg + 1, dtype=torch.int32, device="cuda")
        self.perm = torch.empty(max(wl.n, 1), dtype=torch.int32, device="cuda")
        npm = wl.n_per_modality()
        self.npm = npm
        self.outs = [torch.empty((c, H, D), dtype=dt, device="cuda") for c in npm]
        self.idxs = [torch.empty(c, dtype=torch.int32, device="cuda") for c in npm]
        self.ws_pack = h3.workspace(h3.pack_workspace_bytes(wl.n, wl.n_seg), "cuda")
        self.ws_attn = h3.workspace(h3.attn_workspace_bytes(wl.n, wl.n_seg), "cuda")
        self.ws_unpack = h3.workspace(h3.unpack_workspace_bytes(wl.n), "cuda")
        self.max_len = int(wl.segment_lengths().max())

    def run(self):
        wl, d = self.wl, self.d
        h3.pack_rope(d["q"], d["k"], d["v"], d["tags"], d["pos"], d["seg"], wl.n_seg, wl.rope, wl.time_offset,
                     capacity=wl.capacity, q_out=self.qo, k_out=self.ko, v_out=self.vo, cu=self.cu,
                     perm=self.perm, ws=self.ws_pack)
        h3.varlen_attn_fwd(self.qo, self.ko, self.vo, self.cu, total_rows=wl.n, max_seqlen=self.max_len,
                           o=self.o, ws=self.ws_attn)
        h3.unpack_by_modality(self.o, self.perm, d["tags"], self.npm, outs=self.outs, idxs=self.idxs,
                              ws=self.ws_unpack)

    def results(self):
        n = self.wl.n
        return [t.clone() for t in [self.o[:n], self.cu, self.perm[:n]] + self.outs + self.idxs]

    def clear(self):
        for t in (self.o, self.qo, self.ko, self.vo):
            t.fill_(float("nan"))
        for t in self.outs:
            t.zero_()
        for t in self.idxs + [self.cu, self.perm]:
            t.fill_(-7)


def _same(a, b):
    return len(a) == len(b) and all(torch.equal(x, y) for x, y in zip(a, b))


def test_two_streams_match_one_after_the_other():
    A = Step(W.make_custom([300, 129, 64, 1, 700], H=4, D=128, time_offset=238.0), seed=21)
    B = Step(W.make_custom([2000, 77, 513], H=3, D=64), seed=22)
    A.run()
    B.run()
    torch.cuda.synchronize()
    ref_a, ref_b = A.results(), B.results()
    A.clear()
    B.clear()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        with torch.cuda.stream(s1):
            A.run()
        with torch.cuda.stream(s2):
            B.run()
        torch.cuda.synchronize()
        assert _same(A.results(), ref_a)
        assert _same(B.results(), ref_b)


def test_step_captured_in_a_hip_graph_replays_exactly():
    S = Step(W.make_custom([300, 129, 64, 1, 700], H=4, D=128, time_offset=238.0), seed=23)
    S.run()
    torch.cuda.synchronize()
    ref = S.results()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):     # one run on the capture stream before capturing
        S.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        S.run()
    torch.cuda.synchronize()

    for _ in range(3):                # eager work and synchronisation between replays
        S.clear()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(S.results(), ref)

    # new inputs in the same buffers: a replay must recompute, matching an eager run
    S.d["q"].mul_(-1.5)
    S.d["v"].add_(0.25)
    S.clear()
    S.run()
    torch.cuda.synchronize()
    ref2 = S.results()
    assert not torch.equal(ref2[0], ref[0])
    for _ in range(2):
        S.clear()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(S.results(), ref2)


def _fp8_and_vsa_buffers(seed):
    lengths, H = [700, 65, 1300], 3
    rows = sum(lengths)
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q, k, v = ((torch.randn((rows, H, 128), generator=g) * 0.5).to(torch.bfloat16).cuda() for _ in range(3))
    cu = torch.tensor([0, 700, 765, rows], dtype=torch.int32, device="cuda")
    b = dict(q=q, k=k, v=v, cu=cu, rows=rows, H=H, max_len=max(lengths), topk=5)
    b["q8"] = torch.empty((rows, H, 128), dtype=torch.uint8, device="cuda")
    b["k8"] = torch.empty_like(b["q8"])
    b["qe"] = torch.empty((rows, H, 4), dtype=torch.uint8, device="cuda")
    b["ke"] = torch.empty_like(b["qe"])
    b["o8"] = torch.empty_like(v)
    b["ws"] = h3.workspace(h3.attn_workspace_bytes(rows, 3), "cuda")
    nb = h3.vsa_blocks_bound(rows, 3)
    b["sel"] = torch.full((H, nb, 5), -1, dtype=torch.int32, device="cuda")
    b["ov"] = torch.empty_like(v)
    b["wsv"] = h3.workspace(h3.load().h3_vsa_workspace_bytes(rows, 3, H), "cuda")
    return b


def _fp8_and_vsa_run(b):
    h3.quantize_qk_fp8(b["q"], b["k"], b["rows"], q8=b["q8"], qe=b["qe"], k8=b["k8"], ke=b["ke"])
    h3.varlen_attn_fwd_fp8qk(b["q8"], b["qe"], b["k8"], b["ke"], b["v"], b["cu"], b["rows"], b["max_len"],
                             o=b["o8"], ws=b["ws"])
    h3.vsa_select(b["q"], b["k"], b["cu"], b["rows"], b["topk"], max_seqlen=b["max_len"], sel=b["sel"], ws=b["wsv"])
    h3.vsa_attn_fwd(b["q"], b["k"], b["v"], b["cu"], b["rows"], b["sel"], b["topk"], o=b["ov"], ws=b["wsv"])


def _fp8_and_vsa_results(b):
    return [b[n].clone() for n in ("q8", "qe", "k8", "ke", "o8", "sel", "ov")]


def _fp8_and_vsa_clear(b):
    for n in ("q8", "qe", "k8", "ke"):
        b[n].fill_(0x55)
    b["sel"].fill_(-1)
    b["o8"].fill_(float("nan"))
    b["ov"].fill_(float("nan"))


def test_fp8_and_vsa_calls_captured_in_a_hip_graph():
    b = _fp8_and_vsa_buffers(31)
    _fp8_and_vsa_run(b)
    torch.cuda.synchronize()
    ref = _fp8_and_vsa_results(b)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _fp8_and_vsa_run(b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _fp8_and_vsa_run(b)
    torch.cuda.synchronize()
    for _ in range(3):
        _fp8_and_vsa_clear(b)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(_fp8_and_vsa_results(b), ref)
    b["k"].mul_(-0.5)                      # new inputs in place: replays recompute
    _fp8_and_vsa_clear(b)
    _fp8_and_vsa_run(b)
    torch.cuda.synchronize()
    ref2 = _fp8_and_vsa_results(b)
    assert not torch.equal(ref2[4], ref[4])
    _fp8_and_vsa_clear(b)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert _same(_fp8_and_vsa_results(b), ref2)
