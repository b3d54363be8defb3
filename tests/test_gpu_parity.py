"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Element-by-element at sizes the oracle finishes in seconds (several tiles and
ragged tails); sampled rows at the full workload sizes, in the same launch
configuration bench.py times; integers bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from oracle.cache import cached
import packed_varlen_attention_amd as h3
import workloads as W
from gpu_common import assert_close, device_inputs, f64, run_path, sample_rows

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _oracle_full(wl, q, k, v, heads=None):
    """The oracle's whole path; `heads` restricts it to some heads (each head
    is independent), to bound host time and memory at large sizes."""
    if heads is not None:
        q, k, v = q[:, heads], k[:, heads], v[:, heads]
    return oracle.run(W.to_f64(q), W.to_f64(k), W.to_f64(v), wl.tags, wl.pos, wl.seg, wl.n_seg,
                      wl.rope, wl.time_offset)


def _check_full(wl, g, r, stagewise=True, heads=None):
    n = wl.n
    hs = slice(None) if heads is None else heads
    assert g["cu"].cpu().numpy().tolist() == r["cu"].tolist()
    assert np.array_equal(g["perm"][:n].cpu().numpy(), r["perm"])
    assert_close(g["q"][:n, hs], r["q"], wl.dtype, "packed Q'")
    assert_close(g["k"][:n, hs], r["k"], wl.dtype, "packed K'")
    assert torch.equal(g["v"][:n, hs].cpu().double(), torch.from_numpy(r["v"]))   # exact copy
    assert_close(g["o"][:n, hs], r["o"], wl.dtype, "O end-to-end")
    for m in range(3):
        assert np.array_equal(g["idxs"][m].cpu().numpy(), r["idxs"][m])
        assert torch.equal(g["outs"][m], g["o"][g["idxs"][m].long()])       # exact gather
    if stagewise:   # the oracle's attention on the GPU's own Q', K', V
        ref = oracle.attention(f64(g["q"][:n, hs]), f64(g["k"][:n, hs]), f64(g["v"][:n, hs]), r["cu"])
        assert_close(g["o"][:n, hs], ref, wl.dtype, "O stage-wise")
    # pad rows past the effective length stay untouched (NaN prefill)
    for key in ("q", "k", "v", "o"):
        assert torch.isnan(g[key][n:].float()).all()


def test_tiny_fp32_end_to_end():
    wl = W.make_workload(0)
    q, k, v = W.make_qkv(wl)
    g = run_path(wl, device_inputs(wl, q, k, v))
    r = _oracle_full(wl, q, k, v)
    assert g["cu"].cpu().tolist() == [0, 10, 30, 45]
    _check_full(wl, g, r)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_segments(D, dtype):
    # every residue of the 64-key tile count mod 3 and mod 4 (the kernel's
    # main loop is unrolled by its LDS ring size), each ragged and aligned
    lengths = [1, 0, 33, 64, 65, 127, 128, 129, 191, 192, 193, 255, 256, 257, 300, 320, 321,
               383, 384, 385, 449, 450, 513, 577, 640, 641, 1100]
    wl = W.make_custom(lengths, H=3, D=D, dtype=dtype, q_scale=0.5 if dtype == "bf16" else 1.0,
                       time_offset=17.0)
    q, k, v = W.make_qkv(wl, seed=77)
    g = run_path(wl, device_inputs(wl, q, k, v))
    r = _oracle_full(wl, q, k, v)
    _check_full(wl, g, r)


@pytest.mark.parametrize("D", [64, 128])
def test_many_short_segments(D):
    # thousands of segments of 0..12 rows: one query tile each, the segment
    # search over a long prefix, pack counts spread over many (segment, block)
    # cells, empty segments between non-empty ones
    rng = np.random.default_rng(21)
    lengths = [int(x) for x in rng.integers(0, 13, size=3000)]
    wl = W.make_custom(lengths, H=2, D=D, time_offset=3.0)
    q, k, v = W.make_qkv(wl, seed=78)
    g = run_path(wl, device_inputs(wl, q, k, v))
    r = _oracle_full(wl, q, k, v)
    _check_full(wl, g, r)


def test_out_of_range_segment_ids_end_to_end():
    """Tokens whose segment id is outside 0..n_seg-1 get no packed row: perm is
    -1 past cu[n_seg] (pre-filled with a stale in-range value here), their
    per-modality slot keeps idx -1 and an unwritten row, and their Euler state
    is not stepped; every other output matches the oracle."""
    wl = W.make_custom([40, 70, 25, 66], H=2, D=128, time_offset=5.0)
    seg = wl.seg.copy()
    seg[[3, 50, 51, 130]] = [7, -1, 4, -100]           # four tokens of three modalities dropped
    wl.seg = seg
    q, k, v = W.make_qkv(wl, seed=81)
    d = device_inputs(wl, q, k, v)
    n, H, D = wl.n, wl.H, wl.D
    perm = torch.full((n,), 5, dtype=torch.int32, device="cuda")     # stale values
    mk = lambda: torch.full((wl.capacity, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    qp, kp, vp, cu, perm = h3.pack_rope(d["q"], d["k"], d["v"], d["tags"], d["pos"], d["seg"], wl.n_seg,
                                        wl.rope, wl.time_offset, capacity=wl.capacity, q_out=mk(),
                                        k_out=mk(), v_out=mk(), perm=perm)
    r = _oracle_full(wl, q, k, v)
    total = int(r["cu"][-1])
    assert total == n - 4
    assert cu.cpu().numpy().tolist() == r["cu"].tolist()
    assert perm.cpu().numpy().tolist() == r["perm"].tolist()          # -1 tail included
    o = mk()
    h3.varlen_attn_fwd(qp, kp, vp, cu, total_rows=total, max_seqlen=70, o=o)
    npm = wl.n_per_modality()
    outs = [torch.full((c, H, D), 3.0, dtype=torch.bfloat16, device="cuda") for c in npm]
    idxs = [torch.full((c,), 1234, dtype=torch.int32, device="cuda") for c in npm]
    h3.unpack_by_modality(o, perm, d["tags"], npm, outs=outs, idxs=idxs)
    torch.cuda.synchronize()
    assert_close(o[:total], r["o"], "bf16", "O with dropped tokens")
    for m in range(3):
        want = r["idxs"][m]
        assert np.array_equal(idxs[m].cpu().numpy(), want)
        have = torch.from_numpy(want >= 0).cuda()
        assert torch.equal(outs[m][have], o[idxs[m][have].long()])
        assert (outs[m][~have] == 3.0).all()                          # dropped: row not written
    assert sum(int((x < 0).sum()) for x in r["idxs"]) == 4
    # the epilogue: dropped tokens keep their state, idx -1
    z, anchor = W.make_states(wl, seed=82)
    zd = [x.cuda() for x in z]
    sig, nxt = (0.0, 0.7, 0.6), (0.0, 0.65, 0.5)
    idx2 = [torch.full((c,), 1234, dtype=torch.int32, device="cuda") for c in npm]
    h3.unpack_euler(o, perm, d["tags"], npm, [None, zd[1], zd[2]], sig, nxt, idxs=idx2)
    torch.cuda.synchronize()
    new, ridx = oracle.unpack_euler(f64(o[:total]), r["perm"], wl.tags,
                                    [None, z[1].double().numpy(), z[2].double().numpy()], sig, nxt)
    for m in (1, 2):
        assert np.array_equal(idx2[m].cpu().numpy(), ridx[m])
        assert np.max(np.abs(zd[m].cpu().double().numpy() - new[m])) <= 1e-5
        dropped = torch.from_numpy(ridx[m] < 0)
        assert torch.equal(zd[m].cpu()[dropped], z[m][dropped])       # not stepped, bit for bit


def test_medium_8527_tokens_full():
    wl = W.make_workload(1)
    q, k, v = W.make_qkv(wl)
    g = run_path(wl, device_inputs(wl, q, k, v))
    r = _oracle_full(wl, q, k, v)
    _check_full(wl, g, r, stagewise=False)
    heads = [0, 11, 23]
    ref = oracle.attention(f64(g["q"][:wl.n, heads]), f64(g["k"][:wl.n, heads]),
                           f64(g["v"][:wl.n, heads]), r["cu"])
    assert_close(g["o"][:wl.n, heads], ref, "bf16", "O stage-wise, 3 heads")


@pytest.mark.parametrize("shifted", [False, True])
def test_window_partitions_full(shifted):
    wl = W.make_workload(4, shifted=shifted)
    q, k, v = W.make_qkv(wl)
    g = run_path(wl, device_inputs(wl, q, k, v))
    heads = [0, 9, 23]
    r = _oracle_full(wl, q, k, v, heads)
    _check_full(wl, g, r, heads=heads)
    # unpack restores grid (source) order: video index of source token i is inv_perm[i]
    inv = np.empty(wl.n, np.int64)
    inv[r["perm"]] = np.arange(wl.n)
    assert np.array_equal(g["idxs"][W.VIDEO].cpu().numpy(), inv)


def _sampled_full_size(index, heads, n_random):
    wl = W.make_workload(index)
    q, k, v = W.make_qkv(wl)
    g = run_path(wl, device_inputs(wl, q, k, v))
    n = wl.n
    cu, perm = oracle.pack(wl.seg, wl.n_seg)
    assert np.array_equal(g["cu"].cpu().numpy(), cu)
    assert np.array_equal(g["perm"][:n].cpu().numpy(), perm)
    rows = sample_rows(cu, n_random=n_random, seed=index)
    rows_d = torch.from_numpy(rows).cuda()
    # RoPE on the sampled source rows (RoPE is per token)
    src = perm[rows]
    qs, ks = W.to_f64(q[src]), W.to_f64(k[src])
    qr, kr = oracle.rope_qk(qs, ks, wl.tags[src], wl.pos[src], wl.rope, wl.time_offset)
    assert_close(g["q"][rows_d], qr, "bf16", "packed Q' sampled rows")
    assert_close(g["k"][rows_d], kr, "bf16", "packed K' sampled rows")
    # attention, end to end: oracle RoPE of every token for the sampled heads
    qh, kh, vh = W.to_f64(q[:, heads]), W.to_f64(k[:, heads]), W.to_f64(v[:, heads])
    qrh, krh = oracle.rope_qk(qh, kh, wl.tags, wl.pos, wl.rope, wl.time_offset)
    ref = cached(oracle.attention_rows, qrh[perm], krh[perm], vh[perm], cu, rows)
    got = g["o"][rows_d][:, heads]
    assert_close(got, ref, "bf16", "O end-to-end sampled rows")
    # attention, stage-wise on the GPU's own packed tensors
    ref2 = cached(oracle.attention_rows, f64(g["q"][:n, heads]), f64(g["k"][:n, heads]),
                  f64(g["v"][:n, heads]), cu, rows)
    assert_close(got, ref2, "bf16", "O stage-wise sampled rows")
    # unpack: indices bit-exact, values an exact gather, pad rows untouched
    _, idxs = oracle.unpack(np.zeros((n, 1, 1)), perm, wl.tags)
    for m in range(3):
        assert np.array_equal(g["idxs"][m].cpu().numpy(), idxs[m])
        assert torch.equal(g["outs"][m], g["o"][g["idxs"][m].long()])
    assert torch.isnan(g["o"][n:].float()).all()
    assert torch.isfinite(g["o"][:n].float()).all()


def test_h3_step_58758_tokens_sampled():
    _sampled_full_size(2, heads=[0, 17, 39], n_random=48)


def test_continuation_153735_tokens_sampled():
    _sampled_full_size(3, heads=[0, 25], n_random=32)


# ------------------------------------------------------------ GPU properties
def _packed_inputs(wl, seed=5, scale=None):
    q, k, v = W.make_qkv(wl, seed=seed)
    if scale is not None:
        q = (q.float() * scale).to(q.dtype)
    return [t.cuda() for t in (q, k, v)]


def test_segments_bit_identical_alone_and_poisoned():
    wl = W.make_custom([300, 129, 64, 1, 700], H=2, D=128)
    q, k, v = _packed_inputs(wl)
    cu, _ = oracle.pack(wl.seg, wl.n_seg)
    cu_d = torch.from_numpy(cu).cuda()
    o = h3.varlen_attn_fwd(q, k, v, cu_d, total_rows=wl.n)
    o2 = h3.varlen_attn_fwd(q, k, v, cu_d, total_rows=wl.n)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)                                   # repeat run: bit-identical
    for s in range(wl.n_seg):
        a, b = int(cu[s]), int(cu[s + 1])
        alone = h3.varlen_attn_fwd(q[a:b].contiguous(), k[a:b].contiguous(), v[a:b].contiguous(),
                                   torch.tensor([0, b - a], dtype=torch.int32, device="cuda"),
                                   total_rows=b - a)
        assert torch.equal(alone, o[a:b])                       # packed == alone, bit for bit
        qp, kp, vp = q.clone(), k.clone(), v.clone()
        for t in (qp, kp, vp):
            t[:a] = float("nan")
            t[b:] = float("nan")
        op = h3.varlen_attn_fwd(qp, kp, vp, cu_d, total_rows=wl.n)
        assert torch.equal(op[a:b], o[a:b])                     # out-of-segment poison: no effect


def test_nan_pad_rows_are_never_read():
    wl = W.make_custom([256, 3661], H=2, D=128)
    cap = wl.n + 58                                              # the page's 58 pad rows
    q, k, v = _packed_inputs(wl)
    cu_d = torch.from_numpy(oracle.pack(wl.seg, wl.n_seg)[0]).cuda()
    pad = lambda t, val: torch.cat([t, torch.full((cap - wl.n,) + tuple(t.shape[1:]), val, dtype=t.dtype,
                                                  device="cuda")])
    clean = h3.varlen_attn_fwd(pad(q, 0.0), pad(k, 0.0), pad(v, 0.0), cu_d, total_rows=wl.n)
    dirty = h3.varlen_attn_fwd(pad(q, float("nan")), pad(k, float("inf")), pad(v, float("nan")), cu_d,
                               total_rows=wl.n)
    torch.cuda.synchronize()
    assert torch.equal(clean[:wl.n], dirty[:wl.n])
    assert torch.isfinite(dirty[:wl.n].float()).all()


@pytest.mark.parametrize("case", ["peaked", "large_logit"])
def test_online_softmax_stress(case):
    """Peaked softmax (Q x 4) and one key per segment with a large logit, which
    forces the running max to move late in the segment."""
    wl = W.make_custom([700, 129, 1000], H=2, D=128)
    q, k, v = _packed_inputs(wl, scale=4.0 if case == "peaked" else None)
    cu, _ = oracle.pack(wl.seg, wl.n_seg)
    if case == "large_logit":
        for a, b in zip(cu[:-1], cu[1:]):
            j = int(b) - 3
            k[j] = (q[a:b].float().mean(0) * 20.0).to(k.dtype)
    o = h3.varlen_attn_fwd(q, k, v, torch.from_numpy(cu).cuda(), total_rows=wl.n)
    torch.cuda.synchronize()
    ref = oracle.attention(f64(q), f64(k), f64(v), cu)
    assert_close(o, ref, "bf16", "O " + case)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("rate", [0.3, 0.04])
def test_online_softmax_rescale_every_few_tiles(D, rate):
    """Logits that climb along each segment by `rate` (log2 units) per key, so
    the running max moves and the accumulators are rescaled every one
    (rate 0.3) or every few (rate 0.04) 32-key halves, deep inside the
    kernel's main loop; every row checked against the oracle."""
    wl = W.make_custom([3000, 1500, 200], H=2, D=D)
    q, k, v = W.make_qkv(wl, seed=11)
    cu, _ = oracle.pack(wl.seg, wl.n_seg)
    amp = 4.0
    qf, kf = q.float() * 0.1, k.float() * 0.1
    qf[:, :, 0] += amp
    ramp = rate / (D ** -0.5 * np.log2(np.e) * amp)        # k[:, :, 0] step per key
    for a, b in zip(cu[:-1], cu[1:]):
        kf[a:b, :, 0] += (torch.arange(b - a, dtype=torch.float32) * ramp)[:, None]
    q, k = qf.to(q.dtype).cuda(), kf.to(k.dtype).cuda()
    v = v.cuda()
    o = h3.varlen_attn_fwd(q, k, v, torch.from_numpy(cu).cuda(), total_rows=wl.n)
    torch.cuda.synchronize()
    ref = oracle.attention(f64(q), f64(k), f64(v), cu)
    assert_close(o, ref, "bf16", "O rescale rate %g D %d" % (rate, D))


@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "bf16"), (128, "f32")])
def test_maximum_head_count(D, dtype):
    # H = 4096, the most the ABI accepts: a token row is H*D elements (1 MiB in
    # bf16 at D = 128) and a 64-row tile 64 MiB, the reach that the kernels'
    # 32-bit tile-relative offsets are sized for.  Ragged segments of 70 and
    # 130 rows, NaN pad rows up to the capacity; the oracle checks the first,
    # a middle and the last heads (heads are independent).
    # Inputs come from the seeded device generator (the CPU one takes ~45 s
    # at this size); only the checked heads are copied to the host.
    wl = W.make_custom([70, 130], H=4096, D=D, dtype=dtype, q_scale=0.5 if dtype == "bf16" else 1.0, index=7)
    q, k, v = W.make_qkv_on_device(wl, "cuda")
    g = run_path(wl, device_inputs(wl, q, k, v))
    heads = [0, 1, 2047, 4094, 4095]
    qh, kh, vh = (t[:, heads].cpu() for t in (q, k, v))
    _check_full(wl, g, _oracle_full(wl, qh, kh, vh), heads=heads)


def test_softmax_scale_argument():
    wl = W.make_custom([200, 77], H=2, D=64)
    q, k, v = _packed_inputs(wl)
    cu, _ = oracle.pack(wl.seg, wl.n_seg)
    o = h3.varlen_attn_fwd(q, k, v, torch.from_numpy(cu).cuda(), total_rows=wl.n, softmax_scale=0.3)
    torch.cuda.synchronize()
    ref = oracle.attention(f64(q), f64(k), f64(v), cu, softmax_scale=0.3)
    assert_close(o, ref, "bf16", "O scale 0.3")


def test_empty_inputs_and_validation():
    dev = "cuda"
    wl = W.make_custom([0, 0], H=2, D=128)
    e = torch.empty((0, 2, 128), dtype=torch.bfloat16, device=dev)
    _, _, _, cu, _ = h3.pack_rope(e, e, e, torch.empty(0, dtype=torch.uint8, device=dev),
                                  torch.empty((0, 3), dtype=torch.int32, device=dev),
                                  torch.empty(0, dtype=torch.int32, device=dev), 2, wl.rope, 0.0,
                                  capacity=0)
    torch.cuda.synchronize()
    assert cu.cpu().tolist() == [0, 0, 0]
    z = torch.zeros((4, 2, 128), dtype=torch.bfloat16, device=dev)
    o = torch.full_like(z, 7.0)
    h3.varlen_attn_fwd(z, z, z, torch.zeros(3, dtype=torch.int32, device=dev), total_rows=0, o=o)
    torch.cuda.synchronize()
    assert (o == 7.0).all()                                       # nothing written
    good = torch.tensor([0, 3, 3, 10], dtype=torch.int32, device=dev)
    assert h3.validate_seqlens(good, capacity=10) == 0
    assert h3.validate_seqlens(good, capacity=9) == 5             # H3_ERR_CAPACITY
    assert h3.validate_seqlens(torch.tensor([0, 4, 3], dtype=torch.int32, device=dev), 10) == 4
    assert h3.validate_seqlens(torch.tensor([1, 4], dtype=torch.int32, device=dev), 10) == 4


def test_short_segment_kernel_matches_main_kernel_bit_for_bit():
    """Segments up to 512 rows with max_seqlen given, and few 128-row items
    (here 147 for 512 workgroup slots), go to the short-segment kernel
    (128-row tiles, 32-key K/V tiles, two workgroups per CU); without
    the hint the main kernel runs.  Per row both do the same arithmetic in the
    same order, so the outputs must be identical, and match the oracle."""
    lengths = [1, 31, 32, 33, 63, 64, 65, 0, 127, 128, 129, 255, 256, 257, 300, 511, 512]
    wl = W.make_custom(lengths, H=3, D=128)
    q, k, v = W.make_qkv(wl, seed=81)
    cu, _ = oracle.pack(wl.seg, wl.n_seg)
    # planted large logits so the lazy rescale runs inside short segments too
    qf, kf = q.float(), k.float()
    qf[:, :, 0] += 3.0
    kf[::37, :, 0] += 40.0
    q, k = qf.to(q.dtype).cuda(), kf.to(k.dtype).cuda()
    v = v.cuda()
    dcu = torch.from_numpy(cu).cuda()
    o_main = h3.varlen_attn_fwd(q, k, v, dcu, total_rows=wl.n, max_seqlen=0)
    o_short = h3.varlen_attn_fwd(q, k, v, dcu, total_rows=wl.n, max_seqlen=512)
    torch.cuda.synchronize()
    assert torch.equal(o_main[:wl.n], o_short[:wl.n])
    ref = oracle.attention(f64(q), f64(k), f64(v), cu)
    assert_close(o_short[:wl.n], ref, "bf16", "short-segment kernel")


@pytest.mark.parametrize("H,repeats", [(24, 8), (1, 50)])
def test_multi_item_kernel_matches_main_kernel_bit_for_bit(H, repeats):
    """With many short segments (at least four 128-row items per workgroup
    slot), the short-segment call runs the several-items-per-workgroup
    kernel: each workgroup walks a strided list of items, and the K/V tile
    ring and the next item's Q loads run across item boundaries.  Ragged
    tails, one-tile items, empty segments and planted rescales inside a
    workgroup's item sequence; outputs identical to the main kernel's, and
    to the oracle on two heads.  At H = 1 a row is one 256-byte head slice,
    so the range check that drops an item's stores past its segment end
    (rows of the next segment) has no slack."""
    base = [1, 31, 32, 33, 63, 64, 65, 0, 127, 128, 129, 255, 256, 257, 300, 511, 512]
    lengths = [base[(7 * i) % len(base)] for i in range(repeats * len(base))]
    wl = W.make_custom(lengths, H=H, D=128)
    q, k, v = W.make_qkv(wl, seed=82)
    cu, _ = oracle.pack(wl.seg, wl.n_seg)
    qf, kf = q.float(), k.float()
    qf[:, :, 0] += 3.0
    kf[::37, :, 0] += 40.0
    q, k = qf.to(q.dtype).cuda(), kf.to(k.dtype).cuda()
    v = v.cuda()
    dcu = torch.from_numpy(cu).cuda()
    o_main = h3.varlen_attn_fwd(q, k, v, dcu, total_rows=wl.n, max_seqlen=0)
    o_multi = h3.varlen_attn_fwd(q, k, v, dcu, total_rows=wl.n, max_seqlen=512)
    o_again = h3.varlen_attn_fwd(q, k, v, dcu, total_rows=wl.n, max_seqlen=512)
    torch.cuda.synchronize()
    assert torch.equal(o_main[:wl.n], o_multi[:wl.n])
    assert torch.equal(o_multi, o_again)
    heads = sorted({0, H - 1})
    ref = oracle.attention(f64(q[:, heads]), f64(k[:, heads]), f64(v[:, heads]), cu)
    assert_close(o_multi[:wl.n, heads], ref, "bf16", "several-items-per-workgroup kernel")


@pytest.mark.parametrize("repeats", [1, 12])
def test_max_seqlen_hint_below_a_segment_length_changes_nothing(repeats):
    """The hint only selects kernels: with max_seqlen = 512 but segments of up
    to 3,000 rows, the short-segment kernels (one item per workgroup for the
    few-item case, several for the many-item case) still walk every key tile
    of every segment, and the output equals the main kernel's bit for bit."""
    lengths = [3000, 17, 512, 1300, 0, 129, 2049, 64] * repeats
    wl = W.make_custom(lengths, H=8, D=128)
    q, k, v = (t.cuda() for t in W.make_qkv(wl, seed=83))
    cu, _ = oracle.pack(wl.seg, wl.n_seg)
    dcu = torch.from_numpy(cu).cuda()
    o_main = h3.varlen_attn_fwd(q, k, v, dcu, total_rows=wl.n, max_seqlen=0)
    o_hint = h3.varlen_attn_fwd(q, k, v, dcu, total_rows=wl.n, max_seqlen=512)
    torch.cuda.synchronize()
    assert torch.equal(o_main[:wl.n], o_hint[:wl.n])
