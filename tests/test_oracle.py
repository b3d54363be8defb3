"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: every check is a printed page
value, a closed form, an identity of rotations / softmax, an independent
formulation (complex numbers, torch's float64 SDPA) or brute force in pure
Python on tiny inputs.
"""
import cmath
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = []


def _f64(wl, seed=None):
    q, k, v = W.make_qkv(wl, seed=seed)
    return W.to_f64(q), W.to_f64(k), W.to_f64(v)


# ---------------------------------------------------------------- page values
def test_page_cu_seqlens_examples(golden):
    ex2 = golden["cu_seqlens_text_video"]
    wl = W.make_custom([10, 20], H=1, D=64, modalities=[W.TEXT, W.VIDEO])
    cu, perm = oracle.pack(wl.seg, wl.n_seg)
    assert cu.tolist() == ex2["cu_seqlens"]
    ex3 = golden["cu_seqlens_text_video_audio"]
    wl0 = W.make_workload(0)
    cu, perm = oracle.pack(wl0.seg, wl0.n_seg)
    assert cu.tolist() == ex3["cu_seqlens"]
    assert perm.tolist() == list(range(45))
    assert [(g[0], g[2]) for g in wl0.groups] == [tuple(x) for x in ex3["groups"]]


def test_page_exact_zero_weights(golden):
    """Token 15 (video) dots only with keys 10..29; keys 0..9 get weight exactly 0."""
    ex = golden["cu_seqlens_text_video"]
    wl = W.make_workload(0)
    q, k, v = _f64(wl)
    qr, kr = oracle.rope_qk(q, k, wl.tags, wl.pos, wl.rope, wl.time_offset)
    cu, perm = oracle.pack(wl.seg, wl.n_seg)
    P = oracle.attention_weights(qr[perm], kr[perm], cu)
    lo, hi = ex["visible_keys"]
    z0, z1 = ex["zero_weight_keys"]
    i = ex["query"]
    for h in range(wl.H):
        assert np.all(P[h, i, z0:z1 + 1] == 0.0)
        assert np.all(P[h, i, hi + 1:] == 0.0)
        assert np.all(P[h, i, lo:hi + 1] > 0.0)
        assert abs(P[h, i, lo:hi + 1].sum() - 1.0) < 1e-15
    # every off-diagonal block is exactly zero; every row sums to one
    mask = np.zeros((wl.n, wl.n), bool)
    for a, b in zip(cu[:-1], cu[1:]):
        mask[a:b, a:b] = True
    assert np.all(P[:, ~mask] == 0.0)
    assert np.allclose(P.sum(axis=2), 1.0, atol=1e-15, rtol=0)


def test_attention_weights_in_block_values():
    """Inside the segment blocks the weight matrix is the softmax itself: each
    diagonal block equals torch's float64 softmax of that segment's scaled
    scores (a library routine), and P.V equals the attention output, which is
    pinned to torch's scaled_dot_product_attention separately.  A wrong scale,
    a transposed block or weights taken from the wrong segment fail one of
    these."""
    wl = W.make_workload(0)
    q, k, v = _f64(wl)
    r = oracle.run(q, k, v, wl.tags, wl.pos, wl.seg, wl.n_seg, wl.rope, wl.time_offset)
    qp, kp, vp, cu = r["q"], r["k"], r["v"], r["cu"]
    P = oracle.attention_weights(qp, kp, cu)
    D = qp.shape[2]
    for h in range(wl.H):
        assert np.allclose(P[h] @ vp[:, h], r["o"][:, h], atol=1e-14, rtol=0)
        for a, b in zip(cu[:-1], cu[1:]):
            S = torch.from_numpy(qp[a:b, h]) @ torch.from_numpy(kp[a:b, h]).T
            want = torch.softmax(S * (1.0 / np.sqrt(D)), dim=1).numpy()
            assert np.allclose(P[h, a:b, a:b], want, atol=1e-15, rtol=0)
    # a non-default scale moves the weights the same way
    P2 = oracle.attention_weights(qp, kp, cu, softmax_scale=0.3)
    a, b = int(cu[1]), int(cu[2])
    S = torch.from_numpy(qp[a:b, 1]) @ torch.from_numpy(kp[a:b, 1]).T
    assert np.allclose(P2[1, a:b, a:b], torch.softmax(S * 0.3, dim=1).numpy(), atol=1e-15, rtol=0)
    assert not np.allclose(P2[1, a:b, a:b], P[1, a:b, a:b], atol=1e-3)


def test_page_trim_numbers(golden):
    ex = golden["trim_padding"]
    assert ex["aligned_length"] - ex["effective_tokens"] == ex["padding"]
    assert ex["aligned_length"] == 919 * W.ALIGN
    wl2 = W.make_workload(2)
    assert wl2.n == ex["effective_tokens"] and wl2.capacity == ex["aligned_length"]
    # aligned already: trimming is a no-op
    wl4 = W.make_workload(4)
    assert wl4.capacity == wl4.n


def test_page_time_shift(golden):
    ex = golden["time_shift"]
    s = ex["window_start_frame"]
    d = oracle.time_shift(s)
    assert abs(d - 1190.0 / 3.0) < 1e-12            # 238 * 40 / 24 = 396.666...
    assert round(d, ex["printed_decimals"]) == ex["shift_printed"]
    assert d != int(d)                              # the fraction is kept


def test_page_continuation_order(golden):
    ex = golden["continuation_order"]
    wl = W.make_workload(3)
    mods = [g[1] for g in wl.groups]
    assert mods == [W.TEXT, W.AUDIO, W.VIDEO, W.AUDIO, W.VIDEO]
    assert len(ex["order"]) == len(wl.groups) == 5
    assert wl.groups[2][2] == ex["video_reference_frames"] * 48 * 84
    assert wl.n_seg == 1 and wl.time_offset == golden["time_shift"]["window_start_frame"]


def test_window_partition_closed_forms():
    """Regular 4x8x8 windows over 16x64x112: 4*8*14 = 448 windows of 256.
    Half-shifted: 5*9*15 = 675 edge-cropped windows; sizes 256/128/64/32 occur
    3*7*13 / (2*7*13 + 3*2*13 + 3*7*2) / (2*2*13 + 2*7*2 + 3*2*2) / 2*2*2 times."""
    reg = W.make_workload(4, shifted=False)
    L = reg.segment_lengths()
    assert reg.n_seg == 448 and np.all(L == 256)
    sh = W.make_workload(4)
    L = sh.segment_lengths()
    assert sh.n_seg == 675 and L.sum() == 114688
    sizes, counts = np.unique(L, return_counts=True)
    expect = {256: 3 * 7 * 13, 128: 2 * 7 * 13 + 3 * 2 * 13 + 3 * 7 * 2,
              64: 2 * 2 * 13 + 2 * 7 * 2 + 3 * 2 * 2, 32: 2 * 2 * 2}
    assert dict(zip(sizes.tolist(), counts.tolist())) == expect


# ---------------------------------------------------------------------- pack
def _pack_brute(seg, n_seg):
    perm, cu = [], [0]
    for s in range(n_seg):
        members = [i for i in range(len(seg)) if seg[i] == s]
        perm += members
        cu.append(cu[-1] + len(members))
    return cu, perm + [-1] * (len(seg) - len(perm))


@pytest.mark.parametrize("case", ["c4_shifted", "random", "empty_segments", "dropped", "all_dropped"])
def test_pack_stable_bruteforce(case):
    rng = np.random.default_rng(7)
    if case == "c4_shifted":
        wl = W.make_workload(4)
        seg, n_seg = wl.seg[:6000], wl.n_seg      # a prefix: still unsorted windows
    elif case == "random":
        seg, n_seg = rng.integers(0, 13, size=500).astype(np.int32), 13
    elif case == "empty_segments":
        seg, n_seg = np.array([3, 3, 0, 5, 0, 3], np.int32), 7
    elif case == "dropped":                       # ids outside 0..n_seg-1 belong to no segment
        seg, n_seg = np.array([2, -1, 0, 9, 2, 7, 0, -5, 1], np.int32), 7
    else:
        seg, n_seg = np.array([4, -1, 4], np.int32), 3
    cu, perm = oracle.pack(seg, n_seg)
    cu_b, perm_b = _pack_brute(seg.tolist(), n_seg)
    assert cu.tolist() == cu_b and perm.tolist() == perm_b
    assert cu.dtype == np.int32 and perm.dtype == np.int32


# ---------------------------------------------------------------------- RoPE
def test_rope_frequencies_textbook_values():
    """RoFormer: pair j of a d-wide slice turns by pos * 10000^(-2j/d).
    Values below are written out, not recomputed with the oracle's formula."""
    wl = W.make_custom([4], H=1, D=64, modalities=[W.TEXT])
    th = oracle.rope_angles(wl.tags, wl.pos, wl.rope, 0.0, 64)
    assert np.all(th[0] == 0.0)                              # position 0: no rotation
    assert th[1, 0] == 1.0                                   # pair 0 turns 1 rad per unit
    assert abs(th[1, 1] - 0.7498942093324559) < 1e-15        # 10000^(-1/32)
    assert abs(th[1, 16] - 0.01) < 1e-15                     # 10000^(-1/2)
    assert abs(th[3, 31] - 3 * 1.333521432163324e-4) < 1e-18  # 3 * 10000^(-31/32)


def test_rope_complex_form_bruteforce():
    """The rotation equals (x0 + i x1) * exp(i theta) (pure-Python complex)."""
    wl = W.make_workload(0)
    q, k, v = _f64(wl)
    th = oracle.rope_angles(wl.tags, wl.pos, wl.rope, 0.0, wl.D)
    qr = oracle.apply_rope(q, th)
    for i in range(0, wl.n, 7):
        for h in range(wl.H):
            for j in range(wl.D // 2):
                z = complex(q[i, h, 2 * j], q[i, h, 2 * j + 1]) * cmath.exp(1j * th[i, j])
                assert abs(z.real - qr[i, h, 2 * j]) < 1e-14
                assert abs(z.imag - qr[i, h, 2 * j + 1]) < 1e-14


def test_rope_norm_and_relative_position():
    """|pair| is kept; <R(p) q, R(p') k> = <q, R(p'-p) k> for one 1-D scheme."""
    rng = np.random.default_rng(3)
    D = 64
    wl = W.make_custom([50], H=1, D=D, modalities=[W.TEXT])
    th = oracle.rope_angles(wl.tags, wl.pos, wl.rope, 0.0, D)
    x = rng.standard_normal((50, 1, D))
    xr = oracle.apply_rope(x, th)
    n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n1 = xr[..., 0::2] ** 2 + xr[..., 1::2] ** 2
    assert np.allclose(n0, n1, rtol=1e-13, atol=0)
    q = np.repeat(rng.standard_normal((1, 1, D)), 50, axis=0)
    k = np.repeat(rng.standard_normal((1, 1, D)), 50, axis=0)
    qr, kr = oracle.apply_rope(q, th), oracle.apply_rope(k, th)
    for p, pp in [(3, 10), (20, 27), (0, 7), (40, 47), (12, 5), (30, 23)]:
        lhs = float(qr[p, 0] @ kr[pp, 0])
        if pp >= p:       # R(pp - p) k is k rotated to text position pp - p
            rhs = float(q[0, 0] @ kr[pp - p, 0])
        else:             # negative offset: rotate k backwards by position p - pp
            back = oracle.apply_rope(k[:1], -th[p - pp:p - pp + 1])
            rhs = float(q[0, 0] @ back[0, 0])
        assert abs(lhs - rhs) < 1e-12
    # same offset, different absolute positions: same score
    assert abs(float(qr[3, 0] @ kr[10, 0]) - float(qr[20, 0] @ kr[27, 0])) < 1e-12


def test_rope_video_slices_and_audio_scale():
    D = 64
    wl = W.make_workload(0)          # video grid t 0..4, h 0..1, w 0..1; audio ticks 0..14
    th = oracle.rope_angles(wl.tags, wl.pos, wl.rope, 0.0, D)
    vid = np.nonzero(wl.tags == W.VIDEO)[0]
    d_t, d_h, d_w = 16, 24, 24
    for i in vid:
        t, h, w = wl.pos[i]
        assert th[i, 0] == t and th[i, d_t // 2] == h and th[i, (d_t + d_h) // 2] == w
        if h == 0 and w == 0:
            assert np.all(th[i, d_t // 2:] == 0.0)
        # t slice is 1-D RoPE of width 16: pair j turns t * 10000^(-2j/16)
        assert abs(th[i, 1] - t * 10000 ** (-1 / 8)) < 1e-14
        assert abs(th[i, d_t // 2 + 1] - h * 10000 ** (-1 / 12)) < 1e-14
    # audio tick 5 at 40 Hz is 3.0 video frames: same angles as text index 3
    aud = np.nonzero(wl.tags == W.AUDIO)[0]
    txt = np.nonzero(wl.tags == W.TEXT)[0]
    assert np.allclose(th[aud[5]], th[txt[3]], rtol=1e-15, atol=0)


def test_rope_time_shift_applies_to_time_axis_only():
    D = 64
    wl = W.make_workload(0)
    th0 = oracle.rope_angles(wl.tags, wl.pos, wl.rope, 0.0, D)
    th1 = oracle.rope_angles(wl.tags, wl.pos, wl.rope, 238.0, D)
    delta = 1190.0 / 3.0
    txt = wl.tags == W.TEXT
    vid = wl.tags == W.VIDEO
    aud = wl.tags == W.AUDIO
    assert np.array_equal(th0[txt], th1[txt])                       # text: no shift
    assert np.allclose(th1[vid, 0] - th0[vid, 0], delta, rtol=0, atol=1e-12)
    assert np.array_equal(th0[vid, 8:], th1[vid, 8:])               # h, w untouched
    assert np.allclose(th1[aud, 0] - th0[aud, 0], delta, rtol=0, atol=1e-12)


# ----------------------------------------------------------------- attention
def _sdpa_per_segment(q, k, v, cu):
    out = np.zeros_like(q)
    for a, b in zip(cu[:-1], cu[1:]):
        if b <= a:
            continue
        Q = torch.from_numpy(q[a:b]).permute(1, 0, 2).unsqueeze(0)
        K = torch.from_numpy(k[a:b]).permute(1, 0, 2).unsqueeze(0)
        V = torch.from_numpy(v[a:b]).permute(1, 0, 2).unsqueeze(0)
        O = torch.nn.functional.scaled_dot_product_attention(Q, K, V)
        out[a:b] = O[0].permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("lengths", [[10, 20, 15], [1, 0, 33, 64, 65, 3], [200]])
def test_attention_vs_torch_sdpa(lengths):
    wl = W.make_custom(lengths, H=3, D=64, dtype="f32", q_scale=1.0)
    q, k, v = _f64(wl)
    cu, perm = oracle.pack(wl.seg, wl.n_seg)
    o = oracle.attention(q[perm], k[perm], v[perm], cu)
    ref = _sdpa_per_segment(q[perm], k[perm], v[perm], cu)
    assert np.max(np.abs(o - ref)) < 1e-13
    rows = np.arange(0, wl.n, 5)
    o_rows = oracle.attention_rows(q[perm], k[perm], v[perm], cu, rows, heads=[2, 0])
    assert np.max(np.abs(o_rows - ref[rows][:, [2, 0]])) < 1e-13


def test_attention_bruteforce_tiny():
    """Pure-Python triple loop with math.exp on the 45-token workload."""
    wl = W.make_workload(0)
    q, k, v = _f64(wl)
    cu, perm = oracle.pack(wl.seg, wl.n_seg)
    o = oracle.attention(q, k, v, cu)
    D = wl.D
    for (a, b) in zip(cu[:-1].tolist(), cu[1:].tolist()):
        for h in range(wl.H):
            for i in range(a, b):
                s = [sum(q[i, h, d] * k[j, h, d] for d in range(D)) / math.sqrt(D) for j in range(a, b)]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                z = sum(e)
                for d in range(0, D, 9):
                    ref = sum(e[j - a] * v[j, h, d] for j in range(a, b)) / z
                    assert abs(ref - o[i, h, d]) < 1e-13


def test_attention_closed_forms():
    rng = np.random.default_rng(11)
    H, D = 2, 64
    cu = np.array([0, 1, 9, 40], np.int32)          # a length-1 segment, then two more
    q = rng.standard_normal((40, H, D))
    k = rng.standard_normal((40, H, D))
    v = rng.standard_normal((40, H, D))
    o = oracle.attention(q, k, v, cu)
    assert np.array_equal(o[0], v[0])                                   # L = 1 -> V
    o = oracle.attention(np.zeros_like(q), k, v, cu)                     # Q = 0 -> mean V
    assert np.allclose(o[1:9], v[1:9].mean(axis=0, keepdims=True), atol=1e-14, rtol=0)
    assert np.allclose(o[9:40], v[9:40].mean(axis=0, keepdims=True), atol=1e-14, rtol=0)
    vc = np.full_like(v, 0.375)                                          # constant V
    assert np.allclose(oracle.attention(q, k, vc, cu), 0.375, atol=1e-15, rtol=0)
    ks = np.repeat(k[9:10], 40, axis=0)                                  # identical keys
    o = oracle.attention(q, ks, v, cu)
    assert np.allclose(o[9:40], v[9:40].mean(axis=0, keepdims=True), atol=1e-14, rtol=0)


def test_attention_packed_equals_segments_alone_and_pad_rows_unread():
    wl = W.make_workload(0)
    q, k, v = _f64(wl)
    cu, perm = oracle.pack(wl.seg, wl.n_seg)
    cap = wl.capacity
    pad = lambda x: np.concatenate([x, np.full((cap - wl.n,) + x.shape[1:], np.nan)])
    o = oracle.attention(pad(q), pad(k), pad(v), cu)
    assert np.all(o[wl.n:] == 0.0) and np.all(np.isfinite(o))
    for a, b in zip(cu[:-1], cu[1:]):
        alone = oracle.attention(q[a:b], k[a:b], v[a:b], np.array([0, b - a]))
        assert np.array_equal(alone, o[a:b])


def test_attention_key_permutation_invariance():
    wl = W.make_workload(0)
    q, k, v = _f64(wl)
    cu, _ = oracle.pack(wl.seg, wl.n_seg)
    o = oracle.attention(q, k, v, cu)
    rng = np.random.default_rng(5)
    p = np.arange(wl.n)
    for a, b in zip(cu[:-1], cu[1:]):
        p[a:b] = a + rng.permutation(b - a)
    o2 = oracle.attention(q, k[p], v[p], cu)
    assert np.max(np.abs(o - o2)) < 1e-13


@pytest.mark.parametrize("which", ["tiny", "windows"])
def test_time_shift_invariance_end_to_end(which):
    """Shifting every time coordinate of a single-modality segment by a
    constant leaves attention unchanged (RoPE depends on differences only)."""
    if which == "tiny":
        wl = W.make_workload(0)
    else:
        wl = W.make_custom([40, 24, 37], H=2, D=64, dtype="f32", q_scale=1.0)
    q, k, v = _f64(wl)
    r0 = oracle.run(q, k, v, wl.tags, wl.pos, wl.seg, wl.n_seg, wl.rope, 0.0)
    r1 = oracle.run(q, k, v, wl.tags, wl.pos, wl.seg, wl.n_seg, wl.rope, 238.0)
    pos2 = wl.pos.copy()
    pos2[:, 0] += 17
    r2 = oracle.run(q, k, v, wl.tags, pos2, wl.seg, wl.n_seg, wl.rope, 0.0)
    for r in (r1, r2):
        assert np.max(np.abs(r["o"] - r0["o"])) < 1e-12
        assert np.max(np.abs(r["q"] - r0["q"])) > 1e-3      # RoPE itself did change


# -------------------------------------------------------------------- unpack
def test_unpack_bruteforce_and_grid_order():
    wl = W.make_workload(4)
    n = 3000
    seg = wl.seg[:n]
    cu, perm = oracle.pack(seg, wl.n_seg)
    o = np.arange(n, dtype=np.float64)[:, None, None] * np.ones((1, 1, 2))
    o = o[perm]                                   # packed copy of a source-indexed ramp
    tags = wl.tags[:n].copy()
    tags[::7] = W.TEXT
    tags[3::11] = W.AUDIO
    outs, idxs = oracle.unpack(o, perm, tags)
    perm_l = perm.tolist()
    for m in (W.TEXT, W.VIDEO, W.AUDIO):
        expect_idx = [perm_l.index(i) for i in range(n) if tags[i] == m]
        assert idxs[m].tolist() == expect_idx
        # source order restored: the ramp reads back as the source indices of modality m
        assert outs[m][:, 0, 0].tolist() == [float(i) for i in range(n) if tags[i] == m]
    assert sorted(np.concatenate(idxs).tolist()) == list(range(n))


def test_unpack_and_epilogue_with_dropped_tokens_bruteforce():
    """Tokens whose segment id is out of range have no packed row: pure-Python
    loops give their place in the modality slice index -1 and no value, and
    leave their state unstepped."""
    seg = np.array([0, 5, 1, -1, 0, 1, 2, 0], np.int32)          # tokens 1 and 3 dropped (n_seg 3)
    tags = np.array([0, 1, 1, 2, 2, 1, 0, 1], np.uint8)
    n = seg.shape[0]
    cu, perm = oracle.pack(seg, 3)
    assert cu.tolist() == [0, 3, 5, 6] and perm.tolist() == [0, 4, 7, 2, 5, 6, -1, -1]
    o = np.arange(6, dtype=np.float64)[:, None, None] * 10.0 + 1.0   # packed rows 0..5
    outs, idxs = oracle.unpack(o, perm, tags)
    row_of = {int(perm[p]): p for p in range(n) if perm[p] >= 0}
    for m in range(3):
        src = [i for i in range(n) if tags[i] == m]
        assert idxs[m].tolist() == [row_of.get(i, -1) for i in src]
        for kk, i in enumerate(src):
            if i in row_of:
                assert outs[m][kk, 0, 0] == 10.0 * row_of[i] + 1.0
            else:
                assert np.isnan(outs[m][kk]).all()
    z = [None, np.ones((4, 1, 1)), np.full((2, 1, 1), 2.0)]
    new, _ = oracle.unpack_euler(o, perm, tags, z, (0.0, 0.5, 0.5), (0.0, 0.25, 0.25))
    # video tokens 1 (dropped), 2, 5, 7 -> rows -, 3, 4, 2;  audio tokens 3 (dropped), 4 -> rows -, 1
    assert new[1][:, 0, 0].tolist() == [1.0, 1.0 - 0.25 * 31.0, 1.0 - 0.25 * 41.0, 1.0 - 0.25 * 21.0]
    assert new[2][:, 0, 0].tolist() == [2.0, 2.0 - 0.25 * 11.0]


def test_run_end_to_end_tiny():
    wl = W.make_workload(0)
    q, k, v = _f64(wl)
    r = oracle.run(q, k, v, wl.tags, wl.pos, wl.seg, wl.n_seg, wl.rope, wl.time_offset)
    assert r["cu"].tolist() == [0, 10, 30, 45]
    assert [x.shape[0] for x in r["outs"]] == [10, 20, 15]
    ref = _sdpa_per_segment(r["q"], r["k"], r["v"], r["cu"])
    assert np.max(np.abs(r["o"] - ref)) < 1e-13


# ------------------------------------------- denoising-step epilogue (Euler)
def test_sigma_schedule_page_values_and_closed_forms(golden):
    sp = golden["sigma_points"]
    ex = golden["denoise_three_step_example"]
    for shift in (sp["video_flow_shift"], sp["audio_flow_shift"]):
        s = oracle.sigma_schedule(sp["sigma_points"], shift)
        assert s.shape == (sp["sigma_points"] + 1,)
        assert s[0] == 1.0 and s[-1] == ex["last_target_sigma"]     # pure noise down to clean
        assert np.all(np.diff(s) < 0)
    # the three-step example: sigma_3 (max) -> sigma_2 -> sigma_1 -> 0
    s3 = oracle.sigma_schedule(ex["steps"], 3.0)
    assert s3.shape == (4,) and s3[0] == 1.0 and s3[-1] == 0.0
    # shift 1 is the plain even grid
    assert np.allclose(oracle.sigma_schedule(4, 1.0), [1.0, 0.75, 0.5, 0.25, 0.0], atol=0, rtol=0)
    # closed forms of the shift map at u = 1/2 (4 points: u = 1, 3/4, 1/2, 1/4)
    assert oracle.sigma_schedule(4, 3.0)[2] == pytest.approx(0.75, abs=1e-15)        # 1.5 / 2
    assert oracle.sigma_schedule(4, 12.0)[2] == pytest.approx(12.0 / 13.0, abs=1e-15)
    assert oracle.sigma_schedule(4, 3.0)[1] == pytest.approx(9.0 / 10.0, abs=1e-15)  # 2.25 / 2.5
    # a larger shift keeps more noise at every interior point: video above audio
    v = oracle.sigma_schedule(sp["sigma_points"], sp["video_flow_shift"])
    a = oracle.sigma_schedule(sp["sigma_points"], sp["audio_flow_shift"])
    assert np.all(v[1:-1] > a[1:-1])


def test_euler_step_lands_on_the_straight_flow_path():
    # z_sigma = (1 - sigma) x0 + sigma * noise, v = noise - x0: one eta = 0 step
    # with the exact velocity reaches the path point at sigma_next.
    rng = np.random.default_rng(5)
    x0 = rng.standard_normal((7, 3, 16))
    noise = rng.standard_normal((7, 3, 16))
    v = noise - x0
    for sig, nxt in ((1.0, 0.9), (0.6, 0.25), (0.3, 0.0)):
        z = (1 - sig) * x0 + sig * noise
        assert np.allclose(oracle.x0_from_velocity(z, v, sig), x0, atol=1e-13, rtol=0)
        got = oracle.euler_step(z, v, sig, nxt)
        assert np.allclose(got, (1 - nxt) * x0 + nxt * noise, atol=1e-13, rtol=0)


def test_euler_whole_schedule_telescopes():
    rng = np.random.default_rng(6)
    x0 = rng.standard_normal((5, 8))
    noise = rng.standard_normal((5, 8))
    for shift in (12.0, 3.0):
        s = oracle.sigma_schedule(50, shift)
        # constant velocity: the steps sum to sigma_end - sigma_start = -1
        z = noise.copy()
        for i in range(50):
            z = oracle.euler_step(z, x0, s[i], s[i + 1])
        assert np.allclose(z, noise - x0, atol=1e-12, rtol=0)
        # exact rectified-flow velocity from pure noise ends at the clean sample
        z = noise.copy()
        for i in range(50):
            z = oracle.euler_step(z, noise - x0, s[i], s[i + 1])
        assert np.allclose(z, x0, atol=1e-12, rtol=0)


def test_euler_repin_and_degenerate_steps():
    rng = np.random.default_rng(7)
    z = rng.standard_normal((6, 4))
    v = rng.standard_normal((6, 4))
    anchor = rng.standard_normal((6, 4))
    pinned = np.array([True, False, False, True, False, True])
    out = oracle.euler_step(z, v, 0.8, 0.5, pinned, anchor)
    assert np.array_equal(out[pinned], anchor[pinned])                  # restored exactly
    assert np.allclose(out[~pinned], z[~pinned] - 0.3 * v[~pinned], atol=1e-15, rtol=0)
    kept = oracle.euler_step(z, v, 0.8, 0.5, pinned, None)             # no anchor: pinned rows keep z
    assert np.array_equal(kept[pinned], z[pinned])
    # zero step (x0 = z - sigma v, then + sigma v: equal up to one rounding)
    assert np.allclose(oracle.euler_step(z, v, 0.4, 0.4), z, atol=1e-15, rtol=0)
    assert np.array_equal(oracle.euler_step(z, np.zeros_like(v), 0.9, 0.1), z)   # zero velocity


def test_unpack_euler_bruteforce():
    # pure-Python loops over tokens against the vectorised epilogue
    wl = W.make_workload(0)
    rng = np.random.default_rng(8)
    n = wl.n
    perm = rng.permutation(n).astype(np.int32)
    o = rng.standard_normal((n, 2, 4))
    tags = wl.tags
    npm = wl.n_per_modality()
    z = [None, rng.standard_normal((npm[1], 2, 4)), rng.standard_normal((npm[2], 2, 4))]
    anchor = [None, rng.standard_normal((npm[1], 2, 4)), rng.standard_normal((npm[2], 2, 4))]
    pinned = rng.random(n) < 0.3
    sig, nxt = (0.0, 0.7, 0.5), (0.0, 0.6, 0.2)
    new, idxs = oracle.unpack_euler(o, perm, tags, z, sig, nxt, pinned, anchor)
    inv = {int(perm[p]): p for p in range(n)}
    for m in (1, 2):
        k = 0
        for i in range(n):
            if int(tags[i]) != m:
                continue
            p = inv[i]
            assert idxs[m][k] == p
            for h in range(2):
                for d in range(4):
                    want = anchor[m][k, h, d] if pinned[i] else \
                        z[m][k, h, d] + (nxt[m] - sig[m]) * o[p, h, d]
                    assert abs(new[m][k, h, d] - want) <= 1e-15
            k += 1
        assert k == npm[m]
    assert new[0] is None


# ------------------------------------------------ VSA block-sparse attention
def _rand_qkv(rows, H, D, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((rows, H, D)), rng.standard_normal((rows, H, D)),
            rng.standard_normal((rows, H, D)))


def test_vsa_block_size_from_page_and_layout(golden):
    vb = golden["vsa_block"]
    assert int(np.prod(vb["block_dims"])) == vb["tokens_per_block"] == 64
    import inspect
    for f in (oracle.block_layout, oracle.block_means, oracle.vsa_select, oracle.vsa_attention):
        assert inspect.signature(f).parameters["block"].default == vb["tokens_per_block"]
    bstart, bseg, bcu = oracle.block_layout(np.array([0, 70, 70, 200, 201]))
    assert bstart.tolist() == [0, 64, 70, 134, 198, 200, 201]
    assert bseg.tolist() == [0, 0, 2, 2, 2, 3]
    assert bcu.tolist() == [0, 2, 2, 5, 6]


def test_vsa_block_means_bruteforce():
    q, _, _ = _rand_qkv(141, 2, 3, 1)
    cu = np.array([0, 77, 141])
    got = oracle.block_means(q, cu)
    bounds = [(0, 64), (64, 77), (77, 141)]
    for j, (a, b) in enumerate(bounds):
        for h in range(2):
            for d in range(3):
                acc = 0.0
                for r in range(a, b):
                    acc += q[r, h, d]
                assert abs(got[j, h, d] - acc / (b - a)) <= 1e-15


def test_vsa_select_bruteforce_with_ties():
    q, k, _ = _rand_qkv(300, 2, 4, 2)
    k[128:192] = k[0:64]                  # blocks 0 and 2 of segment 0 score equally
    cu = np.array([0, 300])
    topk = 2
    sel = oracle.vsa_select(q, k, cu, topk)
    nb = 5
    bounds = [(64 * j, min(300, 64 * j + 64)) for j in range(nb)]
    for h in range(2):
        qm = [[sum(q[r, h, d] for r in range(a, b)) / (b - a) for d in range(4)] for a, b in bounds]
        km = [[sum(k[r, h, d] for r in range(a, b)) / (b - a) for d in range(4)] for a, b in bounds]
        for bq in range(nb):
            sc = [sum(qm[bq][d] * km[c][d] for d in range(4)) / 2.0 for c in range(nb)]
            ranked = sorted(range(nb), key=lambda c: (-sc[c], c))
            assert sel[h, bq].tolist() == sorted(ranked[:topk])
    # the tie: whenever block 2 is kept and block 0 is not, block 0 must have lost on score
    S = oracle.vsa_scores(q, k, cu)[0]
    assert np.array_equal(S[:, :, 0], S[:, :, 2])
    for h in range(2):
        for bq in range(nb):
            s = sel[h, bq].tolist()
            assert not (2 in s and 0 not in s)


def test_vsa_keep_every_block_is_dense_attention():
    q, k, v = _rand_qkv(333, 3, 8, 3)
    cu = np.array([0, 50, 50, 333])
    sel = oracle.vsa_select(q, k, cu, topk=16)
    assert (sel[:, 0, 0] == 0).all() and (sel[:, 0, 1:] == -1).all()   # segment 0: one block
    assert (sel[:, 1:, 5:] == -1).all() and (sel[:, 1:, :5] >= 1).all()  # segment 2: five blocks
    got = oracle.vsa_attention(q, k, v, cu, sel)
    assert np.allclose(got, oracle.attention(q, k, v, cu), atol=1e-13, rtol=0)


def test_vsa_attention_matches_masked_sdpa():
    q, k, v = _rand_qkv(260, 2, 16, 4)
    cu = np.array([0, 260])
    rng = np.random.default_rng(5)
    sel = np.full((2, 5, 3), -1, np.int32)
    for h in range(2):
        for b in range(5):
            n = rng.integers(1, 4)
            sel[h, b, :n] = np.sort(rng.choice(5, size=n, replace=False))
    got = oracle.vsa_attention(q, k, v, cu, sel)
    bstart = [0, 64, 128, 192, 256, 260]
    for h in range(2):
        mask = torch.zeros((260, 260), dtype=torch.bool)
        for b in range(5):
            for c in sel[h, b]:
                if c >= 0:
                    mask[bstart[b]:bstart[b + 1], bstart[c]:bstart[c + 1]] = True
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[:, h])[None], torch.from_numpy(k[:, h])[None], torch.from_numpy(v[:, h])[None],
            attn_mask=mask[None])
        assert np.allclose(got[:, h], ref[0].numpy(), atol=1e-12, rtol=0)


def test_vsa_attention_blocks_is_the_restriction():
    q, k, v = _rand_qkv(333, 4, 8, 9)
    cu = np.array([0, 50, 50, 333])
    sel = oracle.vsa_select(q, k, cu, topk=3)
    full = oracle.vsa_attention(q, k, v, cu, sel)
    bstart, _, _ = oracle.block_layout(cu)
    heads = [3, 1]
    blocks = [0, 2, 5]                                  # a one-block segment, a full block, the short last one
    got = oracle.vsa_attention_blocks(q, k, v, cu, sel[heads], blocks, heads)
    for b, ob in zip(blocks, got):
        assert np.array_equal(ob, full[bstart[b]:bstart[b + 1]][:, heads])


def test_vsa_key_permutation_inside_a_kept_block():
    q, k, v = _rand_qkv(256, 2, 8, 6)
    cu = np.array([0, 256])
    sel = oracle.vsa_select(q, k, cu, topk=2)
    o = oracle.vsa_attention(q, k, v, cu, sel)
    perm = np.arange(256)
    perm[64:128] = 64 + np.random.default_rng(7).permutation(64)
    o2 = oracle.vsa_attention(q, k[perm], v[perm], cu, sel)     # block means and key sets unchanged
    assert np.array_equal(oracle.vsa_select(q, k[perm], cu, topk=2), sel)
    assert np.allclose(o, o2, atol=1e-13, rtol=0)


# ---------------------------------------------------------------------------
# FP8 Q.K attention: E4M3 values, rounding, MX block exponents, quantization,
# and the attention on dequantized operands
# ---------------------------------------------------------------------------
def test_e4m3_values_from_the_format_definition():
    # OCP 8-bit floating point E4M3: bias 7, max normal S.1111.110 = 448,
    # min normal 2^-6, min subnormal 2^-9, S.1111.111 = NaN, no infinities
    assert oracle.e4m3_value(0x7E) == 448.0 and oracle.e4m3_value(0xFE) == -448.0
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x38) == 1.0 and oracle.e4m3_value(0x40) == 2.0
    assert oracle.e4m3_value(0x3C) == 1.5 and oracle.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))
    assert oracle.e4m3_value(0x80) == 0.0 and math.copysign(1.0, oracle.e4m3_value(0x80)) < 0
    pos = [oracle.e4m3_value(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:]))            # codes 0x00..0x7E increase
    assert all(oracle.e4m3_value(c | 0x80) == -oracle.e4m3_value(c) for c in range(0x7F))
    # spacing: 8 values per binade, ulp 2^(e-3); subnormals spaced 2^-9
    for e in range(-6, 9):
        grid = [v for v in pos if 2.0 ** e <= v < 2.0 ** (e + 1)]
        assert len(grid) == (8 if e < 8 else 7) and np.allclose(np.diff(grid), 2.0 ** (e - 3))


def test_e4m3_round_nearest_ties_to_even():
    for c in range(256):
        if c not in (0x7F, 0xFF):
            assert oracle.e4m3_round(oracle.e4m3_value(c)) == c   # every finite code round-trips
    # midpoints go to the even mantissa: 1.0625 between 1.0 (m=0) and 1.125 (m=1);
    # 1.1875 between 1.125 (m=1) and 1.25 (m=2); 432 between 416 (m=5) and 448 (m=6);
    # 2^-10 between 0 and the smallest subnormal
    assert oracle.e4m3_round(1.0625) == 0x38
    assert oracle.e4m3_round(1.1875) == 0x3A
    assert oracle.e4m3_round(432.0) == 0x7E and oracle.e4m3_round(-432.0) == 0xFE
    assert oracle.e4m3_round(2.0 ** -10) == 0x00 and oracle.e4m3_round(-(2.0 ** -10)) == 0x80
    assert oracle.e4m3_round(1.0625 + 1e-9) == 0x39 and oracle.e4m3_round(1.0625 - 1e-9) == 0x38
    # nearest value against a sorted table searched independently
    table = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    rng = np.random.default_rng(3)
    for x in np.concatenate([rng.uniform(-448, 448, 300), rng.standard_normal(300) * 0.01]):
        got = oracle.e4m3_value(oracle.e4m3_round(x))
        j = np.searchsorted(table, abs(x))
        cand = table[max(j - 1, 0):j + 1]
        assert abs(abs(got) - abs(x)) == np.abs(cand - abs(x)).min()
        assert math.copysign(1.0, got) == math.copysign(1.0, x)
    with pytest.raises(ValueError):
        oracle.e4m3_round(449.0)


def test_mx_exponent_closed_form():
    # the smallest e with amax <= 448 * 2^e: then amax * 2^-e lies in (224, 448]
    assert oracle.mx_exponent(448.0) == 0 and oracle.mx_exponent(448.0001) == 1
    assert oracle.mx_exponent(224.0) == -1 and oracle.mx_exponent(224.0001) == 0
    assert oracle.mx_exponent(1.0) == -8 and oracle.mx_exponent(0.0) == -127
    rng = np.random.default_rng(4)
    for amax in np.exp(rng.uniform(-60, 60, 500)):
        e = oracle.mx_exponent(float(amax))
        assert 224.0 < amax * 2.0 ** -e <= 448.0


def test_mx_quantization_error_bound_and_exact_grid():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((5, 3, 128)) * np.exp(rng.uniform(-8, 8, (5, 3, 1)))).astype(np.float32)
    x[0, 0, :32] = 0.0                                   # an all-zero block
    codes, exps = oracle.quantize_mx_e4m3(x)
    assert codes.shape == x.shape and exps.shape == (5, 3, 4)
    assert (exps[0, 0, 0] == -127) and (codes[0, 0, :32] & 0x7F == 0).all()
    deq = oracle.dequantize_mx_e4m3(codes, exps)
    scale = np.repeat(np.ldexp(1.0, exps.astype(np.int64)), 32, axis=-1)
    xs = np.abs(x.astype(np.float64)) / scale             # the block-scaled magnitudes, <= 448
    assert xs.max() <= 448.0
    err = np.abs(deq - x)
    normal = xs >= 2.0 ** -6
    # half an ulp: 3 mantissa bits give 2^-4 relative for normals, 2^-10 * scale below
    assert (err[normal] <= 2.0 ** -4 * np.abs(x[normal]) + 0.0).all()
    assert (err[~normal] <= 2.0 ** -10 * scale[~normal]).all()
    # values already on a block's grid come back unchanged
    g = rng.choice([c for c in range(0x7F) if oracle.e4m3_value(c) <= 256.0], size=(2, 2, 128))
    y = np.array([[[oracle.e4m3_value(c) for c in r] for r in m] for m in g]) * 2.0 ** -8
    y[..., ::32] = 1.0                                    # amax 1.0 in every block: exponent -8
    yc, ye = oracle.quantize_mx_e4m3(y)
    assert (ye == -8).all() and np.array_equal(oracle.dequantize_mx_e4m3(yc, ye), y)


def test_fp8qk_attention_reduces_to_plain_attention_on_grid_values():
    # softmax_scale = 1 / log2(e) makes the Q factor scale * log2 e exactly 1 in
    # float32; with Q and K on an MX grid the quantization is exact, and base-2
    # exponentials of the logits are the natural softmax at scale ln 2
    rng = np.random.default_rng(9)
    cands = [c for c in range(0x7F) if oracle.e4m3_value(c) <= 256.0]
    def grid(rows):
        g = rng.choice(cands, size=(rows, 2, 64)) | (rng.integers(0, 2, (rows, 2, 64)) << 7)
        y = np.vectorize(oracle.e4m3_value)(g) * 2.0 ** -8
        y[..., ::32] = 1.0
        return y
    rows = 150
    q, k = grid(rows), grid(rows)
    v = rng.standard_normal((rows, 2, 64))
    cu = np.array([0, 37, 37, 150])
    s = 1.0 / 1.4426950408889634
    assert np.float32(s * 1.4426950408889634) == np.float32(1.0)
    got = oracle.attention_fp8qk(q, k, v, cu, softmax_scale=s)
    want = oracle.attention(q, k, v, cu, softmax_scale=math.log(2.0))
    assert np.allclose(got, want, atol=1e-12, rtol=0)


def test_fp8qk_attention_error_against_exact_attention():
    # E4M3's 3 mantissa bits bound the logit error; on this workload's
    # N(0, 0.25) rows the output stays within a few percent of exact attention
    rng = np.random.default_rng(10)
    q, k, v = (rng.standard_normal((300, 2, 128)) * 0.5 for _ in range(3))
    cu = np.array([0, 300])
    got = oracle.attention_fp8qk(q.astype(np.float32), k.astype(np.float32), v, cu)
    want = oracle.attention(q.astype(np.float32).astype(np.float64), k.astype(np.float32).astype(np.float64), v, cu)
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert 1e-4 < rel < 5e-2


def test_attention_base2_rows_is_the_restriction():
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((200, 3, 16)) for _ in range(3))
    cu = np.array([0, 70, 70, 200])
    full = oracle.attention_base2(q, k, v, cu)
    rows = [0, 5, 69, 70, 150, 199]
    assert np.allclose(oracle.attention_base2_rows(q, k, v, cu, rows, heads=[2, 0]), full[rows][:, [2, 0]],
                       atol=1e-14, rtol=0)
    # base-2 logits are natural logits times ln 2
    assert np.allclose(full, oracle.attention(q, k, v, cu, softmax_scale=math.log(2.0)), atol=1e-12, rtol=0)
