"""GPU parity of VSA-style block-sparse attention (h3_vsa_select and
h3_vsa_attn_fwd through the C ABI) against the CPU oracle.

The selection is an integer result decided by floating-point scores: block
means are compared at fp32 tolerance, the GPU's selection must be a valid
top-k of the oracle's fp64 scores (every kept block scores at least as high
as every dropped one, up to a rounding margin far below the score spread) and
equal to the oracle's selection wherever the k-th and (k+1)-th scores are
separated by more than that margin; exact ties are broken by lower block
number on both sides.  Attention is checked stage-wise (the oracle's sparse
attention on the GPU's own selection) at the bf16 tolerances."""
import numpy as np
import pytest
import torch

import oracle
from oracle.cache import cached
import packed_varlen_attention_amd as h3
import workloads as W
from gpu_common import F32_MAX_ABS, assert_close, errors, f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

MARGIN = 1e-6      # fp32 rounding of a 128-term dot product of block means, with room


def _packed(lengths, H, seed, dup=None):
    """Packed bf16 Q, K, V [rows, H, 128] for segments of `lengths` (RoPE
    plays no part in the block-sparse path, so the rows are drawn packed)."""
    rows = int(sum(lengths))
    cap = max(64, (rows + 63) // 64 * 64)
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    t = [(torch.randn((cap, H, 128), generator=g) * 0.5).to(torch.bfloat16) for _ in range(3)]
    if dup is not None:                      # copy key block dup[0] over dup[1] (exact score ties)
        a, b = dup
        t[1][b * 64:(b + 1) * 64] = t[1][a * 64:(a + 1) * 64]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return t, cu, rows


def _check_selection(sel_gpu, q, k, cu, topk):
    sel_o = oracle.vsa_select(q, k, cu, topk)
    scores = oracle.vsa_scores(q, k, cu)
    _, _, bcu = oracle.block_layout(cu)
    H = q.shape[1]
    n_exact = 0
    for s, S in enumerate(scores):
        a = int(bcu[s])
        n_s = S.shape[1]
        for h in range(H):
            for bl in range(n_s):
                got = sel_gpu[h, a + bl]
                kept = [int(c) for c in got if c >= 0]
                assert kept == sorted(set(kept)) and len(kept) == min(topk, n_s)
                assert all(a <= c < a + n_s for c in kept)
                assert (got[len(kept):] == -1).all()
                row = S[h, bl]
                loc = [c - a for c in kept]
                drop = [c for c in range(n_s) if c not in loc]
                if drop:
                    assert row[loc].min() >= row[drop].max() - MARGIN
                srt = np.sort(row)[::-1]
                if n_s <= topk or srt[topk - 1] - srt[topk] > MARGIN:
                    assert got.tolist() == sel_o[h, a + bl].tolist()
                    n_exact += 1
    return n_exact


@pytest.mark.parametrize("topk", [1, 3, 8])
def test_vsa_ragged_segments_means_selection_attention(topk):
    lengths = [1, 63, 64, 65, 0, 200, 129, 700]
    H = 3
    (q, k, v), cu, rows = _packed(lengths, H, seed=11)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    dcu = torch.from_numpy(cu).cuda()
    sel, qm, km = h3.vsa_select(dq, dk, dcu, rows, topk, max_seqlen=max(lengths), means=True)
    o = torch.full_like(dq, float("nan"))
    h3.vsa_attn_fwd(dq, dk, dv, dcu, rows, sel, topk, o=o)
    torch.cuda.synchronize()
    q64, k64, v64 = W.to_f64(q[:rows]), W.to_f64(k[:rows]), W.to_f64(v[:rows])
    nb = oracle.block_layout(cu)[2][-1]
    for got, x in ((qm, q64), (km, k64)):
        max_abs, _ = errors(got[:nb], oracle.block_means(x, cu))
        assert max_abs <= F32_MAX_ABS
    sel_np = sel[:, :nb].cpu().numpy()
    n_exact = _check_selection(sel_np, q64, k64, cu, topk)
    assert n_exact > 0
    ref = oracle.vsa_attention(q64, k64, v64, cu, sel_np)
    assert_close(o[:rows], ref, "bf16", "VSA O stage-wise")
    assert torch.isnan(o[rows:].float()).all()          # rows past total_rows untouched


@pytest.mark.parametrize("topk", [3, 40])
def test_vsa_grouped_and_per_block_selection_agree(topk):
    # Up to 1,280 key blocks per segment the scores of 8 query blocks are
    # formed together (key means read once per group); longer segments take
    # one workgroup per query block.  max_seqlen is only an upper bound, so a
    # larger one selects the per-block kernel on the same inputs: both must
    # give the same selection bit for bit (same fmaf order per score), and it
    # must pass the oracle check.  Segment lengths cover partial groups
    # (1..7 blocks), exact groups (8, 16) and a long one (18 blocks = 8+8+2).
    lengths = [1, 63, 64 * 8, 65, 0, 200, 64 * 16, 129, 64 * 17 + 5, 700]
    H = 3
    (q, k, v), cu, rows = _packed(lengths, H, seed=14, dup=(3, 5))
    dq, dk = q.cuda(), k.cuda()
    dcu = torch.from_numpy(cu).cuda()
    grouped = h3.vsa_select(dq, dk, dcu, rows, topk, max_seqlen=max(lengths))
    per_block = h3.vsa_select(dq, dk, dcu, rows, topk, max_seqlen=64 * 1281)
    torch.cuda.synchronize()
    assert torch.equal(grouped, per_block)
    nb = oracle.block_layout(cu)[2][-1]
    assert _check_selection(grouped[:, :nb].cpu().numpy(), W.to_f64(q[:rows]), W.to_f64(k[:rows]), cu, topk) > 0


def test_vsa_exact_ties_break_to_lower_block():
    (q, k, v), cu, rows = _packed([64 * 6], 2, seed=12, dup=(1, 4))
    dcu = torch.from_numpy(cu).cuda()
    sel = h3.vsa_select(q.cuda(), k.cuda(), dcu, rows, 2, max_seqlen=rows)
    torch.cuda.synchronize()
    got = sel[:, :6].cpu().numpy()
    want = oracle.vsa_select(W.to_f64(q[:rows]), W.to_f64(k[:rows]), cu, 2)
    assert np.array_equal(got, want)
    for h in range(2):
        for b in range(6):
            assert not (4 in got[h, b] and 1 not in got[h, b])


def test_vsa_keep_every_block_equals_dense_attention():
    lengths = [300, 64, 5]
    (q, k, v), cu, rows = _packed(lengths, 2, seed=13)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    dcu = torch.from_numpy(cu).cuda()
    sel = h3.vsa_select(dq, dk, dcu, rows, 16, max_seqlen=300)
    o = h3.vsa_attn_fwd(dq, dk, dv, dcu, rows, sel, 16)
    torch.cuda.synchronize()
    ref = oracle.attention(W.to_f64(q[:rows]), W.to_f64(k[:rows]), W.to_f64(v[:rows]), cu)
    assert_close(o[:rows], ref, "bf16", "VSA keep-all vs dense oracle")


def test_vsa_full_size_cube_grid_sampled():
    # the measured configuration: 59,904 cube-ordered video tokens, 40 heads,
    # 936 blocks, top-117 (one block in eight); sampled query blocks of three
    # heads against the oracle's scores and its block-restricted attention
    wl = W.make_vsa_workload()
    q, k, v = W.make_qkv_on_device(wl, "cuda", seed=5)
    cu = torch.tensor([0, wl.n], dtype=torch.int32, device="cuda")
    topk = 117
    sel = h3.vsa_select(q, k, cu, wl.n, topk, max_seqlen=wl.n)
    o = h3.vsa_attn_fwd(q, k, v, cu, wl.n, sel, topk)
    torch.cuda.synchronize()
    heads = [0, 21, 39]
    qs, ks, vs = f64(q[:, heads]), f64(k[:, heads]), f64(v[:, heads])
    sel_np = sel[heads].cpu().numpy()
    cu_np = np.array([0, wl.n])
    scores = oracle.vsa_scores(qs, ks, cu_np)[0]             # [3 heads, 936, 936]
    rng = np.random.default_rng(1)
    blocks = np.unique(np.concatenate([[0, 935], rng.integers(0, 936, 10)]))
    for hi in range(3):
        for b in blocks:
            row = scores[hi, b]
            kept = sel_np[hi, b]
            assert len(set(kept.tolist())) == topk and (kept >= 0).all()
            drop = np.setdiff1d(np.arange(936), kept)
            assert row[kept].min() >= row[drop].max() - MARGIN
    ref = cached(oracle.vsa_attention_blocks, qs, ks, vs, cu_np, sel_np, blocks, heads=[0, 1, 2])
    for b, rb in zip(blocks, ref):
        assert_close(o[64 * b:64 * b + 64, heads], rb, "bf16", "VSA O full size, block %d" % b)


def test_vsa_selection_does_not_depend_on_the_hint():
    """max_seqlen only sizes the scores' on-chip buffer: with a hint below a
    segment's length that segment is scored on demand, which must give the
    same selection bit for bit, in the grouped kernel (hints up to 1,280
    blocks) and in the per-block kernel (longer hints; a first segment of
    1,301 blocks needs one); and it must pass the oracle check."""
    lengths = [64 * 1300 + 17, 64 * 40, 5]
    H, topk = 1, 9
    (q, k, v), cu, rows = _packed(lengths, H, seed=15)
    dq, dk = q.cuda(), k.cuda()
    dcu = torch.from_numpy(cu).cuda()
    hints = {"exact": max(lengths), "unknown": 0, "grouped_below": 64 * 1280, "tiny": 1,
             "per_block_below": 64 * 1290}
    sels = {name: h3.vsa_select(dq, dk, dcu, rows, topk, max_seqlen=hint) for name, hint in hints.items()}
    torch.cuda.synchronize()
    for name, s in sels.items():
        assert torch.equal(s, sels["exact"]), name
    nb = oracle.block_layout(cu)[2][-1]
    assert _check_selection(sels["exact"][:, :nb].cpu().numpy(), W.to_f64(q[:rows]), W.to_f64(k[:rows]), cu,
                            topk) > 0


@pytest.mark.parametrize("rate", [0.3, 0.04])
def test_vsa_online_softmax_rescale_under_rotated_walks(rate):
    """Logits that climb along each segment by `rate` (log2 units) per key, so
    the running max moves and the accumulators are rescaled every one (rate
    0.3) or every few (0.04) 32-key halves.  24 heads x 43 blocks put about
    129 items on each XCD, so the walks start at positions spread over the
    whole segment and wrap around to lower blocks (whose logits then lie far
    below the reference).  Both the gate's top-k and caller lists of every
    block are checked against the oracle."""
    lengths = [64 * 20, 64 * 12 + 20, 64 * 9 + 3]
    H = 24
    (q, k, v), cu, rows = _packed(lengths, H, seed=41)
    amp = 4.0
    qf, kf = q.float() * 0.1, k.float() * 0.1
    qf[:, :, 0] += amp
    ramp = rate / (128 ** -0.5 * np.log2(np.e) * amp)        # k[:, :, 0] step per key
    for a, b in zip(cu[:-1], cu[1:]):
        kf[a:b, :, 0] += (torch.arange(b - a, dtype=torch.float32) * ramp)[:, None]
    q, k = qf.to(torch.bfloat16), kf.to(torch.bfloat16)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    dcu = torch.from_numpy(cu).cuda()
    _, bseg, bcu = oracle.block_layout(cu)
    nb = int(bcu[-1])
    nb_cap = h3.vsa_blocks_bound(rows, len(lengths))
    every = np.full((H, nb_cap, 20), -1, np.int32)
    for b in range(nb):
        s = int(bseg[b])
        own = np.arange(bcu[s], bcu[s + 1])
        every[:, b, :len(own)] = own
    q64, k64, v64 = W.to_f64(q[:rows]), W.to_f64(k[:rows]), W.to_f64(v[:rows])
    sel = h3.vsa_select(dq, dk, dcu, rows, 8, max_seqlen=max(lengths))
    for lists, topk in ((torch.from_numpy(every).cuda(), 20), (sel, 8)):
        o = torch.full_like(dq, float("nan"))
        h3.vsa_attn_fwd(dq, dk, dv, dcu, rows, lists, topk, o=o)
        torch.cuda.synchronize()
        ref = oracle.vsa_attention(q64, k64, v64, cu, lists[:, :nb].cpu().numpy())
        assert_close(o[:rows], ref, "bf16", "VSA rescale rate %g, top-%d" % (rate, topk))


def test_vsa_attention_on_caller_lists():
    """h3_vsa_attn_fwd on selection lists the caller made: any order, repeated
    blocks (attended once per listing, as the oracle's key concatenation does),
    blocks of other segments (ignored), and a negative entry that ends the list
    before later entries.  Each workgroup starts its walk of the list at a
    position tied to its index, so these lists also check that every entry is
    visited exactly once whatever the start.  The expected output is the
    oracle's attention on the lists reduced by the documented rules."""
    lengths = [300, 64, 5, 700, 130]
    H, topk = 3, 7
    (q, k, v), cu, rows = _packed(lengths, H, seed=31)
    _, bseg, bcu = oracle.block_layout(cu)
    nb = int(bcu[-1])
    nb_cap = h3.vsa_blocks_bound(rows, len(lengths))
    rng = np.random.default_rng(5)
    sel = np.full((H, nb_cap, topk), -1, np.int32)
    ref_sel = np.full((H, nb, 2 * topk), -1, np.int32)
    for h in range(H):
        for b in range(nb):
            s = int(bseg[b])
            own = np.arange(bcu[s], bcu[s + 1])
            others = np.setdiff1d(np.arange(nb), own)
            lst = list(rng.permutation(own)[:rng.integers(1, min(len(own), topk) + 1)])
            if rng.random() < 0.3:                     # a repeated block
                lst.append(lst[0])
            if len(others) and rng.random() < 0.5:     # a block of another segment
                lst.insert(int(rng.integers(0, len(lst) + 1)), int(rng.choice(others)))
            lst = lst[:topk]
            if len(lst) < topk - 1 and rng.random() < 0.5:   # -1, then an entry that must be ignored
                lst += [-1, int(own[0])]
            sel[h, b, :len(lst)] = lst
            kept = []
            for c in lst:
                if c < 0:
                    break
                if bcu[s] <= c < bcu[s + 1]:
                    kept.append(c)
            assert kept                                 # every list starts with a block of its own segment
            ref_sel[h, b, :len(kept)] = kept
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    o = torch.full_like(dq, float("nan"))
    h3.vsa_attn_fwd(dq, dk, dv, torch.from_numpy(cu).cuda(), rows, torch.from_numpy(sel).cuda(), topk, o=o)
    torch.cuda.synchronize()
    ref = oracle.vsa_attention(W.to_f64(q[:rows]), W.to_f64(k[:rows]), W.to_f64(v[:rows]), cu, ref_sel)
    assert_close(o[:rows], ref, "bf16", "VSA attention on caller-made lists")


def test_vsa_attention_out_of_segment_runs_and_keyless_blocks():
    """Runs of one to three blocks of other segments anywhere in a caller's
    list (before, between and after its own blocks, so before and after the
    first own block of any rotated walk), and lists that keep no block of
    their own segment.  Kept keys: the oracle on the reduced lists; a query
    block with no kept key has no softmax, and its rows of o keep the value
    they had (documented: not written)."""
    lengths = [200, 64, 450, 70]
    H, topk = 2, 9
    (q, k, v), cu, rows = _packed(lengths, H, seed=47)
    _, bseg, bcu = oracle.block_layout(cu)
    nb = int(bcu[-1])
    nb_cap = h3.vsa_blocks_bound(rows, len(lengths))
    rng = np.random.default_rng(11)
    sel = np.full((H, nb_cap, topk), -1, np.int32)
    ref_sel = np.full((H, nb, topk), -1, np.int32)
    keyless = np.zeros((H, nb), bool)
    for h in range(H):
        for b in range(nb):
            s = int(bseg[b])
            own = np.arange(bcu[s], bcu[s + 1])
            others = np.setdiff1d(np.arange(nb), own)
            if rng.random() < 0.2:                       # no block of its own segment
                lst = [int(c) for c in rng.choice(others, size=int(rng.integers(1, 4)))]
            else:
                mine = [int(c) for c in rng.permutation(own)[:int(rng.integers(1, min(len(own), 3) + 1))]]
                lst = []
                for c in mine:                           # a run of foreign blocks before each own block
                    lst += [int(x) for x in rng.choice(others, size=int(rng.integers(0, 3)))]
                    lst.append(c)
                lst += [int(x) for x in rng.choice(others, size=int(rng.integers(0, 4)))]
            lst = lst[:topk]
            sel[h, b, :len(lst)] = lst
            kept = [c for c in lst if bcu[s] <= c < bcu[s + 1]]
            if kept:
                ref_sel[h, b, :len(kept)] = kept
            else:
                keyless[h, b] = True
                ref_sel[h, b, 0] = int(own[0])           # any block: these rows are not compared
    assert keyless.any() and (~keyless).any()
    sentinel = 3.0
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    o = torch.full_like(dq, sentinel)
    h3.vsa_attn_fwd(dq, dk, dv, torch.from_numpy(cu).cuda(), rows, torch.from_numpy(sel).cuda(), topk, o=o)
    torch.cuda.synchronize()
    got = o[:rows].float().cpu().numpy()
    ref = oracle.vsa_attention(W.to_f64(q[:rows]), W.to_f64(k[:rows]), W.to_f64(v[:rows]), cu, ref_sel)
    bstart, _, _ = oracle.block_layout(cu)
    row_mask = np.zeros((rows, H), bool)                 # (row, head) pairs with kept keys
    for h in range(H):
        for b in range(nb):
            r0, r1 = int(bstart[b]), int(bstart[b + 1])
            if keyless[h, b]:
                assert (got[r0:r1, h, :] == sentinel).all(), "keyless query block %d head %d was written" % (b, h)
            else:
                row_mask[r0:r1, h] = True
    assert_close(torch.from_numpy(got[row_mask]), ref[row_mask], "bf16",
                 "VSA attention with out-of-segment runs")
