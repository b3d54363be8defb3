"""GPU test of h3_varlen_attn_fwd_noalloc, the attention entry point that
allocates nothing (its scratch is a fixed buffer the library holds per GPU).

Its output must equal h3_varlen_attn_fwd's bit for bit (same kernels, same
tile list), on consecutive calls that reuse the one buffer, the second with a
smaller problem, on each of the kernel routes (long segments, short segments
by the max_seqlen hint, the fp32 path), and rows past total_rows must stay
untouched."""
import numpy as np
import pytest
import torch

import packed_varlen_attention_amd as h3

pytestmark = pytest.mark.gpu


def _case(lengths, H, D, dtype, seed, pad=3):
    """Random packed Q/K/V for the given segment lengths, `pad` NaN rows past
    the last segment."""
    g = torch.Generator("cpu").manual_seed(seed)
    total = int(sum(lengths))
    rows = total + pad
    mk = lambda: (torch.randn((rows, H, D), generator=g) * 0.5).to(dtype)
    q, k, v = mk(), mk(), mk()
    for t in (q, k, v):
        t[total:] = float("nan")
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))
    return q.cuda(), k.cuda(), v.cuda(), cu.cuda(), total, int(max(lengths))


def _both(case, hint):
    q, k, v, cu, total, longest = case
    max_seqlen = longest if hint else 0
    o_ws = torch.full_like(q, 7.0)
    o_na = torch.full_like(q, 7.0)
    h3.varlen_attn_fwd(q, k, v, cu, total_rows=total, max_seqlen=max_seqlen, o=o_ws)
    h3.varlen_attn_fwd_noalloc(q, k, v, cu, total_rows=total, max_seqlen=max_seqlen, o=o_na)
    torch.cuda.synchronize()
    return o_ws, o_na, total


@pytest.mark.parametrize("route", ["long", "short", "f32"])
def test_noalloc_matches_workspace_call_on_two_calls(route):
    if route == "long":
        big = _case([300, 0, 1000, 64, 5, 257], H=4, D=128, dtype=torch.bfloat16, seed=11)
        small = _case([129, 40], H=2, D=128, dtype=torch.bfloat16, seed=12)
    elif route == "short":
        big = _case([256, 37, 0, 128, 255, 1, 512] * 3, H=3, D=128, dtype=torch.bfloat16, seed=13)
        small = _case([64, 31], H=2, D=128, dtype=torch.bfloat16, seed=14)
    else:
        big = _case([10, 20, 15, 70], H=2, D=64, dtype=torch.float32, seed=15)
        small = _case([9], H=1, D=64, dtype=torch.float32, seed=16)
    for case in (big, small):                       # the second call is smaller
        o_ws, o_na, total = _both(case, hint=(route == "short"))
        assert torch.equal(o_na[:total], o_ws[:total]), route
        assert torch.isfinite(o_na[:total].float()).all()
        assert (o_na[total:] == 7.0).all()           # rows past total_rows untouched


def test_noalloc_after_many_segments_then_few():
    """A call with many segments fills much of the scratch; a following call
    with fewer segments must not see the stale tile counts."""
    many = _case([1, 2, 3, 65] * 500, H=2, D=128, dtype=torch.bfloat16, seed=17)
    few = _case([70, 3], H=2, D=128, dtype=torch.bfloat16, seed=18)
    for case in (many, few):
        o_ws, o_na, total = _both(case, hint=False)
        assert torch.equal(o_na[:total], o_ws[:total])


def test_noalloc_rejects_too_many_segments():
    q, k, v, _, _, _ = _case([4], H=1, D=128, dtype=torch.bfloat16, seed=19)
    cu = torch.zeros(65473, dtype=torch.int32, device="cuda")        # 65,472 segments
    with pytest.raises(h3.H3Error) as e:
        h3.varlen_attn_fwd_noalloc(q, k, v, cu, total_rows=4)
    assert e.value.status == 10
