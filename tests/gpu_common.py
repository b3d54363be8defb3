"""Shared helpers of the GPU tests: run the HIP path on a workload and compare
against the oracle at the stated tolerances."""
import numpy as np
import torch

import packed_varlen_attention_amd as h3
import workloads as W

# Tolerances of the path: integers bit-exact; fp32 max-abs 1e-5; bf16 max-abs
# 2e-2 and relative RMS 5e-3 (both must hold).
F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_REL_RMS = 5e-3


def errors(gpu, ref):
    g = gpu.detach().to("cpu", torch.float64).numpy() if torch.is_tensor(gpu) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    d = np.abs(g - r)
    max_abs = float(d.max()) if d.size else 0.0
    den = float(np.sqrt((r * r).sum()))
    rel_rms = float(np.sqrt((d * d).sum()) / den) if den > 0 else 0.0
    return max_abs, rel_rms


def assert_close(gpu, ref, dtype: str, what: str):
    max_abs, rel_rms = errors(gpu, ref)
    assert np.all(np.isfinite(gpu.detach().float().cpu().numpy())), what + ": non-finite values"
    if dtype == "f32":
        assert max_abs <= F32_MAX_ABS, "%s: max-abs %.3e > %.0e" % (what, max_abs, F32_MAX_ABS)
    else:
        assert max_abs <= BF16_MAX_ABS and rel_rms <= BF16_REL_RMS, \
            "%s: max-abs %.3e (<= %.0e), rel-RMS %.3e (<= %.0e)" % (what, max_abs, BF16_MAX_ABS, rel_rms,
                                                                   BF16_REL_RMS)
    return max_abs, rel_rms


def device_inputs(wl, q, k, v, dev="cuda"):
    return dict(q=q.to(dev), k=k.to(dev), v=v.to(dev),
                tags=torch.from_numpy(wl.tags).to(dev),
                pos=torch.from_numpy(wl.pos).to(dev),
                seg=torch.from_numpy(wl.seg).to(dev))


def run_path(wl, d, pad_value=float("nan")):
    """pack -> attention -> unpack on device inputs `d`; packed buffers have the
    workload's capacity and their pad rows are pre-filled with `pad_value`."""
    dt = d["q"].dtype
    cap, H, D = wl.capacity, wl.H, wl.D
    mk = lambda: torch.full((cap, H, D), pad_value, dtype=dt, device="cuda")
    qo, ko, vo = mk(), mk(), mk()
    qp, kp, vp, cu, perm = h3.pack_rope(d["q"], d["k"], d["v"], d["tags"], d["pos"], d["seg"], wl.n_seg,
                                        wl.rope, wl.time_offset, capacity=cap, q_out=qo, k_out=ko, v_out=vo)
    o = mk()
    max_len = int(wl.segment_lengths().max()) if wl.n_seg else 0
    h3.varlen_attn_fwd(qp, kp, vp, cu, total_rows=wl.n, max_seqlen=max_len, o=o)
    outs, idxs = h3.unpack_by_modality(o, perm, d["tags"], wl.n_per_modality())
    torch.cuda.synchronize()
    return dict(q=qp, k=kp, v=vp, cu=cu, perm=perm, o=o, outs=outs, idxs=idxs)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def sample_rows(cu, n_random=32, seed=0, edges=2):
    """Packed rows to check at full size: the first and last `edges` rows of
    every segment plus seeded random rows."""
    cu = np.asarray(cu, np.int64)
    rows = set()
    for a, b in zip(cu[:-1], cu[1:]):
        for r in list(range(a, min(b, a + edges))) + list(range(max(a, b - edges), b)):
            rows.add(int(r))
    rng = np.random.default_rng(seed)
    if cu[-1] > 0:
        rows.update(int(x) for x in rng.integers(0, cu[-1], size=n_random))
    return np.array(sorted(rows), np.int64)
