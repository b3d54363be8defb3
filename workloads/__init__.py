"""Seeded synthetic inputs for packed varlen modality-RoPE attention.

This module builds the *inputs* of the path only: per-token modality tags,
(t, h, w) positions, segment ids, the per-modality RoPE parameters and seeded
Q/K/V tensors.  It holds none of the method's arithmetic (no sort, no rotation,
no softmax); both the CPU oracle (``oracle/``) and the HIP path receive what it
builds, and neither imports the other.

The five workloads follow the packed-sequence description of the MiniMax-H3
write-up ("生产环境下的音视频联合生成：MiniMax-H3 与 vLLM-Omni 架构解析",
section 三, the cu_seqlens example and the 58,758-token sequence of section 一)
and the continuation / window-attention sections of "突破视频生成大模型的工程瓶颈"
(long-video continuation: five-group order and the time shift; window-aligned
SP: regular and half-shifted 3-D windows).  Shapes, head layouts and value
scales are the workload definitions this library is measured on; where those
are garbled the plainest reading is taken (see the module-level notes below).

Readings taken here (all are inputs, so both sides see the same ones):
  * text tokens: position (index, 0, 0); video tokens: (t, h, w) of a row-major
    latent grid, t slowest; audio tokens: (tick, 0, 0) at 40 Hz, converted to
    video-frame time by the audio RoPE time scale 24/40.
  * the 58,758-token workload's video rows are the first 58,295 rows of a
    24 x 48 x 51 row-major grid (the printed "24x48x50.6-equivalent ... padded
    to total" is not an integer grid).
  * continuation groups each start their local time at 0; the shift
    s = 238 frames is applied to video and audio time only.
  * shifted windows are edge-cropped, not cyclic: a half-window offset
    (2, 4, 4) leaves boundaries {0,2,6,10,14,16} x {0,4,12,...,60,64} x
    {0,4,12,...,108,112}; windows are numbered row-major, which is the
    segment id of every token inside.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

TEXT, VIDEO, AUDIO = 0, 1, 2
MODALITY_NAMES = ("text", "video", "audio")
BASE_SEED = 1101          # the seed of the request example on the deployment page
ALIGN = 64                # the page's aligned length 58,816 = 919 * 64


@dataclasses.dataclass(frozen=True)
class RopeModality:
    """RoPE parameters of one modality (inputs to both sides)."""
    base: float           # theta_j = coord * base ** (-2 j / d_axis)
    time_scale: float     # tau = t * time_scale (+ shift)
    shift_time: int       # 1: add the continuation shift s * 40 / 24 to tau
    d_t: int              # width of the time slice of the head dim
    d_h: int              # width of the height slice
    d_w: int              # width of the width slice


def default_rope(D: int, base: float = 10000.0) -> Tuple[RopeModality, RopeModality, RopeModality]:
    """Per-modality RoPE of the tiny fp32 workload, scaled to head dim D.

    Text: 1-D over all of D.  Video: 3-D, split D/4 : 3D/8 : 3D/8 over t:h:w
    (16/24/24 at D = 64, 32/48/48 at D = 128).  Audio: 1-D over all of D on
    40 Hz ticks, time scaled by 24/40 into video-frame units.  Video and audio
    take the continuation time shift; text does not.
    """
    assert D % 8 == 0
    text = RopeModality(base, 1.0, 0, D, 0, 0)
    video = RopeModality(base, 1.0, 1, D // 4, 3 * D // 8, 3 * D // 8)
    audio = RopeModality(base, 24.0 / 40.0, 1, D, 0, 0)
    return (text, video, audio)


@dataclasses.dataclass
class Workload:
    name: str
    index: int
    n: int
    n_seg: int
    H: int
    D: int
    dtype: str            # "f32" or "bf16"
    capacity: int
    time_offset: float    # s, in video frames
    q_scale: float        # Q/K/V ~ N(0,1) * q_scale
    tags: np.ndarray      # uint8 [n]
    pos: np.ndarray       # int32 [n, 3]
    seg: np.ndarray       # int32 [n]
    rope: Tuple[RopeModality, RopeModality, RopeModality]
    groups: List[Tuple[str, int, int]]   # (label, modality, count) in source order
    note: str = ""

    @property
    def seed(self) -> int:
        return BASE_SEED + self.index

    def n_per_modality(self) -> Tuple[int, int, int]:
        return tuple(int((self.tags == m).sum()) for m in (TEXT, VIDEO, AUDIO))

    def segment_lengths(self) -> np.ndarray:
        return np.bincount(self.seg, minlength=self.n_seg).astype(np.int64)

    def unmasked_flops(self) -> float:
        """4 * sum_k L_k^2 * D * H: QK^T and PV inside each segment only."""
        L = self.segment_lengths().astype(np.float64)
        return float(4.0 * (L * L).sum() * self.D * self.H)


class _Builder:
    def __init__(self):
        self.tags: List[np.ndarray] = []
        self.pos: List[np.ndarray] = []
        self.seg: List[np.ndarray] = []
        self.groups: List[Tuple[str, int, int]] = []

    def text(self, label: str, count: int, seg: int):
        p = np.zeros((count, 3), np.int32)
        p[:, 0] = np.arange(count)
        self._add(label, TEXT, p, seg)

    def audio(self, label: str, count: int, seg: int):
        p = np.zeros((count, 3), np.int32)
        p[:, 0] = np.arange(count)
        self._add(label, AUDIO, p, seg)

    def video(self, label: str, T: int, Hh: int, W: int, seg, keep: Optional[int] = None):
        t, h, w = np.meshgrid(np.arange(T), np.arange(Hh), np.arange(W), indexing="ij")
        p = np.stack([t.ravel(), h.ravel(), w.ravel()], axis=1).astype(np.int32)
        if keep is not None:
            p = p[:keep]
        self._add(label, VIDEO, p, seg)

    def _add(self, label, modality, p, seg):
        n = p.shape[0]
        self.tags.append(np.full(n, modality, np.uint8))
        self.pos.append(p)
        if np.isscalar(seg):
            self.seg.append(np.full(n, seg, np.int32))
        else:
            self.seg.append(np.asarray(seg, np.int32))
        self.groups.append((label, modality, n))

    def arrays(self):
        return (np.concatenate(self.tags), np.concatenate(self.pos, axis=0),
                np.concatenate(self.seg))


def _round_up(x: int, a: int) -> int:
    return (x + a - 1) // a * a


def window_boundaries(extent: int, window: int, offset: int) -> List[int]:
    """Edge-cropped window boundaries along one axis.

    offset 0 gives the regular partition; offset = window / 2 gives the
    half-shifted partition whose first and last windows are cropped.
    """
    b = [0]
    x = offset if offset > 0 else window
    while x < extent:
        b.append(x)
        x += window
    b.append(extent)
    return b


def window_segments(T: int, Hh: int, W: int, win: Sequence[int], shift: Sequence[int]) -> Tuple[np.ndarray, int]:
    """Segment id (row-major window index) of every token of a row-major grid."""
    ids = []
    for extent, w, s in zip((T, Hh, W), win, shift):
        bnd = np.asarray(window_boundaries(extent, w, s))
        ids.append((np.searchsorted(bnd, np.arange(extent), side="right") - 1, len(bnd) - 1))
    (it, nt), (ih, nh), (iw, nw) = ids
    seg = (it[:, None, None] * nh + ih[None, :, None]) * nw + iw[None, None, :]
    return seg.ravel().astype(np.int32), nt * nh * nw


def make_workload(index: int, *, shifted: bool = True) -> Workload:
    """The five workloads, by index 0..4."""
    b = _Builder()
    s = 0.0
    if index == 0:
        # cu_seqlens = [0, 10, 30, 45]: text 10, video 20, audio 15 (section 三 example).
        H, D, dtype, scale = 2, 64, "f32", 1.0
        b.text("text", 10, 0)
        b.video("video", 5, 2, 2, 1)
        b.audio("audio", 15, 2)
        n_seg, name, note = 3, "tiny_fp32_cu[0,10,30,45]", ""
    elif index == 1:
        H, D, dtype, scale = 24, 128, "bf16", 0.5
        b.text("text", 256, 0)
        b.audio("audio", 207, 1)
        b.video("video", 21, 16, 24, 2)
        n_seg, name, note = 3, "medium_8527tok_3seg", ""
    elif index == 2:
        H, D, dtype, scale = 40, 128, "bf16", 0.5
        b.text("text", 256, 0)
        b.audio("audio", 207, 1)
        b.video("video", 24, 48, 51, 1, keep=58758 - 256 - 207)
        n_seg, name = 2, "h3_step_58758tok"
        note = "video rows: first 58,295 of a 24x48x51 row-major grid"
    elif index == 3:
        H, D, dtype, scale = 40, 128, "bf16", 0.5
        s = 238.0
        b.text("text", 256, 0)
        b.audio("audio_ref", 56, 0)
        b.video("video_ref", 7, 48, 84, 0)
        b.audio("audio_tgt", 207, 0)
        b.video("video_tgt", 31, 48, 84, 0)
        n_seg, name, note = 1, "continuation_153735tok_s238", "five groups, one segment"
    elif index == 4:
        H, D, dtype, scale = 24, 128, "bf16", 0.5
        T, Hh, W = 16, 64, 112
        seg, n_seg = window_segments(T, Hh, W, (4, 8, 8), (2, 4, 4) if shifted else (0, 0, 0))
        b.video("video_grid", T, Hh, W, seg)
        name = "window_%s_114688tok" % ("shifted" if shifted else "regular")
        note = "windows 4x8x8" + (", half-shifted (2,4,4), edge-cropped" if shifted else "")
    else:
        raise ValueError("workload index must be 0..4")
    tags, pos, segv = b.arrays()
    n = tags.shape[0]
    return Workload(name=name, index=index, n=n, n_seg=n_seg, H=H, D=D, dtype=dtype,
                    capacity=_round_up(n, ALIGN), time_offset=s, q_scale=scale,
                    tags=tags, pos=pos, seg=segv, rope=default_rope(D), groups=b.groups,
                    note=note)


def make_custom(lengths: Sequence[int], H: int, D: int, dtype: str = "bf16",
                modalities: Optional[Sequence[int]] = None, time_offset: float = 0.0,
                q_scale: float = 0.5, index: int = 100, capacity: Optional[int] = None) -> Workload:
    """Small ragged workloads for parity tests: one group per segment.

    Segment k holds `lengths[k]` tokens of modality `modalities[k]` (cycling
    text, video, audio by default).  Video groups use a (L/4 .. ) x 2 x 2
    grid truncated to L rows.
    """
    b = _Builder()
    if modalities is None:
        modalities = [(TEXT, VIDEO, AUDIO)[k % 3] for k in range(len(lengths))]
    for k, (L, m) in enumerate(zip(lengths, modalities)):
        if m == TEXT:
            b.text("text%d" % k, L, k)
        elif m == AUDIO:
            b.audio("audio%d" % k, L, k)
        else:
            T = max(1, (L + 3) // 4)
            b.video("video%d" % k, T, 2, 2, k, keep=L)
    if sum(lengths) == 0:
        tags = np.zeros(0, np.uint8); pos = np.zeros((0, 3), np.int32); segv = np.zeros(0, np.int32)
    else:
        tags, pos, segv = b.arrays()
    n = tags.shape[0]
    return Workload(name="custom_%s" % "_".join(map(str, lengths)), index=index, n=n,
                    n_seg=len(lengths), H=H, D=D, dtype=dtype,
                    capacity=capacity if capacity is not None else _round_up(max(n, 1), ALIGN),
                    time_offset=time_offset, q_scale=q_scale, tags=tags, pos=pos, seg=segv,
                    rope=default_rope(D), groups=b.groups)


def make_qkv(wl: Workload, seed: Optional[int] = None, chunk_rows: int = 4096):
    """Seeded Q, K, V in source order, as CPU torch tensors [n, H, D].

    Definition: one torch CPU generator seeded with `seed` (default
    1101 + workload index) draws float32 N(0, 1) values for Q, then K, then V,
    each in row chunks of `chunk_rows` tokens; values are multiplied by the
    workload's scale and rounded (RNE) to bfloat16 unless the workload is fp32.
    """
    import torch
    g = torch.Generator(device="cpu")
    g.manual_seed(wl.seed if seed is None else int(seed))
    out_dtype = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    tensors = []
    for _ in range(3):
        t = torch.empty((wl.n, wl.H, wl.D), dtype=out_dtype)
        for r0 in range(0, wl.n, chunk_rows):
            r1 = min(wl.n, r0 + chunk_rows)
            x = torch.randn((r1 - r0, wl.H, wl.D), generator=g, dtype=torch.float32)
            if wl.q_scale != 1.0:
                x.mul_(wl.q_scale)
            t[r0:r1] = x.to(out_dtype)
        tensors.append(t)
    return tuple(tensors)


def make_qkv_on_device(wl: Workload, device, seed: Optional[int] = None):
    """Seeded Q, K, V drawn directly on `device` (fast for the large
    workloads).  Same recipe as make_qkv but with torch's device generator, so
    the values differ from make_qkv's; they are deterministic for a seed."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed if seed is None else int(seed))
    out_dtype = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    tensors = []
    for _ in range(3):
        x = torch.randn((wl.n, wl.H, wl.D), generator=g, dtype=torch.float32, device=device)
        if wl.q_scale != 1.0:
            x.mul_(wl.q_scale)
        tensors.append(x.to(out_dtype))
        del x
    return tuple(tensors)


def to_f64(t) -> np.ndarray:
    """Exact upcast of a CPU torch tensor (fp32 or bf16) to a float64 array."""
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()


# ---------------------------------------------------------------------------
# Inputs of the denoising-step epilogue: per-modality latent states, anchor
# values and the pinned-row flags.  The continuation layout's reference groups
# (labels ending in "_ref") are the anchor rows ([P1] section 四: reference
# frames / audio clips are pinned and restored after every update).
# ---------------------------------------------------------------------------
def pinned_rows(wl: Workload) -> np.ndarray:
    """uint8 [n] in source order: 1 for tokens of a reference group."""
    flags = []
    for label, _m, count in wl.groups:
        flags.append(np.full(count, 1 if label.endswith("_ref") else 0, np.uint8))
    return np.concatenate(flags) if flags else np.zeros(0, np.uint8)


def make_states(wl: Workload, seed: int, scale: float = 1.0):
    """Seeded float32 N(0, 1) * scale states and anchors per modality, each
    [n_m, H, D] (tokens of that modality in source order), as CPU torch
    tensors: returns (z[3], anchor[3]).  One generator draws z for text,
    video, audio, then the anchors in the same order."""
    import torch
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    npm = wl.n_per_modality()
    z = [torch.randn((c, wl.H, wl.D), generator=g, dtype=torch.float32) * scale for c in npm]
    a = [torch.randn((c, wl.H, wl.D), generator=g, dtype=torch.float32) * scale for c in npm]
    return z, a


def make_continuation_small(H: int = 4, D: int = 128, T_ref: int = 3, T_tgt: int = 5, Hh: int = 6,
                            W: int = 7, audio_ref: int = 13, audio_tgt: int = 37) -> Workload:
    """The continuation window's five groups (text, audio reference, video
    reference, audio target, video target) at a size the oracle finishes in
    seconds; one segment, shift s = 238."""
    b = _Builder()
    b.text("text", 19, 0)
    b.audio("audio_ref", audio_ref, 0)
    b.video("video_ref", T_ref, Hh, W, 0)
    b.audio("audio_tgt", audio_tgt, 0)
    b.video("video_tgt", T_tgt, Hh, W, 0)
    tags, pos, segv = b.arrays()
    n = tags.shape[0]
    return Workload(name="continuation_small_%dtok" % n, index=103, n=n, n_seg=1, H=H, D=D,
                    dtype="bf16", capacity=_round_up(n, ALIGN), time_offset=238.0, q_scale=0.5,
                    tags=tags, pos=pos, seg=segv, rope=default_rope(D), groups=b.groups)


# ---------------------------------------------------------------------------
# Block-sparse (VSA) layout: a video latent grid listed cube by cube, so that
# every 64 consecutive tokens form one 4 x 4 x 4 block ("突破视频生成大模型的
# 工程瓶颈", sparse-attention section: VSA cuts the video tensor into 4 x 4 x 4
# = 64-token blocks).  Positions keep the grid coordinates, so RoPE is the same
# as for the row-major layout.
# ---------------------------------------------------------------------------
def cube_order_video(T: int, Hh: int, W: int, cube: int = 4) -> np.ndarray:
    """int32 [T*Hh*W, 3] (t, h, w) positions, cube-major: cubes row-major
    over (t, h, w), tokens row-major inside a cube.  Dims must be multiples
    of `cube`."""
    assert T % cube == 0 and Hh % cube == 0 and W % cube == 0
    ct, ch, cw, it, ih, iw = np.meshgrid(np.arange(T // cube), np.arange(Hh // cube), np.arange(W // cube),
                                         np.arange(cube), np.arange(cube), np.arange(cube), indexing="ij")
    t = (ct * cube + it).ravel()
    h = (ch * cube + ih).ravel()
    w = (cw * cube + iw).ravel()
    return np.stack([t, h, w], axis=1).astype(np.int32)


def make_vsa_workload(T: int = 24, Hh: int = 48, W: int = 52, H: int = 40, D: int = 128,
                      index: int = 200) -> Workload:
    """One segment of video tokens in cube order (T x Hh x W grid; the default
    24 x 48 x 52 = 59,904 tokens is the 58,758-token step's video grid rounded
    up to whole 4 x 4 x 4 cubes: 936 blocks)."""
    p = cube_order_video(T, Hh, W)
    n = p.shape[0]
    tags = np.full(n, VIDEO, np.uint8)
    seg = np.zeros(n, np.int32)
    return Workload(name="vsa_video_%dx%dx%d_%dtok" % (T, Hh, W, n), index=index, n=n, n_seg=1, H=H, D=D,
                    dtype="bf16", capacity=_round_up(n, ALIGN), time_offset=0.0, q_scale=0.5,
                    tags=tags, pos=p, seg=seg, rope=default_rope(D), groups=[("video_cubes", VIDEO, n)])
