"""Seeded synthetic inputs for the mShortConv + KDA forward.

This module only draws random numbers and lays out token segments. It holds
none of the method's arithmetic: no convolution, no recurrence. Both the CPU
oracle (through the tests and the bench) and the HIP library consume what it
returns, so the two sides always see bit-identical inputs.

Six workloads, each named by what it is:

* ``tiny_text_fp32``   B=1, H=2,  d=32,  T=256 text tokens, fp32.
* ``image_1024``       B=1, H=16, d=128, 256 text + 64x64 image grid (4,352 tokens), bf16.
* ``image_4096``       B=1, H=16, d=128, 256 text + 256x256 image grid (65,792 tokens), bf16.
* ``video_5s``         B=2, H=16, d=128, 256 text + 21x32x56 video grid (37,888 tokens), bf16, S0 != 0.
* ``video_30s``        B=1, H=16, d=128, 256 text + 126x45x45 video grid (255,406 tokens), bf16.
* ``packed_mixed``     one row of 40 packed samples, H=16, d=128, bf16: the 256^2, 512^2 and
  1024^2 image buckets at 4:2:2 (16x16, 32x32 and 64x64 grids), each after its own text
  prompt of 32..300 tokens (62,796 tokens in all); the state restarts at every sample.

Grid sizes follow the packing the Chimera pages describe (page 1, section 3.2
and Eq. 12): text tokens first, then visual tokens in time-first raster order.
A 4096x4096 image patchified at 16x16 gives the 256x256 grid (page 1,
section 1).

Recipe (one fixed draw order per workload, ``numpy.random.default_rng(seed)``
with seed = workload index):

1. q, k, v ~ N(0, 1), each [B, T, H, d]; q and k are then divided by their
   Euclidean norm over d for every (token, head).
2. alpha: log(alpha) = -s * softplus(N(0, 1)), [B, T, H, d]; s = 1 for the
   tiny workload and 0.05 for the others (long memory).
3. beta = sigmoid(N(0, 1)), [B, T, H].
4. S0 ~ N(0, 0.1^2), [B, H, d, d], only for ``video_5s`` (else no S0).
5. Text conv weights ~ N(0, 0.5^2), [C, 4]; visual conv weights ~ N(0, 0.5^2),
   [C, 27], with C = 3*H*d channels (the q|k|v blocks side by side).

Every bf16 workload rounds each drawn fp32 value once to bf16 (round to
nearest, ties to even); both sides consume the rounded values. Conv weights
stay fp32.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

TEXT, IMAGE, VIDEO = 0, 1, 2
KIND_NAMES = {TEXT: "text", IMAGE: "image", VIDEO: "video"}


@dataclasses.dataclass(frozen=True)
class Segment:
    """One modality segment of the packed stream: [start, start + length)."""
    kind: int
    start: int
    length: int
    frames: int = 0
    height: int = 0
    width: int = 0


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    B: int
    H: int
    d: int
    dtype: str            # "f32" or "bf16"
    segments: tuple       # tuple of Segment
    log_alpha_scale: float
    s0_std: Optional[float]
    chunk: int = 64
    samples: Optional[tuple] = None   # packed sample offsets (N + 1, from 0 to T), or None

    @property
    def T(self) -> int:
        return sum(s.length for s in self.segments)

    @property
    def C(self) -> int:
        return 3 * self.H * self.d


def text_then_grid(n_text: int, frames: int, height: int, width: int) -> tuple:
    """Text prefix followed by one visual grid in time-first raster order."""
    segs = [Segment(TEXT, 0, n_text)]
    kind = IMAGE if frames == 1 else VIDEO
    segs.append(Segment(kind, n_text, frames * height * width, frames, height, width))
    return tuple(segs)


def packed_samples(groups: int = 5, seed: int = 5) -> tuple:
    """Segments and sample offsets of a row of packed image samples: per group of eight, four
    16x16, two 32x32 and two 64x64 grids (the 256^2 / 512^2 / 1024^2 buckets at 4:2:2 after
    16x16 patches), each after a text prompt of 32..300 tokens drawn from its own stream."""
    rng = np.random.default_rng(seed + 2000)
    sides = [16, 16, 16, 16, 32, 32, 64, 64]
    segs, cu, off = [], [0], 0
    for _ in range(groups):
        for side in sides:
            n_text = int(rng.integers(32, 301))
            segs.append(Segment(TEXT, off, n_text))
            segs.append(Segment(IMAGE, off + n_text, side * side, 1, side, side))
            off += n_text + side * side
            cu.append(off)
    return tuple(segs), tuple(cu)


_PACKED_SEGS, _PACKED_CU = packed_samples()

WORKLOADS: List[Workload] = [
    Workload(0, "tiny_text_fp32", 1, 2, 32, "f32", (Segment(TEXT, 0, 256),), 1.0, None),
    Workload(1, "image_1024", 1, 16, 128, "bf16", text_then_grid(256, 1, 64, 64), 0.05, None),
    Workload(2, "image_4096", 1, 16, 128, "bf16", text_then_grid(256, 1, 256, 256), 0.05, None),
    Workload(3, "video_5s", 2, 16, 128, "bf16", text_then_grid(256, 21, 32, 56), 0.05, 0.1),
    Workload(4, "video_30s", 1, 16, 128, "bf16", text_then_grid(256, 126, 45, 45), 0.05, None),
    Workload(5, "packed_mixed", 1, 16, 128, "bf16", _PACKED_SEGS, 0.05, None, samples=_PACKED_CU),
]


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = ((u + bias) & np.uint32(0xFFFF0000)).view(np.float32)
    return r


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of fp32 values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / n).astype(np.float32)


def _softplus(x):
    return np.logaddexp(np.float32(0.0), x).astype(np.float32)


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def make_inputs(w: Workload, T: Optional[int] = None, segments=None, seed: Optional[int] = None):
    """Draw one workload's inputs.

    ``T``/``segments`` override the token count and layout (for small parity
    cases with the same distributions); ``seed`` overrides the workload index.
    Returns a dict of numpy arrays (fp32 storage; bf16 workloads hold
    bf16-representable values):

    x      [B, T, 3*H*d]  conv input, channel = part*H*d + h*d + i (part 0=q, 1=k, 2=v)
    alpha  [B, T, H, d]
    beta   [B, T, H]
    S0     [B, H, d, d] or None
    w_text [3*H*d, 4]
    w_vis  [3*H*d, 27]
    """
    segs = tuple(segments) if segments is not None else w.segments
    T = sum(s.length for s in segs) if T is None else T
    assert sum(s.length for s in segs) == T
    rng = np.random.default_rng(w.index if seed is None else seed)
    B, H, d = w.B, w.H, w.d
    q = _unit_rows(_normal(rng, (B, T, H, d)))
    k = _unit_rows(_normal(rng, (B, T, H, d)))
    v = _normal(rng, (B, T, H, d))
    log_alpha = -np.float32(w.log_alpha_scale) * _softplus(_normal(rng, (B, T, H, d)))
    alpha = np.exp(log_alpha).astype(np.float32)
    beta = _sigmoid(_normal(rng, (B, T, H)))
    S0 = None
    if w.s0_std is not None:
        S0 = (np.float32(w.s0_std) * _normal(rng, (B, H, d, d))).astype(np.float32)
    C = 3 * H * d
    w_text = (np.float32(0.5) * _normal(rng, (C, 4))).astype(np.float32)
    w_vis = (np.float32(0.5) * _normal(rng, (C, 27))).astype(np.float32)
    x = np.concatenate([q.reshape(B, T, H * d), k.reshape(B, T, H * d), v.reshape(B, T, H * d)], axis=-1)
    del q, k, v
    if w.dtype == "bf16":
        x = round_to_bf16(x)
        alpha = round_to_bf16(alpha)
        beta = round_to_bf16(beta)
    return dict(x=x, alpha=alpha, beta=beta, S0=S0, w_text=w_text, w_vis=w_vis, segments=segs)


def small_layout(kind: str, n_text: int, frames: int = 1, height: int = 1, width: int = 1) -> tuple:
    """A reduced layout of the same kind, for parity cases the oracle runs in seconds."""
    if kind == "text":
        return (Segment(TEXT, 0, n_text),)
    return text_then_grid(n_text, frames, height, width)


def make_gate(w: Workload, T: Optional[int] = None, seed: Optional[int] = None):
    """Inputs of the output gate and norm (Eq. 15): the gate projection g [B, T, H, d]
    ~ N(0, 1) and the norm gain [d] ~ 1 + 0.1 N(0, 1) (fp32). Drawn from their own
    stream (seed + 1000), so the workload's other inputs do not change. The gate is
    bf16-representable for bf16 workloads."""
    T = w.T if T is None else T
    rng = np.random.default_rng((w.index if seed is None else seed) + 1000)
    gate = _normal(rng, (w.B, T, w.H, w.d))
    weight = (np.float32(1.0) + np.float32(0.1) * _normal(rng, (w.d,))).astype(np.float32)
    if w.dtype == "bf16":
        gate = round_to_bf16(gate)
    return gate, weight
