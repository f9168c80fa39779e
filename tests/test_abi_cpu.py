"""The C-ABI library on the host: exported symbols, the host neighbour table
against the oracle (bit-exact), and argument checking (CPU only, no kernel runs)."""
import ctypes
import json
import os
import re
import subprocess

import numpy as np
import pytest

import workloads as wl
from oracle import neighbours_ref
import linear_attention_recurrence_mshortconv_amd as chm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "chimera_mshortconv.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(chimera_[a-z_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_function():
    L = chm.lib()
    names = _declared_functions()
    assert "chimera_kda_fwd" in names and "chimera_mshortconv_fwd" in names and len(names) >= 6
    out = subprocess.run(["nm", "-D", "--defined-only", chm.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (chimera_\w+)", out))
    for n in names:
        assert n in exported, n
        assert getattr(L, n) is not None


def test_status_strings():
    for s in range(8):
        assert len(chm.status_string(s)) > 0
    assert chm.status_string(0) == "ok"


def _layouts():
    out = [w.segments for w in wl.WORKLOADS]
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "neighbours_worked_example.json")))
    out.append(tuple(wl.Segment(**{"kind": s["kind"], "start": s["start"], "length": s["length"],
                                    "frames": s.get("frames", 0), "height": s.get("height", 0),
                                    "width": s.get("width", 0)}) for s in g["layout"]))
    rng = np.random.default_rng(1234)
    for _ in range(25):                                   # random packed layouts
        segs, start = [], 0
        for _ in range(int(rng.integers(1, 6))):
            kind = int(rng.integers(0, 3))
            if kind == wl.TEXT:
                n = int(rng.integers(1, 40))
                segs.append(wl.Segment(wl.TEXT, start, n))
            else:
                F = 1 if kind == wl.IMAGE else int(rng.integers(1, 6))
                Hh, Ww = int(rng.integers(1, 9)), int(rng.integers(1, 9))
                n = F * Hh * Ww
                segs.append(wl.Segment(kind, start, n, F, Hh, Ww))
            start += n
        out.append(tuple(segs))
    return out


def test_host_index_bit_exact_against_oracle():
    for segs in _layouts():
        T = sum(s.length for s in segs)
        got = chm.mshortconv_index(segs, T)
        want = neighbours_ref(segs, T)
        assert got.dtype == np.int32 and np.array_equal(got, want), segs[:3]


def test_host_index_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "neighbours_worked_example.json")))
    idx = chm.mshortconv_index(g["layout"], g["T"])
    for pos, row in g["rows"].items():
        assert idx[int(pos)].tolist() == row


def _status(fn, *args):
    return fn(*args)


def test_segment_validation_errors():
    L = chm.lib()
    buf = np.zeros((64, 27), dtype=np.int32)
    p = buf.ctypes.data
    cases = [
        ([dict(kind=0, start=1, length=4)], 5, 4),                      # does not start at 0
        ([dict(kind=0, start=0, length=4)], 5, 4),                      # does not reach T
        ([dict(kind=0, start=0, length=3), dict(kind=0, start=2, length=3)], 5, 4),   # overlap
        ([dict(kind=1, start=0, length=6, frames=2, height=1, width=3)], 6, 4),       # image with 2 frames
        ([dict(kind=2, start=0, length=7, frames=1, height=2, width=3)], 7, 4),       # length != grid
        ([dict(kind=0, start=0, length=4, height=2)], 4, 4),            # text with a grid
        ([dict(kind=9, start=0, length=4)], 4, 4),                      # unknown kind
        ([dict(kind=0, start=0, length=0)], 0, 4),                      # empty segment
    ]
    for segs, T, want in cases:
        arr = chm.segment_array(segs)
        assert L.chimera_mshortconv_index(arr, len(segs), T, p) == want, segs
        assert L.chimera_mshortconv_fwd(1, 2, 1, T, 8, 1, 3, 4, arr, len(segs), None) == want, segs
    arr = chm.segment_array([dict(kind=0, start=0, length=4)])
    assert L.chimera_mshortconv_index(arr, 1, 4, None) == 1               # null output
    assert L.chimera_mshortconv_index(None, 1, 4, p) == 1                 # null table
    assert L.chimera_mshortconv_index(arr, 1, -1, p) == 2                 # negative T
    assert L.chimera_mshortconv_index(chm.segment_array([]), 0, 0, None) == 0   # empty stream is fine


def test_conv_argument_errors():
    L = chm.lib()
    arr = chm.segment_array([dict(kind=0, start=0, length=4)])
    assert L.chimera_mshortconv_fwd(1, 2, 1, 4, 8, 7, 3, 4, arr, 1, None) == 3       # dtype
    assert L.chimera_mshortconv_fwd(1, 2, 1, 4, 12, 1, 3, 4, arr, 1, None) == 2      # C % 8
    assert L.chimera_mshortconv_fwd(None, 2, 1, 4, 8, 1, 3, 4, arr, 1, None) == 1    # null x
    assert L.chimera_mshortconv_fwd(1, 2, 1, 4, 8, 1, None, 4, arr, 1, None) == 1    # text weights
    assert L.chimera_mshortconv_fwd(1, 1, 1, 4, 8, 1, 3, 4, arr, 1, None) == 5       # in place
    assert L.chimera_mshortconv_fwd(1, 2, -1, 4, 8, 1, 3, 4, arr, 1, None) == 2      # negative B
    assert L.chimera_mshortconv_fwd(1, 2, 0, 4, 8, 1, 3, 4, arr, 1, None) == 0       # empty batch: no-op
    vis = chm.segment_array([dict(kind=1, start=0, length=4, frames=1, height=2, width=2)])
    assert L.chimera_mshortconv_fwd(1, 2, 1, 4, 8, 1, 3, None, vis, 1, None) == 1    # visual weights


def test_kda_argument_errors():
    L = chm.lib()
    args = lambda **kw: dict(dict(q=1, k=2, v=3, stride=256, a=4, b=5, S0=None, o=6, Sf=None, B=1, T=8, H=2,
                                  dk=128, dv=128, dt=1, flags=1, ws=None, wsb=0), **kw)

    def call(**kw):
        a = args(**kw)
        return L.chimera_kda_fwd(a["q"], a["k"], a["v"], a["stride"], a["a"], a["b"], a["S0"], a["o"], a["Sf"],
                                 a["B"], a["T"], a["H"], a["dk"], a["dv"], a["dt"], a["flags"], a["ws"], a["wsb"],
                                 None)
    assert call(dt=5) == 3
    assert call(dk=0) == 2 and call(dv=300) == 2 and call(T=-1) == 2
    assert call(q=None) == 1 and call(o=None) == 1 and call(b=None) == 1
    assert call(stride=100) == 2                                        # stride below H*d
    assert call(flags=64) == 5                                          # unknown flag
    assert call(B=0) == 0 and call(H=0) == 0                            # nothing to do


def test_kda_gated_argument_errors():
    """chimera_kda_fwd_gated checks its gate arguments before any launch (no kernel runs here)."""
    L = chm.lib()
    f = ctypes.c_float

    def call(gate=7, gstride=256, eps=1e-6, T=8, B=1):
        return L.chimera_kda_fwd_gated(1, 2, 3, 256, 4, 5, None, gate, gstride, None, f(eps), 6, None, B, T, 2, 128,
                                       128, 1, 1, None, 0, None)
    assert call(gate=None) == 1                                         # gate required when T > 0
    assert call(gstride=200) == 2                                       # stride below H*dv
    assert call(eps=-1.0) == 2 and call(eps=float("nan")) == 2 and call(eps=float("inf")) == 2
    assert call(B=0) == 0                                               # nothing to do
    ev = (ctypes.c_void_p * 8)()
    names = (ctypes.c_char_p * 8)()
    used = ctypes.c_int32(3)
    timed = lambda cap: L.chimera_kda_fwd_gated_timed(1, 2, 3, 256, 4, 5, None, 7, 256, None, f(1e-6), 6, None, 1,
                                                      8, 2, 128, 128, 1, 1, None, 0, None, ev, names, cap,
                                                      ctypes.byref(used))
    assert timed(5) == 2 and used.value == 0                            # needs 5 kernels + 1


def test_kda_varlen_argument_errors_and_workspace():
    """chimera_kda_fwd_varlen checks the sample offsets before any launch (no kernel runs here);
    its workspace for equal samples equals the batched call's."""
    L = chm.lib()
    f = ctypes.c_float

    def call(cu, nseq=None):
        arr = np.ascontiguousarray(np.asarray(cu, dtype=np.int64))
        n = len(cu) - 1 if nseq is None else nseq
        return L.chimera_kda_fwd_varlen(1, 2, 3, 256, 4, 5, None, None, 0, None, f(1e-6), 6, None, arr.ctypes.data,
                                        n, 2, 128, 128, 1, 1, None, 0, None)
    assert call([1, 5]) == 2                                            # must start at 0
    assert call([0, 9, 4]) == 2                                         # decreasing
    assert call([0, 4], nseq=-1) == 2
    assert L.chimera_kda_fwd_varlen(1, 2, 3, 256, 4, 5, None, None, 0, None, f(1e-6), 6, None, None, 1, 2, 128,
                                    128, 1, 1, None, 0, None) == 1      # no offsets
    assert call([0]) == 0                                               # no sample: nothing to do
    big = 64 * 300
    need = chm.kda_varlen_workspace_size([0, big, 2 * big, 3 * big], 16, 128, 128, chm.BF16, chm.KDA_L2NORM_QK)
    assert need > 0
    assert need == chm.kda_workspace_size(3, big, 16, 128, 128, chm.BF16, chm.KDA_L2NORM_QK)
    mixed = [0, 1000, 1000, 5000, 5300, 20000]
    assert chm.kda_varlen_workspace_size(mixed, 16, 128, 128, chm.BF16, chm.KDA_SEQUENTIAL) == 0
    assert chm.kda_varlen_workspace_size(mixed, 16, 128, 128, chm.BF16, chm.KDA_L2NORM_QK) > 0
    assert chm.kda_varlen_workspace_size([0, 3, 2], 16, 128, 128, chm.BF16, 0) == 0     # invalid offsets
    ev = (ctypes.c_void_p * 16)()
    names = (ctypes.c_char_p * 16)()
    used = ctypes.c_int32(3)
    arr = np.array([0, 5, 9], dtype=np.int64)
    timed = lambda cap: L.chimera_kda_fwd_varlen_timed(1, 2, 3, 256, 4, 5, None, None, 0, None, f(1e-6), 6, None,
                                                       arr.ctypes.data, 2, 2, 128, 128, 1, 1, None, 0, None, ev,
                                                       names, cap, ctypes.byref(used))
    assert timed(7) == 2 and used.value == 0                            # needs 2 * nseq + 4 = 8


def test_backward_argument_errors():
    """The backward entry points check their arguments before any launch (no kernel runs here)."""
    L = chm.lib()
    call = lambda **kw: L.chimera_kda_bwd(*[kw.get(n, d) for n, d in (
        ("q", 1), ("k", 2), ("v", 3), ("stride", 256), ("a", 4), ("b", 5), ("S0", None), ("do", 6), ("dS", None),
        ("dq", 7), ("dk", 8), ("dv", 9), ("da", 10), ("db", 11), ("dS0", None), ("B", 1), ("T", 8), ("H", 2),
        ("dkk", 128), ("dvv", 128), ("dt", 1), ("flags", 1), ("ws", None), ("wsb", 0), ("stream", None))])
    assert call(dt=7) == 3
    assert call(dkk=256, stride=1024) == 5                              # the backward takes dk <= 128
    assert call(do=None) == 1 and call(dq=None) == 1 and call(db=None) == 1
    assert call(stride=100) == 2
    assert call() == 6                                                  # workspace missing
    assert call(B=0) == 0
    # bf16 heads of 128 run the chunked backward: here 5 segments of 272 tokens (17 chunks of 16) per
    # head, each split in two parts whose checkpoints are kept one part at a time: the bf16 state
    # before each chunk of the longer part (9 slots per segment), 1 KiB of T fragments per chunk,
    # and 13 fp32 matrices per segment (its L, M, start, E, G and a spare; at its part boundary L and
    # M in two slots each, the start in two slots, dS)
    n = int(L.chimera_kda_bwd_workspace_size(1, 64 * 20 + 3, 16, 128, 128, 1, 1))
    assert n == 2 * 16 * 5 * 9 * 128 * 128 + 16 * 81 * 1024 + 4 * 13 * 16 * 5 * 128 * 128
    # one segment (sequences too short to cut): the state before every chunk, no per-segment matrices
    n1 = int(L.chimera_kda_bwd_workspace_size(1, 200, 16, 128, 128, 1, 1))
    assert n1 == 2 * 16 * 13 * 128 * 128 + 16 * 13 * 1024
    # the token-by-token backward (CHIMERA_KDA_SEQUENTIAL, or fp32): fp32 checkpoints + slice partials
    for dt, fl in ((1, 3), (0, 1)):
        n = int(L.chimera_kda_bwd_workspace_size(1, 64 * 20 + 3, 16, 128, 128, dt, fl))
        assert n >= 4 * (16 * 81 * 128 * 128 + 8 * 1283 * 16 * (3 * 128 + 1))
    # the chunked backward reads q, k, v, alpha and dout as 8-byte pieces: other layouts are refused
    small = int(L.chimera_kda_bwd_workspace_size(1, 8, 2, 128, 128, 1, 1))
    big = np.zeros(small + 256, dtype=np.uint8)
    wsp = (big.ctypes.data + 255) // 256 * 256
    assert call(ws=wsp, wsb=small) == 5                                 # q = 1: misaligned
    assert call(ws=wsp, wsb=small, stride=258, q=8, k=16, v=24, a=32, do=40) == 5   # stride % 4
    arr = chm.segment_array([dict(kind=0, start=0, length=4)])
    cb = lambda **kw: L.chimera_mshortconv_bwd(kw.get("x", 1), kw.get("dy", 2), kw.get("dx", 3), kw.get("dwt", 4),
                                               kw.get("dwv", 5), 1, 4, kw.get("C", 8), 1, 6, 7, arr, 1, None)
    assert cb(C=12) == 2 and cb(dwt=None) == 1 and cb(dx=None) == 1 and cb(dx=1) == 5


def test_backward_varlen_argument_errors():
    """chimera_kda_bwd_varlen checks its arguments before any launch (no kernel runs here)."""
    L = chm.lib()
    cu = np.array([0, 5, 5, 12], dtype=np.int64)
    bad0 = np.array([1, 5], dtype=np.int64)
    down = np.array([0, 5, 4], dtype=np.int64)
    def call(cu_arr=cu, nseq=3, **kw):
        a = dict(q=1, k=2, v=3, stride=256, al=4, be=5, S0=None, do=6, dS=None, dq=7, dk=8, dv=9, da=10, db=11,
                 dS0=None, H=2, dkk=128, dvv=128, dt=1, flags=1, ws=None, wsb=0)
        a.update(kw)
        ptr = None if cu_arr is None else cu_arr.ctypes.data
        return L.chimera_kda_bwd_varlen(a["q"], a["k"], a["v"], a["stride"], a["al"], a["be"], a["S0"], a["do"],
                                        a["dS"], a["dq"], a["dk"], a["dv"], a["da"], a["db"], a["dS0"], ptr, nseq,
                                        a["H"], a["dkk"], a["dvv"], a["dt"], a["flags"], a["ws"], a["wsb"], None)
    assert call(dt=7) == 3
    assert call(cu_arr=None) == 1
    assert call(cu_arr=bad0, nseq=1) == 2 and call(cu_arr=down, nseq=2) == 2 and call(nseq=-1) == 2
    assert call(dkk=256, stride=1024) == 5
    assert call(do=None) == 1 and call(db=None) == 1
    assert call(stride=100) == 2
    assert call() == 6                                                  # workspace missing
    assert call(nseq=0) == 0
    need = int(L.chimera_kda_bwd_varlen_workspace_size(cu.ctypes.data, 3, 2, 128, 128, 1, 1))
    one = int(L.chimera_kda_bwd_workspace_size(1, 7, 2, 128, 128, 1, 1))
    assert need >= one > 0                                              # the largest run's need


def test_fused_conv_argument_errors():
    """chimera_kda_fwd_conv checks its arguments before any launch (no kernel runs here)."""
    L = chm.lib()
    text = chm.segment_array([dict(kind=0, start=0, length=8)])
    img = chm.segment_array([dict(kind=1, start=0, length=8, frames=1, height=2, width=4)])
    many = chm.segment_array([dict(kind=0, start=i, length=1) for i in range(33)])
    def call(segs=text, nseg=None, **kw):
        a = dict(x=1, wt=2, wv=3, al=4, be=5, S0=None, o=6, Sf=None, B=1, T=8, H=2, dk=32, dv=32, dt=1, flags=1)
        a.update(kw)
        n = len(segs) if nseg is None else nseg
        return L.chimera_kda_fwd_conv(a["x"], a["wt"], a["wv"], segs, n, a["al"], a["be"], a["S0"], a["o"], a["Sf"],
                                      a["B"], a["T"], a["H"], a["dk"], a["dv"], a["dt"], a["flags"],
                                      a.get("ws"), a.get("wsb", 0), None)
    assert call(dt=7) == 3
    assert call(dk=256) == 5                                            # the conv weights of dk > 128 do not fit
    assert call(flags=8) == 5                                           # an unknown flag
    assert call(T=9) == 4                                               # segments must tile [0, T)
    assert call(segs=many, T=33) == 5                                   # more than 32 segments
    assert call(x=None) == 1 and call(o=None) == 1 and call(al=None) == 1
    assert call(wt=None) == 1 and call(segs=img, wv=None) == 1          # the weights the layout uses
    assert call(x=6) == 5                                               # o aliasing x
    assert call(B=0) == 0
    # bf16 with dk = dv = 128 (x and alpha 8-byte aligned) runs the chunked kernels, which need the workspace
    need = int(L.chimera_kda_conv_workspace_size(img, 1, 1, 8, 2, 128, 128, 1, 1))
    assert need > 0
    big = dict(segs=img, dk=128, dv=128, x=8, o=16, al=32)
    assert call(**big) == 6
    assert call(**big, ws=16, wsb=need - 1) == 6
    assert call(**dict(big, x=None), ws=16, wsb=need) == 1                # argument checks come first


def test_fused_conv_workspace_size_rules():
    """The fused call's workspace: the chunked path's states plus the transposed weights and
    the segment table; zero on the token-by-token kernel."""
    L = chm.lib()
    img = chm.segment_array([dict(kind=0, start=0, length=256), dict(kind=1, start=256, length=65536, frames=1,
                                                                      height=256, width=256)])
    size = lambda *a: int(L.chimera_kda_conv_workspace_size(img, 2, *a))
    T, H, d = 65792, 16, 128
    full = size(1, T, H, d, d, 1, 1)
    states = chm.kda_workspace_size(1, T, H, d, d, chm.BF16, chm.KDA_L2NORM_QK)
    assert full == states + (31 * 3 * H * d * 4 + 255) // 256 * 256 + 2 * 32
    assert size(1, T, H, d, d, 1, 1 | 2) == 0                             # CHIMERA_KDA_SEQUENTIAL
    assert size(1, T, H, d, d, 0, 1) == 0                                 # fp32: token by token
    assert size(1, T, H, 64, 64, 1, 1) == 0                               # d = 64: the conv is fused only at 128
    assert size(1, T + 1, H, d, d, 1, 1) == 0                             # segments that do not tile T
    no_split = size(1, T, H, d, d, 1, 1 | 4)
    assert no_split == (31 * 3 * H * d * 4 + 255) // 256 * 256 + 2 * 32   # one segment: no states


def test_workspace_size_rules():
    n = chm.kda_workspace_size(1, 65792, 16, 128, 128, chm.BF16, chm.KDA_L2NORM_QK)
    assert n >= 0
    # bf16 heads up to 128 in steps of 8 run the chunked kernels at 128 channels: the same states
    for dk, dv in ((64, 64), (32, 32), (8, 128), (128, 96)):
        assert chm.kda_workspace_size(1, 65792, 16, dk, dv, chm.BF16, chm.KDA_L2NORM_QK) == n
    # token by token: sequences cut into P segments (about 2048 blocks of 16 columns, segments of
    # at least 256 tokens and whole 16-token batches), 4 (2 dk dv + dk dk) bytes per (head, segment)
    # (P = 32, 15, 2, 16 below: e.g. 16 heads of 4 column slices want 32 segments of 2064 tokens)
    assert chm.kda_workspace_size(1, 65792, 16, 60, 64, chm.BF16, chm.KDA_L2NORM_QK) == 16 * 32 * (2 * 60 * 64 + 60 * 60) * 4
    assert chm.kda_workspace_size(1, 65792, 16, 64, 132, chm.BF16, 0) == 16 * 15 * (2 * 64 * 132 + 64 * 64) * 4
    assert chm.kda_workspace_size(1, 600, 2, 32, 32, chm.F32, 0) == 2 * 2 * (3 * 32 * 32) * 4
    assert chm.kda_workspace_size(1, 65792, 16, 128, 128, chm.BF16, chm.KDA_SEQUENTIAL) == 16 * 16 * 3 * 128 * 128 * 4
    assert chm.kda_workspace_size(1, 65792, 16, 256, 256, chm.BF16, 0) == 0     # d_k > 128: no cut
    assert chm.kda_workspace_size(1, 600, 2, 32, 32, chm.F32, chm.KDA_NO_SPLIT) == 0
    assert chm.kda_workspace_size(1, 256, 2, 32, 32, chm.F32, 0) == 0            # one segment
    assert chm.kda_workspace_size(256, 4096, 16, 32, 32, chm.F32, 0) == 0        # heads fill the chip
    assert chm.kda_workspace_size(1, 10, 1, 0, 128, chm.BF16, 0) == 0            # invalid sizes


def test_timed_variants_check_their_marks_first():
    """The timing variants refuse missing or too few marks before any launch."""
    L = chm.lib()
    arr = chm.segment_array([dict(kind=0, start=0, length=4), dict(kind=1, start=4, length=4, frames=1, height=2,
                                                                    width=2)])
    ev = (ctypes.c_void_p * 8)()
    names = (ctypes.c_char_p * 8)()
    used = ctypes.c_int32(5)
    conv = lambda ev_, cap: L.chimera_mshortconv_fwd_timed(1, 2, 1, 8, 8, 1, 3, 4, arr, 2, None, ev_, names, cap,
                                                           ctypes.byref(used))
    assert conv(None, 8) == 1
    assert conv(ev, 2) == 2 and used.value == 0                          # needs nseg + 1 = 3
    kda = lambda ev_, cap: L.chimera_kda_fwd_timed(1, 2, 3, 256, 4, 5, None, 6, None, 1, 8, 2, 128, 128, 1, 1,
                                                   None, 0, None, ev_, names, cap, ctypes.byref(used))
    assert kda(None, 8) == 1
    assert kda(ev, 4) == 2                                                 # needs 4 kernels + 1
    fused = lambda ev_, cap: L.chimera_kda_fwd_conv_timed(1, 2, 3, arr, 2, 4, 5, None, 6, None, 1, 8, 2, 128, 128, 1,
                                                          1, None, 0, None, ev_, names, cap, ctypes.byref(used))
    assert fused(None, 8) == 1
    assert fused(ev, 4) == 2                                               # needs 4 kernels + 1
    used.value = 9
    assert L.chimera_kda_fwd_timed(1, 2, 3, 256, 4, 5, None, 6, None, 0, 8, 2, 128, 128, 1, 1, None, 0, None, ev,
                                   names, 5, ctypes.byref(used)) == 0 and used.value == 0   # B = 0: nothing launched
