"""Pins for the mShortConv oracle (CPU only).

Each test checks the oracle against something other than itself: hand-derived
fixtures from Eq. 12 and Fig. 4 (tests/golden/), a closed form (a centred
delta kernel is the identity), a library routine (torch's grouped conv1d /
conv2d / conv3d in fp64 with explicit padding), or a second formulation (the
gather through the neighbour table).
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import neighbours_ref, conv_ref, conv_gather_ref, TEXT, IMAGE, VIDEO


def _segs(layout):
    return [dict(l) for l in layout]


def test_neighbours_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "neighbours_worked_example.json")))
    idx = neighbours_ref(_segs(g["layout"]), g["T"])
    assert idx.dtype == np.int32 and idx.shape == (g["T"], 27)
    for pos, row in g["rows"].items():
        assert idx[int(pos)].tolist() == row, pos


def test_neighbours_fig4_raster(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "raster_fig4.json")))
    Fr, Hh, Ww = g["frames"], g["height"], g["width"]
    seg = [dict(kind=VIDEO, start=0, length=Fr * Hh * Ww, frames=Fr, height=Hh, width=Ww)]
    idx = neighbours_ref(seg, Fr * Hh * Ww)
    # the centre tap of the printed token n (1-based) is raster position n - 1
    grid = np.array(g["printed_fragments"]["frame1_grid"])
    for h in range(Hh):
        for w in range(Ww):
            n = grid[h, w]
            assert idx[n - 1, 22] == n - 1
            assert n - 1 == 0 * Hh * Ww + h * Ww + w          # Eq. 12 for frame 0
    for name, first in (("frame2_head", 26), ("frame3_head", 51)):
        assert g["printed_fragments"][name][0] == first
    assert g["printed_fragments"]["frame3_tail"][-1] == Fr * Hh * Ww
    for fact in g["neighbour_facts"]:
        kt, kh, kw = fact["tap"]
        got = int(idx[fact["token"] - 1, kt * 9 + kh * 3 + kw])
        want = -1 if fact["expect"] is None else fact["expect"] - 1
        assert got == want, fact["what"]


def test_conv_hand_examples(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "conv_hand_examples.json")))
    t = g["text"]
    x = np.array(t["x"], dtype=np.float64)[None, :, None]
    w = np.array(t["w"], dtype=np.float64)[None, :]
    seg = [dict(kind=TEXT, start=0, length=len(t["x"]))]
    y = conv_ref(x, w, np.zeros((1, 27)), seg)
    assert y[0, :, 0].tolist() == t["y"]
    yg = conv_gather_ref(x, w, np.zeros((1, 27)), seg)
    assert yg[0, :, 0].tolist() == t["y"]

    for kind_name, kind in (("image", IMAGE), ("video", VIDEO)):
        e = g[kind_name]
        xs = np.array(e["x"], dtype=np.float64)
        Fr = e.get("frames", 1)
        Hh, Ww = e["height"], e["width"]
        L = Fr * Hh * Ww
        seg = [dict(kind=kind, start=0, length=L, frames=Fr, height=Hh, width=Ww)]
        for tap, want in e["one_hot_taps"].items():
            wv = np.zeros((1, 27))
            wv[0, int(tap)] = 1.0
            y = conv_ref(xs.reshape(1, L, 1), np.zeros((1, 4)), wv, seg)
            assert y.reshape(np.array(want).shape).tolist() == want, (kind_name, tap)
            yg = conv_gather_ref(xs.reshape(1, L, 1), np.zeros((1, 4)), wv, seg)
            assert yg.reshape(np.array(want).shape).tolist() == want, (kind_name, tap)


def _mixed_layout():
    # text, image, text, video: every kind, segment edges not aligned to anything
    segs = [dict(kind=TEXT, start=0, length=7),
            dict(kind=IMAGE, start=7, length=5 * 6, frames=1, height=5, width=6),
            dict(kind=TEXT, start=37, length=3),
            dict(kind=VIDEO, start=40, length=4 * 3 * 5, frames=4, height=3, width=5)]
    return segs, 100


def test_conv_centred_delta_is_identity():
    rng = np.random.default_rng(1)
    segs, T = _mixed_layout()
    C = 5
    x = rng.standard_normal((2, T, C))
    wt = np.zeros((C, 4)); wt[:, 3] = 1.0
    wv = np.zeros((C, 27)); wv[:, 2 * 9 + 1 * 3 + 1] = 1.0
    assert np.array_equal(conv_ref(x, wt, wv, segs), x)
    assert np.array_equal(conv_gather_ref(x, wt, wv, segs), x)


def test_conv_matches_torch_grouped_conv():
    rng = np.random.default_rng(2)
    segs, T = _mixed_layout()
    B, C = 2, 6
    x = rng.standard_normal((B, T, C))
    wt = rng.standard_normal((C, 4))
    wv = rng.standard_normal((C, 27))
    y = conv_ref(x, wt, wv, segs)
    xt = torch.from_numpy(x)
    for s in segs:
        a, L = s["start"], s["length"]
        xs = xt[:, a:a + L, :]                                   # [B, L, C]
        if s["kind"] == TEXT:
            inp = F.pad(xs.permute(0, 2, 1), (3, 0))             # causal: 3 zeros in front
            ref = F.conv1d(inp, torch.from_numpy(wt)[:, None, :], groups=C)
            ref = ref.permute(0, 2, 1)
        elif s["kind"] == IMAGE:
            g = xs.reshape(B, s["height"], s["width"], C).permute(0, 3, 1, 2)
            w2 = torch.from_numpy(wv).reshape(C, 3, 3, 3)[:, 2][:, None]   # kt = 2 slice
            ref = F.conv2d(F.pad(g, (1, 1, 1, 1)), w2, groups=C).permute(0, 2, 3, 1).reshape(B, L, C)
        else:
            g = xs.reshape(B, s["frames"], s["height"], s["width"], C).permute(0, 4, 1, 2, 3)
            w3 = torch.from_numpy(wv).reshape(C, 1, 3, 3, 3)
            ref = F.conv3d(F.pad(g, (1, 1, 1, 1, 2, 0)), w3, groups=C)   # time: 2 in front, 0 behind
            ref = ref.permute(0, 2, 3, 4, 1).reshape(B, L, C)
        np.testing.assert_allclose(y[:, a:a + L], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_conv_gather_equals_segment_views():
    rng = np.random.default_rng(3)
    segs, T = _mixed_layout()
    x = rng.standard_normal((1, T, 4))
    wt = rng.standard_normal((4, 4))
    wv = rng.standard_normal((4, 27))
    np.testing.assert_allclose(conv_gather_ref(x, wt, wv, segs), conv_ref(x, wt, wv, segs),
                               rtol=1e-13, atol=1e-13)


def test_conv_segments_do_not_mix():
    rng = np.random.default_rng(4)
    segs, T = _mixed_layout()
    x = rng.standard_normal((1, T, 3))
    wt = rng.standard_normal((3, 4))
    wv = rng.standard_normal((3, 27))
    y = conv_ref(x, wt, wv, segs)
    for s in segs:
        a, L = s["start"], s["length"]
        x2 = x.copy()
        x2[:, a:a + L] += 100.0                                  # perturb one segment only
        y2 = conv_ref(x2, wt, wv, segs)
        outside = np.ones(T, dtype=bool); outside[a:a + L] = False
        assert np.array_equal(y2[:, outside], y[:, outside])


def test_conv_linear_in_x_and_w():
    rng = np.random.default_rng(5)
    segs, T = _mixed_layout()
    x1, x2 = rng.standard_normal((2, 1, T, 3))
    wt1, wt2 = rng.standard_normal((2, 3, 4))
    wv1, wv2 = rng.standard_normal((2, 3, 27))
    lhs = conv_ref(x1 + 2 * x2, wt1, wv1, segs)
    np.testing.assert_allclose(lhs, conv_ref(x1, wt1, wv1, segs) + 2 * conv_ref(x2, wt1, wv1, segs), atol=1e-12)
    lhs = conv_ref(x1, wt1 - wt2, wv1 - wv2, segs)
    np.testing.assert_allclose(lhs, conv_ref(x1, wt1, wv1, segs) - conv_ref(x1, wt2, wv2, segs), atol=1e-12)


def test_neighbours_bounds_and_causality():
    segs, T = _mixed_layout()
    idx = neighbours_ref(segs, T)
    for s in segs:
        a, L = s["start"], s["length"]
        rows = idx[a:a + L]
        valid = rows[rows >= 0]
        assert valid.min() >= a and valid.max() < a + L         # never leaves its segment
        if s["kind"] == TEXT:
            assert (rows[:, 4:] == -1).all()
            assert (rows[:, :4][rows[:, :4] >= 0] <= np.arange(a, a + L)[:, None].repeat(4, 1)[rows[:, :4] >= 0]).all()
        else:
            HW = s["height"] * s["width"]
            frame_of = lambda p: (p - a) // HW
            for t in range(27):
                ok = rows[:, t] >= 0
                dt = frame_of(rows[ok, t]) - frame_of(np.arange(a, a + L)[ok])
                assert (dt == t // 9 - 2).all()                  # causal in time: -2, -1, 0
