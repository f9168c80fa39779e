"""Input generator sanity and the oracle's bf16 rounding (CPU only)."""
import numpy as np
import torch

import workloads as wl
from oracle import round_bf16_ref


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-20, 20, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -2.5e-38])])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_bf16_ref(x), want)
    np.testing.assert_array_equal(wl.round_to_bf16(x.astype(np.float32)).astype(np.float64), want)


def test_ties_go_to_even():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: even mantissa wins (1)
    assert round_bf16_ref(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert round_bf16_ref(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6


def test_small_inputs_deterministic_and_shaped():
    w = wl.WORKLOADS[1]
    segs = wl.small_layout("image", 16, 1, 8, 8)
    a = wl.make_inputs(w, segments=segs)
    b = wl.make_inputs(w, segments=segs)
    T = 16 + 64
    assert a["x"].shape == (1, T, 3 * 16 * 128)
    assert a["alpha"].shape == (1, T, 16, 128) and a["beta"].shape == (1, T, 16)
    for key in ("x", "alpha", "beta", "w_text", "w_vis"):
        np.testing.assert_array_equal(a[key], b[key])
    for key in ("x", "alpha", "beta"):
        assert (a[key].view(np.uint32) & 0xFFFF == 0).all()        # bf16-representable
    assert (a["alpha"] > 0).all() and (a["alpha"] <= 1).all()
    assert (a["beta"] > 0).all() and (a["beta"] < 1).all()


def test_workload_sizes():
    T = [w.T for w in wl.WORKLOADS]
    assert T == [256, 4352, 65792, 37888, 255406, 62796]
    assert wl.WORKLOADS[3].B == 2 and wl.WORKLOADS[3].s0_std == 0.1
    assert wl.WORKLOADS[0].dtype == "f32" and wl.WORKLOADS[0].d == 32


def test_packed_workload_layout():
    """The packed row: 40 samples, each a text segment then an image grid, the sample offsets
    on the text starts, segments tiling the row."""
    w = wl.WORKLOADS[5]
    cu = w.samples
    assert len(cu) == 41 and cu[0] == 0 and cu[-1] == w.T
    segs = w.segments
    assert len(segs) == 80
    for n in range(40):
        t, g = segs[2 * n], segs[2 * n + 1]
        assert t.kind == wl.TEXT and t.start == cu[n] and 32 <= t.length <= 300
        assert g.kind == wl.IMAGE and g.start == t.start + t.length and g.start + g.length == cu[n + 1]
        assert g.height == g.width and g.height in (16, 32, 64)
    sides = [segs[2 * n + 1].height for n in range(8)]
    assert sides == [16, 16, 16, 16, 32, 32, 64, 64]                 # 4:2:2 per group of eight
