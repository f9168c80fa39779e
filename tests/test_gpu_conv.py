"""GPU parity of mShortConv and its device neighbour arithmetic (through the C ABI)."""
import numpy as np
import pytest

import workloads as wl
from oracle import neighbours_ref, conv_ref
from tests.gpu_util import assert_rel_l2, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def chm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_recurrence_mshortconv_amd as m
    m.lib()
    return m


def _mixed_layout():
    # every kind; grids with ragged edges against the 8x32 / 8x16 tiles
    S = wl.Segment
    return (S(wl.TEXT, 0, 19), S(wl.IMAGE, 19, 37 * 45, 1, 37, 45), S(wl.TEXT, 19 + 1665, 5),
            S(wl.VIDEO, 1689, 5 * 19 * 23, 5, 19, 23))


def _layouts():
    out = [_mixed_layout()] + [w.segments for w in wl.WORKLOADS]
    S = wl.Segment
    out.append((S(wl.VIDEO, 0, 1 * 1 * 1, 1, 1, 1),))                  # a one-token video
    out.append((S(wl.IMAGE, 0, 1 * 70, 1, 1, 70), S(wl.TEXT, 70, 1)))  # one-row image, one-token text
    return out


def test_device_neighbour_arithmetic_bit_exact(chm):
    for segs in _layouts():
        T = sum(s.length for s in segs)
        got = chm.mshortconv_index_device(segs, T).cpu().numpy()
        assert np.array_equal(got, neighbours_ref(segs, T)), segs[:2]


def _position_code(B, T, C):
    """x[b, p, c] = digit (c mod 3) of b*T + p in base 256, plus 1: integers 1..256, exact in bf16
    and fp32, so that a conv with a single unit tap copies its source token's code unchanged
    (zero padding reads as 0, which no code takes)."""
    pos = np.arange(B * T, dtype=np.int64).reshape(B, T, 1)
    digit = np.arange(C) % 3
    return ((pos >> (8 * digit)) & 255).astype(np.float32) + 1.0


def _decode(y):
    """Source token (b*T + p) of every output row from its first three channels, -1 for all-zero
    rows; every channel must carry the code of the same source."""
    y = np.asarray(y, dtype=np.float64)
    C = y.shape[-1]
    assert np.array_equal(y, y[..., np.arange(C) % 3]), "channels of one row gathered different sources"
    d = y[..., :3].astype(np.int64)
    zero = (d == 0).all(-1)
    assert ((d >= 1) | zero[..., None]).all(), "partly padded row"
    src = (d[..., 0] - 1) + ((d[..., 1] - 1) << 8) + ((d[..., 2] - 1) << 16)
    return np.where(zero, -1, src)


@pytest.mark.parametrize("dtype,C,kernels", [
    ("bf16", 64, {"conv_text_kernel", "conv_rows_kernel", "conv_tile_kernel"}),
    ("bf16", 72, {"conv_text_kernel", "conv_gather_kernel"}),
    ("f32", 64, {"conv_text_kernel", "conv_gather_kernel"}),
])
def test_conv_gathers_bit_exact_one_hot(chm, dtype, C, kernels):
    """The taps the product conv kernels actually read, bit for bit: for each tap, weights that are
    1 on that tap and 0 elsewhere make y a copy of the tap's source token (Eq. 13 with a one-hot
    kernel), and the inputs encode every token's position exactly, so decoding y gives the
    neighbour table each kernel used. Compared with neighbours_ref (Eq. 12 raster order, zero
    padding at segment edges, causal in time) for all 4 text and 27 visual taps, two batch items."""
    import torch
    S = wl.Segment
    segs = _mixed_layout() + (S(wl.IMAGE, 1689 + 5 * 19 * 23, 1 * 70, 1, 1, 70),)
    T = sum(s.length for s in segs)
    B = 2
    table = neighbours_ref(segs, T)
    is_text = np.zeros(T, dtype=bool)
    for sg in segs:
        if sg.kind == wl.TEXT:
            is_text[sg.start:sg.start + sg.length] = True
    x = to_device(_position_code(B, T, C), dtype)
    ran = set()
    for part, ntaps in (("text", 4), ("vis", 27)):
        for j in range(ntaps):
            wt = np.zeros((C, 4), np.float32)
            wv = np.zeros((C, 27), np.float32)
            (wt if part == "text" else wv)[:, j] = 1.0
            marks = chm.Marks(len(segs) + 1)
            y = chm.mshortconv_fwd(x, torch.from_numpy(wt), torch.from_numpy(wv), segs, marks=marks)
            torch.cuda.synchronize()
            ran |= {n for n, _ in marks.kernels()}
            got = _decode(to_host(y))
            mine = is_text if part == "text" else ~is_text
            want = np.where(mine, table[:, j], -1)
            for b in range(B):
                exp_b = np.where(want >= 0, want + b * T, -1)
                bad = np.nonzero(got[b] != exp_b)[0]
                assert bad.size == 0, (f"{part} tap {j}, batch {b}: token {bad[0]} read {got[b][bad[0]]}, "
                                       f"expected {exp_b[bad[0]]}")
    assert ran == kernels, ran


def _conv_bound(x, wt, wv, segs, dtype):
    """Element-wise error bound: fp32 accumulation of up to 27 terms plus one
    rounding to the output dtype (half an ulp: 2^-8 relative for bf16, 2^-24 for fp32)."""
    ref = conv_ref(x, wt, wv, segs)
    mag = conv_ref(np.abs(x), np.abs(wt), np.abs(wv), segs)
    unit = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -24
    return ref, unit * np.abs(ref) + 28 * 2.0 ** -24 * mag + 1e-30


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("C", [64, 192])
def test_conv_parity_mixed_layout(chm, dtype, C):
    segs = _mixed_layout()
    T = sum(s.length for s in segs)
    rng = np.random.default_rng(C)
    x = rng.standard_normal((2, T, C)).astype(np.float32)
    if dtype == "bf16":
        x = wl.round_to_bf16(x)
    wt = (0.5 * rng.standard_normal((C, 4))).astype(np.float32)
    wv = (0.5 * rng.standard_normal((C, 27))).astype(np.float32)
    import torch
    y = chm.mshortconv_fwd(to_device(x, dtype), torch.from_numpy(wt), torch.from_numpy(wv), segs)
    got = to_host(y)
    ref, bound = _conv_bound(x, wt, wv, segs, dtype)
    err = np.abs(got - ref)
    assert (err <= bound).all(), f"worst excess {np.max(err - bound):.3e}"
    assert_rel_l2(got, ref, dtype, "conv")


def test_conv_centred_delta_is_identity_on_gpu(chm):
    import torch
    segs = _mixed_layout()
    T = sum(s.length for s in segs)
    C = 128
    x = wl.round_to_bf16(np.random.default_rng(3).standard_normal((1, T, C)).astype(np.float32))
    wt = np.zeros((C, 4), np.float32); wt[:, 3] = 1
    wv = np.zeros((C, 27), np.float32); wv[:, 22] = 1
    y = chm.mshortconv_fwd(to_device(x, "bf16"), torch.from_numpy(wt), torch.from_numpy(wv), segs)
    assert np.array_equal(to_host(y), x.astype(np.float64))


@pytest.mark.parametrize("wi", [1, 2, 3, 4])
def test_conv_full_workload_sampled_channels(chm, wi):
    """Full-size workloads in the bench's launch configuration; the oracle recomputes every channel
    of a middle head's q, k and v blocks and every 4th channel of the first and last heads'."""
    import torch
    w = wl.WORKLOADS[wi]
    inp = wl.make_inputs(w)
    x = inp["x"]
    segs = inp["segments"]
    y = chm.mshortconv_fwd(to_device(x, "bf16"), torch.from_numpy(inp["w_text"]), torch.from_numpy(inp["w_vis"]), segs)
    HD = w.H * w.d
    mid = w.H // 2 - 1
    edge = np.concatenate([part * HD + h * w.d + np.arange(w.d) for part in range(3) for h in (0, w.H - 1)])
    full = np.concatenate([part * HD + mid * w.d + np.arange(w.d) for part in range(3)])
    sub = np.sort(np.concatenate([edge[::4], full]))
    got = to_host(y[:, :, torch.from_numpy(sub).to(y.device)])
    ref, bound = _conv_bound(x[:, :, sub], inp["w_text"][sub], inp["w_vis"][sub], segs, "bf16")
    err = np.abs(got - ref)
    assert (err <= bound).all(), f"worst excess {np.max(err - bound):.3e}"
    assert_rel_l2(got, ref, "bf16", w.name)


@pytest.mark.parametrize("height,kernel", [(2, "conv_tile_kernel"), (4, "conv_gather_kernel")])
def test_conv_wide_grid_fallbacks(chm, height, kernel):
    """A 4096-wide image with 65,536 channels. The rows kernel's buffers (six staged
    rows) would pass 2 GiB, so at height 2 the frame-tile kernel runs; at height 4 a
    whole frame passes 2 GiB as well and the gather kernel runs. Sampled channels
    (every token) against the oracle."""
    import torch
    W, C = 4096, 65536
    segs = (wl.Segment(wl.IMAGE, 0, height * W, 1, height, W),)
    T = height * W
    g = torch.Generator(device="cuda")
    g.manual_seed(11 + height)
    x = torch.randn(1, T, C, device="cuda", generator=g).to(torch.bfloat16)
    rng = np.random.default_rng(height)
    wt = (0.5 * rng.standard_normal((C, 4))).astype(np.float32)
    wv = (0.5 * rng.standard_normal((C, 27))).astype(np.float32)
    marks = chm.Marks(2)
    y = chm.mshortconv_fwd(x, torch.from_numpy(wt), torch.from_numpy(wv), segs, marks=marks)
    torch.cuda.synchronize()
    assert [n for n, _ in marks.kernels()] == [kernel]
    sub = np.unique(np.concatenate([np.arange(0, C, C // 16) + np.arange(16) * 37, [C - 1]]))
    idx = torch.from_numpy(sub).to("cuda")
    got = to_host(y[:, :, idx])
    xs = to_host(x[:, :, idx])
    del x, y
    ref, bound = _conv_bound(xs, wt[sub], wv[sub], segs, "bf16")
    err = np.abs(got - ref)
    assert (err <= bound).all(), f"worst excess {np.max(err - bound):.3e}"
    assert_rel_l2(got, ref, "bf16", f"wide grid h={height}")
