"""GPU parity of the fused conv + recurrence (chimera_kda_fwd_conv): q|k|v computed from x
in the recurrence's load stage and never stored, on the token-by-token kernel and on the
chunked MFMA kernels, against the oracle chain conv_ref -> rounding to the storage type ->
L2 norm -> kda_ref, and against the two-call path (conv, then the recurrence on the stored
q|k|v)."""
import numpy as np
import pytest

import workloads as wl
from oracle import conv_ref, kda_ref, l2norm_ref, round_bf16_ref
from tests.gpu_util import assert_close, rel_l2, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def chm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_recurrence_mshortconv_amd as m
    m.lib()
    return m


def _case(rng, B, T, H, dk, dv, dtype, with_s0):
    rnd = (lambda a: wl.round_to_bf16(a.astype(np.float32))) if dtype == "bf16" else (lambda a: a.astype(np.float32))
    C = H * (2 * dk + dv)
    x = rnd(rng.standard_normal((B, T, C)))
    wt = (0.5 * rng.standard_normal((C, 4))).astype(np.float32)
    wv = (0.5 * rng.standard_normal((C, 27))).astype(np.float32)
    alpha = rnd(np.exp(-0.05 * np.logaddexp(0, rng.standard_normal((B, T, H, dk)))))
    beta = rnd(1 / (1 + np.exp(-rng.standard_normal((B, T, H)))))
    S0 = (0.1 * rng.standard_normal((B, H, dk, dv))).astype(np.float32) if with_s0 else None
    return x, wt, wv, alpha, beta, S0


def _oracle(x, wt, wv, segs, alpha, beta, S0, H, dk, dv, dtype):
    y = conv_ref(x, wt, wv, segs)
    if dtype == "bf16":
        y = round_bf16_ref(y)
    B, T = x.shape[:2]
    q = y[..., :H * dk].reshape(B, T, H, dk)
    k = y[..., H * dk:2 * H * dk].reshape(B, T, H, dk)
    v = y[..., 2 * H * dk:].reshape(B, T, H, dv)
    return kda_ref(l2norm_ref(q), l2norm_ref(k), v, alpha, beta, S0)


def _fused(chm, x, wt, wv, segs, alpha, beta, S0, H, dk, dv, dtype, **kw):
    import torch
    s0 = None if S0 is None else torch.from_numpy(S0).cuda()
    return chm.kda_fwd_conv(to_device(x, dtype), torch.from_numpy(wt).cuda(), torch.from_numpy(wv).cuda(), segs,
                            to_device(alpha, dtype), to_device(beta, dtype), s0, H=H, dk=dk, dv=dv, **kw)


def test_fused_text_fp32_tiny(chm):
    """The tiny text workload's shapes: fp32, 256 text tokens, two 32-wide heads."""
    rng = np.random.default_rng(140)
    segs = (wl.Segment(wl.TEXT, 0, 256),)
    args = _case(rng, 1, 256, 2, 32, 32, "f32", False)
    o, Sf = _fused(chm, *args[:3], segs, *args[3:], 2, 32, 32, "f32")
    o_ref, S_ref = _oracle(*args[:3], segs, *args[3:], 2, 32, 32, "f32")
    assert_close(to_host(o), o_ref, "f32", "o")
    assert_close(to_host(Sf), S_ref, "f32", "S_final")


def test_fused_mixed_layout_bf16(chm):
    """Text, image, text, video segments (the video's first frames read zero in time), two
    batch items with their own S0, dk = 32, dv = 40 (a partial 16-column slice)."""
    S = wl.Segment
    segs = (S(wl.TEXT, 0, 9), S(wl.IMAGE, 9, 7 * 6, 1, 7, 6), S(wl.TEXT, 51, 3), S(wl.VIDEO, 54, 3 * 4 * 5, 3, 4, 5))
    rng = np.random.default_rng(141)
    H, dk, dv = 2, 32, 40
    args = _case(rng, 2, 114, H, dk, dv, "bf16", True)
    o, Sf = _fused(chm, *args[:3], segs, *args[3:], H, dk, dv, "bf16")
    o_ref, S_ref = _oracle(*args[:3], segs, *args[3:], H, dk, dv, "bf16")
    assert_close(to_host(o), o_ref, "bf16", "o")
    assert_close(to_host(Sf), S_ref, "bf16", "S_final")


def test_fused_image_d128_matches_two_calls(chm):
    """The token-by-token fused kernel at d = 128, the image_1024 layout (256 text + 64 x 64
    image) on two heads: against the oracle, and against the two-call path (conv, then the
    token-by-token recurrence)."""
    import torch
    rng = np.random.default_rng(142)
    segs = wl.text_then_grid(256, 1, 64, 64)
    H, d, T = 2, 128, 256 + 64 * 64
    x, wt, wv, alpha, beta, S0 = _case(rng, 1, T, H, d, d, "bf16", False)
    o, Sf = _fused(chm, x, wt, wv, segs, alpha, beta, S0, H, d, d, "bf16", sequential=True)
    o_ref, S_ref = _oracle(x, wt, wv, segs, alpha, beta, S0, H, d, d, "bf16")
    assert_close(to_host(o), o_ref, "bf16", "o")
    assert_close(to_host(Sf), S_ref, "bf16", "S_final")
    y = chm.mshortconv_fwd(to_device(x, "bf16"), torch.from_numpy(wt).cuda(), torch.from_numpy(wv).cuda(), segs)
    o2, S2 = chm.kda_fwd(*chm.split_qkv(y, H, d), to_device(alpha, "bf16"), to_device(beta, "bf16"), None,
                         sequential=True)
    assert rel_l2(to_host(o), to_host(o2)) <= 1e-3 and rel_l2(to_host(Sf), to_host(S2)) <= 1e-3


# ---- the chunked MFMA kernels with the conv in their load stage (bf16, d = 128) ----------

def _layouts_chunked():
    S = wl.Segment
    return {
        # every kind in one row; ragged grids against the 64-token chunks; the video's first two
        # frames read zero in time
        "mixed": (S(wl.TEXT, 0, 19), S(wl.IMAGE, 19, 37 * 45, 1, 37, 45), S(wl.TEXT, 19 + 1665, 5),
                  S(wl.VIDEO, 1689, 5 * 19 * 23, 5, 19, 23)),
        "text_image": wl.text_then_grid(256, 1, 24, 40),
        "video2": (S(wl.VIDEO, 0, 2 * 8 * 9, 2, 8, 9), S(wl.TEXT, 144, 70)),   # two frames: kt = 1, 2 only
        "one_chunk": (S(wl.TEXT, 0, 37),),
        "one_token": (S(wl.IMAGE, 0, 1, 1, 1, 1),),
    }


def _dev_case(chm, rng, B, T, H, d, with_s0):
    import torch
    x, wt, wv, alpha, beta, S0 = _case(rng, B, T, H, d, d, "bf16", with_s0)
    dev = dict(x=to_device(x, "bf16"), wt=torch.from_numpy(wt).cuda(), wv=torch.from_numpy(wv).cuda(),
               al=to_device(alpha, "bf16"), be=to_device(beta, "bf16"),
               s0=None if S0 is None else torch.from_numpy(S0).cuda())
    return (x, wt, wv, alpha, beta, S0), dev


def _two_calls(chm, dv, segs, H, d, **kw):
    y = chm.mshortconv_fwd(dv["x"], dv["wt"], dv["wv"], segs)
    return chm.kda_fwd(*chm.split_qkv(y, H, d), dv["al"], dv["be"], dv["s0"], **kw)


@pytest.mark.parametrize("name,B,with_s0,no_split", [
    ("mixed", 2, True, False), ("mixed", 1, False, True), ("text_image", 2, False, False),
    ("video2", 2, True, False), ("one_chunk", 2, True, False), ("one_token", 1, True, False),
])
def test_fused_chunked_equals_two_calls_bit_for_bit(chm, name, B, with_s0, no_split):
    """The conv in the chunked kernels' load stage sums the taps in the conv kernels' order and
    rounds once, so o and S_final equal the two-call path (conv, then the chunked recurrence on
    the stored q|k|v) bit for bit: split into one-chunk segments (small inputs on the chip's
    256 blocks) and unsplit (one block runs the whole sequence)."""
    import torch
    segs = _layouts_chunked()[name]
    T = sum(s.length for s in segs)
    H, d = 2, 128
    rng = np.random.default_rng(150 + len(name) + B)
    host, dv = _dev_case(chm, rng, B, T, H, d, with_s0)
    print(f"fused chunked {name}: B={B} T={T} no_split={no_split}", flush=True)
    marks = chm.Marks(8)
    o1, S1 = chm.kda_fwd_conv(dv["x"], dv["wt"], dv["wv"], segs, dv["al"], dv["be"], dv["s0"], H=H, dk=d, dv=d,
                              no_split=no_split, marks=marks)
    torch.cuda.synchronize()
    names = [n for n, _ in marks.kernels()]
    assert "kda_out_conv_kernel" in names, names   # the chunked path ran
    o2, S2 = _two_calls(chm, dv, segs, H, d, no_split=no_split)
    assert torch.equal(o1, o2), f"o differs at {torch.nonzero(o1 != o2)[:3].tolist()}"
    assert torch.equal(S1, S2)


def test_fused_chunked_mixed_vs_oracle(chm):
    """The chunked fused path on the mixed layout (two batch items, S0) against the oracle."""
    segs = _layouts_chunked()["mixed"]
    T = sum(s.length for s in segs)
    H, d = 2, 128
    rng = np.random.default_rng(160)
    args = _case(rng, 2, T, H, d, d, "bf16", True)
    o, Sf = _fused(chm, *args[:3], segs, *args[3:], H, d, d, "bf16")
    o_ref, S_ref = _oracle(*args[:3], segs, *args[3:], H, d, d, "bf16")
    assert_close(to_host(o), o_ref, "bf16", "o")
    assert_close(to_host(Sf), S_ref, "bf16", "S_final")


@pytest.mark.parametrize("wi", [2, 3])
def test_fused_chunked_full_size(chm, wi):
    """image_4096 and video_5s at full size in the bench's launch configuration: the fused call
    equals the two calls bit for bit on every head; a middle head against the oracle."""
    import torch
    w = wl.WORKLOADS[wi]
    inp = wl.make_inputs(w)
    print(f"fused chunked full size {w.name}", flush=True)
    x = to_device(inp["x"], "bf16")
    wt, wv = torch.from_numpy(inp["w_text"]).cuda(), torch.from_numpy(inp["w_vis"]).cuda()
    al, be = to_device(inp["alpha"], "bf16"), to_device(inp["beta"], "bf16")
    s0 = None if inp["S0"] is None else torch.from_numpy(inp["S0"]).cuda()
    segs = inp["segments"]
    o1, S1 = chm.kda_fwd_conv(x, wt, wv, segs, al, be, s0, H=w.H, dk=w.d, dv=w.d)
    y = chm.mshortconv_fwd(x, wt, wv, segs)
    o2, S2 = chm.kda_fwd(*chm.split_qkv(y, w.H, w.d), al, be, s0)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    head = w.H // 2 - 1
    o_got, S_got = to_host(o1[:, :, [head]]), to_host(S1[:, [head]])
    del x, y, o1, o2, S1, S2
    HD = w.H * w.d
    chans = np.concatenate([part * HD + head * w.d + np.arange(w.d) for part in range(3)])
    y_ref = round_bf16_ref(conv_ref(inp["x"][:, :, chans], inp["w_text"][chans], inp["w_vis"][chans], segs))
    parts = y_ref.reshape(w.B, w.T, 3, 1, w.d)
    S0 = None if inp["S0"] is None else inp["S0"][:, [head]]
    o_ref, S_ref = kda_ref(l2norm_ref(parts[:, :, 0]), l2norm_ref(parts[:, :, 1]), parts[:, :, 2],
                           inp["alpha"][:, :, [head]], inp["beta"][:, :, [head]], S0)
    assert_close(o_got, o_ref, "bf16", f"{w.name} o")
    assert_close(S_got, S_ref, "bf16", f"{w.name} S_final")
