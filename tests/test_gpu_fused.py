"""GPU parity of the fused conv + recurrence (chimera_kda_fwd_conv): q|k|v computed from x
inside the token-by-token kernel's load stage, never stored, against the oracle chain
conv_ref -> rounding to the storage type -> L2 norm -> kda_ref."""
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


def _fused(chm, x, wt, wv, segs, alpha, beta, S0, H, dk, dv, dtype):
    import torch
    s0 = None if S0 is None else torch.from_numpy(S0).cuda()
    return chm.kda_fwd_conv(to_device(x, dtype), torch.from_numpy(wt).cuda(), torch.from_numpy(wv).cuda(), segs,
                            to_device(alpha, dtype), to_device(beta, dtype), s0, H=H, dk=dk, dv=dv)


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
    """d = 128, the image_1024 layout (256 text + 64 x 64 image) on two heads: against the
    oracle, and against the two-call path (conv, then the token-by-token recurrence)."""
    import torch
    rng = np.random.default_rng(142)
    segs = wl.text_then_grid(256, 1, 64, 64)
    H, d, T = 2, 128, 256 + 64 * 64
    x, wt, wv, alpha, beta, S0 = _case(rng, 1, T, H, d, d, "bf16", False)
    o, Sf = _fused(chm, x, wt, wv, segs, alpha, beta, S0, H, d, d, "bf16")
    o_ref, S_ref = _oracle(x, wt, wv, segs, alpha, beta, S0, H, d, d, "bf16")
    assert_close(to_host(o), o_ref, "bf16", "o")
    assert_close(to_host(Sf), S_ref, "bf16", "S_final")
    y = chm.mshortconv_fwd(to_device(x, "bf16"), torch.from_numpy(wt).cuda(), torch.from_numpy(wv).cuda(), segs)
    o2, S2 = chm.kda_fwd(*chm.split_qkv(y, H, d), to_device(alpha, "bf16"), to_device(beta, "bf16"), None,
                         sequential=True)
    assert rel_l2(to_host(o), to_host(o2)) <= 1e-3 and rel_l2(to_host(Sf), to_host(S2)) <= 1e-3
