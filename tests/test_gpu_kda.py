"""GPU parity of the KDA forward (through the C ABI) against the fp64 oracle."""
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


def _split(x, B, T, H, d):
    parts = x.reshape(B, T, 3, H, d)
    return parts[:, :, 0], parts[:, :, 1], parts[:, :, 2]


def _oracle_kda(x, alpha, beta, S0, B, T, H, d, heads=None):
    q, k, v = _split(x, B, T, H, d)
    sel = slice(None) if heads is None else heads
    q, k, v = l2norm_ref(q[:, :, sel]), l2norm_ref(k[:, :, sel]), v[:, :, sel]
    a, b = alpha[:, :, sel], beta[:, :, sel]
    s0 = None if S0 is None else S0[:, sel]
    return kda_ref(q, k, v, a, b, s0)


def _run_kda(chm, x_dev, alpha, beta, S0, w, **kw):
    import torch
    B, T = x_dev.shape[:2]
    q, k, v = chm.split_qkv(x_dev, w.H, w.d)
    a = to_device(alpha, w.dtype)
    b = to_device(beta, w.dtype)
    s0 = None if S0 is None else torch.from_numpy(S0).cuda()
    return chm.kda_fwd(q, k, v, a, b, s0, l2norm=True, **kw)


def test_tiny_text_fp32_pipeline(chm):
    """The fp32 text workload end to end: conv then KDA, against the oracle pipeline."""
    import torch
    w = wl.WORKLOADS[0]
    inp = wl.make_inputs(w)
    x_dev = to_device(inp["x"], "f32")
    y = chm.mshortconv_fwd(x_dev, torch.from_numpy(inp["w_text"]), torch.from_numpy(inp["w_vis"]), inp["segments"])
    o, Sf = _run_kda(chm, y, inp["alpha"], inp["beta"], inp["S0"], w)
    y_ref = conv_ref(inp["x"], inp["w_text"], inp["w_vis"], inp["segments"])
    o_ref, S_ref = _oracle_kda(y_ref, inp["alpha"], inp["beta"], inp["S0"], w.B, w.T, w.H, w.d)
    assert_close(to_host(y), y_ref, "f32", "conv")
    assert_close(to_host(o), o_ref, "f32", "o")
    assert_close(to_host(Sf), S_ref, "f32", "S_final")


@pytest.mark.parametrize("sequential", [True, False])
def test_kda_bf16_small(chm, sequential):
    """bf16 inputs, fp32 state, d=128, several chunks and a ragged tail, nonzero S0."""
    w = wl.WORKLOADS[3]
    T = 64 * 5 + 23
    segs = wl.small_layout("text", T)
    inp = wl.make_inputs(w, segments=segs, seed=11)
    S0 = inp["S0"]
    x_dev = to_device(inp["x"], "bf16")
    o, Sf = _run_kda(chm, x_dev, inp["alpha"], inp["beta"], S0, w, sequential=sequential)
    o_ref, S_ref = _oracle_kda(inp["x"], inp["alpha"], inp["beta"], S0, w.B, T, w.H, w.d, heads=[0, 5, 15])
    got_o = to_host(o)[:, :, [0, 5, 15]]
    got_S = to_host(Sf)[:, [0, 5, 15]]
    assert_close(got_o, o_ref, "bf16", "o")
    assert_close(got_S, S_ref, "bf16", "S_final")


def test_kda_fp32_small_dims(chm):
    """fp32, odd head dims (dk != dv, not multiples of 16), several batch items."""
    rng = np.random.default_rng(5)
    B, T, H, dk, dv = 2, 77, 3, 20, 37
    q = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    alpha = np.exp(-np.logaddexp(0, rng.standard_normal((B, T, H, dk)))).astype(np.float32)
    beta = (1 / (1 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32)
    S0 = (0.1 * rng.standard_normal((B, H, dk, dv))).astype(np.float32)
    import torch
    o, Sf = chm.kda_fwd(*(torch.from_numpy(a).cuda() for a in (q, k, v, alpha, beta, S0)), l2norm=True)
    o_ref, S_ref = kda_ref(l2norm_ref(q), l2norm_ref(k), v, alpha, beta, S0)
    assert_close(to_host(o), o_ref, "f32", "o")
    assert_close(to_host(Sf), S_ref, "f32", "S_final")


def test_kda_empty_sequence_copies_state(chm):
    import torch
    B, H, d = 1, 2, 128
    S0 = torch.randn(B, H, d, d, device="cuda")
    e = torch.empty(B, 0, H, d, dtype=torch.bfloat16, device="cuda")
    o, Sf = chm.kda_fwd(e, e, e, e, torch.empty(B, 0, H, dtype=torch.bfloat16, device="cuda"), S0)
    assert o.shape == (B, 0, H, d)
    assert torch.equal(Sf, S0)
