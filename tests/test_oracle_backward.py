"""Pins for the backward oracle (CPU only).

The torch restatements of the forward steps are checked against the numpy
oracle (``kda_ref``, ``conv_ref``, pinned elsewhere); the autograd gradients
are checked against central finite differences of the numpy forward (fp64,
random directions), which shares no code with torch's reverse mode, and
against closed forms (no write: dv = dk = 0, dS0 = sum_t q_t do_t^T; identity
conv: dx = dy).
"""
import numpy as np
import torch

import workloads as wl
from oracle import conv_ref, kda_ref, l2norm_ref
from oracle.backward import conv_backward_ref, conv_torch, kda_backward_ref, kda_torch


def _inputs(rng, B=1, T=9, H=2, dk=4, dv=3):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    alpha = np.exp(-np.logaddexp(0, rng.standard_normal((B, T, H, dk))))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    S0 = rng.standard_normal((B, H, dk, dv))
    return q, k, v, alpha, beta, S0


def _loss_np(q, k, v, alpha, beta, S0, do, dS):
    o, S = kda_ref(l2norm_ref(q), l2norm_ref(k), v, alpha, beta, S0)
    return float((o * do).sum() + (S * dS).sum())


def test_torch_restatement_matches_the_numpy_oracle():
    rng = np.random.default_rng(90)
    q, k, v, alpha, beta, S0 = _inputs(rng)
    f = lambda a: torch.tensor(a, dtype=torch.float64)
    o, S = kda_torch(*(f(a) for a in (q, k, v, alpha, beta, S0)))
    o2, S2 = kda_ref(q, k, v, alpha, beta, S0)
    np.testing.assert_allclose(o.numpy(), o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S.numpy(), S2, rtol=1e-12, atol=1e-13)
    segs = wl.text_then_grid(5, 3, 3, 4)
    x = rng.standard_normal((2, 41, 8))
    wt, wv = rng.standard_normal((8, 4)), rng.standard_normal((8, 27))
    np.testing.assert_allclose(conv_torch(f(x), f(wt), f(wv), segs).numpy(), conv_ref(x, wt, wv, segs), rtol=1e-12,
                               atol=1e-13)


def test_kda_gradients_match_finite_differences():
    rng = np.random.default_rng(91)
    q, k, v, alpha, beta, S0 = _inputs(rng)
    do = rng.standard_normal(v.shape)
    dS = rng.standard_normal(S0.shape)
    g = kda_backward_ref(q, k, v, alpha, beta, S0, do, dS)
    args = [q, k, v, alpha, beta, S0]
    names = ["dq", "dk", "dv", "dalpha", "dbeta", "dS0"]
    h = 1e-6
    for i, name in enumerate(names):
        for _ in range(3):
            e = rng.standard_normal(args[i].shape)
            plus = [a + h * e if j == i else a for j, a in enumerate(args)]
            minus = [a - h * e if j == i else a for j, a in enumerate(args)]
            fd = (_loss_np(*plus, do, dS) - _loss_np(*minus, do, dS)) / (2 * h)
            np.testing.assert_allclose((g[name] * e).sum(), fd, rtol=2e-6, atol=1e-8, err_msg=name)


def test_conv_gradients_match_finite_differences():
    rng = np.random.default_rng(92)
    segs = wl.text_then_grid(6, 3, 3, 4) + (wl.Segment(wl.IMAGE, 42, 12, 1, 3, 4),)
    T = 54
    x = rng.standard_normal((2, T, 8))
    wt, wv = rng.standard_normal((8, 4)), rng.standard_normal((8, 27))
    dy = rng.standard_normal(x.shape)
    g = conv_backward_ref(x, wt, wv, segs, dy)
    loss = lambda x_, wt_, wv_: float((conv_ref(x_, wt_, wv_, segs) * dy).sum())
    h = 1e-6
    for name, i in (("dx", 0), ("dw_text", 1), ("dw_vis", 2)):
        args = [x, wt, wv]
        e = rng.standard_normal(args[i].shape)
        plus = [a + h * e if j == i else a for j, a in enumerate(args)]
        minus = [a - h * e if j == i else a for j, a in enumerate(args)]
        fd = (loss(*plus) - loss(*minus)) / (2 * h)
        np.testing.assert_allclose((g[name] * e).sum(), fd, rtol=1e-7, atol=1e-8, err_msg=name)


def test_no_write_closed_form():
    """beta = 0, alpha = 1: o_t = S0^T q^_t, so dv = dk = 0, dS0 = sum_t q^_t do_t^T and
    dq_t = (S0 do_t) pulled back through the norm."""
    rng = np.random.default_rng(93)
    q, k, v, _, _, S0 = _inputs(rng, T=7)
    alpha = np.ones_like(k)
    beta = np.zeros(k.shape[:3])
    do = rng.standard_normal(v.shape)
    g = kda_backward_ref(q, k, v, alpha, beta, S0, do, None)
    assert np.array_equal(g["dv"], np.zeros_like(v)) and np.abs(g["dk"]).max() < 1e-15
    qn = l2norm_ref(q)
    np.testing.assert_allclose(g["dS0"], np.einsum("bthk,bthv->bhkv", qn, do), rtol=1e-13)


def test_identity_conv_passes_the_gradient_through():
    rng = np.random.default_rng(94)
    segs = wl.text_then_grid(5, 2, 3, 3)
    x = rng.standard_normal((1, 23, 8))
    wt = np.zeros((8, 4)); wt[:, 3] = 1.0
    wv = np.zeros((8, 27)); wv[:, 2 * 9 + 1 * 3 + 1] = 1.0
    dy = rng.standard_normal(x.shape)
    g = conv_backward_ref(x, wt, wv, segs, dy)
    np.testing.assert_array_equal(g["dx"], dy)


def test_gate_norm_restatement_and_gradients():
    """The torch restatement equals the numpy gated_rmsnorm_ref; its gradients match central
    differences of the numpy function; with a constant row and no gain the norm's gradient is
    the closed form do = s (dy - mean(dy)) / |c| (c the constant, s = Sigmoid(gate))."""
    from oracle import gated_rmsnorm_ref
    from oracle.backward import gate_norm_backward_ref, gated_rmsnorm_torch
    rng = np.random.default_rng(95)
    o, g = rng.standard_normal((3, 2, 12)), rng.standard_normal((3, 2, 12))
    w, dy = 1 + 0.1 * rng.standard_normal(12), rng.standard_normal((3, 2, 12))
    f = lambda a: torch.tensor(a, dtype=torch.float64)
    np.testing.assert_allclose(gated_rmsnorm_torch(f(o), f(g), f(w), 1e-6).numpy(), gated_rmsnorm_ref(o, g, w, 1e-6),
                               rtol=1e-13, atol=1e-14)
    got = gate_norm_backward_ref(o, g, w, dy, 1e-6)
    loss = lambda o_, g_, w_: float((gated_rmsnorm_ref(o_, g_, w_, 1e-6) * dy).sum())
    h = 1e-6
    for name, i in (("do", 0), ("dgate", 1), ("dweight", 2)):
        args = [o, g, w]
        e = rng.standard_normal(args[i].shape)
        plus = [a + h * e if j == i else a for j, a in enumerate(args)]
        minus = [a - h * e if j == i else a for j, a in enumerate(args)]
        fd = (loss(*plus) - loss(*minus)) / (2 * h)
        np.testing.assert_allclose((got[name] * e).sum(), fd, rtol=1e-7, atol=1e-9, err_msg=name)
    c, gc = -2.5, rng.standard_normal((1, 8))
    dyc = rng.standard_normal((1, 8))
    r = gate_norm_backward_ref(np.full((1, 8), c), gc, None, dyc, 0.0)
    s = 1 / (1 + np.exp(-gc))
    # y = s * sign(c): dy . dy/do_j = s_j dy_j / |c| - sign(c) sum_i s_i dy_i sign(c) / (8 |c|)
    want = (s * dyc - (s * dyc).sum() / 8) / abs(c)
    np.testing.assert_allclose(r["do"], want, rtol=1e-12)
