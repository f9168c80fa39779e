"""GPU parity of the backward pass (chimera_kda_bwd, chimera_kda_bwd_varlen,
chimera_gate_norm_bwd, chimera_mshortconv_bwd) against the fp64 autograd oracle
(oracle.backward)."""
import numpy as np
import pytest

import workloads as wl
from oracle import kda_ref, l2norm_ref
from oracle.backward import conv_backward_ref, gate_norm_backward_ref, kda_backward_ref
from tests.gpu_util import assert_close, rel_l2, to_device, to_host

pytestmark = pytest.mark.gpu

# bf16 storage of the inputs and of the gradients: each gradient tensor within rel-L2 2e-2 of
# the fp64 gradient of the same (bf16-valued) inputs, and every element within 2% of the
# tensor's largest magnitude (one bf16 rounding is 2^-9 relative; the rest is fp32 reduction
# order over d and over the sequence)
BF16_BWD_REL_L2 = 2e-2
BF16_BWD_MAX_REL = 2e-2


def _close_bf16(got, want, what):
    r = rel_l2(got, want)
    m = float(np.max(np.abs(got - want)) / max(np.max(np.abs(want)), 1e-30))
    assert r <= BF16_BWD_REL_L2 and m <= BF16_BWD_MAX_REL, f"{what}: rel-L2 {r:.3e}, max/max {m:.3e}"


@pytest.fixture(scope="module")
def chm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_recurrence_mshortconv_amd as m
    m.lib()
    return m


def _case(rng, B, T, H, dk, dv, dtype):
    rnd = (lambda a: wl.round_to_bf16(a.astype(np.float32))) if dtype == "bf16" else (lambda a: a.astype(np.float32))
    q, k = rnd(rng.standard_normal((B, T, H, dk))), rnd(rng.standard_normal((B, T, H, dk)))
    v = rnd(rng.standard_normal((B, T, H, dv)))
    alpha = rnd(np.exp(-0.3 * np.logaddexp(0, rng.standard_normal((B, T, H, dk)))))
    beta = rnd(1 / (1 + np.exp(-rng.standard_normal((B, T, H)))))
    S0 = (0.1 * rng.standard_normal((B, H, dk, dv))).astype(np.float32)
    do = rnd(rng.standard_normal((B, T, H, dv)))
    dS = (0.1 * rng.standard_normal((B, H, dk, dv))).astype(np.float32)
    return q, k, v, alpha, beta, S0, do, dS


def _run(chm, dtype, q, k, v, alpha, beta, S0, do, dS):
    import torch
    dev = lambda a: to_device(a, dtype)
    g = chm.kda_bwd(dev(q), dev(k), dev(v), dev(alpha), dev(beta), torch.from_numpy(S0).cuda(), dev(do),
                    torch.from_numpy(dS).cuda())
    return {n: to_host(t) for n, t in g.items()}


def _run_fused_fp32(chm, q, k, v, alpha, beta, S0, do, dS):
    """q, k, v and their gradients as views into fused [B, T, H*(2 dk + dv)] tensors (the
    shared token stride the entry point requires when dk != dv)."""
    import torch
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    W = H * (2 * dk + dv)
    fused = torch.from_numpy(np.concatenate([q.reshape(B, T, -1), k.reshape(B, T, -1), v.reshape(B, T, -1)],
                                            axis=-1)).cuda()
    views = lambda t: (t[:, :, :H * dk].view(B, T, H, dk), t[:, :, H * dk:2 * H * dk].view(B, T, H, dk),
                       t[:, :, 2 * H * dk:].view(B, T, H, dv))
    gfused = torch.zeros(B, T, W, device="cuda")
    dev = lambda a: torch.from_numpy(a).cuda()
    g = chm.kda_bwd(*views(fused), dev(alpha), dev(beta), dev(S0), dev(do), dev(dS), grads=views(gfused))
    return {n: to_host(t) for n, t in g.items()}


def test_kda_bwd_fp32_odd_dims(chm):
    """fp32, dk != dv (not multiples of 16), two batch items; q, k, v and their gradients are
    views into fused tensors (the shared token stride)."""
    rng = np.random.default_rng(120)
    args = _case(rng, 2, 77, 3, 20, 37, "f32")
    got = _run_fused_fp32(chm, *args)
    ref = kda_backward_ref(*args)
    for n in ("dq", "dk", "dv", "dalpha", "dbeta", "dS0"):
        assert_close(got[n], ref[n], "f32", n)


@pytest.mark.parametrize("T", [1, 16, 300])
def test_kda_bwd_bf16_d128(chm, T):
    rng = np.random.default_rng(121 + T)
    args = _case(rng, 1, T, 2, 128, 128, "bf16")
    got = _run(chm, "bf16", *args)
    ref = kda_backward_ref(*args)
    for n in ("dq", "dk", "dv", "dalpha", "dbeta", "dS0"):
        _close_bf16(got[n], ref[n], f"{n} T={T}")


@pytest.mark.parametrize("B,T,H,l2norm,init,decay", [
    (1, 1000, 2, True, True, 0.3),     # three segments of 336, 336 and 328 tokens; a ragged last chunk
    (1, 4357, 1, True, True, 0.3),     # 17 segments of 272 tokens, the last of 5: its second part is empty
    (2, 600, 2, True, True, 0.3),      # two batch items of two heads, two segments each
    (2, 77, 3, True, False, 0.3),      # one segment with a ragged chunk, two batch items, no S0 / dS_final
    (1, 16, 1, False, True, 0.3),      # exactly one chunk, no normalisation
    (1, 600, 1, True, True, 3.0),      # strong decay (alpha down to about e^-8 within a chunk), 2 segments
])
def test_kda_bwd_chunked_bf16(chm, B, T, H, l2norm, init, decay):
    """The chunked MFMA backward (bf16, d = 128; 16-token chunks, segments joined by chains, each
    segment's checkpoint and gradient passes run per half) against the fp64 autograd oracle, and the
    token-by-token backward (CHIMERA_KDA_SEQUENTIAL) on the same inputs against it too."""
    import torch
    rng = np.random.default_rng(300 + T + H)
    q, k, v, alpha, beta, S0, do, dS = _case(rng, B, T, H, 128, 128, "bf16")
    alpha = wl.round_to_bf16(np.exp(-decay * np.logaddexp(0, rng.standard_normal(alpha.shape))).astype(np.float32))
    # raised to the chunked kernels' floor (bf16 0x3A11, about e^-7.5), so that their clamp changes nothing
    alpha = np.maximum(alpha, np.array([0x3A110000], dtype=np.uint32).view(np.float32)[0])
    if not l2norm:   # unit-norm scale without the normalisation, so that the recurrence stays bounded
        q, k = wl.round_to_bf16(q / np.float32(np.sqrt(128))), wl.round_to_bf16(k / np.float32(np.sqrt(128)))
    if not init:
        S0 = dS = None
    dev = lambda a: to_device(a, "bf16")
    opt = lambda a: None if a is None else torch.from_numpy(a).cuda()
    ref = kda_backward_ref(q, k, v, alpha, beta, S0, do, dS, l2norm=l2norm)
    for seq in (False, True):
        g = chm.kda_bwd(dev(q), dev(k), dev(v), dev(alpha), dev(beta), opt(S0), dev(do), opt(dS), l2norm=l2norm,
                        sequential=seq)
        got = {n: to_host(t) for n, t in g.items()}
        for n in ("dq", "dk", "dv", "dalpha", "dbeta", "dS0"):
            _close_bf16(got[n], ref[n], f"{n} (sequential={seq})")


def test_kda_bwd_fp32_segments(chm):
    """fp32, T = 700 on two 32-wide heads: the sequence is cut into segments of 80 tokens (the
    last 60) whose reverse passes run at once, joined by the chains of transition products;
    with S0 and dS_final."""
    rng = np.random.default_rng(124)
    args = _case(rng, 1, 700, 2, 32, 32, "f32")
    got = _run(chm, "f32", *args)
    ref = kda_backward_ref(*args)
    for n in ("dq", "dk", "dv", "dalpha", "dbeta", "dS0"):
        assert_close(got[n], ref[n], "f32", n)


def test_kda_bwd_fp32_odd_dims_segments(chm):
    """fp32, dk = 20, dv = 37 (the last 16-column slice partly outside), T = 400: five segments
    of 80 tokens; chains over a ragged column slice."""
    rng = np.random.default_rng(127)
    args = _case(rng, 1, 400, 1, 20, 37, "f32")
    got = _run_fused_fp32(chm, *args)
    ref = kda_backward_ref(*args)
    for n in ("dq", "dk", "dv", "dalpha", "dbeta", "dS0"):
        assert_close(got[n], ref[n], "f32", n)


def test_kda_bwd_fp32_extreme_dims(chm):
    """fp32, dk = 16 (one row per thread) with dv = 256 (the largest: sixteen column slices), and
    dk = 128 with dv = 1; T = 70 (ragged last checkpoint block)."""
    rng = np.random.default_rng(134)
    for dk, dv in ((16, 256), (128, 1)):
        args = _case(rng, 1, 70, 2, dk, dv, "f32")
        got = _run_fused_fp32(chm, *args)
        ref = kda_backward_ref(*args)
        for n in ("dq", "dk", "dv", "dalpha", "dbeta", "dS0"):
            assert_close(got[n], ref[n], "f32", f"{n} dk={dk} dv={dv}")


def test_kda_bwd_bf16_segments_batch(chm):
    """bf16 d = 128, two sequences of 1000 tokens: 13 segments of 80 tokens per sequence."""
    rng = np.random.default_rng(125)
    args = _case(rng, 2, 1000, 2, 128, 128, "bf16")
    got = _run(chm, "bf16", *args)
    ref = kda_backward_ref(*args)
    for n in ("dq", "dk", "dv", "dalpha", "dbeta", "dS0"):
        _close_bf16(got[n], ref[n], f"{n} segmented")


def test_kda_bwd_empty_sequence(chm):
    """T = 0: nothing to carry back, so dS0 = dS_final and the token gradients are empty."""
    rng = np.random.default_rng(128)
    args = _case(rng, 1, 0, 2, 128, 128, "bf16")
    got = _run(chm, "bf16", *args)
    assert np.array_equal(got["dS0"], args[-1].astype(np.float64))
    assert got["dq"].shape == (1, 0, 2, 128) and got["dbeta"].shape == (1, 0, 2)


def test_kda_bwd_full_size_directional(chm):
    """The image_4096 sizes in the training-step bench's configuration (65,792 tokens, 16 heads,
    d = 128, q|k|v as views into one fused bf16 tensor: 16 segments of 4,112 tokens, both chains).
    For head 5: the GPU gradients of all five inputs, paired with a random direction over the whole
    sequence, against the central difference of the fp64 oracle's loss sum(o * do) +
    sum(S_final * dS_final) along it; and the gradients of the last 2,048 tokens element by element
    against the fp64 autograd oracle run from the oracle's state before them."""
    import torch
    T, H, d, hd, tail = 65792, 16, 128, 5, 2048
    rng = np.random.default_rng(129)
    y = wl.round_to_bf16(rng.standard_normal((1, T, 3 * H * d), dtype=np.float32))
    alpha = wl.round_to_bf16(np.exp(-0.05 * np.logaddexp(0, rng.standard_normal((1, T, H, d), dtype=np.float32))))
    beta = wl.round_to_bf16(1 / (1 + np.exp(-rng.standard_normal((1, T, H), dtype=np.float32))))
    do = wl.round_to_bf16(rng.standard_normal((1, T, H, d), dtype=np.float32))
    dS = (0.1 * rng.standard_normal((1, H, d, d))).astype(np.float32)
    yd = to_device(y, "bf16")
    dy = torch.zeros_like(yd)
    g = chm.kda_bwd(*chm.split_qkv(yd, H, d), to_device(alpha, "bf16"), to_device(beta, "bf16"), None,
                    to_device(do, "bf16"), torch.from_numpy(dS).cuda(), grads=chm.split_qkv(dy, H, d))
    gy = to_host(dy.view(T, 3, H, d)[:, :, hd])
    grad = [gy[:, 0], gy[:, 1], gy[:, 2], to_host(g["dalpha"][0, :, hd]), to_host(g["dbeta"][0, :, hd])]
    del yd, dy, g
    y5 = y.reshape(T, 3, H, d)[:, :, hd].astype(np.float64)
    theta = [y5[:, 0], y5[:, 1], y5[:, 2], alpha[0, :, hd].astype(np.float64), beta[0, :, hd].astype(np.float64)]
    do5, dS5 = do[0, :, hd].astype(np.float64), dS[0, hd].astype(np.float64)

    def loss(x):
        e = lambda a: a[None, :, None]
        o, S = kda_ref(l2norm_ref(e(x[0])), l2norm_ref(e(x[1])), e(x[2]), e(x[3]), x[4][None, :, None])
        return float((o[0, :, 0] * do5).sum() + (S[0, 0] * dS5).sum())

    h = 1e-5
    dirs = [rng.standard_normal(t.shape) for t in theta]
    fd = (loss([t + h * dd for t, dd in zip(theta, dirs)]) - loss([t - h * dd for t, dd in zip(theta, dirs)])) / (2 * h)
    gpu = sum(float((gi * di).sum()) for gi, di in zip(grad, dirs))
    print(f"all inputs, whole sequence: GPU {gpu:.6e}, oracle {fd:.6e}", flush=True)
    assert abs(gpu - fd) <= 1e-2 * abs(fd), (gpu, fd)
    # the last `tail` tokens element by element: their gradients depend on the tokens before
    # them only through the state there
    lo = T - tail
    e = lambda a: a[None, :lo, None]
    _, S_mid = kda_ref(l2norm_ref(e(theta[0])), l2norm_ref(e(theta[1])), e(theta[2]), e(theta[3]),
                       theta[4][None, :lo, None])
    t4 = lambda a: a[None, lo:, None]
    ref = kda_backward_ref(t4(theta[0]), t4(theta[1]), t4(theta[2]), t4(theta[3]), theta[4][None, lo:, None], S_mid,
                           t4(do5), dS5[None, None])
    for i, name in enumerate(("dq", "dk", "dv", "dalpha", "dbeta")):
        _close_bf16(grad[i][lo:], ref[name][0, :, 0], f"{name}, last {tail} tokens")


def _packed(rng, cu, H, dk, dv, dtype):
    rnd = (lambda a: wl.round_to_bf16(a.astype(np.float32))) if dtype == "bf16" else (lambda a: a.astype(np.float32))
    T, N = cu[-1], len(cu) - 1
    q, k = rnd(rng.standard_normal((T, H, dk))), rnd(rng.standard_normal((T, H, dk)))
    v = rnd(rng.standard_normal((T, H, dv)))
    alpha = rnd(np.exp(-0.05 * np.logaddexp(0, rng.standard_normal((T, H, dk)))))
    beta = rnd(1 / (1 + np.exp(-rng.standard_normal((T, H)))))
    S0 = (0.1 * rng.standard_normal((N, H, dk, dv))).astype(np.float32)
    do = rnd(rng.standard_normal((T, H, dv)))
    dS = (0.1 * rng.standard_normal((N, H, dk, dv))).astype(np.float32)
    return q, k, v, alpha, beta, S0, do, dS


def _check_packed(chm, cu, args, dtype):
    import torch
    q, k, v, alpha, beta, S0, do, dS = args
    dev = lambda a: to_device(a, dtype)
    g = chm.kda_bwd_varlen(dev(q), dev(k), dev(v), dev(alpha), dev(beta), cu, torch.from_numpy(S0).cuda(), dev(do),
                           torch.from_numpy(dS).cuda())
    got = {n: to_host(t) for n, t in g.items()}
    for n in range(len(cu) - 1):
        s, e = cu[n], cu[n + 1]
        one = lambda a: a[None, s:e]
        ref = kda_backward_ref(one(q), one(k), one(v), one(alpha), one(beta), S0[n:n + 1], one(do), dS[n:n + 1])
        names = ("dq", "dk", "dv", "dalpha", "dbeta") if e > s else ()
        for name in names:
            if dtype == "bf16":
                _close_bf16(got[name][s:e], ref[name][0], f"{name} of sample {n}")
            else:
                assert_close(got[name][s:e], ref[name][0], "f32", f"{name} of sample {n}")
        if e == s:
            assert np.array_equal(got["dS0"][n], dS[n].astype(np.float64))
        elif dtype == "bf16":
            _close_bf16(got["dS0"][n], ref["dS0"][0], f"dS0 of sample {n}")
        else:
            assert_close(got["dS0"][n], ref["dS0"][0], "f32", f"dS0 of sample {n}")


def test_kda_bwd_varlen_mixed_lengths_bf16(chm):
    """Samples of 1, 63, 65, 0, 371 and 200 tokens packed in one row, each with its own S0 and
    dS_final (the 371-token sample cut into segments): every sample against the autograd oracle
    on that sample alone."""
    cu = [0, 1, 64, 129, 129, 500, 700]
    _check_packed(chm, cu, _packed(np.random.default_rng(130), cu, 2, 128, 128, "bf16"), "bf16")


def test_kda_bwd_varlen_equal_runs_fp32(chm):
    """fp32, 32-wide heads: three samples of 50 tokens (one batched run of three), one of 1, one of 149."""
    cu = [0, 50, 100, 150, 151, 300]
    _check_packed(chm, cu, _packed(np.random.default_rng(131), cu, 3, 32, 32, "f32"), "f32")


@pytest.mark.parametrize("dtype,weighted", [("f32", True), ("bf16", True), ("bf16", False)])
def test_gate_norm_bwd(chm, dtype, weighted):
    """Eq. 15's gate and norm, backward: do, dgate (the gate a view with a wider token stride) and
    the summed gain gradient against fp64 autograd of the definition."""
    import torch
    rng = np.random.default_rng(132)
    B, T, H, dv = 2, 77, 3, 40
    rnd = (lambda a: wl.round_to_bf16(a.astype(np.float32))) if dtype == "bf16" else (lambda a: a.astype(np.float32))
    o, g, dy = (rnd(rng.standard_normal((B, T, H, dv))) for _ in range(3))
    w = (1 + 0.1 * rng.standard_normal(dv)).astype(np.float32) if weighted else None
    wide = torch.zeros(B, T, H * dv + 8, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
    wide[:, :, 8:] = to_device(g.reshape(B, T, H * dv), dtype)
    gd = wide[:, :, 8:].view(B, T, H, dv)
    dout, dgate, dw = chm.gate_norm_bwd(to_device(o, dtype), gd, None if w is None else torch.from_numpy(w).cuda(),
                                        to_device(dy, dtype), 1e-6)
    ref = gate_norm_backward_ref(o, g, w, dy, 1e-6)
    check = (lambda a, b, n: assert_close(a, b, "f32", n)) if dtype == "f32" else _close_bf16
    check(to_host(dout), ref["do"], "do")
    check(to_host(dgate), ref["dgate"], "dgate")
    assert rel_l2(to_host(dw), ref["dweight"]) <= (1e-4 if dtype == "f32" else 1e-3)


def test_gated_chain_backward_fp32(chm):
    """The gated output's gradient through both backward calls: the KDA output, the gate and
    norm's backward into dL/do, the KDA backward from it; against the oracle's chain rule in fp64
    (its own output, the gate and norm's autograd, then the KDA autograd)."""
    import torch
    rng = np.random.default_rng(133)
    B, T, H, d = 1, 150, 2, 32
    q, k, v, alpha, beta, S0, _, _ = _case(rng, B, T, H, d, d, "f32")
    g = rng.standard_normal((B, T, H, d)).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    dy = rng.standard_normal((B, T, H, d)).astype(np.float32)
    dev = lambda a: torch.from_numpy(a).cuda()
    o, _ = chm.kda_fwd(dev(q), dev(k), dev(v), dev(alpha), dev(beta), dev(S0))
    do, dgate, dw = chm.gate_norm_bwd(o, dev(g), dev(w), dev(dy), 1e-6)
    got = {n: to_host(t) for n, t in chm.kda_bwd(dev(q), dev(k), dev(v), dev(alpha), dev(beta), dev(S0), do).items()}
    o_ref, _ = kda_ref(l2norm_ref(q), l2norm_ref(k), v, alpha, beta, S0)
    gn = gate_norm_backward_ref(o_ref, g, w, dy, 1e-6)
    ref = kda_backward_ref(q, k, v, alpha, beta, S0, gn["do"])
    assert_close(to_host(dgate), gn["dgate"], "f32", "dgate")
    for n in ("dq", "dk", "dv", "dalpha", "dbeta", "dS0"):
        assert_close(got[n], ref[n], "f32", n)


def test_conv_bwd_fp32_mixed_layout(chm):
    import torch
    S = wl.Segment
    segs = (S(wl.TEXT, 0, 9), S(wl.IMAGE, 9, 7 * 6, 1, 7, 6), S(wl.TEXT, 51, 3), S(wl.VIDEO, 54, 3 * 4 * 5, 3, 4, 5))
    T, C = 114, 24
    rng = np.random.default_rng(122)
    x = rng.standard_normal((2, T, C)).astype(np.float32)
    dy = rng.standard_normal((2, T, C)).astype(np.float32)
    wt = (0.5 * rng.standard_normal((C, 4))).astype(np.float32)
    wv = (0.5 * rng.standard_normal((C, 27))).astype(np.float32)
    dx, dwt, dwv = chm.mshortconv_bwd(to_device(x, "f32"), to_device(dy, "f32"), torch.from_numpy(wt),
                                      torch.from_numpy(wv), segs)
    ref = conv_backward_ref(x, wt, wv, segs, dy)
    np.testing.assert_allclose(to_host(dx), ref["dx"], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(to_host(dwt), ref["dw_text"], rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(to_host(dwv), ref["dw_vis"], rtol=1e-5, atol=1e-4)


def test_conv_bwd_bf16_grids(chm):
    """bf16: image grids take the image conv's kernel with mirrored taps for dx (one launch for
    both images), the video the tile kernel's adjoint, the text the gather kernel; dx within one
    bf16 rounding of the fp64 adjoint, dw within fp32 summation error."""
    import torch
    S = wl.Segment
    segs = (S(wl.TEXT, 0, 5), S(wl.IMAGE, 5, 20 * 33, 1, 20, 33), S(wl.VIDEO, 665, 2 * 5 * 6, 2, 5, 6),
            S(wl.IMAGE, 725, 7 * 64, 1, 7, 64))
    T, C = 725 + 448, 128
    rng = np.random.default_rng(126)
    x = wl.round_to_bf16(rng.standard_normal((2, T, C)).astype(np.float32))
    dy = wl.round_to_bf16(rng.standard_normal((2, T, C)).astype(np.float32))
    wt = (0.5 * rng.standard_normal((C, 4))).astype(np.float32)
    wv = (0.5 * rng.standard_normal((C, 27))).astype(np.float32)
    dx, dwt, dwv = chm.mshortconv_bwd(to_device(x, "bf16"), to_device(dy, "bf16"), torch.from_numpy(wt),
                                      torch.from_numpy(wv), segs)
    ref = conv_backward_ref(x, wt, wv, segs, dy)
    np.testing.assert_allclose(to_host(dx), ref["dx"], rtol=2.0 ** -8, atol=1e-4)
    for got, want in ((dwt, ref["dw_text"]), (dwv, ref["dw_vis"])):
        np.testing.assert_allclose(to_host(got), want, rtol=1e-4, atol=1e-4 * np.abs(want).max())


@pytest.mark.parametrize("frames,height,width", [(11, 6, 19), (2, 9, 17), (3, 4, 4)])
def test_conv_bwd_bf16_video_adjoint(chm, frames, height, width):
    """bf16 video dx on the tile kernel's adjoint (mirrored spatial taps, frames walked from the
    last one back): 11 frames make two frame ranges of a block (the second starts from staged
    frames after it), grids that are not a multiple of the 4 x 16 tile, and a grid smaller than
    one tile, against the fp64 adjoint (dy outside the segment, a text prefix and a trailing text,
    must not leak in)."""
    import torch
    S = wl.Segment
    n = frames * height * width
    segs = (S(wl.TEXT, 0, 7), S(wl.VIDEO, 7, n, frames, height, width), S(wl.TEXT, 7 + n, 5))
    T, C = 7 + n + 5, 192
    rng = np.random.default_rng(frames * 100 + height * 10 + width)
    x = wl.round_to_bf16(rng.standard_normal((1, T, C)).astype(np.float32))
    dy = wl.round_to_bf16(rng.standard_normal((1, T, C)).astype(np.float32))
    wt = (0.5 * rng.standard_normal((C, 4))).astype(np.float32)
    wv = (0.5 * rng.standard_normal((C, 27))).astype(np.float32)
    dx, dwt, dwv = chm.mshortconv_bwd(to_device(x, "bf16"), to_device(dy, "bf16"), torch.from_numpy(wt),
                                      torch.from_numpy(wv), segs)
    ref = conv_backward_ref(x, wt, wv, segs, dy)
    np.testing.assert_allclose(to_host(dx), ref["dx"], rtol=2.0 ** -8, atol=1e-4)
    np.testing.assert_allclose(to_host(dwv), ref["dw_vis"], rtol=1e-4, atol=1e-4 * np.abs(ref["dw_vis"]).max())


def test_pipeline_backward_bf16(chm):
    """conv -> KDA forward, then the KDA gradients written straight into one fused q|k|v
    gradient and the conv's backward on it, against the oracle's chain of the two."""
    import torch
    S = wl.Segment
    H, d = 2, 128
    segs = (S(wl.TEXT, 0, 30), S(wl.IMAGE, 30, 12 * 11, 1, 12, 11))
    T, C = 162, 3 * H * d
    rng = np.random.default_rng(123)
    x = wl.round_to_bf16(rng.standard_normal((1, T, C)).astype(np.float32))
    wt = (0.5 * rng.standard_normal((C, 4))).astype(np.float32)
    wv = (0.5 * rng.standard_normal((C, 27))).astype(np.float32)
    alpha = wl.round_to_bf16(np.exp(-0.05 * np.logaddexp(0, rng.standard_normal((1, T, H, d)))).astype(np.float32))
    beta = wl.round_to_bf16((1 / (1 + np.exp(-rng.standard_normal((1, T, H))))).astype(np.float32))
    do = wl.round_to_bf16(rng.standard_normal((1, T, H, d)).astype(np.float32))
    xd = to_device(x, "bf16")
    y = chm.mshortconv_fwd(xd, torch.from_numpy(wt), torch.from_numpy(wv), segs)
    q, k, v = chm.split_qkv(y, H, d)
    dy = torch.zeros_like(y)
    gq, gk, gv = chm.split_qkv(dy, H, d)
    g = chm.kda_bwd(q, k, v, to_device(alpha, "bf16"), to_device(beta, "bf16"), None, to_device(do, "bf16"),
                    grads=(gq, gk, gv))
    dx, dwt, dwv = chm.mshortconv_bwd(xd, dy, torch.from_numpy(wt), torch.from_numpy(wv), segs)
    # oracle chain, from the inputs alone: the conv output rounded once to bf16, the KDA
    # gradients in fp64, then the conv's backward of those
    from oracle import conv_ref, round_bf16_ref
    y_ref = round_bf16_ref(conv_ref(x, wt, wv, segs))
    parts = y_ref.reshape(1, T, 3, H, d)
    ref = kda_backward_ref(parts[:, :, 0], parts[:, :, 1], parts[:, :, 2], alpha, beta, None, do)
    _close_bf16(to_host(g["dalpha"]), ref["dalpha"], "dalpha")
    _close_bf16(to_host(g["dbeta"]), ref["dbeta"], "dbeta")
    dy_ref = np.concatenate([ref[n].reshape(1, T, H * d) for n in ("dq", "dk", "dv")], axis=-1)
    _close_bf16(to_host(dy), dy_ref, "dy")
    cref = conv_backward_ref(x, wt, wv, segs, dy_ref)
    _close_bf16(to_host(dx), cref["dx"], "dx")
    _close_bf16(to_host(dwt), cref["dw_text"], "dw_text")
    _close_bf16(to_host(dwv), cref["dw_vis"], "dw_vis")
