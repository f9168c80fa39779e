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
    """fp32, odd head dims (dk != dv, not multiples of 16), several batch items; q, k, v
    are views into one fused tensor (the ABI's shared token stride)."""
    import torch
    rng = np.random.default_rng(5)
    B, T, H, dk, dv = 2, 77, 3, 20, 37
    fused = rng.standard_normal((B, T, H * (2 * dk + dv))).astype(np.float32)
    q = fused[:, :, :H * dk].reshape(B, T, H, dk)
    k = fused[:, :, H * dk:2 * H * dk].reshape(B, T, H, dk)
    v = fused[:, :, 2 * H * dk:].reshape(B, T, H, dv)
    alpha = np.exp(-np.logaddexp(0, rng.standard_normal((B, T, H, dk)))).astype(np.float32)
    beta = (1 / (1 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32)
    S0 = (0.1 * rng.standard_normal((B, H, dk, dv))).astype(np.float32)
    fd = torch.from_numpy(fused).cuda()
    qd = fd[:, :, :H * dk].view(B, T, H, dk)
    kd = fd[:, :, H * dk:2 * H * dk].view(B, T, H, dk)
    vd = fd[:, :, 2 * H * dk:].view(B, T, H, dv)
    o, Sf = chm.kda_fwd(qd, kd, vd, *(torch.from_numpy(a).cuda() for a in (alpha, beta, S0)), l2norm=True)
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


def _small_case(rng, B, T, H, d, s0, strong=False):
    q = wl.round_to_bf16(rng.standard_normal((B, T, H, d)).astype(np.float32))
    k = wl.round_to_bf16(rng.standard_normal((B, T, H, d)).astype(np.float32))
    v = wl.round_to_bf16(rng.standard_normal((B, T, H, d)).astype(np.float32))
    if strong:
        la = np.full((B, T, H, d), -5.0, np.float32)          # log alpha = -5 everywhere
    else:
        la = -0.05 * np.logaddexp(0, rng.standard_normal((B, T, H, d))).astype(np.float32)
    alpha = wl.round_to_bf16(np.exp(la).astype(np.float32))
    beta = wl.round_to_bf16((1 / (1 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32))
    S0 = (0.1 * rng.standard_normal((B, H, d, d))).astype(np.float32) if s0 else None
    return q, k, v, alpha, beta, S0


def _gpu_kda(chm, q, k, v, alpha, beta, S0, **kw):
    import torch
    dev = lambda a: to_device(a, "bf16")
    s0 = None if S0 is None else torch.from_numpy(S0).cuda()
    return chm.kda_fwd(dev(q), dev(k), dev(v), dev(alpha), dev(beta), s0, l2norm=True, **kw)


@pytest.mark.parametrize("T", [1, 17, 64, 65, 200, 343, 1000])
@pytest.mark.parametrize("no_split", [False, True])
def test_kda_chunked_shapes(chm, T, no_split):
    rng = np.random.default_rng(T)
    B, H, d = 2, 2, 128
    q, k, v, alpha, beta, S0 = _small_case(rng, B, T, H, d, s0=True)
    o, Sf = _gpu_kda(chm, q, k, v, alpha, beta, S0, no_split=no_split)
    o_ref, S_ref = kda_ref(l2norm_ref(q), l2norm_ref(k), v, alpha, beta, S0)
    assert_close(to_host(o), o_ref, "bf16", f"o T={T}")
    assert_close(to_host(Sf), S_ref, "bf16", f"S_final T={T}")


def test_kda_chunked_zero_state_and_no_norm(chm):
    rng = np.random.default_rng(77)
    B, T, H, d = 1, 300, 3, 128
    q, k, v, alpha, beta, _ = _small_case(rng, B, T, H, d, s0=False)
    q, k = (wl.round_to_bf16(l2norm_ref(x).astype(np.float32)) for x in (q, k))
    o, Sf = _gpu_kda(chm, q, k, v, alpha, beta, None)
    o2, Sf2 = chm.kda_fwd(*(to_device(a, "bf16") for a in (q, k, v, alpha, beta)), None, l2norm=False)
    o_ref, S_ref = kda_ref(q, k, v, alpha, beta, None)
    assert_close(to_host(o2), o_ref, "bf16", "o (no norm)")
    assert_close(to_host(Sf2), S_ref, "bf16", "S (no norm)")
    assert_close(to_host(o), o_ref, "bf16", "o (norm of unit rows)")


def test_kda_chunked_strong_decay(chm):
    """log alpha = -5 for every token and channel: the factored decays stay finite."""
    rng = np.random.default_rng(5)
    B, T, H, d = 1, 260, 2, 128
    q, k, v, alpha, beta, S0 = _small_case(rng, B, T, H, d, s0=True, strong=True)
    o, Sf = _gpu_kda(chm, q, k, v, alpha, beta, S0)
    o_ref, S_ref = kda_ref(l2norm_ref(q), l2norm_ref(k), v, alpha, beta, S0)
    assert np.isfinite(to_host(o)).all()
    assert_close(to_host(o), o_ref, "bf16", "o strong decay")
    assert_close(to_host(Sf), S_ref, "bf16", "S strong decay")


@pytest.mark.parametrize("no_split", [False, True])
def test_kda_chunked_degenerate_decay(chm, no_split):
    """Decays far beyond the blocked factorisation's range: log alpha uniform in [-30, 0],
    a tenth of the entries exactly 0 (complete forgetting), and one chunk with alpha = 1.
    The chunked kernel raises alpha to e^-7.5 as it loads it; against the exact oracle
    the result stays finite and within the bf16 tolerances."""
    rng = np.random.default_rng(31)
    B, T, H, d = 1, 64 * 9 + 17, 2, 128
    q, k, v, _, beta, S0 = _small_case(rng, B, T, H, d, s0=True)
    la = rng.uniform(-30.0, 0.0, (B, T, H, d)).astype(np.float32)
    alpha = np.exp(la).astype(np.float32)
    alpha[rng.random((B, T, H, d)) < 0.1] = 0.0
    alpha[:, 64 * 3:64 * 4] = 1.0
    alpha = wl.round_to_bf16(alpha)
    o, Sf = _gpu_kda(chm, q, k, v, alpha, beta, S0, no_split=no_split)
    o_ref, S_ref = kda_ref(l2norm_ref(q), l2norm_ref(k), v, alpha, beta, S0)
    assert np.isfinite(to_host(o)).all() and np.isfinite(to_host(Sf)).all()
    assert_close(to_host(o), o_ref, "bf16", "o degenerate decay")
    assert_close(to_host(Sf), S_ref, "bf16", "S degenerate decay")


@pytest.mark.parametrize("no_split", [False, True])
def test_kda_chunked_mixed_decay_rates(chm, no_split):
    """Per-channel decay rates from e^-0.01 to e^-0.45 per token (within a chunk some channels fall
    below e^-25 while others barely move), every fifth chunk with log alpha = -1 (the blocked
    factorisation), and a chunk with alpha = 1, in one sequence; against the oracle."""
    rng = np.random.default_rng(41)
    B, T, H, d = 2, 64 * 21 + 30, 2, 128
    q, k, v, _, beta, S0 = _small_case(rng, B, T, H, d, s0=True)
    rate = np.exp(rng.uniform(np.log(0.01), np.log(0.45), (1, 1, H, d))).astype(np.float32)
    la = -rate * (0.5 + rng.random((B, T, H, d), dtype=np.float32))
    for c in range(4, T // 64, 5):
        la[:, 64 * c:64 * (c + 1)] = -1.0
    la[:, 64 * 7:64 * 8] = 0.0
    alpha = wl.round_to_bf16(np.exp(la).astype(np.float32))
    o, Sf = _gpu_kda(chm, q, k, v, alpha, beta, S0, no_split=no_split)
    o_ref, S_ref = kda_ref(l2norm_ref(q), l2norm_ref(k), v, alpha, beta, S0)
    assert np.isfinite(to_host(o)).all() and np.isfinite(to_host(Sf)).all()
    assert_close(to_host(o), o_ref, "bf16", "o mixed rates")
    assert_close(to_host(Sf), S_ref, "bf16", "S mixed rates")


@pytest.mark.parametrize("dk,dv", [(64, 64), (32, 32), (64, 128), (128, 96), (8, 16)])
@pytest.mark.parametrize("no_split", [False, True])
def test_kda_chunked_head_sizes(chm, dk, dv, no_split):
    """bf16 heads below 128 channels on the chunked kernels (zero-padded inside them to 128):
    q, k, v as views into one fused tensor, several chunks and a ragged tail, S0; every head
    against the oracle, and the kernel names show the chunked path ran."""
    import torch
    rng = np.random.default_rng(dk * 1000 + dv)
    B, T, H = 2, 64 * 5 + 23, 3
    C = H * (2 * dk + dv)
    x = wl.round_to_bf16(rng.standard_normal((B, T, C)).astype(np.float32))
    q = x[:, :, :H * dk].reshape(B, T, H, dk)
    k = x[:, :, H * dk:2 * H * dk].reshape(B, T, H, dk)
    v = x[:, :, 2 * H * dk:].reshape(B, T, H, dv)
    la = -0.05 * np.logaddexp(0, rng.standard_normal((B, T, H, dk))).astype(np.float32)
    alpha = wl.round_to_bf16(np.exp(la).astype(np.float32))
    beta = wl.round_to_bf16((1 / (1 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32))
    S0 = (0.1 * rng.standard_normal((B, H, dk, dv))).astype(np.float32)
    xd = to_device(x, "bf16")
    qd = xd[:, :, :H * dk].view(B, T, H, dk)
    kd = xd[:, :, H * dk:2 * H * dk].view(B, T, H, dk)
    vd = xd[:, :, 2 * H * dk:].view(B, T, H, dv)
    marks = chm.Marks(8)
    o, Sf = chm.kda_fwd(qd, kd, vd, to_device(alpha, "bf16"), to_device(beta, "bf16"), torch.from_numpy(S0).cuda(),
                        no_split=no_split, marks=marks)
    torch.cuda.synchronize()
    assert "kda_out_kernel" in [n for n, _ in marks.kernels()]
    o_ref, S_ref = kda_ref(l2norm_ref(q), l2norm_ref(k), v, alpha, beta, S0)
    assert_close(to_host(o), o_ref, "bf16", f"o dk={dk} dv={dv}")
    assert_close(to_host(Sf), S_ref, "bf16", f"S_final dk={dk} dv={dv}")


def test_kda_chunked_split_invariance(chm):
    """Segmenting the sequence (three passes) and not segmenting it agree closely."""
    rng = np.random.default_rng(8)
    B, T, H, d = 1, 64 * 40 + 9, 4, 128
    q, k, v, alpha, beta, S0 = _small_case(rng, B, T, H, d, s0=True)
    o1, S1 = _gpu_kda(chm, q, k, v, alpha, beta, S0, no_split=False)
    o2, S2 = _gpu_kda(chm, q, k, v, alpha, beta, S0, no_split=True)
    assert rel_l2(to_host(o1), to_host(o2)) < 5e-3
    assert rel_l2(to_host(S1), to_host(S2)) < 5e-3


@pytest.mark.parametrize("wi", [1, 2, 3, 4])
def test_pipeline_full_workload_sampled_heads(chm, wi):
    """conv then chunked KDA at full size in the bench's launch configuration;
    the oracle recomputes whole heads (every token) for the first, a middle and the last head
    (the first and last at the 255K-token video)."""
    import torch
    w = wl.WORKLOADS[wi]
    inp = wl.make_inputs(w)
    heads = [0, w.H - 1] if wi == 4 else [0, w.H // 2 - 1, w.H - 1]
    x_dev = to_device(inp["x"], "bf16")
    y = chm.mshortconv_fwd(x_dev, torch.from_numpy(inp["w_text"]), torch.from_numpy(inp["w_vis"]), inp["segments"])
    del x_dev
    o, Sf = _run_kda(chm, y, inp["alpha"], inp["beta"], inp["S0"], w)
    o_got = to_host(o[:, :, heads])
    S_got = to_host(Sf[:, heads])
    del y, o, Sf
    HD = w.H * w.d
    chans = np.concatenate([part * HD + h * w.d + np.arange(w.d) for part in range(3) for h in heads])
    y_ref = round_bf16_ref(conv_ref(inp["x"][:, :, chans], inp["w_text"][chans], inp["w_vis"][chans], inp["segments"]))
    nh = len(heads)
    parts = y_ref.reshape(w.B, w.T, 3, nh, w.d)
    S0 = None if inp["S0"] is None else inp["S0"][:, heads]
    o_ref, S_ref = kda_ref(l2norm_ref(parts[:, :, 0]), l2norm_ref(parts[:, :, 1]), parts[:, :, 2],
                           inp["alpha"][:, :, heads], inp["beta"][:, :, heads], S0)
    assert_close(o_got, o_ref, "bf16", f"{w.name} o")
    assert_close(S_got, S_ref, "bf16", f"{w.name} S_final")


def test_kda_chunked_matches_token_by_token(chm):
    """The chunk-size invariance of the method on the GPU: the chunked MFMA path (64-token chunks, the
    sequence cut into segments) and the token-by-token kernel (one token per step, fp32) on the same
    bf16 inputs give the same o and S_final within the bf16 tolerance, and each is within it of the
    oracle."""
    rng = np.random.default_rng(21)
    B, T, H, d = 2, 64 * 23 + 37, 4, 128
    q, k, v, alpha, beta, S0 = _small_case(rng, B, T, H, d, s0=True)
    o1, S1 = _gpu_kda(chm, q, k, v, alpha, beta, S0)
    o2, S2 = _gpu_kda(chm, q, k, v, alpha, beta, S0, sequential=True)
    assert_close(to_host(o1), to_host(o2), "bf16", "o chunked vs token-by-token")
    assert_close(to_host(S1), to_host(S2), "bf16", "S_final chunked vs token-by-token")
    o_ref, S_ref = kda_ref(l2norm_ref(q), l2norm_ref(k), v, alpha, beta, S0)
    for o, S, name in ((o1, S1, "chunked"), (o2, S2, "token-by-token")):
        assert_close(to_host(o), o_ref, "bf16", f"{name} o")
        assert_close(to_host(S), S_ref, "bf16", f"{name} S_final")


def test_timed_variants_match_untimed(chm):
    """The timing entry points launch the same kernels: identical outputs, one mark per kernel."""
    import torch
    w = wl.WORKLOADS[1]
    inp = wl.make_inputs(w)
    x_dev = to_device(inp["x"], "bf16")
    wt, wv = torch.from_numpy(inp["w_text"]), torch.from_numpy(inp["w_vis"])
    y1 = chm.mshortconv_fwd(x_dev, wt, wv, inp["segments"])
    mc = chm.Marks(len(inp["segments"]) + 1)
    y2 = chm.mshortconv_fwd(x_dev, wt, wv, inp["segments"], marks=mc)
    o1, S1 = _run_kda(chm, y1, inp["alpha"], inp["beta"], inp["S0"], w)
    mk = chm.Marks(5)
    o2, S2 = _run_kda(chm, y1, inp["alpha"], inp["beta"], inp["S0"], w, marks=mk)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(o1, o2) and torch.equal(S1, S2)
    conv_k, kda_k = mc.kernels(), mk.kernels()
    assert [n for n, _ in conv_k] == ["conv_text_kernel", "conv_rows_kernel"]
    assert [n for n, _ in kda_k] == ["kda_sum_kernel", "kda_combine_kernel", "kda_out_kernel"]
    assert all(ms > 0 for _, ms in conv_k + kda_k)


@pytest.mark.parametrize("B,T,H,dk,dv", [(1, 1000, 2, 128, 128), (2, 517, 3, 96, 40), (1, 600, 1, 32, 32)])
def test_kda_token_by_token_split(chm, B, T, H, dk, dv):
    """The token-by-token kernel on a sequence cut into segments (end states from zero and
    transition products per segment, the chain of start states, then the readout from them;
    ragged last segments here) against the oracle, and against the same kernel unsplit to fp32
    rounding: fp32 inputs with a nonzero S0, and bf16 inputs with the same cut."""
    import torch
    rng = np.random.default_rng(T + dk)
    q = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    alpha = np.exp(-0.2 * np.logaddexp(0, rng.standard_normal((B, T, H, dk)))).astype(np.float32)
    beta = (1 / (1 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32)
    S0 = (0.1 * rng.standard_normal((B, H, dk, dv))).astype(np.float32)
    assert chm.kda_workspace_size(B, T, H, dk, dv, chm.F32, chm.KDA_L2NORM_QK) > 0   # the cut applies
    dev = lambda a: torch.from_numpy(a).cuda()

    def qkv(fd):   # q, k, v as views of one fused tensor: the ABI's one token stride
        return (fd[:, :, :H * dk].view(B, T, H, dk), fd[:, :, H * dk:2 * H * dk].view(B, T, H, dk),
                fd[:, :, 2 * H * dk:].view(B, T, H, dv))
    fused = np.concatenate([a.reshape(B, T, -1) for a in (q, k, v)], axis=2)
    args = (*qkv(dev(fused)), dev(alpha), dev(beta), dev(S0))
    o, Sf = chm.kda_fwd(*args, l2norm=True)
    o1, S1 = chm.kda_fwd(*args, l2norm=True, no_split=True)
    o_ref, S_ref = kda_ref(l2norm_ref(q), l2norm_ref(k), v, alpha, beta, S0)
    torch.cuda.synchronize()
    assert_close(to_host(o), o_ref, "f32", "o")
    assert_close(to_host(Sf), S_ref, "f32", "S_final")
    assert rel_l2(to_host(o), to_host(o1)) < 1e-5 and rel_l2(to_host(Sf), to_host(S1)) < 1e-5
    # bf16 storage on the same cut (the chunked kernel set aside): the rounded inputs' oracle
    rb = lambda a: round_bf16_ref(a)
    ob, Sb = chm.kda_fwd(*qkv(to_device(rb(fused), "bf16")), *(to_device(rb(a), "bf16") for a in (alpha, beta)),
                         dev(S0), l2norm=True, sequential=True)
    ob_ref, Sb_ref = kda_ref(l2norm_ref(rb(q)), l2norm_ref(rb(k)), rb(v), rb(alpha), rb(beta), S0)
    assert_close(to_host(ob), ob_ref, "bf16", "o bf16")
    assert_close(to_host(Sb), Sb_ref, "bf16", "S_final bf16")
