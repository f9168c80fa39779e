"""GPU parity of KDA over samples packed in one row (chimera_kda_fwd_varlen), the state
restarting at every sample boundary, against the fp64 oracle (kda_varlen_ref)."""
import numpy as np
import pytest

import workloads as wl
from oracle import conv_ref, gated_rmsnorm_ref, kda_varlen_ref, l2norm_ref, round_bf16_ref
from tests.gpu_util import assert_close, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def chm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_recurrence_mshortconv_amd as m
    m.lib()
    return m


def _case(rng, T, H, d, N, dtype="bf16"):
    rnd = (lambda a: wl.round_to_bf16(a.astype(np.float32))) if dtype == "bf16" else (lambda a: a.astype(np.float32))
    q, k, v = (rnd(rng.standard_normal((T, H, d))) for _ in range(3))
    alpha = rnd(np.exp(-0.05 * np.logaddexp(0, rng.standard_normal((T, H, d)))))
    beta = rnd(1 / (1 + np.exp(-rng.standard_normal((T, H)))))
    S0 = (0.1 * rng.standard_normal((N, H, d, d))).astype(np.float32)
    return q, k, v, alpha, beta, S0


def _run(chm, q, k, v, alpha, beta, S0, cu, dtype="bf16", **kw):
    import torch
    dev = lambda a: to_device(a, dtype)
    s0 = None if S0 is None else torch.from_numpy(S0).cuda()
    return chm.kda_fwd_varlen(dev(q), dev(k), dev(v), dev(alpha), dev(beta), cu, s0, **kw)


@pytest.mark.parametrize("no_split", [False, True])
def test_varlen_mixed_lengths(chm, no_split):
    """Lengths 1, 63, 65, 0 (an empty sample), 371 and 200 in one row, each with its own S0."""
    rng = np.random.default_rng(70)
    cu = [0, 1, 64, 129, 129, 500, 700]
    H, d = 2, 128
    q, k, v, alpha, beta, S0 = _case(rng, cu[-1], H, d, len(cu) - 1)
    o, Sf = _run(chm, q, k, v, alpha, beta, S0, cu, no_split=no_split)
    o_ref, S_ref = kda_varlen_ref(l2norm_ref(q), l2norm_ref(k), v, alpha, beta, cu, S0)
    assert_close(to_host(o), o_ref, "bf16", "o")
    assert_close(to_host(Sf), S_ref, "bf16", "S_final")
    assert np.array_equal(to_host(Sf)[3], S0[3].astype(np.float64))    # the empty sample keeps its S0


def test_varlen_head_size_64(chm):
    """Packed samples with 64-channel heads on the chunked kernels (zero-padded inside them)."""
    rng = np.random.default_rng(72)
    cu = [0, 70, 70, 333, 400]
    H, d = 3, 64
    q, k, v, alpha, beta, S0 = _case(rng, cu[-1], H, d, len(cu) - 1)
    o, Sf = _run(chm, q, k, v, alpha, beta, S0, cu)
    o_ref, S_ref = kda_varlen_ref(l2norm_ref(q), l2norm_ref(k), v, alpha, beta, cu, S0)
    assert_close(to_host(o), o_ref, "bf16", "o d=64")
    assert_close(to_host(Sf), S_ref, "bf16", "S_final d=64")


def test_varlen_equal_samples_match_the_batched_call(chm):
    """Three samples of equal length in one row launch exactly as a batch of three."""
    import torch
    rng = np.random.default_rng(71)
    L, H, d, N = 64 * 40 + 9, 4, 128, 3
    q, k, v, alpha, beta, S0 = _case(rng, N * L, H, d, N)
    o1, S1 = _run(chm, q, k, v, alpha, beta, S0, [0, L, 2 * L, 3 * L])
    dev = lambda a: to_device(a, "bf16")
    b = lambda a: dev(a).view((N, L) + a.shape[1:])
    o2, S2 = chm.kda_fwd(b(q), b(k), b(v), b(alpha), b(beta), torch.from_numpy(S0).cuda())
    torch.cuda.synchronize()
    assert torch.equal(o1.view(N, L, H, d), o2) and torch.equal(S1, S2)


def test_varlen_more_runs_than_one_launch_holds(chm):
    """60 samples of 60 different lengths: the run table goes to the kernels in two launches."""
    rng = np.random.default_rng(72)
    lens = rng.permutation(np.arange(1, 61)) * 7
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    H, d = 1, 128
    q, k, v, alpha, beta, S0 = _case(rng, cu[-1], H, d, len(lens))
    o, Sf = _run(chm, q, k, v, alpha, beta, S0, cu)
    o_ref, S_ref = kda_varlen_ref(l2norm_ref(q), l2norm_ref(k), v, alpha, beta, cu, S0)
    assert_close(to_host(o), o_ref, "bf16", "o")
    assert_close(to_host(Sf), S_ref, "bf16", "S_final")


@pytest.mark.parametrize("fused", [True, False])
def test_varlen_gated(chm, fused):
    import torch
    rng = np.random.default_rng(73)
    cu = [0, 300, 301, 1100]
    H, d = 2, 128
    q, k, v, alpha, beta, S0 = _case(rng, cu[-1], H, d, 3)
    gate = wl.round_to_bf16(rng.standard_normal((cu[-1], H, d)).astype(np.float32))
    w = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    if fused:
        g = to_device(gate, "bf16")
    else:                       # token stride H*d + 4, 8 bytes past 16-byte alignment: the separate pass
        wide = torch.zeros(cu[-1], H * d + 4, dtype=torch.bfloat16, device="cuda")
        wide[:, 4:] = to_device(gate.reshape(cu[-1], H * d), "bf16")
        g = wide[:, 4:].view(cu[-1], H, d)
    o, Sf = _run(chm, q, k, v, alpha, beta, S0, cu, gate=g, norm_weight=torch.from_numpy(w).cuda(), norm_eps=1e-6)
    o_ref, S_ref = kda_varlen_ref(l2norm_ref(q), l2norm_ref(k), v, alpha, beta, cu, S0)
    assert_close(to_host(o), gated_rmsnorm_ref(o_ref, gate, w, 1e-6), "bf16", "gated o")
    assert_close(to_host(Sf), S_ref, "bf16", "S_final")


def test_varlen_fp32_token_by_token(chm):
    """fp32 with small head dims runs the token-by-token kernel, one launch per run of equal lengths."""
    rng = np.random.default_rng(74)
    cu = [0, 40, 80, 80, 157, 160]
    H, d = 3, 32
    q, k, v, alpha, beta, S0 = _case(rng, cu[-1], H, d, len(cu) - 1, dtype="f32")
    o, Sf = _run(chm, q, k, v, alpha, beta, S0, cu, dtype="f32")
    o_ref, S_ref = kda_varlen_ref(l2norm_ref(q), l2norm_ref(k), v, alpha, beta, cu, S0)
    assert_close(to_host(o), o_ref, "f32", "o")
    assert_close(to_host(Sf), S_ref, "f32", "S_final")


def test_varlen_timed_marks(chm):
    import torch
    rng = np.random.default_rng(75)
    cu = [0, 64 * 20, 64 * 20 + 333]
    H, d = 16, 128
    q, k, v, alpha, beta, S0 = _case(rng, cu[-1], H, d, 2)
    o1, S1 = _run(chm, q, k, v, alpha, beta, S0, cu)
    m = chm.Marks(8)
    o2, S2 = _run(chm, q, k, v, alpha, beta, S0, cu, marks=m)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    assert [n for n, _ in m.kernels()] == ["kda_sum_kernel", "kda_combine_kernel", "kda_out_kernel"]


def test_packed_row_conv_then_varlen_kda(chm):
    """Three samples packed in one row, each its own text and grid segments (an image, a
    wider image, a short video): the conv works per segment, the recurrence restarts per
    sample; against conv_ref over the packed segments and kda_varlen_ref."""
    import torch
    w = wl.WORKLOADS[2]
    a = wl.text_then_grid(77, 1, 16, 20)                 # 77 + 320 tokens
    b = wl.text_then_grid(40, 1, 32, 32)                 # 40 + 1024
    c = wl.text_then_grid(13, 3, 8, 8)                   # 13 + 192
    segs, cu, off = [], [0], 0
    for sample in (a, b, c):
        for sg in sample:
            segs.append(wl.Segment(sg.kind, off + sg.start, sg.length, sg.frames, sg.height, sg.width))
        off += sum(sg.length for sg in sample)
        cu.append(off)
    inp = wl.make_inputs(w, segments=tuple(segs), seed=76)
    T, H, d = cu[-1], w.H, w.d
    y = chm.mshortconv_fwd(to_device(inp["x"], "bf16"), torch.from_numpy(inp["w_text"]),
                           torch.from_numpy(inp["w_vis"]), segs)
    q, k, v = chm.split_qkv(y, H, d)
    o, Sf = chm.kda_fwd_varlen(q[0], k[0], v[0], to_device(inp["alpha"][0], "bf16"),
                               to_device(inp["beta"][0], "bf16"), cu, None)
    y_ref = round_bf16_ref(conv_ref(inp["x"], inp["w_text"], inp["w_vis"], segs))
    parts = y_ref.reshape(1, T, 3, H, d)[0]
    o_ref, S_ref = kda_varlen_ref(l2norm_ref(parts[:, 0]), l2norm_ref(parts[:, 1]), parts[:, 2],
                                  inp["alpha"][0], inp["beta"][0], cu, None)
    assert_close(to_host(o), o_ref, "bf16", "o")
    assert_close(to_host(Sf), S_ref, "bf16", "S_final")
