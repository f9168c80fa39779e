"""GPU parity of the KDA forward with the output gate and norm of Eq. 15 (through
chimera_kda_fwd_gated) against the fp64 oracle: kda_ref, then gated_rmsnorm_ref."""
import numpy as np
import pytest

import workloads as wl
from oracle import conv_ref, gated_rmsnorm_ref, kda_ref, l2norm_ref, round_bf16_ref
from tests.gpu_util import assert_close, to_device, to_host

pytestmark = pytest.mark.gpu

EPS = 1e-6


@pytest.fixture(scope="module")
def chm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_recurrence_mshortconv_amd as m
    m.lib()
    return m


def _bf16_case(rng, B, T, H, d):
    r = lambda *s: wl.round_to_bf16(rng.standard_normal(s).astype(np.float32))
    q, k, v, gate = r(B, T, H, d), r(B, T, H, d), r(B, T, H, d), r(B, T, H, d)
    la = -0.05 * np.logaddexp(0, rng.standard_normal((B, T, H, d))).astype(np.float32)
    alpha = wl.round_to_bf16(np.exp(la).astype(np.float32))
    beta = wl.round_to_bf16((1 / (1 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32))
    S0 = (0.1 * rng.standard_normal((B, H, d, d))).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    return q, k, v, alpha, beta, S0, gate, w


def _gate_view(gate, fused: bool):
    """The gate on the device: contiguous (the fused path), or a view 4 elements into a
    wider row (token stride H*d + 4, base 8 bytes past 16-byte alignment: the separate pass)."""
    import torch
    B, T, H, d = gate.shape
    if fused:
        return to_device(gate, "bf16")
    wide = torch.zeros(B, T, H * d + 4, dtype=torch.bfloat16, device="cuda")
    wide[:, :, 4:] = to_device(gate.reshape(B, T, H * d), "bf16")
    return wide[:, :, 4:].view(B, T, H, d)


@pytest.mark.parametrize("T", [65, 343, 1000])
@pytest.mark.parametrize("no_split", [False, True])
@pytest.mark.parametrize("fused", [True, False])
def test_gated_chunked(chm, T, no_split, fused):
    import torch
    rng = np.random.default_rng(100 + T)
    B, H, d = 2, 2, 128
    q, k, v, alpha, beta, S0, gate, w = _bf16_case(rng, B, T, H, d)
    dev = lambda a: to_device(a, "bf16")
    o, Sf = chm.kda_fwd(dev(q), dev(k), dev(v), dev(alpha), dev(beta), torch.from_numpy(S0).cuda(),
                        no_split=no_split, gate=_gate_view(gate, fused), norm_weight=torch.from_numpy(w).cuda(),
                        norm_eps=EPS)
    o_ref, S_ref = kda_ref(l2norm_ref(q), l2norm_ref(k), v, alpha, beta, S0)
    y_ref = gated_rmsnorm_ref(o_ref, gate, w, EPS)
    assert np.isfinite(to_host(o)).all()
    assert_close(to_host(o), y_ref, "bf16", f"gated o T={T}")
    assert_close(to_host(Sf), S_ref, "bf16", f"S_final T={T}")


def test_gated_head_size_64(chm):
    """64-channel heads: the chunked kernels, then the separate gate and norm pass (the fused one
    takes 128-channel heads); the norm runs over each head's 64 channels."""
    import torch
    rng = np.random.default_rng(99)
    B, T, H, d = 2, 300, 3, 64
    q, k, v, alpha, beta, S0, gate, w = _bf16_case(rng, B, T, H, d)
    dev = lambda a: to_device(a, "bf16")
    marks = chm.Marks(8)
    o, Sf = chm.kda_fwd(dev(q), dev(k), dev(v), dev(alpha), dev(beta), torch.from_numpy(S0).cuda(),
                        gate=dev(gate), norm_weight=torch.from_numpy(w).cuda(), norm_eps=EPS, marks=marks)
    torch.cuda.synchronize()
    names = [n for n, _ in marks.kernels()]
    assert "kda_out_kernel" in names and "kda_gate_norm_kernel" in names, names
    o_ref, S_ref = kda_ref(l2norm_ref(q), l2norm_ref(k), v, alpha, beta, S0)
    assert_close(to_host(o), gated_rmsnorm_ref(o_ref, gate, w, EPS), "bf16", "gated o d=64")
    assert_close(to_host(Sf), S_ref, "bf16", "S_final d=64")


def test_gated_tiny_fp32_pipeline(chm):
    """The fp32 text workload end to end with the gate (token-by-token kernel, then the
    gate/norm pass)."""
    import torch
    w = wl.WORKLOADS[0]
    inp = wl.make_inputs(w)
    gate, nw = wl.make_gate(w)
    y = chm.mshortconv_fwd(to_device(inp["x"], "f32"), torch.from_numpy(inp["w_text"]),
                           torch.from_numpy(inp["w_vis"]), inp["segments"])
    q, k, v = chm.split_qkv(y, w.H, w.d)
    o, Sf = chm.kda_fwd(q, k, v, to_device(inp["alpha"], "f32"), to_device(inp["beta"], "f32"), None,
                        gate=to_device(gate, "f32"), norm_weight=torch.from_numpy(nw).cuda(), norm_eps=EPS)
    y_ref = conv_ref(inp["x"], inp["w_text"], inp["w_vis"], inp["segments"])
    parts = y_ref.reshape(w.B, w.T, 3, w.H, w.d)
    o_ref, S_ref = kda_ref(l2norm_ref(parts[:, :, 0]), l2norm_ref(parts[:, :, 1]), parts[:, :, 2],
                           inp["alpha"], inp["beta"], None)
    assert_close(to_host(o), gated_rmsnorm_ref(o_ref, gate, nw, EPS), "f32", "gated o")
    assert_close(to_host(Sf), S_ref, "f32", "S_final")


def test_gated_sequential_bf16_no_weight(chm):
    """bf16 on the token-by-token kernel (dk = dv = 64), no gain, a large epsilon."""
    rng = np.random.default_rng(9)
    B, T, H, d = 1, 150, 3, 64
    q, k, v, alpha, beta, S0, gate, _ = _bf16_case(rng, B, T, H, d)
    dev = lambda a: to_device(a, "bf16")
    import torch
    o, _ = chm.kda_fwd(dev(q), dev(k), dev(v), dev(alpha), dev(beta), torch.from_numpy(S0).cuda(),
                       gate=dev(gate), norm_eps=0.05)
    o_ref, _ = kda_ref(l2norm_ref(q), l2norm_ref(k), v, alpha, beta, S0)
    assert_close(to_host(o), gated_rmsnorm_ref(o_ref, gate, None, 0.05), "bf16", "gated o")


@pytest.mark.parametrize("fused", [True, False])
def test_gated_timed_marks(chm, fused):
    """The gated timing entry point names its kernels and matches the untimed call."""
    import torch
    rng = np.random.default_rng(12)
    B, T, H, d = 1, 64 * 12 + 5, 16, 128
    q, k, v, alpha, beta, S0, gate, w = _bf16_case(rng, B, T, H, d)
    dev = lambda a: to_device(a, "bf16")
    args = [dev(a) for a in (q, k, v, alpha, beta)] + [torch.from_numpy(S0).cuda()]
    g = _gate_view(gate, fused)
    kw = dict(gate=g, norm_weight=torch.from_numpy(w).cuda(), norm_eps=EPS)
    o1, S1 = chm.kda_fwd(*args, **kw)
    m = chm.Marks(6)
    o2, S2 = chm.kda_fwd(*args, marks=m, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    names = [n for n, _ in m.kernels()]
    tail = ["kda_out_gated_kernel"] if fused else ["kda_out_kernel", "kda_gate_norm_kernel"]
    assert names == ["kda_sum_kernel", "kda_combine_kernel"] + tail


def test_gated_full_image_workload_sampled_head(chm):
    """conv then gated KDA at the full image workload (65,792 tokens, 16 heads) in the
    bench's launch configuration; the oracle recomputes one whole head."""
    import torch
    w = wl.WORKLOADS[2]
    inp = wl.make_inputs(w)
    gate, nw = wl.make_gate(w)
    head = 7
    y = chm.mshortconv_fwd(to_device(inp["x"], "bf16"), torch.from_numpy(inp["w_text"]),
                           torch.from_numpy(inp["w_vis"]), inp["segments"])
    q, k, v = chm.split_qkv(y, w.H, w.d)
    o, _ = chm.kda_fwd(q, k, v, to_device(inp["alpha"], "bf16"), to_device(inp["beta"], "bf16"), None,
                       gate=to_device(gate, "bf16"), norm_weight=torch.from_numpy(nw).cuda(), norm_eps=EPS)
    o_got = to_host(o[:, :, [head]])
    del y, o
    HD = w.H * w.d
    chans = np.concatenate([part * HD + head * w.d + np.arange(w.d) for part in range(3)])
    y_ref = round_bf16_ref(conv_ref(inp["x"][:, :, chans], inp["w_text"][chans], inp["w_vis"][chans],
                                    inp["segments"]))
    parts = y_ref.reshape(w.B, w.T, 3, 1, w.d)
    o_ref, _ = kda_ref(l2norm_ref(parts[:, :, 0]), l2norm_ref(parts[:, :, 1]), parts[:, :, 2],
                       inp["alpha"][:, :, [head]], inp["beta"][:, :, [head]], None)
    assert_close(o_got, gated_rmsnorm_ref(o_ref, gate[:, :, [head]], nw, EPS), "bf16", "gated o, image_4096")
