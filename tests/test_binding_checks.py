"""The Python binding rejects bad tensors before any call reaches the library (CPU only).

Every tensor here lives in host memory: a wrapper that let one through would hand a host
pointer to a kernel. Each case breaks one argument of an otherwise valid call and expects a
ValueError naming it; the valid call itself stops at the GPU check.
"""
import pytest
import torch

import linear_attention_recurrence_mshortconv_amd as chm

B, T, H, D = 1, 6, 2, 4
bf = torch.bfloat16


def _kda_args():
    y = torch.zeros(B, T, 3 * H * D, dtype=bf)
    q, k, v = chm.split_qkv(y, H, D)
    return dict(q=q, k=k, v=v, alpha=torch.ones(B, T, H, D, dtype=bf), beta=torch.zeros(B, T, H, dtype=bf))


def _fwd(**over):
    a = _kda_args()
    a.update(over)
    return chm.kda_fwd(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a.get("S0"), out=a.get("out"),
                       state_out=a.get("state_out"))


def test_kda_fwd_valid_layout_stops_at_gpu_check():
    with pytest.raises(ValueError, match="GPU tensor"):
        _fwd()


@pytest.mark.parametrize("name,bad,msg", [
    ("alpha", torch.ones(1, 1, H, D, dtype=bf).expand(B, T, H, D), "alpha must be contiguous"),
    ("alpha", torch.ones(B, T, H, D, dtype=torch.float32), "alpha: dtype"),
    ("beta", torch.zeros(B, T, H + 1, dtype=bf), "beta: shape"),
    ("S0", torch.zeros(B, H, D, D, dtype=bf), "S0: dtype"),
    ("S0", torch.zeros(B, H, D, 1).expand(B, H, D, D), "S0 must be contiguous"),
    ("out", torch.zeros(B, T, H, D + 1, dtype=bf), "out: shape"),
    ("state_out", torch.zeros(B, H, D, D, dtype=torch.float64), "state_out: dtype"),
])
def test_kda_fwd_rejects(name, bad, msg):
    with pytest.raises(ValueError, match=msg):
        _fwd(**{name: bad})


def test_kda_fwd_rejects_overlapping_tokens():
    a = _kda_args()
    k = torch.zeros(B, 1, H, D, dtype=bf).expand(B, T, H, D)        # every token at one address
    with pytest.raises(ValueError):
        chm.kda_fwd(k, k, k, a["alpha"], a["beta"])


def test_kda_bwd_rejects_expanded_gradients():
    a = _kda_args()
    dout = torch.zeros(1, 1, 1, D, dtype=bf).expand(B, T, H, D)     # stride 0: would read past the buffer
    with pytest.raises(ValueError, match="dout must be contiguous"):
        chm.kda_bwd(a["q"], a["k"], a["v"], a["alpha"], a["beta"], None, dout, grads=chm.split_qkv(
            torch.zeros(B, T, 3 * H * D, dtype=bf), H, D))
    with pytest.raises(ValueError, match="dS_final: dtype"):
        chm.kda_bwd(a["q"], a["k"], a["v"], a["alpha"], a["beta"], None, torch.zeros(B, T, H, D, dtype=bf),
                    torch.zeros(B, H, D, D, dtype=bf))
    with pytest.raises(ValueError, match="alpha must be contiguous"):
        chm.kda_bwd(a["q"], a["k"], a["v"], torch.ones(B, T, H, 2 * D, dtype=bf)[..., ::2], a["beta"], None,
                    torch.zeros(B, T, H, D, dtype=bf))


def test_kda_bwd_varlen_rejects():
    y = torch.zeros(T, 3 * H * D, dtype=bf)
    q, k, v = y.view(T, 3, H, D).unbind(1)
    al, be = torch.ones(T, H, D, dtype=bf), torch.zeros(T, H, dtype=bf)
    with pytest.raises(ValueError, match="dout must be contiguous"):
        chm.kda_bwd_varlen(q, k, v, al, be, [0, 2, T], None, torch.zeros(1, 1, D, dtype=bf).expand(T, H, D),
                           grads=(torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)))
    with pytest.raises(ValueError, match="cu_seqlens"):
        chm.kda_bwd_varlen(q, k, v, al, be, [0, 4, 2, T], None, torch.zeros(T, H, D, dtype=bf))


def test_kda_fwd_varlen_rejects():
    y = torch.zeros(T, 3 * H * D, dtype=bf)
    q, k, v = y.view(T, 3, H, D).unbind(1)
    al, be = torch.ones(T, H, D, dtype=bf), torch.zeros(T, H, dtype=bf)
    with pytest.raises(ValueError, match="cu_seqlens"):
        chm.kda_fwd_varlen(q, k, v, al, be, [0, 3, T - 1])
    with pytest.raises(ValueError, match="S0: shape"):
        chm.kda_fwd_varlen(q, k, v, al, be, [0, 3, T], torch.zeros(3, H, D, D))


def test_gate_norm_bwd_rejects():
    o = torch.zeros(B, T, H, D, dtype=bf)
    with pytest.raises(ValueError, match="dy must be contiguous"):
        chm.gate_norm_bwd(o, o, None, torch.zeros(1, 1, 1, D, dtype=bf).expand(B, T, H, D))
    with pytest.raises(ValueError, match="norm_weight: dtype"):
        chm.gate_norm_bwd(o, o, torch.ones(D, dtype=bf), o)


def test_conv_wrappers_reject():
    C = 3 * H * D
    x = torch.zeros(B, T, C, dtype=bf)
    segs = [dict(kind=0, start=0, length=T)]
    wt, wv = torch.zeros(C, 4), torch.zeros(C, 27)
    with pytest.raises(ValueError, match="dy must be contiguous"):
        chm.mshortconv_bwd(x, torch.zeros(1, 1, C, dtype=bf).expand(B, T, C), wt, wv, segs)
    with pytest.raises(ValueError, match="w_vis: shape"):
        chm.mshortconv_fwd(x, wt, torch.zeros(C, 9), segs)
    with pytest.raises(ValueError, match="x must be contiguous"):
        chm.mshortconv_fwd(torch.zeros(B, T, 2 * C, dtype=bf)[..., ::2], wt, wv, segs)
    with pytest.raises(ValueError, match="GPU tensor"):
        chm.mshortconv_fwd(x, wt, wv, segs)


def test_kda_fwd_conv_rejects():
    C = 3 * H * D
    x = torch.zeros(B, T, C, dtype=bf)
    segs = [dict(kind=0, start=0, length=T)]
    wt, wv = torch.zeros(C, 4), torch.zeros(C, 27)
    al, be = torch.ones(B, T, H, D, dtype=bf), torch.zeros(B, T, H, dtype=bf)
    with pytest.raises(ValueError, match="beta must be contiguous"):
        chm.kda_fwd_conv(x, wt, wv, segs, al, torch.zeros(B, T, 1, dtype=bf).expand(B, T, H), H=H, dk=D, dv=D)
    with pytest.raises(ValueError, match="channels"):
        chm.kda_fwd_conv(x, wt, wv, segs, al, be, H=H, dk=D, dv=2 * D)
    with pytest.raises(ValueError, match="w_text: shape"):
        chm.kda_fwd_conv(x, torch.zeros(C, 3), wv, segs, al, be, H=H, dk=D, dv=D)
    with pytest.raises(ValueError, match="GPU tensor"):
        chm.kda_fwd_conv(x, wt, wv, segs, al, be, H=H, dk=D, dv=D)
