"""Oracle for the backward pass of mShortConv, KDA and Eq. 15's gate and norm, fp64 (torch autograd).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The backward of a step is the derivative of its plain definition. The forward
definitions are restated here in torch fp64 ops, as written in ``kda.py`` and
``mshortconv.py`` (Eq. 13, Eq. 14 with page 2's parentheses, the inner
readout of Eq. 15, and Fig. 2's per-head L2 normalisation; page 1, section
3.3), and torch's reverse-mode autodiff supplies the vector-Jacobian products.
No step is blocked, fused or reordered.

``conv_torch`` is the gather formulation: y[b, p, c] = sum over taps of
w[c, tap] * x[b, idx[p, tap], c], with idx the neighbour table of
``neighbours_ref`` (-1 = zero padding); text tokens use the 4 text weights on
taps 0..3, visual tokens the 27 visual weights.
"""
from __future__ import annotations

import numpy as np
import torch

from .kda import L2_EPS, RMS_EPS
from .mshortconv import TEXT, neighbours_ref, _seg_fields

_F64 = torch.float64


def l2norm_torch(x, eps: float = L2_EPS):
    return x / torch.sqrt((x * x).sum(-1, keepdim=True) + eps)


def kda_torch(q, k, v, alpha, beta, S0=None):
    """Token loop of Eq. 14 and o_t = S_t^T q_t, differentiable. Shapes as kda_ref."""
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    S = torch.zeros(B, H, dk, dv, dtype=_F64) if S0 is None else S0
    outs = []
    for t in range(T):
        S = alpha[:, t, :, :, None] * S                              # Diag(alpha_t) S_{t-1}
        kt = k[:, t]
        u = beta[:, t, :, None] * (v[:, t] - torch.einsum("bhkv,bhk->bhv", S, kt))
        S = S + kt[:, :, :, None] * u[:, :, None, :]
        outs.append(torch.einsum("bhkv,bhk->bhv", S, q[:, t]))
    o = torch.stack(outs, dim=1) if T > 0 else torch.zeros(B, 0, H, dv, dtype=_F64)
    return o, S


def conv_torch(x, w_text, w_vis, segments):
    """mShortConv by gathering through the neighbour table (differentiable in x and w)."""
    B, T, C = x.shape
    idx = torch.from_numpy(neighbours_ref(segments, T).astype(np.int64))   # [T, 27]
    text = torch.zeros(T, dtype=torch.bool)
    for seg in segments:
        kind, start, length, _, _, _ = _seg_fields(seg)
        if kind == TEXT:
            text[start:start + length] = True
    xz = torch.cat([x, torch.zeros(B, 1, C, dtype=x.dtype)], dim=1)       # row T reads as zero
    src = torch.where(idx >= 0, idx, torch.full_like(idx, T))
    g = xz[:, src]                                                       # [B, T, 27, C]
    yv = (g * w_vis.t()[None, None]).sum(2)
    yt = (g[:, :, :4] * w_text.t()[None, None]).sum(2)
    return torch.where(text[None, :, None], yt, yv)


def kda_backward_ref(q, k, v, alpha, beta, S0, do, dS_final=None, l2norm: bool = True):
    """Gradients of (o, S_final) = KDA(normalise(q), normalise(k), v, alpha, beta, S0)
    against do [B, T, H, dv] and dS_final [B, H, dk, dv] (or None = 0).

    Returns a dict of fp64 numpy arrays: dq, dk, dv, dalpha, dbeta, dS0 (dS0 even when S0 is
    None, as the gradient of a zero initial state)."""
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), dtype=_F64, requires_grad=True)
    B, T, H, dk = np.shape(k)
    dv = np.shape(v)[-1]
    qt, kt, vt, at, bt = t(q), t(k), t(v), t(alpha), t(beta)
    s0 = t(np.zeros((B, H, dk, dv)) if S0 is None else S0)
    qn, kn = (l2norm_torch(qt), l2norm_torch(kt)) if l2norm else (qt, kt)
    o, S = kda_torch(qn, kn, vt, at, bt, s0)
    loss = (o * torch.as_tensor(np.asarray(do, dtype=np.float64))).sum()
    if dS_final is not None:
        loss = loss + (S * torch.as_tensor(np.asarray(dS_final, dtype=np.float64))).sum()
    grads = torch.autograd.grad(loss, [qt, kt, vt, at, bt, s0], allow_unused=True)
    names = ["dq", "dk", "dv", "dalpha", "dbeta", "dS0"]
    shapes = [qt.shape, kt.shape, vt.shape, at.shape, bt.shape, s0.shape]
    return {n: (np.zeros(sh) if g is None else g.detach().numpy()) for n, g, sh in zip(names, grads, shapes)}


def conv_backward_ref(x, w_text, w_vis, segments, dy):
    """Gradients of y = mShortConv(x) against dy: dict of dx [B, T, C], dw_text [C, 4],
    dw_vis [C, 27] (fp64 numpy)."""
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), dtype=_F64, requires_grad=True)
    xt, wt, wv = t(x), t(w_text), t(w_vis)
    y = conv_torch(xt, wt, wv, segments)
    loss = (y * torch.as_tensor(np.asarray(dy, dtype=np.float64))).sum()
    dx, dwt, dwv = torch.autograd.grad(loss, [xt, wt, wv], allow_unused=True)
    z = lambda g, ref: np.zeros(ref.shape) if g is None else g.detach().numpy()
    return {"dx": z(dx, xt), "dw_text": z(dwt, wt), "dw_vis": z(dwv, wv)}


def gated_rmsnorm_torch(o, gate, weight=None, eps: float = RMS_EPS):
    """Sigmoid(gate) * RMSNorm(o) over the last axis (Eq. 15 without W_o), differentiable."""
    rms = torch.sqrt((o * o).mean(-1, keepdim=True) + eps)
    y = o / rms
    if weight is not None:
        y = y * weight
    return y * torch.sigmoid(gate)


def gate_norm_backward_ref(o, gate, weight, dy, eps: float = RMS_EPS):
    """Gradients of y = Sigmoid(gate) * RMSNorm(o) * weight against dy: dict of do, dgate (the
    shapes of o and gate) and dweight ([dv], summed over all rows; with weight None, the
    gradient with respect to a gain of ones), fp64 numpy."""
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), dtype=_F64, requires_grad=True)
    ot, gt = t(o), t(gate)
    wt = t(np.ones(np.shape(o)[-1]) if weight is None else weight)
    y = gated_rmsnorm_torch(ot, gt, wt, eps)
    loss = (y * torch.as_tensor(np.asarray(dy, dtype=np.float64))).sum()
    do, dg, dw = torch.autograd.grad(loss, [ot, gt, wt])
    return {"do": do.detach().numpy(), "dgate": dg.detach().numpy(), "dweight": dw.detach().numpy()}
