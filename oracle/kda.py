"""Oracle for the Kimi Delta Attention (KDA) recurrence, fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition (Chimera, page 1, section 3.3, Eq. 14 and the inner term of
Eq. 15; Eq. 14's parentheses are garbled on page 1 and printed cleanly in
page 2's LaTeX):

    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
    o_t = S_t^T q_t

per head, with S_t in R^{d_k x d_v}, alpha_t in (0, 1)^{d_k} one decay per key
channel, beta_t in (0, 1) one scalar per head and token. The readout uses the
state after token t. The state starts from S0 (zero at a sample boundary,
page 1, section 3.3).

Expanding the product gives the form the loop uses, with no other change:

    S <- Diag(alpha_t) S                      (decay first)
    S <- S + beta_t k_t (v_t - S^T k_t)^T     (erase and write on the decayed state)
    o_t = S^T q_t

``l2norm_ref`` is the per-(token, head) L2 normalisation that Fig. 2 (page 1)
draws between mShortConv and the recurrence; its epsilon (1e-6 inside the
square root) is a reading made here, not the pages'.

``kda_varlen_ref`` runs several samples packed into one token row: the state
restarts (from that sample's S0, zero by default) at every packed sample
boundary (page 1, section 3.3), so each sample is the plain recurrence on its
own tokens.

``gated_rmsnorm_ref`` is the rest of the KDA output in Eq. 15 (page 1, section
3.3) short of the output projection W_o: Sigmoid(gate) times RMSNorm(S_t^T q_t),
where gate is the W_gate projection of the layer input (taken as an input
here). Eq. 15 does not say over which channels the norm runs, whether it has a
gain or what its epsilon is; the reading here is the usual one for a
multi-head output: each head's d_v channels on their own, a gain vector of
length d_v shared by the heads, epsilon inside the square root.
"""
from __future__ import annotations

import numpy as np

L2_EPS = 1e-6
RMS_EPS = 1e-6


def l2norm_ref(x: np.ndarray, eps: float = L2_EPS) -> np.ndarray:
    """x / sqrt(sum(x^2) + eps) over the last axis, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def kda_ref(q, k, v, alpha, beta, S0=None):
    """Token-by-token KDA forward.

    q, k, alpha: [B, T, H, dk]; v: [B, T, H, dv]; beta: [B, T, H];
    S0: [B, H, dk, dv] or None (zeros). Everything is used exactly in fp64.
    Returns (o [B, T, H, dv], S_final [B, H, dk, dv]), both fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    a = np.asarray(alpha, dtype=np.float64)
    b = np.asarray(beta, dtype=np.float64)
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64, copy=True)
    o = np.empty((B, T, H, dv))
    for t in range(T):
        S *= a[:, t, :, :, None]                                   # Diag(alpha_t) S_{t-1}
        kt = k[:, t]                                               # [B, H, dk]
        pred = np.einsum("bhkv,bhk->bhv", S, kt)                   # S^T k_t
        u = b[:, t, :, None] * (v[:, t] - pred)                    # beta_t (v_t - S^T k_t)
        S += kt[:, :, :, None] * u[:, :, None, :]                  # + k_t u^T
        o[:, t] = np.einsum("bhkv,bhk->bhv", S, q[:, t])           # S_t^T q_t
    return o, S


def gated_rmsnorm_ref(o, gate, weight=None, eps: float = RMS_EPS):
    """Sigmoid(gate) * RMSNorm(o) per (token, head), in fp64 (Eq. 15 without W_o).

    o, gate: [..., dv]; weight: [dv] or None (ones).
    RMSNorm(x) = x / sqrt(mean(x^2) + eps) * weight over the last axis.
    """
    o = np.asarray(o, dtype=np.float64)
    g = np.asarray(gate, dtype=np.float64)
    w = np.ones(o.shape[-1]) if weight is None else np.asarray(weight, dtype=np.float64)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o / rms * w / (1.0 + np.exp(-g))


def kda_varlen_ref(q, k, v, alpha, beta, cu_seqlens, S0=None):
    """Packed samples: q, k, alpha [T, H, dk]; v [T, H, dv]; beta [T, H]; cu_seqlens the N + 1
    sample offsets (0 = c_0 <= c_1 <= ... <= c_N = T); S0 [N, H, dk, dv] or None.
    Sample n is kda_ref on tokens [c_n, c_{n+1}) from S0[n] (zeros if None).
    Returns (o [T, H, dv], S_final [N, H, dk, dv]) in fp64."""
    v = np.asarray(v, dtype=np.float64)
    T, H, dv = v.shape
    dk = np.shape(k)[-1]
    cu = [int(c) for c in cu_seqlens]
    N = len(cu) - 1
    o = np.empty((T, H, dv))
    S = np.empty((N, H, dk, dv))
    for n in range(N):
        a, b = cu[n], cu[n + 1]
        s0 = None if S0 is None else np.asarray(S0, dtype=np.float64)[n:n + 1]
        on, Sn = kda_ref(np.asarray(q)[None, a:b], np.asarray(k)[None, a:b], v[None, a:b],
                         np.asarray(alpha)[None, a:b], np.asarray(beta)[None, a:b], s0)
        o[a:b] = on[0]
        S[n] = Sn[0]
    return o, S
