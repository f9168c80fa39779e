"""The chunked form the HIP kernels compute, checked in numpy against the oracle (CPU only).

This is a design check, not part of the oracle: it restates, in fp64 (and
once in fp32 to check the exponent ranges), the chunk algorithm the kernels
implement, derived from Eq. 14 (Chimera page 1, section 3.3):

Within a chunk of n tokens entering with state S, let g_r = sum_{i<=r} log a_i
(per key channel). Then, with u_r = beta_r (v_r - S_{r-1}^T Diag(a_r) k_r),

    S_r = Diag(e^{g_r}) (S + sum_{i<=r} (k_i * e^{-g_i}) u_i^T)
    (I + A) U = diag(beta) V - diag(beta) (K * e^{g}) S,
        A_ri = beta_r sum_c k_rc k_ic e^{g_rc - g_ic}   (i < r)
    O = (Q * e^{g}) S + Aqk U,  Aqk_ri = sum_c q_rc k_ic e^{g_rc - g_ic}   (i <= r)
    S_next = Diag(e^{g_n}) S + (K * e^{g_n - g})^T U

The pairwise factors e^{g_r - g_i} are split around a reference point inside
each 16-token row block, so no factored operand leaves the range of a
16-token span. The sequence-parallel variant runs each segment of chunks from
[S | M] = [0 | I] to get (S_seg, M_seg), combines S_start(p+1) = M_p S_start(p)
+ S_p, and reruns each segment from its S_start.
"""
import numpy as np
import pytest

from oracle import kda_ref, l2norm_ref

SUB = 16


def _chunk_step(Q, K, V, la, beta, S, dt=np.float64):
    """One chunk (rows padded to a multiple of SUB with k=q=v=0, log a=0, beta=0)."""
    n, dk = K.shape
    g = np.cumsum(la.astype(dt), axis=0).astype(dt)
    nb = n // SUB
    ref_rows = np.minimum(np.arange(nb) * SUB + SUB // 2, n - 1)
    ref = g[ref_rows]                                          # [nb, dk]
    blk = np.arange(n) // SUB
    e_row = np.exp(g - ref[blk]).astype(dt)                   # e^{g_r - m_I}
    e_col = np.exp(ref[blk] - g).astype(dt)                   # e^{m_J - g_i}
    Kr, Qr, Kcb = K * e_row, Q * e_row, K * e_col
    A = np.zeros((n, n), dt)
    Aqk = np.zeros((n, n), dt)
    for I in range(nb):
        ri = slice(I * SUB, (I + 1) * SUB)
        for J in range(I + 1):
            cj = slice(J * SUB, (J + 1) * SUB)
            P = np.exp(ref[I] - ref[J]).astype(dt)            # <= 1 for J <= I
            Kc = Kcb[cj] * P
            A[ri, cj] = Kr[ri] @ Kc.T
            Aqk[ri, cj] = Qr[ri] @ Kc.T
    A = np.tril(A, -1) * beta[:, None]
    Aqk = np.tril(Aqk, 0)
    Tm = np.linalg.inv(np.eye(n, dtype=dt) + A).astype(dt)
    eg = np.exp(g).astype(dt)
    W = Tm @ (beta[:, None] * K * eg)
    Ut = Tm @ (beta[:, None] * V)
    U = Ut - W @ S
    O = (Q * eg) @ S + Aqk @ U
    Kt = K * np.exp(g[-1] - g).astype(dt)
    S_next = eg[-1][:, None] * S + Kt.T @ U
    return O, S_next


def _pad(a, n, fill=0.0):
    out = np.full((n,) + a.shape[1:], fill, dtype=a.dtype)
    out[:a.shape[0]] = a
    return out


def chunked_head(q, k, v, alpha, beta, S0, C=64, dt=np.float64):
    T, dk = k.shape
    S = S0.astype(dt).copy()
    o = np.zeros(v.shape, dt)
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        sl = slice(c0, c0 + n)
        O, S = _chunk_step(_pad(q[sl].astype(dt), C), _pad(k[sl].astype(dt), C), _pad(v[sl].astype(dt), C),
                           _pad(np.log(alpha[sl]).astype(dt), C), _pad(beta[sl].astype(dt), C), S, dt)
        o[sl] = O[:n]
    return o, S


def segmented_head(q, k, v, alpha, beta, S0, C=64, seg_chunks=3):
    T, dk = k.shape
    dv = v.shape[1]
    n_chunks = -(-T // C)
    bounds = [(p * seg_chunks * C, min(T, (p + 1) * seg_chunks * C)) for p in range(-(-n_chunks // seg_chunks))]
    summaries = []
    for a, b in bounds:                                        # phase 1: [S | M] from [0 | I]
        SM = np.concatenate([np.zeros((dk, dv)), np.eye(dk)], axis=1)
        vv = np.concatenate([v[a:b], np.zeros((b - a, dk))], axis=1)
        _, SM = chunked_head(q[a:b], k[a:b], vv, alpha[a:b], beta[a:b], SM, C)
        summaries.append((SM[:, :dv], SM[:, dv:]))
    starts = [S0]
    for S_p, M_p in summaries:                                 # phase 2: combine
        starts.append(M_p @ starts[-1] + S_p)
    o = np.zeros((T, dv))
    for (a, b), S_st in zip(bounds, starts):                   # phase 3: rerun from S_start
        o[a:b], _ = chunked_head(q[a:b], k[a:b], v[a:b], alpha[a:b], beta[a:b], S_st, C)
    return o, starts[-1]


def _inputs(rng, T, dk, dv, scale):
    q = l2norm_ref(rng.standard_normal((1, T, 1, dk)))
    k = l2norm_ref(rng.standard_normal((1, T, 1, dk)))
    v = rng.standard_normal((1, T, 1, dv))
    alpha = np.exp(-scale * np.logaddexp(0, rng.standard_normal((1, T, 1, dk))))
    beta = 1 / (1 + np.exp(-rng.standard_normal((1, T, 1))))
    S0 = 0.1 * rng.standard_normal((1, 1, dk, dv))
    return q, k, v, alpha, beta, S0


@pytest.mark.parametrize("T,scale", [(200, 1.0), (64, 0.05), (130, 0.05), (17, 1.0)])
def test_chunked_equals_token_loop(T, scale):
    rng = np.random.default_rng(T)
    q, k, v, alpha, beta, S0 = _inputs(rng, T, 32, 24, scale)
    o_ref, S_ref = kda_ref(q, k, v, alpha, beta, S0)
    o, S = chunked_head(q[0, :, 0], k[0, :, 0], v[0, :, 0], alpha[0, :, 0], beta[0, :, 0], S0[0, 0])
    np.testing.assert_allclose(o, o_ref[0, :, 0], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(S, S_ref[0, 0], rtol=1e-10, atol=1e-12)


def test_segmented_equals_token_loop():
    rng = np.random.default_rng(5)
    q, k, v, alpha, beta, S0 = _inputs(rng, 64 * 7 + 23, 16, 16, 0.3)
    o_ref, S_ref = kda_ref(q, k, v, alpha, beta, S0)
    o, S = segmented_head(q[0, :, 0], k[0, :, 0], v[0, :, 0], alpha[0, :, 0], beta[0, :, 0], S0[0, 0])
    np.testing.assert_allclose(o, o_ref[0, :, 0], rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(S, S_ref[0, 0], rtol=1e-9, atol=1e-11)


def test_strong_decay_stays_finite_in_fp32():
    """log a = -5 per token for every channel: spans inside a 16-token block
    reach at most 8 * 5 = 40 in the exponent, far inside fp32's range."""
    rng = np.random.default_rng(9)
    T, dk, dv = 128, 16, 8
    q, k, v, _, beta, S0 = _inputs(rng, T, dk, dv, 1.0)
    alpha = np.full((1, T, 1, dk), np.exp(-5.0))
    o_ref, S_ref = kda_ref(q, k, v, alpha, beta, S0)
    o, S = chunked_head(q[0, :, 0], k[0, :, 0], v[0, :, 0], alpha[0, :, 0], beta[0, :, 0], S0[0, 0],
                        dt=np.float32)
    assert np.isfinite(o).all() and np.isfinite(S).all()
    np.testing.assert_allclose(o, o_ref[0, :, 0], rtol=1e-4, atol=1e-5)
