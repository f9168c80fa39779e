"""Pins for the KDA oracle (CPU only).

The oracle's token loop is checked against: hand-computed fixtures of Eq. 14
/ Eq. 15 (tests/golden/kda_hand_examples.json), closed forms (no write; no
decay and orthonormal keys), an unrolled dense-matrix formulation
S_T = Phi_{T,0} S0 + sum_i Phi_{T,i} beta_i k_i v_i^T evaluated in fp64 and in
exact rational arithmetic, and properties of the definition (linearity in
(V, S0), split/resume, independence of batch items and heads).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import kda_ref, kda_varlen_ref, l2norm_ref


def _rand_inputs(rng, B, T, H, dk, dv, s0=True, log_alpha_scale=1.0):
    q = l2norm_ref(rng.standard_normal((B, T, H, dk)))
    k = l2norm_ref(rng.standard_normal((B, T, H, dk)))
    v = rng.standard_normal((B, T, H, dv))
    alpha = np.exp(-log_alpha_scale * np.logaddexp(0, rng.standard_normal((B, T, H, dk))))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    S0 = rng.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, alpha, beta, S0


def test_hand_examples(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "kda_hand_examples.json")))
    for ex in g["examples"]:
        k = np.array(ex["k"], dtype=np.float64)
        T, dk = k.shape
        dv = len(ex["v"][0])
        sh = lambda a, last: np.array(a, dtype=np.float64).reshape(1, T, 1, last)
        o, S = kda_ref(sh(ex["q"], dk), sh(ex["k"], dk), sh(ex["v"], dv), sh(ex["alpha"], dk),
                       np.array(ex["beta"], dtype=np.float64).reshape(1, T, 1),
                       np.array(ex["S0"], dtype=np.float64).reshape(1, 1, dk, dv))
        np.testing.assert_allclose(o.reshape(T, dv), np.array(ex["o"]), rtol=0, atol=1e-15, err_msg=ex["name"])
        np.testing.assert_allclose(S.reshape(dk, dv), np.array(ex["S_final"]), rtol=0, atol=1e-15, err_msg=ex["name"])


def test_no_decay_no_write_keeps_state():
    rng = np.random.default_rng(10)
    q, k, v, _, _, S0 = _rand_inputs(rng, 2, 9, 3, 4, 5)
    alpha = np.ones_like(k)
    beta = np.zeros(k.shape[:3])
    o, S = kda_ref(q, k, v, alpha, beta, S0)
    assert np.array_equal(S, S0)
    np.testing.assert_allclose(o, np.einsum("bhkv,bthk->bthv", S0, q), atol=1e-14)


def test_no_write_is_pure_channel_decay():
    rng = np.random.default_rng(11)
    q, k, v, alpha, _, S0 = _rand_inputs(rng, 1, 12, 2, 6, 3, log_alpha_scale=3.0)
    beta = np.zeros(k.shape[:3])
    o, S = kda_ref(q, k, v, alpha, beta, S0)
    cum = np.cumprod(alpha, axis=1)                              # prod_{j<=t} alpha_j
    np.testing.assert_allclose(S, cum[:, -1, :, :, None] * S0, rtol=1e-13)
    np.testing.assert_allclose(o, np.einsum("bhkv,bthk->bthv", S0, q * cum), rtol=1e-12, atol=1e-15)


def test_orthonormal_keys_overwrite_exactly():
    rng = np.random.default_rng(12)
    dk, dv, T = 6, 4, 5
    Q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Q[:, :T].T.reshape(1, T, 1, dk)                          # mutually orthonormal keys
    v = rng.standard_normal((1, T, 1, dv))
    q = rng.standard_normal((1, T, 1, dk))
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, S = kda_ref(q, k, v, np.ones((1, T, 1, dk)), np.ones((1, T, 1)), S0)
    K = k.reshape(T, dk)
    V = v.reshape(T, dv)
    np.testing.assert_allclose(K @ S[0, 0], V, atol=1e-12)      # k_t^T S_T = v_t^T for every t
    expect = (np.eye(dk) - K.T @ K) @ S0[0, 0] + K.T @ V
    np.testing.assert_allclose(S[0, 0], expect, atol=1e-12)


def _unrolled(q, k, v, alpha, beta, S0):
    """S_t = Phi_{t,0} S0 + sum_{i<=t} Phi_{t,i} beta_i k_i v_i^T, with
    Phi_{t,i} = prod_{j=i+1..t} (I - beta_j k_j k_j^T) Diag(alpha_j), built as
    explicit dense matrices for one (b, h)."""
    T, dk = k.shape
    mats = [(np.eye(dk) - beta[j] * np.outer(k[j], k[j])) @ np.diag(alpha[j]) for j in range(T)]
    outs, S_t = [], None
    for t in range(T):
        phi = np.eye(dk)
        for j in range(t, -1, -1):
            phi = phi @ mats[j]                                  # Phi_{t,-1} = M_t ... M_0
        S_t = phi @ S0
        for i in range(t + 1):
            phi_ti = np.eye(dk)
            for j in range(t, i, -1):
                phi_ti = phi_ti @ mats[j]
            S_t = S_t + phi_ti @ (beta[i] * np.outer(k[i], v[i]))
        outs.append(S_t.T @ q[t])
    return np.array(outs), S_t


@pytest.mark.parametrize("T", [1, 2, 5, 8])
def test_bruteforce_dense_transitions(T):
    rng = np.random.default_rng(100 + T)
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, 2, T, 2, 4, 3)
    o, S = kda_ref(q, k, v, alpha, beta, S0)
    for b in range(2):
        for h in range(2):
            ob, Sb = _unrolled(q[b, :, h], k[b, :, h], v[b, :, h], alpha[b, :, h], beta[b, :, h], S0[b, h])
            np.testing.assert_allclose(o[b, :, h], ob, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(S[b, h], Sb, rtol=1e-12, atol=1e-13)


def _frac_matmul(A, B):
    return [[sum((A[i][t] * B[t][j] for t in range(len(B))), Fraction(0)) for j in range(len(B[0]))]
            for i in range(len(A))]


def test_exact_rationals():
    """The unrolled product form in exact rational arithmetic vs the fp64 loop."""
    rng = np.random.default_rng(7)
    T, dk, dv = 4, 3, 2
    r = lambda: Fraction(int(rng.integers(-8, 9)), int(rng.integers(1, 9)))
    rp = lambda: Fraction(int(rng.integers(1, 16)), 16)           # in (0, 1)
    k = [[r() for _ in range(dk)] for _ in range(T)]
    v = [[r() for _ in range(dv)] for _ in range(T)]
    q = [[r() for _ in range(dk)] for _ in range(T)]
    alpha = [[rp() for _ in range(dk)] for _ in range(T)]
    beta = [rp() for _ in range(T)]
    S = [[r() for _ in range(dv)] for _ in range(dk)]
    S0 = [row[:] for row in S]
    o_exact = []
    for t in range(T):
        I = [[Fraction(int(i == j)) for j in range(dk)] for i in range(dk)]
        E = [[I[i][j] - beta[t] * k[t][i] * k[t][j] for j in range(dk)] for i in range(dk)]
        D = [[alpha[t][i] if i == j else Fraction(0) for j in range(dk)] for i in range(dk)]
        S = _frac_matmul(_frac_matmul(E, D), S)
        S = [[S[i][j] + beta[t] * k[t][i] * v[t][j] for j in range(dv)] for i in range(dk)]
        o_exact.append([sum((S[i][j] * q[t][i] for i in range(dk)), Fraction(0)) for j in range(dv)])
    f = lambda a: np.array([[float(x) for x in row] for row in a])
    o, Sf = kda_ref(f(q).reshape(1, T, 1, dk), f(k).reshape(1, T, 1, dk), f(v).reshape(1, T, 1, dv),
                    f(alpha).reshape(1, T, 1, dk), np.array([float(b) for b in beta]).reshape(1, T, 1),
                    f(S0).reshape(1, 1, dk, dv))
    np.testing.assert_allclose(o.reshape(T, dv), f(o_exact), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Sf.reshape(dk, dv), f(S), rtol=1e-12, atol=1e-12)


def test_linear_in_values_and_initial_state():
    rng = np.random.default_rng(13)
    q, k, v1, alpha, beta, S01 = _rand_inputs(rng, 1, 20, 2, 5, 4)
    v2 = rng.standard_normal(v1.shape)
    S02 = rng.standard_normal(S01.shape)
    o12, S12 = kda_ref(q, k, v1 + 3 * v2, alpha, beta, S01 + 3 * S02)
    o1, S1 = kda_ref(q, k, v1, alpha, beta, S01)
    o2, S2 = kda_ref(q, k, v2, alpha, beta, S02)
    np.testing.assert_allclose(o12, o1 + 3 * o2, atol=1e-11)
    np.testing.assert_allclose(S12, S1 + 3 * S2, atol=1e-11)


def test_split_and_resume():
    rng = np.random.default_rng(14)
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, 2, 30, 2, 4, 4)
    o, S = kda_ref(q, k, v, alpha, beta, S0)
    t1 = 13
    oa, Sa = kda_ref(q[:, :t1], k[:, :t1], v[:, :t1], alpha[:, :t1], beta[:, :t1], S0)
    ob, Sb = kda_ref(q[:, t1:], k[:, t1:], v[:, t1:], alpha[:, t1:], beta[:, t1:], Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob], 1), o, atol=1e-13)
    np.testing.assert_allclose(Sb, S, atol=1e-13)


def test_batch_and_heads_independent():
    rng = np.random.default_rng(15)
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, 2, 10, 3, 4, 4)
    o, S = kda_ref(q, k, v, alpha, beta, S0)
    o1, S1 = kda_ref(q[1:, :, 2:], k[1:, :, 2:], v[1:, :, 2:], alpha[1:, :, 2:], beta[1:, :, 2:], S0[1:, 2:])
    np.testing.assert_array_equal(o1, o[1:, :, 2:])
    np.testing.assert_array_equal(S1, S[1:, 2:])


def test_zero_initial_state_is_default():
    rng = np.random.default_rng(16)
    q, k, v, alpha, beta, _ = _rand_inputs(rng, 1, 6, 1, 3, 3, s0=False)
    a = kda_ref(q, k, v, alpha, beta, None)
    b = kda_ref(q, k, v, alpha, beta, np.zeros((1, 1, 3, 3)))
    np.testing.assert_array_equal(a[0], b[0])


def test_l2norm_unit_rows_and_eps():
    rng = np.random.default_rng(17)
    x = rng.standard_normal((3, 7, 16)) * 5
    y = l2norm_ref(x)
    n = np.sqrt((x * x).sum(-1))
    np.testing.assert_allclose(y, x / np.sqrt(n[..., None] ** 2 + 1e-6), rtol=1e-15)
    np.testing.assert_allclose(np.sqrt((y * y).sum(-1)), n / np.sqrt(n * n + 1e-6), rtol=1e-14)
    assert np.array_equal(l2norm_ref(np.zeros((2, 4))), np.zeros((2, 4)))


def test_l2norm_hand_examples(golden_dir):
    """l2norm_ref against hand-computed values (tests/golden/l2norm_hand_examples.json): the 3-4-5 and
    1-2-2 triangles, the zero vector, a tiny vector that shows the epsilon inside the square root, signs,
    and two heads of one token normalised on their own."""
    import json
    import os
    g = json.load(open(os.path.join(golden_dir, "l2norm_hand_examples.json")))
    for ex in g["examples"]:
        np.testing.assert_allclose(l2norm_ref(np.array(ex["x"]), g["eps"]), ex["y"], rtol=1e-15, atol=0,
                                   err_msg=ex["name"])
    np.testing.assert_allclose(l2norm_ref(np.array(g["heads"]["x"])), g["heads"]["y"], rtol=1e-15, atol=0)
    # the default epsilon is the fixture's
    np.testing.assert_allclose(l2norm_ref(np.array([3.0, 4.0])), g["examples"][0]["y"], rtol=1e-15, atol=0)


def _variant(q, k, v, alpha, beta, S0, mode):
    """Plausible misreadings of Eq. 14/15, used to show the fixtures catch them."""
    q, k, v, a, b = [np.asarray(z, dtype=np.float64) for z in (q, k, v, alpha, beta)]
    B, T, H, dk = k.shape
    S = np.array(S0, dtype=np.float64)
    o = np.empty(v.shape)
    for t in range(T):
        kt = k[:, t]
        if mode == "erase_then_decay":
            pred = np.einsum("bhkv,bhk->bhv", S, kt)
            S = S - b[:, t, :, None, None] * kt[..., None] * pred[:, :, None, :]
            S = S * a[:, t, :, :, None] + b[:, t, :, None, None] * kt[..., None] * v[:, t][:, :, None, :]
        elif mode == "exclusive_readout":
            o[:, t] = np.einsum("bhkv,bhk->bhv", S, q[:, t])
            S = S * a[:, t, :, :, None]
            pred = np.einsum("bhkv,bhk->bhv", S, kt)
            S = S + b[:, t, :, None, None] * kt[..., None] * (v[:, t] - pred)[:, :, None, :]
            continue
        elif mode == "transposed":
            S = S * a[:, t, :, :, None]
            pred = np.einsum("bhkv,bhv->bhk", S, kt)
            S = S + b[:, t, :, None, None] * kt[..., None] * (v[:, t] - pred)[:, :, None, :]
        o[:, t] = np.einsum("bhkv,bhk->bhv", S, q[:, t])
    return o, S


@pytest.mark.parametrize("mode", ["erase_then_decay", "exclusive_readout", "transposed"])
def test_fixtures_reject_plausible_misreadings(golden_dir, mode):
    g = json.load(open(os.path.join(golden_dir, "kda_hand_examples.json")))
    caught = False
    for ex in g["examples"]:
        k = np.array(ex["k"], dtype=np.float64)
        T, dk = k.shape
        dv = len(ex["v"][0])
        if mode == "transposed" and dk != dv:
            continue
        sh = lambda a, last: np.array(a, dtype=np.float64).reshape(1, T, 1, last)
        o, S = _variant(sh(ex["q"], dk), sh(ex["k"], dk), sh(ex["v"], dv), sh(ex["alpha"], dk),
                        np.array(ex["beta"], dtype=np.float64).reshape(1, T, 1),
                        np.array(ex["S0"], dtype=np.float64).reshape(1, 1, dk, dv), mode)
        if not (np.allclose(o.reshape(T, dv), ex["o"]) and np.allclose(S.reshape(dk, dv), ex["S_final"])):
            caught = True
    assert caught


def test_varlen_one_sample_is_the_plain_recurrence():
    rng = np.random.default_rng(60)
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, 1, 23, 2, 5, 3)
    o, S = kda_ref(q, k, v, alpha, beta, S0)
    o2, S2 = kda_varlen_ref(q[0], k[0], v[0], alpha[0], beta[0], [0, 23], S0)
    assert np.array_equal(o2, o[0]) and np.array_equal(S2, S)


def test_varlen_equal_samples_are_a_batch():
    rng = np.random.default_rng(61)
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, 3, 11, 2, 4, 4)
    o, S = kda_ref(q, k, v, alpha, beta, S0)
    flat = lambda x: x.reshape((33,) + x.shape[2:])
    o2, S2 = kda_varlen_ref(flat(q), flat(k), flat(v), flat(alpha), flat(beta), [0, 11, 22, 33], S0)
    assert np.array_equal(o2, flat(o)) and np.array_equal(S2, S)


def test_varlen_state_restarts_at_every_boundary():
    """A sample's outputs depend on nothing outside it; without the restart (one sample over
    the whole row) the second sample's outputs change."""
    rng = np.random.default_rng(62)
    q, k, v, alpha, beta, _ = _rand_inputs(rng, 1, 30, 2, 4, 3, s0=False)
    cu = [0, 9, 9, 30]                                          # an empty sample in the middle
    o, S = kda_varlen_ref(q[0], k[0], v[0], alpha[0], beta[0], cu)
    v2 = v.copy()
    v2[0, :9] += 5.0                                            # perturb sample 0 only
    o2, S2 = kda_varlen_ref(q[0], k[0], v2[0], alpha[0], beta[0], cu)
    assert np.array_equal(o2[9:], o[9:]) and np.array_equal(S2[1:], S[1:])
    assert np.array_equal(S[1], np.zeros_like(S[1]))            # the empty sample keeps S0 = 0
    oa, _ = kda_ref(q[:, 9:], k[:, 9:], v[:, 9:], alpha[:, 9:], beta[:, 9:], None)
    np.testing.assert_array_equal(o[9:], oa[0])
    ow, _ = kda_ref(q, k, v, alpha, beta, None)                 # no restart
    assert not np.allclose(ow[0, 9:], o[9:])
