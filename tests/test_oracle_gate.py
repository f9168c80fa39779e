"""Pins for the Eq. 15 output gate and norm of the oracle (CPU only).

``gated_rmsnorm_ref`` is checked against torch's own RMSNorm and sigmoid in
fp64 (a library special case), closed forms (a constant row normalises to its
sign times the gain, with epsilon c / sqrt(c^2 + eps); sigmoid(ln 3) = 3/4),
the scale and sign properties of the definition per head, and the output RMS.
"""
import math

import numpy as np
import pytest
import torch

from oracle import gated_rmsnorm_ref


def test_matches_torch_rms_norm_and_sigmoid():
    rng = np.random.default_rng(40)
    o = rng.standard_normal((3, 17, 4, 32)) * rng.uniform(0.01, 5.0, size=(3, 17, 4, 1))
    g = rng.standard_normal((3, 17, 4, 32)) * 3
    w = rng.standard_normal(32)
    for eps in (0.0, 1e-6, 0.3):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(o), (32,), weight=torch.from_numpy(w), eps=eps)
        ref = (ref * torch.sigmoid(torch.from_numpy(g))).numpy()
        np.testing.assert_allclose(gated_rmsnorm_ref(o, g, w, eps), ref, rtol=1e-13, atol=1e-15)


def test_constant_row_closed_form():
    dv = 8
    w = np.arange(1, dv + 1, dtype=np.float64)
    for c in (-2.5, 0.75, 3.0):
        o = np.full((1, dv), c)
        g = np.full((1, dv), math.log(3.0))          # sigmoid(ln 3) = 3/4
        np.testing.assert_allclose(gated_rmsnorm_ref(o, g, w, 0.0), [np.sign(c) * w * 0.75], rtol=1e-15)
        eps = 0.2
        np.testing.assert_allclose(gated_rmsnorm_ref(o, g, w, eps), [c / math.sqrt(c * c + eps) * w * 0.75],
                                   rtol=1e-15)


def test_each_head_is_normalised_on_its_own():
    rng = np.random.default_rng(41)
    o = rng.standard_normal((5, 3, 16))
    g = rng.standard_normal((5, 3, 16))
    w = rng.uniform(0.5, 2.0, 16)
    lam = np.array([1e-3, 1.0, 40.0])[None, :, None]   # a different scale per head
    y = gated_rmsnorm_ref(o, g, w, 0.0)
    np.testing.assert_allclose(gated_rmsnorm_ref(o * lam, g, w, 0.0), y, rtol=1e-13)
    np.testing.assert_allclose(gated_rmsnorm_ref(-o, g, w, 0.0), -y, rtol=1e-15)


def test_unit_output_rms_without_gate_and_gain():
    rng = np.random.default_rng(42)
    o = rng.standard_normal((7, 2, 64)) * 9
    y = gated_rmsnorm_ref(o, np.full(o.shape, 60.0), None, 0.0)   # sigmoid(60) = 1 in fp64
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-14)


def test_zero_row_stays_zero():
    y = gated_rmsnorm_ref(np.zeros((2, 4)), np.zeros((2, 4)), None, 1e-6)
    assert np.array_equal(y, np.zeros((2, 4)))


@pytest.mark.parametrize("wrong", ["all_heads", "no_eps", "sigmoid_of_minus_gate"])
def test_pins_reject_plausible_misreadings(wrong):
    rng = np.random.default_rng(43)
    o = rng.standard_normal((4, 3, 8)) * np.array([0.1, 1.0, 7.0])[None, :, None]
    g = rng.standard_normal((4, 3, 8))
    w = rng.uniform(0.5, 2.0, 8)
    eps = 0.5
    if wrong == "all_heads":
        flat = o.reshape(4, 24)
        bad = (flat / np.sqrt(np.mean(flat * flat, axis=-1, keepdims=True) + eps)).reshape(o.shape) * w
        bad = bad / (1 + np.exp(-g))
    elif wrong == "no_eps":
        bad = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True)) * w / (1 + np.exp(-g))
    else:
        bad = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps) * w / (1 + np.exp(g))
    ref = torch.nn.functional.rms_norm(torch.from_numpy(o), (8,), weight=torch.from_numpy(w), eps=eps)
    ref = (ref * torch.sigmoid(torch.from_numpy(g))).numpy()
    assert not np.allclose(bad, ref, rtol=1e-6)
    np.testing.assert_allclose(gated_rmsnorm_ref(o, g, w, eps), ref, rtol=1e-13)
