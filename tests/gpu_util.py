"""Helpers shared by the GPU parity tests: tolerance checks and input upload."""
from __future__ import annotations

import numpy as np

# Tolerances per output tensor, as fixed for this path: fp32 inputs rel-L2 <= 1e-4;
# bf16 inputs with an fp32 state rel-L2 <= 2e-2 and max-abs <= 5e-2.
TOL_F32_REL_L2 = 1e-4
TOL_BF16_REL_L2 = 2e-2
TOL_BF16_MAX_ABS = 5e-2


def rel_l2(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


def max_abs(got, want) -> float:
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64)))) if np.size(want) else 0.0


def assert_close(got, want, dtype: str, what: str = ""):
    r = rel_l2(got, want)
    if dtype == "f32":
        assert r <= TOL_F32_REL_L2, f"{what}: rel-L2 {r:.3e} > {TOL_F32_REL_L2}"
    else:
        m = max_abs(got, want)
        assert r <= TOL_BF16_REL_L2 and m <= TOL_BF16_MAX_ABS, f"{what}: rel-L2 {r:.3e}, max-abs {m:.3e}"
    return r


def assert_rel_l2(got, want, dtype: str, what: str = ""):
    """The rel-L2 part of assert_close only, for outputs whose every element is already held
    to an error bound of its own (a max-abs figure does not scale with the output's size:
    one bf16 rounding of a value above 16 may move it by more than 5e-2)."""
    r = rel_l2(got, want)
    tol = TOL_F32_REL_L2 if dtype == "f32" else TOL_BF16_REL_L2
    assert r <= tol, f"{what}: rel-L2 {r:.3e} > {tol}"
    return r


def to_device(a: np.ndarray, dtype: str, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to(device)


def to_host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)
