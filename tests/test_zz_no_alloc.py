"""chimera_kda_fwd_noalloc (the KDA forward for callers that cannot allocate) against
chimera_kda_fwd, called through the C ABI: two calls in a row on one GPU, the second smaller,
each equal to the allocating entry point's result on the same inputs (same kernels and plan,
so bit for bit; the bf16 tolerances of the path are checked as well)."""
import ctypes

import numpy as np
import pytest

import workloads as wl
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


def _inputs(chm, T, H, seed, s0):
    import torch
    w = wl.WORKLOADS[1]
    rng = np.random.default_rng(seed)
    d = w.d
    x = wl.round_to_bf16(rng.standard_normal((1, T, 3 * H * d)).astype(np.float32))
    q, k, v = [to_device(x.reshape(1, T, 3, H, d)[:, :, i], "bf16") for i in range(3)]
    alpha = to_device(wl.round_to_bf16(np.exp(-0.05 * np.log1p(np.exp(rng.standard_normal((1, T, H, d)))))
                                       .astype(np.float32)), "bf16")
    beta = to_device(wl.round_to_bf16((1 / (1 + np.exp(-rng.standard_normal((1, T, H))))).astype(np.float32)), "bf16")
    S0 = torch.from_numpy((0.1 * rng.standard_normal((1, H, d, d))).astype(np.float32)).cuda() if s0 else None
    return q, k, v, alpha, beta, S0


def _noalloc(chm, q, k, v, alpha, beta, S0):
    import torch
    B, T, H, d = q.shape
    o = torch.empty_like(q)
    Sf = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
    st = chm.lib().chimera_kda_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), H * d, alpha.data_ptr(),
                                           beta.data_ptr(), None if S0 is None else S0.data_ptr(), o.data_ptr(),
                                           Sf.data_ptr(), B, T, H, d, d, chm.BF16, chm.KDA_L2NORM_QK,
                                           torch.cuda.current_stream().cuda_stream)
    assert st == 0, chm.status_string(st)
    return o, Sf


@pytest.mark.parametrize("first,second", [((4352, 16, True), (1000, 4, False))])
def test_noalloc_matches_allocating_entry_point(chm, first, second):
    import torch
    for n, (T, H, s0) in enumerate((first, second)):
        print(f"noalloc call {n}: T={T} H={H} S0={s0}", flush=True)
        q, k, v, alpha, beta, S0 = _inputs(chm, T, H, 100 + n, s0)
        need = chm.kda_workspace_size(1, T, H, 128, 128, chm.BF16, chm.KDA_L2NORM_QK)
        assert 0 < need <= chm.KDA_NOALLOC_SCRATCH_BYTES
        o_ref, S_ref = chm.kda_fwd(q, k, v, alpha, beta, S0)
        o, Sf = _noalloc(chm, q, k, v, alpha, beta, S0)
        torch.cuda.synchronize()
        assert_close(to_host(o), to_host(o_ref), "bf16", "o")
        assert_close(to_host(Sf), to_host(S_ref), "bf16", "S_final")
        assert torch.equal(o, o_ref) and torch.equal(Sf, S_ref), "not bit-identical to chimera_kda_fwd"


def test_noalloc_empty_and_bad_arguments(chm):
    import torch
    L = chm.lib()
    s = torch.cuda.current_stream().cuda_stream
    # T = 0: nothing to do, no scratch needed
    assert L.chimera_kda_fwd_noalloc(None, None, None, 0, None, None, None, None, None, 1, 0, 2, 128, 128, chm.BF16,
                                     0, s) == 0
    # errors of chimera_kda_fwd are reported unchanged (a null input)
    assert L.chimera_kda_fwd_noalloc(None, None, None, 256, None, None, None, None, None, 1, 8, 2, 128, 128, chm.BF16,
                                     0, s) == 1
