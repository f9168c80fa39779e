"""The boundary's reentrancy on one GPU: two host threads make the process's first calls of the
conv and the chunked recurrence at the same moment, each on its own stream with its own buffers
and workspace (the per-device set-up of both runs concurrently); each thread's results equal the
same calls made again one after the other, bit for bit."""
import subprocess
import sys
import textwrap

import pytest

pytestmark = pytest.mark.gpu

_CHILD = textwrap.dedent(r'''
    import sys, threading
    import numpy as np
    import torch
    import workloads as wl
    import linear_attention_recurrence_mshortconv_amd as chm

    H, d = 4, 128
    segs = wl.text_then_grid(37, 1, 9, 61)
    T = sum(s.length for s in segs)
    dev = torch.device("cuda:0")

    def inputs(seed):
        rng = np.random.default_rng(seed)
        bf = lambda a: torch.from_numpy(wl.round_to_bf16(a.astype(np.float32))).to(torch.bfloat16).to(dev)
        x = bf(rng.standard_normal((2, T, 3 * H * d)))
        wt = torch.from_numpy((0.5 * rng.standard_normal((3 * H * d, 4))).astype(np.float32)).to(dev)
        wv = torch.from_numpy((0.5 * rng.standard_normal((3 * H * d, 27))).astype(np.float32)).to(dev)
        al = bf(np.exp(-0.05 * np.logaddexp(0, rng.standard_normal((2, T, H, d)))))
        be = bf(1 / (1 + np.exp(-rng.standard_normal((2, T, H)))))
        ws = torch.empty(max(chm.kda_workspace_size(2, T, H, d, d, chm.BF16, chm.KDA_L2NORM_QK), 1),
                         dtype=torch.uint8, device=dev)
        return x, wt, wv, al, be, ws

    def run(args, stream):
        x, wt, wv, al, be, ws = args
        with torch.cuda.stream(stream):
            y = chm.mshortconv_fwd(x, wt, wv, segs)
            o, Sf = chm.kda_fwd(*chm.split_qkv(y, H, d), al, be, None, workspace=ws)
        stream.synchronize()
        return y, o, Sf

    cases = [inputs(1), inputs(2)]
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    torch.cuda.synchronize()
    start = threading.Barrier(2)
    out = [None, None]
    err = []

    def worker(i):
        try:
            start.wait()
            out[i] = run(cases[i], streams[i])
        except Exception as e:   # reported by the parent through the exit code
            err.append(repr(e))

    th = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    if err:
        print("thread error:", err, flush=True)
        sys.exit(2)
    for i in range(2):
        again = run(cases[i], streams[0])
        for a, b in zip(out[i], again):
            if not torch.equal(a, b):
                print(f"thread {i}: result differs from the sequential call", flush=True)
                sys.exit(3)
    print("two threads: ok", flush=True)
''')


def test_two_host_threads_one_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    r = subprocess.run([sys.executable, "-c", _CHILD], capture_output=True, text=True, timeout=240,
                       cwd=__import__("os").path.dirname(__import__("os").path.dirname(__file__)))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "two threads: ok" in r.stdout
