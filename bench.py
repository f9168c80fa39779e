"""Benchmark: KDA + mShortConv forward on one MI355X.

One step = one pass of the whole hot path over the 65,792-token workload
(256 text tokens + a 256x256 image grid, the packing of a 4096x4096 image at
16x16 patches; B=1, H=16, d=128, bf16 inputs, fp32 state):

  1. mShortConv on the fused q|k|v tensor (chimera_mshortconv_fwd), and
  2. the KDA forward with per-head q/k L2 normalisation (chimera_kda_fwd).

The neighbour layout is derived arithmetically inside the conv kernel; the
host-side index table is not part of a step. Inputs are synthetic, seeded,
and resident in HBM before the timed region.

Prints one JSON line. Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA+mShortConv fwd tokens/sec/GPU at 65K tok, H=16 d=128; % of roofline"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, published
WORKLOAD_INDEX = 2


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-once", action="store_true",
                    help="for counter runs: one 1 GiB device copy (the scale reference), then one step, then exit")
    ap.add_argument("--cpu-sample-rows", type=int, default=80,
                    help="image rows in the oracle's timed sample (plus the 256 text tokens)")
    return ap.parse_args()


def _cpu_baseline(inp, w, rows: int):
    """The oracle as it stands, on the first 256 + rows*256 tokens of the workload, one host core."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import workloads as wl
    from oracle import conv_ref, kda_ref, l2norm_ref, round_bf16_ref

    img = w.segments[1]
    n_text = w.segments[0].length
    n = n_text + rows * img.width
    segs = (wl.Segment(wl.TEXT, 0, n_text), wl.Segment(wl.IMAGE, n_text, rows * img.width, 1, rows, img.width))
    x = inp["x"][:, :n]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        y = round_bf16_ref(conv_ref(x, inp["w_text"], inp["w_vis"], segs))
        parts = y.reshape(w.B, n, 3, w.H, w.d)
        kda_ref(l2norm_ref(parts[:, :, 0]), l2norm_ref(parts[:, :, 1]), parts[:, :, 2],
                inp["alpha"][:, :n], inp["beta"][:, :n], None)
        dt = time.perf_counter() - t0
    return {"value": n * w.B / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} tokens of the workload (256 text + {rows} image rows x {img.width}), "
                      f"all {w.H} heads, conv + L2 norm + token-by-token KDA in fp64 numpy; {dt:.1f} s on "
                      f"{platform.processor() or platform.machine()}, BLAS limited to 1 thread"}


def main():
    args = _args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); nothing here runs on more than one.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import workloads as wl
    import linear_attention_recurrence_mshortconv_amd as chm

    chm.lib()
    w = wl.WORKLOADS[WORKLOAD_INDEX]
    B, T, H, d = w.B, w.T, w.H, w.d
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = wl.make_inputs(w)
    to_dev = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)
    x = to_dev(inp["x"])
    alpha = to_dev(inp["alpha"])
    beta = to_dev(inp["beta"])
    wt = torch.from_numpy(inp["w_text"]).to(dev)
    wv = torch.from_numpy(inp["w_vis"]).to(dev)
    segs = w.segments
    y = torch.empty_like(x)
    q, k, v = chm.split_qkv(y, H, d)
    o = torch.empty(B, T, H, d, dtype=torch.bfloat16, device=dev)
    need = chm.kda_workspace_size(B, T, H, d, d, chm.BF16, chm.KDA_L2NORM_QK)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def step():
        chm.mshortconv_fwd(x, wt, wv, segs, out=y)
        chm.kda_fwd(q, k, v, alpha, beta, None, workspace=ws, out=o)

    if args.profile_once:
        ref_src = torch.empty(512 * 1024 * 1024, dtype=torch.bfloat16, device=dev)   # 1 GiB
        ref_dst = torch.empty_like(ref_src)
        ref_dst.copy_(ref_src)
        step()
        torch.cuda.synchronize()
        print("profile-once: 1 GiB copy + one step done")
        return

    # the image-grid conv kernel alone: same launch as inside a step, on the image tokens
    img = segs[1]
    x_img = x[:, img.start:]
    y_img = y[:, img.start:]
    img_only = (wl.Segment(wl.IMAGE, 0, img.length, 1, img.height, img.width),)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = e0.elapsed_time(e1) / args.steps

    # per-call split of a step, and the conv grid kernel alone (events on the launch stream)
    def avg_ms(fn, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    n_rep = max(5, args.steps)
    ms_conv = avg_ms(lambda: chm.mshortconv_fwd(x, wt, wv, segs, out=y), n_rep)
    ms_kda = avg_ms(lambda: chm.kda_fwd(q, k, v, alpha, beta, None, workspace=ws, out=o), n_rep)
    ms_conv_grid = avg_ms(lambda: chm.mshortconv_fwd(x_img, wt, wv, img_only, out=y_img), n_rep)

    # algorithmic bytes of the conv grid kernel: read and write every q|k|v channel of every image token once
    conv_bytes = 2 * B * img.length * 3 * H * d * 2
    achieved = conv_bytes / (ms_conv_grid * 1e-3) / 1e9
    kda_bytes = B * T * H * (3 * d * 2 + d * 2 + 2 + d * 2)
    tokens = B * T
    value = tokens / (ms_step * 1e-3)
    src = os.path.join(ROOT, "linear_attention_recurrence_mshortconv_amd", "csrc", "mshortconv.hip")
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; bf16 q|k|v, alpha, beta; fp32 conv weights; fp32 state)",
        "config": {"workload": f"{w.name}: 256 text tokens + 256x256 image grid = {T} tokens, B={B}, H={H}, "
                               f"d_k=d_v={d}, chunk 64, conv 4-tap text / 3x3 image, q/k L2-normalised",
                   "tokens_per_step": tokens, "ms_conv": ms_conv, "ms_kda": ms_kda,
                   "kda_GBps_algorithmic": kda_bytes / (ms_kda * 1e-3) / 1e9,
                   "wall_s_timed": t_wall},
        "roofline": {"bound": "hbm", "kernel": "conv_tile_kernel (image grid, 3x3, bf16)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None, "ms_per_launch": ms_conv_grid,
                     "algorithmic_bytes_per_launch": conv_bytes},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = _cpu_baseline(inp, w, args.cpu_sample_rows)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
