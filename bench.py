"""Benchmark: KDA + mShortConv forward on one MI355X.

One step = one pass of the whole hot path over the 65,792-token workload
(256 text tokens + a 256x256 image grid, the packing of a 4096x4096 image at
16x16 patches; B=1, H=16, d=128, bf16 inputs, fp32 state):

  1. mShortConv on the fused q|k|v tensor (chimera_mshortconv_fwd), and
  2. the KDA forward with per-head q/k L2 normalisation, o and S_final
     (chimera_kda_fwd).

The neighbour layout is derived arithmetically inside the conv kernels; no
host-side index table is part of a step. Inputs are synthetic, seeded, and
resident in HBM before the timed region.

The timed steps call the timing variants of both entry points, which record a
HIP event on the launch stream around every kernel; the per-kernel averages
give the roofline line of the kernel that takes the most time per step.

Prints one JSON line. Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
[--workload NAME] [--gated]; the other four synthetic workloads (tiny_text_fp32,
image_1024, video_5s, video_30s) are measured the same way with --workload.
--gated times the KDA call with the output gate and norm of Eq. 15
(chimera_kda_fwd_gated: Sigmoid(gate) * RMSNorm(o), a synthetic gate input).
--backward times a training step instead: the two forward calls, then
chimera_kda_bwd (writing dq, dk, dv straight into one fused q|k|v gradient) and
chimera_mshortconv_bwd on it, against a synthetic dL/do; each call is bracketed
by HIP events on the stream. --fused times chimera_kda_fwd_conv (the conv computed
in the recurrence's load stage, q|k|v never stored; the chunked kernels for bf16
d = 128) beside the product's two calls (the conv, then the recurrence).

Two helper modes turn rocprofv3 output into the summaries kept with the code:
  python bench.py --summarize-stats <kernel_stats.csv>
  python bench.py --summarize-pmc <fetch counter_collection.csv> <write counter_collection.csv>
"""
from __future__ import annotations

import argparse
import csv
import dataclasses
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA+mShortConv fwd tokens/sec/GPU at 65K tok, H=16 d=128; % of roofline"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, published
WORKLOAD_INDEX = 2
CSRC = os.path.join(ROOT, "linear_attention_recurrence_mshortconv_amd", "csrc")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "image_4096_hbm_traffic.md")
COPY_KERNEL = "__amd_rocclr_copyBuffer"

# kernel -> the source file that defines it (for the staleness check of stored counters)
KERNEL_SOURCE = {
    "conv_rows_kernel": "mshortconv.hip", "conv_tile_kernel": "mshortconv.hip",
    "conv_text_kernel": "mshortconv.hip", "conv_gather_kernel": "mshortconv.hip",
    "kda_sum_kernel": "kda_chunked.hip", "kda_combine_kernel": "kda_chunked.hip",
    "kda_out_kernel": "kda_chunked.hip", "kda_seq_kernel": "kda_sequential.hip",
    "kda_out_gated_kernel": "kda_chunked.hip", "kda_gate_norm_kernel": "kda_sequential.hip",
}


def kda_flops_per_token_head(d: int, C: int = 64) -> float:
    """Algorithmic FLOPs of the chunked KDA per token and head: the intra-chunk products A, Aqk,
    W, U~ (2 C d each) and the triangular inverse (2 C^2 / 3), then U = U~ - W S, Q^ S, the state
    update (2 d^2 each) and Aqk U (2 C d): 182,955 at d = 128, C = 64 (no dense T x T work)."""
    return 6 * d * d + 10 * C * d + 2 * C * C / 3


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def pool_cores() -> int:
    """Host threads for the oracle pool: the cores this process may run on, at most 16 (the host
    share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _oracle_head_job(job):
    """One head of the oracle sample (all batch items or packed samples): the conv of the head's q, k
    and v channels, the rounding to the storage type, the L2 norms and the token loop, in fp64 on one
    core. Runs in a pool worker."""
    from threadpoolctl import threadpool_limits
    from oracle import conv_ref, kda_ref, kda_varlen_ref, l2norm_ref, round_bf16_ref
    x, wt, wv, segs, alpha, beta, S0, bf16, cu = job
    with threadpool_limits(limits=1):
        y = conv_ref(x, wt, wv, segs)
        if bf16:
            y = round_bf16_ref(y)
        B, n = y.shape[:2]
        parts = y.reshape(B, n, 3, 1, -1)
        if cu is not None:
            kda_varlen_ref(l2norm_ref(parts[0, :, 0]), l2norm_ref(parts[0, :, 1]), parts[0, :, 2], alpha[0], beta[0],
                           cu, None)
        else:
            kda_ref(l2norm_ref(parts[:, :, 0]), l2norm_ref(parts[:, :, 1]), parts[:, :, 2], alpha, beta, S0)
    return n * B


def achievable_peaks(dev) -> dict:
    """What this machine reaches outside the path, for context beside the datasheet peaks: a 1 GiB device copy
    (torch's copy kernel: read + write bytes over its time) and a plain 8192^3 bf16 GEMM (torch.matmul on
    contiguous operands, the library's tuned kernel). Each: 2 warm-up runs, then the mean of 10 timed with
    HIP events; after the bench's timed steps, outside them."""
    import torch
    def timed(fn, n=10):
        for _ in range(2):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e-3
    src = torch.empty(512 * 1024 * 1024, dtype=torch.bfloat16, device=dev)   # 1 GiB
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src))
    copy_gbs = 2 * src.numel() * 2 / t_copy / 1e9
    del src, dst
    n = 8192
    a = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    b = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    t_mm = timed(lambda: torch.matmul(a, b))
    gemm_tflops = 2 * n ** 3 / t_mm / 1e12
    del a, b
    torch.cuda.empty_cache()
    return {"copy_GBps": copy_gbs, "gemm_bf16_TFLOPs": gemm_tflops,
            "recipe": "1 GiB bf16 device copy (read + write) and an 8192^3 bf16 torch.matmul, mean of 10 after 2 warm-ups"}


def short_name(full: str) -> str:
    """'void chm::(anonymous namespace)::conv_rows_kernel<4, 32>(...)' -> 'conv_rows_kernel'."""
    s = full.replace("(anonymous namespace)::", "")
    gated = "kda_out_kernel<true>" in s
    s = s.split("(")[0].split("<")[0].strip()
    s = s.split("::")[-1].split(" ")[-1]
    return "kda_out_gated_kernel" if gated else s


def source_hash(kernel: str) -> str:
    f = KERNEL_SOURCE.get(kernel)
    if f is None:
        return "-"
    return hashlib.sha256(open(os.path.join(CSRC, f), "rb").read()).hexdigest()[:16]


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-once", action="store_true",
                    help="for counter runs: one 1 GiB device copy (the scale reference), then one step, then exit")
    ap.add_argument("--workload", default="image_4096",
                    help="synthetic workload (name or index); the metric is quoted on image_4096")
    ap.add_argument("--gated", action="store_true",
                    help="KDA with the output gate and norm of Eq. 15 (Sigmoid(gate) * RMSNorm(o))")
    ap.add_argument("--backward", action="store_true",
                    help="a training step: forward, then the KDA and conv backward (gradients of a synthetic dL/do)")
    ap.add_argument("--fused", action="store_true",
                    help="the conv fused into the recurrence's load stage (chimera_kda_fwd_conv), against the "
                         "two calls (conv, then the recurrence)")
    ap.add_argument("--head-dim", type=int, default=0,
                    help="run the workload with heads of this size at the same width (H * d kept)")
    ap.add_argument("--sequential", action="store_true",
                    help="the KDA call (with --backward: the KDA backward) on the token-by-token kernels (CHIMERA_KDA_SEQUENTIAL)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=20736,
                    help="tokens per sequence in the oracle's timed sample (text + whole grid rows/frames)")
    ap.add_argument("--summarize-stats", metavar="CSV", help="markdown table of a rocprofv3 kernel_stats.csv")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="markdown HBM traffic table from FETCH_SIZE and WRITE_SIZE counter_collection.csv files")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                    help="markdown table of the SQ counters of the KDA kernels (image_4096, one step)")
    return ap.parse_args()


# ----------------------------------------------------------------------------------------------------------
# algorithmic work per launch (bytes that the kernel's job must move, or flops it must do)

KDA_TARGET_BLOCKS = 256   # the library's plan: about one block of each KDA pass per CU


def kda_split(B: int, T: int, H: int, target_blocks: int = KDA_TARGET_BLOCKS):
    """Chunks covered by the summary pass of the chunked KDA: the library cuts every sequence into
    segments of Lo 64-token chunks, Lo chosen so that about 256 output blocks cover the B*H
    sequence-heads, and summarises all segments but the last. Returns (chunks, summarised chunks)."""
    nc = (T + 63) // 64
    lo = max(1, (B * H * nc + target_blocks - 1) // target_blocks)
    p = 1 if nc <= 1 else (nc + lo - 1) // lo
    return nc, (p - 1) * lo


def kda_summarised_tokens(w) -> int:
    """Tokens (per head) that the summary pass reads: every sequence's chunks but those of its last
    output segment, with the library's plan (one Lo for all sequences of the call; for packed samples
    of mixed lengths the library may pick a shorter Lo, which this estimate ignores)."""
    lens = ([w.samples[i + 1] - w.samples[i] for i in range(len(w.samples) - 1)] if w.samples
            else [w.T] * w.B)
    ncs = [(n + 63) // 64 for n in lens]
    lo = max(1, (w.H * sum(ncs) + KDA_TARGET_BLOCKS - 1) // KDA_TARGET_BLOCKS)
    toks = 0
    for n, nc in zip(lens, ncs):
        p = 1 if nc <= 1 else (nc + lo - 1) // lo
        toks += min(n, (p - 1) * lo * 64)
    return toks


def kernel_work(name: str, w) -> dict:
    """Algorithmic bytes (HBM-bound kernels) of one launch on a workload, with the recipe."""
    B, T, H, d, C = w.B, w.T, w.H, w.d, w.C
    text = sum(s.length for s in w.segments if s.kind == 0)
    vis = T - text
    e = 2 if w.dtype == "bf16" else 4
    nseq = len(w.samples) - 1 if w.samples else B
    state = nseq * H * d * d * 4 * (2 if w.s0_std is not None else 1)  # S_final (+ S0) per sequence
    if name in ("conv_rows_kernel", "conv_tile_kernel"):
        return {"bytes": 2 * B * vis * C * e,
                "recipe": f"read + write every q|k|v channel of the {vis} visual tokens once: 2 x {C} x {e} B/token"}
    if name in ("conv_text_kernel", "conv_gather_kernel"):
        n = text if name == "conv_text_kernel" else vis
        return {"bytes": 2 * B * n * C * e, "recipe": f"read + write every channel of the {n} tokens once"}
    if name in ("kda_out_kernel", "kda_seq_kernel", "kda_out_gated_kernel"):
        per = 4 * d * e + e + d * e                               # q, k, v, alpha in; beta in; o out
        gate = d * e if name == "kda_out_gated_kernel" else 0     # + the gate in
        return {"bytes": B * T * H * (per + gate) + state,
                "recipe": f"q, k, v, alpha ({4 * d * e} B) + beta ({e} B)" + (f" + gate ({gate} B)" if gate else "")
                          + f" in, o ({d * e} B) out per token-head, + the fp32 d x d states per head"}
    if name == "kda_gate_norm_kernel":
        return {"bytes": 3 * B * T * H * d * e, "recipe": f"o and the gate in, o out: {3 * d * e} B per token-head"}
    if name == "kda_sum_kernel":
        toks = kda_summarised_tokens(w)
        return {"bytes": toks * H * (3 * d * e + e),
                "recipe": f"k, v, alpha + beta in ({3 * d * e + e} B per token-head) over the {toks} tokens "
                          f"(of {B * T}) the segment summaries cover"}
    return {"bytes": None, "recipe": "workspace only (no algorithmic HBM traffic)"}


def stored_traffic(kernel: str):
    """Scaled HBM bytes per launch from the committed counter summary, or None when the kernel's source
    changed since the counters were taken (or no row exists)."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    for line in open(TRAFFIC_SUMMARY):
        cells = [c.strip().strip("`") for c in line.strip().strip("|").split("|")]
        if len(cells) >= 6 and cells[0] == kernel:
            if cells[1] != source_hash(kernel):
                return None
            try:
                return float(cells[4]) * 1e6
            except ValueError:
                return None
    return None


# ----------------------------------------------------------------------------------------------------------
# summaries of rocprofv3 output

def summarize_stats(path: str):
    rows = list(csv.DictReader(open(path)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    print("| Kernel | Calls | Average (us) | Min (us) | Max (us) | Share |")
    print("|---|---|---|---|---|---|")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        print(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
              f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
              f"{100 * float(r['TotalDurationNs']) / total:.1f}% |")


def _pmc(path: str, counter: str):
    out = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        out.setdefault(short_name(r["Kernel_Name"]) if r["Kernel_Name"] != COPY_KERNEL else COPY_KERNEL,
                       []).append(float(r["Counter_Value"]))
    return out


def summarize_pmc(fetch_csv: str, write_csv: str):
    import workloads as wl
    w = wl.WORKLOADS[WORKLOAD_INDEX]
    f, wr = _pmc(fetch_csv, "FETCH_SIZE"), _pmc(write_csv, "WRITE_SIZE")
    gib_kib = 1024.0 * 1024.0                                    # a 1 GiB copy reads and writes 1 GiB
    f_scale = gib_kib / max(f[COPY_KERNEL])
    w_scale = gib_kib / max(wr[COPY_KERNEL])
    print(f"Scale: the 1 GiB device copy reads FETCH_SIZE = {max(f[COPY_KERNEL]):.0f} KiB and "
          f"WRITE_SIZE = {max(wr[COPY_KERNEL]):.0f} KiB, so the factors are {f_scale:.3f} (fetch) and "
          f"{w_scale:.3f} (write).\n")
    print("| Kernel | Source sha256 (16) | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | Scaled HBM bytes (MB) | "
          "Algorithmic bytes (MB) | Ratio |")
    print("|---|---|---|---|---|---|---|")
    for k in f:
        if k == COPY_KERNEL or k not in KERNEL_SOURCE or k not in wr:
            continue
        fk, wk = sum(f[k]) / len(f[k]), sum(wr[k]) / len(wr[k])
        scaled = (fk * f_scale + wk * w_scale) * 1024.0
        alg = kernel_work(k, w)["bytes"]
        ratio = f"{scaled / alg:.3f}" if alg else "-"
        algs = f"{alg / 1e6:.1f}" if alg else "-"
        print(f"| `{k}` | {source_hash(k)} | {fk:.0f} | {wk:.0f} | {scaled / 1e6:.1f} | {algs} | {ratio} |")


def summarize_counters(paths, chunk_heads: dict):
    """Per-kernel table of SQ counters from rocprofv3 --pmc counter_collection.csv files (several passes).
    Derived figures use the conventions of these counters on gfx9: SQ_WAVE_CYCLES and SQ_ACTIVE_INST_*
    count quad-cycles (4 clocks), SQ_BUSY_CYCLES sums clocks over the 32 shader engines, and
    SQ_VALU_MFMA_BUSY_CYCLES sums clocks over the 1024 SIMDs."""
    vals = {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            k = short_name(r["Kernel_Name"]) if r["Kernel_Name"] != COPY_KERNEL else COPY_KERNEL
            if k not in KERNEL_SOURCE:
                continue
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    avg = {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in vals.items()}
    names = sorted({c for d in avg.values() for c in d})
    ks = [k for k in ("kda_sum_kernel", "kda_combine_kernel", "kda_out_kernel", "kda_out_gated_kernel") if k in avg]
    print("| Counter | " + " | ".join(f"`{k}`" for k in ks) + " |")
    print("|---|" + "---|" * len(ks))
    for c in names:
        print(f"| {c} | " + " | ".join(f"{avg[k].get(c, float('nan')):.4g}" for k in ks) + " |")
    print()
    print("| Derived | " + " | ".join(f"`{k}`" for k in ks) + " |")
    print("|---|" + "---|" * len(ks))

    def row(label, fn):
        out = []
        for k in ks:
            try:
                out.append(fn(avg[k], k))
            except (KeyError, ZeroDivisionError):
                out.append("-")
        print(f"| {label} | " + " | ".join(out) + " |")

    clocks = lambda a: a["SQ_BUSY_CYCLES"] / 32.0       # kernel clocks per shader engine
    row("kernel clocks (SQ_BUSY_CYCLES / 32)", lambda a, k: f"{clocks(a):.3g}")
    row("MFMA busy, share of SIMD clocks", lambda a, k: f"{a['SQ_VALU_MFMA_BUSY_CYCLES'] / (1024 * clocks(a)):.1%}")
    row("VALU issue, share of SIMD clocks", lambda a, k: f"{4 * a['SQ_ACTIVE_INST_VALU'] / (1024 * clocks(a)):.1%}")
    row("LDS issue, share of SIMD clocks", lambda a, k: f"{4 * a['SQ_ACTIVE_INST_LDS'] / (1024 * clocks(a)):.1%}")
    row("LDS bank-conflict clocks / LDS-active clocks",
        lambda a, k: f"{a['SQ_LDS_BANK_CONFLICT'] / (4 * a['SQ_ACTIVE_INST_LDS']):.1%}")
    row("waiting (SQ_WAIT_ANY / SQ_WAVE_CYCLES)", lambda a, k: f"{a['SQ_WAIT_ANY'] / a['SQ_WAVE_CYCLES']:.1%}")
    for c, lab in (("SQ_INSTS_VALU", "VALU"), ("SQ_INSTS_MFMA", "MFMA"), ("SQ_INSTS_LDS", "LDS"),
                   ("SQ_INSTS_SALU", "SALU")):
        row(f"{lab} instructions per chunk-head", lambda a, k, c=c: f"{a[c] / chunk_heads[k]:.0f}"
            if chunk_heads.get(k) else "-")


# ----------------------------------------------------------------------------------------------------------

def _sample_segments(w, budget: int):
    """The first tokens of the workload's layout: the text, then whole grid rows (image) or frames
    (video) up to about `budget` tokens per sequence; for a packed row, its first whole samples."""
    import workloads as wl
    if w.samples:
        k = max(1, sum(1 for c in w.samples[1:] if c <= budget))
        n = w.samples[k]
        return tuple(sg for sg in w.segments if sg.start < n), n
    out, n = [], 0
    for sg in w.segments:
        if sg.kind == wl.TEXT:
            take = min(sg.length, max(budget - n, 0))
            if take > 0:
                out.append(wl.Segment(wl.TEXT, n, take))
                n += take
            continue
        unit = sg.width if sg.frames == 1 else sg.height * sg.width
        k = max(1, min(sg.height if sg.frames == 1 else sg.frames, (budget - n) // unit))
        if sg.frames == 1:
            out.append(wl.Segment(sg.kind, n, k * unit, 1, k, sg.width))
        else:
            out.append(wl.Segment(sg.kind, n, k * unit, k, sg.height, sg.width))
        n += k * unit
        break
    return tuple(out), n


def _cpu_baseline(inp, w, budget: int, gate=None):
    """The oracle as it stands, on the first tokens of the workload, one host core."""
    from threadpoolctl import threadpool_limits
    from oracle import conv_ref, gated_rmsnorm_ref, kda_ref, kda_varlen_ref, l2norm_ref, round_bf16_ref

    segs, n = _sample_segments(w, budget)
    x = inp["x"][:, :n]
    S0 = inp["S0"]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        y = conv_ref(x, inp["w_text"], inp["w_vis"], segs)
        if w.dtype == "bf16":
            y = round_bf16_ref(y)
        parts = y.reshape(w.B, n, 3, w.H, w.d)
        if w.samples:
            cu = [c for c in w.samples if c <= n]
            o_ref, _ = kda_varlen_ref(l2norm_ref(parts[0, :, 0]), l2norm_ref(parts[0, :, 1]), parts[0, :, 2],
                                      inp["alpha"][0, :n], inp["beta"][0, :n], cu, None)
            o_ref = o_ref[None]
        else:
            o_ref, _ = kda_ref(l2norm_ref(parts[:, :, 0]), l2norm_ref(parts[:, :, 1]), parts[:, :, 2],
                               inp["alpha"][:, :n], inp["beta"][:, :n], S0)
        if gate is not None:
            gated_rmsnorm_ref(o_ref, gate[0][:, :n], gate[1], 1e-6)
        dt = time.perf_counter() - t0
    desc = (f"{sum(1 for c in w.samples[1:] if c <= n)} whole packed samples" if w.samples else
            " + ".join(f"{sg.length} {'text' if sg.kind == 0 else 'grid'}" for sg in segs))
    return {"value": n * w.B / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} tokens of each of the {w.B} sequence(s) ({desc}), all {w.H} heads, conv + L2 norm "
                      f"+ token-by-token KDA" + (" + gate and norm" if gate is not None else "") +
                      f" in fp64 numpy; {dt:.1f} s on one core of {cpu_model()} ({os.cpu_count()} logical CPUs "
                      f"reported), BLAS limited to 1 thread"}


def _cpu_baseline_pool(pool, ncores, inp, w, budget: int):
    """The oracle on the same sample as _cpu_baseline, its (batch, head) work split by head over a
    pool of host processes (forked before the GPU was touched), one core each."""
    segs, n = _sample_segments(w, budget)
    H, d = w.H, w.d
    x = inp["x"][:, :n]
    cu = [c for c in w.samples if c <= n] if w.samples else None
    jobs = []
    for h in range(H):
        ch = np.concatenate([np.arange(part * H * d + h * d, part * H * d + (h + 1) * d) for part in range(3)])
        jobs.append((np.ascontiguousarray(x[..., ch]), inp["w_text"][ch], inp["w_vis"][ch], segs,
                     np.ascontiguousarray(inp["alpha"][:, :n, h:h + 1]), np.ascontiguousarray(inp["beta"][:, :n, h:h + 1]),
                     None if inp["S0"] is None else inp["S0"][:, h:h + 1], w.dtype == "bf16", cu))
    t0 = time.perf_counter()
    pool.map(_oracle_head_job, jobs, chunksize=1)
    dt = time.perf_counter() - t0
    return {"value": n * w.B / dt, "unit": "tokens/s", "cores": ncores, "kind": "oracle",
            "sample": f"the same first {n} tokens of each sequence, {H} heads as {H} jobs on a pool of {ncores} "
                      f"processes (one core each, BLAS limited to 1 thread); {dt:.1f} s wall including the transfer "
                      f"of each head's inputs"}


def bench_backward(args, w):
    """One training step on the workload: conv fwd, KDA fwd, KDA bwd (into a fused q|k|v gradient),
    conv bwd. Call-level timing with HIP events on the stream; the oracle baseline times the fp64
    autograd backward on a bounded sample."""
    import torch
    import workloads as wl
    import linear_attention_recurrence_mshortconv_amd as chm
    assert not w.samples, "the backward runs on batched (not packed) workloads"
    B, T, H, d = w.B, w.T, w.H, w.d
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = wl.make_inputs(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    to_dev = lambda a: torch.from_numpy(a).to(tdt).to(dev)
    x, alpha, beta = to_dev(inp["x"]), to_dev(inp["alpha"]), to_dev(inp["beta"])
    S0 = None if inp["S0"] is None else torch.from_numpy(inp["S0"]).to(dev)
    wt, wv = torch.from_numpy(inp["w_text"]).to(dev), torch.from_numpy(inp["w_vis"]).to(dev)
    rng = np.random.default_rng(w.index + 3000)
    do = to_dev(rng.standard_normal((B, T, H, d), dtype=np.float32))
    segs = w.segments
    y, dy, dx = torch.empty_like(x), torch.zeros_like(x), torch.empty_like(x)
    q, k, v = chm.split_qkv(y, H, d)
    gq, gk, gv = chm.split_qkv(dy, H, d)
    o = torch.empty(B, T, H, d, dtype=tdt, device=dev)
    s_final = torch.empty(B, H, d, d, dtype=torch.float32, device=dev)
    dcode = chm.BF16 if w.dtype == "bf16" else chm.F32
    ws = torch.empty(max(chm.kda_workspace_size(B, T, H, d, d, dcode, chm.KDA_L2NORM_QK), 1), dtype=torch.uint8,
                     device=dev)
    bflags = chm.KDA_L2NORM_QK | (chm.KDA_SEQUENTIAL if args.sequential else 0)
    wsb = torch.empty(max(int(chm.lib().chimera_kda_bwd_workspace_size(B, T, H, d, d, dcode, bflags)), 1),
                      dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    calls = ["conv_fwd", "kda_fwd", "kda_bwd", "conv_bwd"]

    def step(ev=None):
        mark = (lambda i: ev[i].record(stream)) if ev else (lambda i: None)
        mark(0)
        chm.mshortconv_fwd(x, wt, wv, segs, out=y)
        mark(1)
        chm.kda_fwd(q, k, v, alpha, beta, S0, workspace=ws, out=o, state_out=s_final)
        mark(2)
        chm.kda_bwd(q, k, v, alpha, beta, S0, do, None, grads=(gq, gk, gv), workspace=wsb, sequential=args.sequential)
        mark(3)
        chm.mshortconv_bwd(x, dy, wt, wv, segs, dx=dx)
        mark(4)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {c: sum(ev[i].elapsed_time(ev[i + 1]) for ev in evs) / args.steps for i, c in enumerate(calls)}
    ms_step = sum(ev[0].elapsed_time(ev[4]) for ev in evs) / args.steps
    e = 2 if w.dtype == "bf16" else 4
    # the KDA backward's minimal traffic per token-head: q, k, v, alpha, beta, dL/do in, dq, dk, dv, dalpha,
    # dbeta out
    bwd_bytes = B * T * H * ((4 * d + 1 + d) * e + (4 * d + 1) * e)
    ms_bwd = per["kda_bwd"]
    chunked_bwd = w.dtype == "bf16" and d == 128 and not args.sequential
    bwd_desc = ("the chunked KDA backward (16-token chunks on MFMA)" if chunked_bwd
                else "the checkpointed token-by-token KDA backward")
    out = {
        "metric": "KDA+mShortConv training step (fwd + bwd) tokens/sec/GPU",
        "value": B * T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": f"synthetic (seeded; {w.dtype} inputs and dL/do; fp32 state)",
        "config": {"workload": f"{w.name}: {T} tokens per sequence, B={B}, H={H}, d={d}; forward (conv, chunked KDA), "
                               f"then {bwd_desc} and the conv backward",
                   "tokens_per_step": B * T, "calls_ms": per, "wall_s_timed": wall,
                   "kda_bwd_workspace_bytes": int(wsb.numel())},
        "roofline": {"bound": "hbm",
                     "kernel": ("kda_bwd (call: chunk factorisation, state passes, chains, gradient pass)" if chunked_bwd
                                else "kda_bwd (call: checkpoint forward, reverse pass, slice sums)"),
                     "achieved": bwd_bytes / (ms_bwd * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": bwd_bytes / (ms_bwd * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": None,
                     "ms_per_launch": ms_bwd, "algorithmic_bytes_per_launch": bwd_bytes,
                     "recipe": f"q, k, v, alpha, beta, dL/do in and dq, dk, dv, dalpha, dbeta out: "
                               f"{(9 * d + 2) * e} B per token-head"},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits
        from oracle.backward import kda_backward_ref
        n = min(T, 64)
        with threadpool_limits(limits=1):
            t1 = time.perf_counter()
            parts = inp["x"][:, :n].reshape(B, n, 3, H, d)
            kda_backward_ref(parts[:, :, 0], parts[:, :, 1], parts[:, :, 2], inp["alpha"][:, :n], inp["beta"][:, :n],
                             None if S0 is None else inp["S0"], do[:, :n].float().cpu().numpy())
            dt = time.perf_counter() - t1
        out["cpu_baseline"] = {"value": B * n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"fp64 autograd KDA backward (with its forward) over the first {n} tokens, "
                                         f"all {H} heads; {dt:.1f} s"}
    print(json.dumps(out), flush=True)


def bench_fused(args, w):
    """The fused conv + recurrence (chimera_kda_fwd_conv: q|k|v computed in the recurrence's load
    stage, never stored) on the workload, timed with HIP events on the stream, each kernel marked;
    beside it the product's two calls (the conv, then the recurrence on the stored q|k|v) on the
    same inputs."""
    import torch
    import workloads as wl
    import linear_attention_recurrence_mshortconv_amd as chm
    assert not w.samples, "the fused call takes batched (not packed) workloads"
    B, T, H, d = w.B, w.T, w.H, w.d
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = wl.make_inputs(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    to_dev = lambda a: torch.from_numpy(a).to(tdt).to(dev)
    x, alpha, beta = to_dev(inp["x"]), to_dev(inp["alpha"]), to_dev(inp["beta"])
    S0 = None if inp["S0"] is None else torch.from_numpy(inp["S0"]).to(dev)
    wt, wv = torch.from_numpy(inp["w_text"]).to(dev), torch.from_numpy(inp["w_vis"]).to(dev)
    segs = w.segments
    o = torch.empty(B, T, H, d, dtype=tdt, device=dev)
    s_final = torch.empty(B, H, d, d, dtype=torch.float32, device=dev)
    dt = chm.BF16 if w.dtype == "bf16" else chm.F32
    need_f = chm.kda_conv_workspace_size(segs, B, T, H, d, d, dt, chm.KDA_L2NORM_QK)
    ws_f = torch.empty(max(need_f, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def fused(m=None):
        chm.kda_fwd_conv(x, wt, wv, segs, alpha, beta, S0, H=H, dk=d, dv=d, out=o, state_out=s_final,
                         workspace=ws_f, marks=m)

    def timed(fn, cap):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        marks = [chm.Marks(cap) for _ in range(args.steps)]
        for m in marks:
            fn(m)
        torch.cuda.synchronize()
        per = {}
        for m in marks:
            for name, t in m.kernels():
                per.setdefault(name, []).append(t)
        return ms, {n: sum(v) / len(v) for n, v in per.items()}

    ms_fused, k_fused = timed(fused, 6)
    peak_fused = int(torch.cuda.max_memory_allocated(dev))
    y = torch.empty_like(x)
    q, k, v = chm.split_qkv(y, H, d)
    need_k = chm.kda_workspace_size(B, T, H, d, d, dt, chm.KDA_L2NORM_QK)
    ws_k = torch.empty(max(need_k, 1), dtype=torch.uint8, device=dev)

    def two_calls(m=None):
        chm.mshortconv_fwd(x, wt, wv, segs, out=y)
        chm.kda_fwd(q, k, v, alpha, beta, S0, out=o, state_out=s_final, workspace=ws_k, marks=m)

    ms_two, k_two = timed(two_calls, 5)
    e = 2 if w.dtype == "bf16" else 4
    # minimal traffic per token-head: x's q|k|v channels, alpha, beta in; o out (plus S_final)
    fused_bytes = B * T * H * (5 * d + 1) * e + B * H * d * d * 4 * (2 if S0 is not None else 1)
    chunked = "kda_out_conv_kernel" in k_fused
    call_ms = sum(k_fused.values()) if chunked else ms_fused
    out = {
        "metric": "KDA+mShortConv fused fwd tokens/sec/GPU",
        "value": B * T / (ms_fused * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_fused, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": f"synthetic (seeded; {w.dtype} x, alpha, beta; fp32 conv weights; fp32 state)",
        "config": {"workload": f"{w.name}: {T} tokens per sequence, B={B}, H={H}, d={d}; the conv computed in the "
                               f"{'chunked' if chunked else 'token-by-token'} recurrence's load stage (q|k|v never "
                               f"stored)",
                   "tokens_per_step": B * T, "kernels_ms": k_fused, "ms_two_calls": ms_two,
                   "two_calls_kernels_ms": k_two, "two_calls_tokens_per_s": B * T / (ms_two * 1e-3),
                   "fused_over_two_calls": ms_two / ms_fused,
                   "memory": {"peak_allocated_bytes_fused": peak_fused, "workspace_bytes_fused": int(need_f),
                              "conv_output_bytes_two_calls": int(y.numel() * y.element_size())}},
        "roofline": {"bound": "hbm", "kernel": "fused call (" + " + ".join(k_fused) + ")", "achieved":
                     fused_bytes / (call_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": fused_bytes / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": None,
                     "ms_per_launch": call_ms, "algorithmic_bytes_per_launch": fused_bytes,
                     "recipe": f"x's q|k|v channels, alpha, beta in and o out: {(5 * d + 1) * e} B per token-head, "
                               f"+ S_final; ms_per_launch is the sum of the call's kernels' average durations"},
        "cpu_baseline": None if args.no_cpu_baseline else _cpu_baseline(inp, w, args.cpu_sample_tokens),
    }
    print(json.dumps(out), flush=True)


def main():
    args = _args()
    if args.summarize_stats:
        summarize_stats(args.summarize_stats)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_counters:
        import workloads as wl
        w = wl.WORKLOADS[WORKLOAD_INDEX]
        nc = (w.T + 63) // 64
        chunks = w.B * w.H * nc
        summ = w.B * kda_summarised_tokens(w) // 64 * w.H
        summarize_counters(args.summarize_counters, {"kda_out_kernel": chunks, "kda_out_gated_kernel": chunks,
                                                     "kda_sum_kernel": summ})
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); nothing here runs on more than one.",
              file=sys.stderr)
        sys.exit(2)
    # the oracle's process pool is forked here, before anything touches the GPU
    pool, ncores = None, pool_cores()
    if not args.no_cpu_baseline and not args.profile_once and not args.backward and not args.fused:
        import multiprocessing as mp
        pool = mp.get_context("fork").Pool(ncores)
    import torch
    import workloads as wl
    import linear_attention_recurrence_mshortconv_amd as chm

    chm.lib()
    by_name = {w.name: w for w in wl.WORKLOADS}
    w = by_name[args.workload] if args.workload in by_name else wl.WORKLOADS[int(args.workload)]
    if args.head_dim:
        if (w.H * w.d) % args.head_dim:
            sys.exit(f"--head-dim {args.head_dim} does not divide the width {w.H * w.d}")
        w = dataclasses.replace(w, H=w.H * w.d // args.head_dim, d=args.head_dim)
    if args.backward:
        bench_backward(args, w)
        return
    if args.fused:
        bench_fused(args, w)
        return
    B, T, H, d = w.B, w.T, w.H, w.d
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = wl.make_inputs(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    to_dev = lambda a: torch.from_numpy(a).to(tdt).to(dev)
    x = to_dev(inp["x"])
    alpha = to_dev(inp["alpha"])
    beta = to_dev(inp["beta"])
    S0 = None if inp["S0"] is None else torch.from_numpy(inp["S0"]).to(dev)
    wt = torch.from_numpy(inp["w_text"]).to(dev)
    wv = torch.from_numpy(inp["w_vis"]).to(dev)
    segs = w.segments
    y = torch.empty_like(x)
    q, k, v = chm.split_qkv(y, H, d)
    o = torch.empty(B, T, H, d, dtype=tdt, device=dev)
    nseq = len(w.samples) - 1 if w.samples else B
    s_final = torch.empty(nseq if w.samples else B, H, d, d, dtype=torch.float32, device=dev)
    dcode = chm.BF16 if w.dtype == "bf16" else chm.F32
    kflags = chm.KDA_L2NORM_QK | (chm.KDA_SEQUENTIAL if args.sequential else 0)
    need = (chm.kda_varlen_workspace_size(w.samples, H, d, d, dcode, kflags) if w.samples else
            chm.kda_workspace_size(B, T, H, d, d, dcode, kflags))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    gate_np = wl.make_gate(w) if args.gated else None
    gkw = {}
    if args.gated:
        gkw = dict(gate=to_dev(gate_np[0]), norm_weight=torch.from_numpy(gate_np[1]).to(dev), norm_eps=1e-6)

    def step(mc=None, mk=None):
        chm.mshortconv_fwd(x, wt, wv, segs, out=y, marks=mc)
        if w.samples:
            chm.kda_fwd_varlen(q[0], k[0], v[0], alpha[0], beta[0], w.samples, None, sequential=args.sequential,
                               workspace=ws, out=o[0],
                               marks=mk, state_out=s_final, **gkw)
        else:
            chm.kda_fwd(q, k, v, alpha, beta, S0, sequential=args.sequential, workspace=ws, out=o, marks=mk,
                        state_out=s_final, **gkw)

    if args.profile_once:
        ref_src = torch.empty(512 * 1024 * 1024, dtype=torch.bfloat16, device=dev)   # 1 GiB
        ref_dst = torch.empty_like(ref_src)
        ref_dst.copy_(ref_src)
        step()
        torch.cuda.synchronize()
        print("profile-once: 1 GiB copy + one step done", flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    # the timed steps: exactly K, between two synchronisations, nothing else on the stream
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    a.record(stream)
    for _ in range(args.steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = a.elapsed_time(b) / args.steps

    # the same steps again with an event after every kernel, for the per-kernel durations (the
    # events add gaps between launches: these steps are reported, not used for the headline)
    kda_cap = 2 * nseq + 4 if w.samples else (6 if args.gated else 5)
    marks = [(chm.Marks(len(segs) + 1), chm.Marks(kda_cap)) for _ in range(args.steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for mc, mk in marks:
        step(mc, mk)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step_marked = e0.elapsed_time(e1) / args.steps

    # per-kernel device time, from the marks of the timed steps
    per_kernel = {}
    for mc, mk in marks:
        for name, ms in mc.kernels() + mk.kernels():
            per_kernel.setdefault(name, []).append(ms)
    kernels = {n: {"ms_per_launch": sum(v) / len(v), "launches_per_step": len(v) / args.steps}
               for n, v in per_kernel.items()}
    dom = max(kernels, key=lambda n: kernels[n]["ms_per_launch"] * kernels[n]["launches_per_step"])


    conv_ms = sum(kernels[n]["ms_per_launch"] * kernels[n]["launches_per_step"] for n in kernels
                  if n.startswith("conv_"))
    kda_names = [n for n in kernels if n.startswith("kda_")]
    kda_ms = sum(kernels[n]["ms_per_launch"] * kernels[n]["launches_per_step"] for n in kda_names)
    e = 2 if w.dtype == "bf16" else 4
    conv_bytes = 2 * B * T * w.C * e
    kda_bytes = B * T * H * (4 * d * e + e + d * e + (d * e if args.gated else 0)) \
        + nseq * H * d * d * 4 * (2 if S0 is not None else 1)
    kda_flops = B * T * H * kda_flops_per_token_head(d)
    # HBM bytes the counters measured for the KDA call: every KDA kernel's stored figure, when all of them
    # are current for this source
    traffic = None
    if w.name == wl.WORKLOADS[WORKLOAD_INDEX].name and not (args.gated or args.head_dim or args.sequential):
        parts = [stored_traffic(n) for n in kda_names]
        traffic = sum(parts) if parts and all(t is not None for t in parts) else None
    t_roof = (conv_bytes + kda_bytes) / (HBM_PEAK_GBS * 1e9)
    mem = {"peak_allocated_bytes": int(torch.cuda.max_memory_allocated(dev)), "workspace_bytes": int(need),
           "note": "torch's peak over the run: inputs, the conv output q|k|v, o, S_final and the KDA workspace (the "
                   "library allocates nothing itself)"}
    tokens = B * T
    if w.samples:
        layout = (f"{nseq} packed samples (a text prompt of 32..300 tokens, then a 16x16, 32x32 or 64x64 image "
                  f"grid at 4:2:2), the state restarting at each sample")
    else:
        layout = " + ".join(("text" if sg.kind == 0 else f"{sg.frames}x{sg.height}x{sg.width} grid") +
                            f" ({sg.length})" for sg in segs)
    out = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": f"synthetic (seeded; {w.dtype} q|k|v, alpha, beta; fp32 conv weights; fp32 state)",
        "config": {"workload": f"{w.name}: {layout} = {T} tokens per sequence, B={B}, H={H}, d_k=d_v={d}, "
                               + ("KDA on the token-by-token kernel, " if args.sequential else "chunk 64, ")
                               + "conv 4-tap text / 3x3 image / 3x3x3 video, q/k L2-normalised, "
                               f"o and S_final written" + (", S0 given" if S0 is not None else "")
                               + (", output gate and per-head RMSNorm of Eq. 15 fused" if args.gated else ""),
                   "tokens_per_step": tokens,
                   "ms_per_step_with_marks": ms_step_marked,
                   "dominant_kernel": dom,
                   "kernels": kernels,
                   "conv_call": {"ms": conv_ms, "GBps_algorithmic": conv_bytes / (conv_ms * 1e-3) / 1e9,
                                 "frac_hbm": conv_bytes / (conv_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
                   "kda_call": {"ms": kda_ms, "GBps_algorithmic": kda_bytes / (kda_ms * 1e-3) / 1e9,
                                "frac_hbm": kda_bytes / (kda_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
                   "memory": mem,
                   "wall_s_timed": t_wall},
        "roofline": {"bound": "hbm", "kernel": "KDA call (" + " + ".join(kda_names) + ")",
                     "achieved": kda_bytes / (kda_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": kda_bytes / (kda_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": traffic, "ms_per_launch": kda_ms, "algorithmic_bytes_per_launch": kda_bytes,
                     "recipe": f"q, k, v, alpha ({4 * d * e} B) + beta ({e} B) in and o ({d * e} B) out per token-head"
                               + (f" + the gate ({d * e} B)" if args.gated else "")
                               + f", x {B * T} tokens x {H} heads, + the fp32 {d}x{d} S_final"
                               + (" and S0" if S0 is not None else "") + " per head; ms_per_launch is the sum of the "
                               "call's kernels' average durations per step",
                     "mfma": {"achieved": kda_flops / (kda_ms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": kda_flops / (kda_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                              "flops_per_launch": kda_flops,
                              "recipe": f"{kda_flops_per_token_head(d):.0f} FLOP per token-head (chunk 64: A, Aqk, W, "
                                        f"U~, the inverse; U, Q^S, Aqk U, the state update)"},
                     "pipeline": {"t_roof_us": t_roof * 1e6, "t_measured_us": ms_step * 1e3,
                                  "frac": t_roof / (ms_step * 1e-3),
                                  "recipe": "conv (read + write q|k|v) + KDA algorithmic bytes at 8 TB/s, against the "
                                            "measured step"}},
        "cpu_baseline": None,
    }
    # the same achieved figures against what this machine reaches with a plain copy and a library GEMM
    ach = achievable_peaks(dev)
    rf = out["roofline"]
    rf["achievable"] = dict(ach, frac_of_copy=rf["achieved"] / ach["copy_GBps"],
                            mfma_frac_of_gemm=rf["mfma"]["achieved"] / ach["gemm_bf16_TFLOPs"],
                            conv_frac_of_copy=out["config"]["conv_call"]["GBps_algorithmic"] / ach["copy_GBps"])
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = _cpu_baseline(inp, w, args.cpu_sample_tokens // max(B, 1), gate_np)
        if pool is not None and gate_np is None:
            out["config"]["cpu_baseline_all_cores"] = _cpu_baseline_pool(pool, ncores, inp, w,
                                                                         args.cpu_sample_tokens // max(B, 1))
            out["config"]["cpu_baseline_all_cores"]["cpu"] = cpu_model()
            out["config"]["cpu_baseline_all_cores"]["os_cpu_count"] = os.cpu_count()
    if pool is not None:
        pool.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
