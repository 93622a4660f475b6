#!/usr/bin/env python
"""Benchmark of the GDN chunked prefill on one MI355X.

A step is one call of the library's forward (gdn_chunk_fwd: intra-chunk kernel,
CP preprocessing, inter-chunk recurrence) over one batch of synthetic inputs
that are already resident in HBM. The default workload is batch-1 agentic
prefill: B=1, H=16, T=32768, dk=dv=128, chunk 64, bf16 q/k/v with fp32 gates,
AutoCP on.

Prints one JSON line with tokens/s, TFLOP/s, the roofline fraction of the
dominant kernel (algorithmic bytes over its HIP-event-timed launch duration)
and the CPU oracle timed on this host's cores.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN chunked-prefill fwd/bwd tokens/s and TFLOP/s (% roofline), B=1 H=16 T=32K"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3       # dense fp32 MFMA


def algorithmic_counts(B, T, H, K, V, esize, N, nseg_total, lengths=None):
    """Algorithmic bytes and flops of the forward, per kernel, for the whole workload.

    Bytes count each input read once and each output written once:
      intra      reads k, v, g, beta; writes w, u, the gate cumsum        ((2K+2V) e + 12 per token-head)
      recur_out  reads q, k, w, u, the gate cumsum; writes o               ((3K+2V) e + 4 per token-head)
                 + the initial / final states and the sub-sequence entry states
    Flops per full chunk of C=64 tokens (triangular products at half):
      intra      Gram C(C-1)K + inverse C(C-1)(C-2)/3 + w,u C(C-1)(K+V)
      recur_out  3 * 2CKV + C(C+1)(K+V)
    """
    C = 64
    toks = B * T if lengths is None else sum(lengths)
    th = toks * H
    b_intra = th * ((2 * K + 2 * V) * esize + 12)
    b_recur = th * ((3 * K + 2 * V) * esize + 4) + N * H * V * K * 4 * 2 + max(nseg_total - N, 0) * H * V * K * 4
    chunks = [((n + C - 1) // C) for n in (lengths if lengths is not None else [T] * B)]
    f_intra = f_recur = 0.0
    for n, nch in zip(lengths if lengths is not None else [T] * B, chunks):
        for j in range(nch):
            c = min(C, n - j * C)
            f_intra += c * (c - 1) * K + c * (c - 1) * (c - 2) / 3 + c * (c - 1) * (K + V)
            f_recur += 3 * 2 * c * K * V + c * (c + 1) * (K + V)
    return dict(bytes=dict(intra=b_intra, recur_out=b_recur),
                flops=dict(intra=f_intra * H, recur_out=f_recur * H), tokens=toks)


def cpu_baseline(inp, tokens):
    from oracle import default_threads, ref_fwd
    threads = default_threads()
    t0 = time.perf_counter()
    ref_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], 1.0, inp["initial_state"],
            cu_seqlens=inp.get("cu_seqlens"), nthreads=threads)
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "seconds": dt,
            "sample": "the whole workload's forward (every head and token) through the fp64 token-by-token "
                      "oracle, OpenMP over sequence x head x 32-row value blocks"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="edge_prefill")
    ap.add_argument("--cp", default=None, help="override the workload's CP mode (auto/off/on/exact/warmup)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the GDN chunked prefill here runs on a single MI355X and has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_deltanet_chunked_04_amd as gdn
    from gdn_inputs import WORKLOADS, make_inputs

    gdn.load_library()
    w = WORKLOADS[args.workload]
    cp = args.cp or w.cp
    inp = make_inputs(w, seed=0)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    q, k, v, g, beta, s0 = (dev[x] for x in ("q", "k", "v", "g", "beta", "initial_state"))
    cu = dev.get("cu_seqlens")
    cu_host = inp.get("cu_seqlens")
    B, T, H, K = q.shape
    V = v.shape[-1]
    lengths = inp["meta"].get("lengths")
    N = B if cu is None else len(lengths)
    desc = gdn.make_desc(q, v, cu_seqlens=cu, cu_seqlens_host=cu_host, cp_mode=cp)
    plan = gdn.gdn_plan(desc)
    ws = torch.empty(plan["fwd_workspace_bytes"], dtype=torch.uint8, device="cuda")
    o = torch.empty((B, T, H, V), dtype=q.dtype, device="cuda")
    sT = torch.empty((N, H, V, K), dtype=torch.float32, device="cuda")

    def step():
        gdn.gdn_chunk_fwd(q, k, v, g, beta, s0, cu_seqlens=cu, cu_seqlens_host=cu_host, cp_mode=cp,
                          workspace=ws, o=o, final_state=sT)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps

    # Per-kernel durations: the same steps with every launch bracketed by HIP events on
    # the launch stream (separate pass, so the events do not perturb ms_per_step).
    gdn.gdn_profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = gdn.gdn_profile_read()
    gdn.gdn_profile_enable(False)
    kernels = {name: {"launches": n, "avg_us": 1e3 * tot / n} for name, (n, tot) in kt.items()}

    esize = 2 if q.dtype == torch.bfloat16 else 4
    counts = algorithmic_counts(B, T, H, K, V, esize, N, plan["total_segments"], lengths)
    tokens = counts["tokens"]
    flops_step = sum(counts["flops"].values())
    dominant = max(("intra", "recur_out"), key=lambda n: kernels.get(n, {"avg_us": 0})["avg_us"])
    dur_s = kernels[dominant]["avg_us"] * 1e-6
    achieved = counts["bytes"][dominant] / dur_s / 1e9
    roofline = {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "algorithmic_bytes": counts["bytes"][dominant], "avg_launch_us": round(dur_s * 1e6, 2)}
    tflops = flops_step / (ms * 1e-3) / 1e12
    peak_mfma = BF16_PEAK_TFLOPS if esize == 2 else FP32_PEAK_TFLOPS
    line = {
        "metric": METRIC,
        "value": round(tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if esize == 2 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "fwd", "B": B, "T": T, "H": H, "K": K, "V": V, "chunk": 64,
                   "cp": cp, "cp_on": plan["cp_on"], "seg_chunks": plan["seg_chunks"],
                   "segments": plan["total_segments"], "tokens": tokens},
        "tflops": round(tflops, 2),
        "mfma_frac": round(tflops / peak_mfma, 4),
        "step_hbm_frac": round(sum(counts["bytes"].values()) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": roofline,
        "kernels_us": {n: round(x["avg_us"], 2) for n, x in kernels.items()},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, tokens)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
