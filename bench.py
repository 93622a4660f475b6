#!/usr/bin/env python
"""Benchmark of the GDN chunked prefill on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic inputs that
are already resident in HBM: the forward (gdn_chunk_fwd: intra-chunk kernel, CP
preprocessing, inter-chunk recurrence) followed by the backward (gdn_chunk_bwd:
recomputation, reverse adjoint pass, per-chunk gradients). The default workload
is batch-1 agentic prefill: B=1, H=16, T=32768, dk=dv=128, chunk 64, bf16
q/k/v with fp32 gates and initial state, AutoCP on; the backward's upstream
gradients are dO ~ N(0,1) (bf16) and d(final state) ~ N(0,0.1).

Prints one JSON line: tokens/s of the step (and of the forward and backward
timed alone), TFLOP/s on algorithmic flops, the roofline fraction of the
step's dominant kernel (algorithmic bytes over its HIP-event-timed launch
duration) and the CPU oracle timed on this host's cores. The headline step
is what the autograd wrapper runs by default: the backward recomputes the
forward's intra-chunk results and CP preprocessing. "reuse_cp" reports the
variant whose forward hands its CP decisions and sub-sequence entry states
(fp32 [segments, H, V, K], 16 MB at the default workload) to the backward,
which skips the forward-direction CP preprocessing; "keep_forward" the
opt-in variant whose backward starts from the forward's kept workspace (more
memory held between the passes, less backward work); "qk_l2norm" the same
step on raw q and k, normalised inside the library.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--pass both|fwd|bwd]
                  [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC_BASE = "GDN chunked-prefill fwd/bwd tokens/s and TFLOP/s (% roofline)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3       # dense fp32 MFMA
FLUSH_BYTES = 1 << 30          # written between flushed calls: 4x the 256 MB Infinity Cache


def metric_name(w, B, T, H, lengths):
    """The metric string with the workload's shape, e.g. "... , B=1 H=16 T=32K"."""
    if lengths is not None:
        return f"{METRIC_BASE}, varlen {len(lengths)} seqs ({sum(lengths)} tokens) H={H}"
    t = f"{T // 1024}K" if T % 1024 == 0 else str(T)
    return f"{METRIC_BASE}, B={B} H={H} T={t}"


def algorithmic_counts(B, T, H, K, V, esize, N, nseg_total, lengths=None, carried=False):
    """Algorithmic bytes and flops per kernel for the whole workload.

    Bytes count each operand a kernel must read once and each result it writes once
    (per token-head unless noted; e = input element size):
      intra        reads k, v, g, beta; writes w, u, gate cumsum            (2K+2V) e + 12
                   (the backward's launch also writes T = (I+A)^-1: + 64 e)
      recur_out    reads q, k, w, u, gate cumsum; writes o                  (3K+2V) e + 4
                   + initial / final states and sub-sequence entry states
      recur_states reads k, w, u, gate cumsum; writes Delta               (2K+2V) e + 4
                   + one V x K state per chunk
      bwd_reverse  reads q, k, w, dO, gate cumsum; writes dDelta          (3K+2V) e + 4
                   + one V x K adjoint per chunk
      bwd_chunk    reads q, k, v, dO, Delta, dDelta, T, gate cumsum, beta and the chunk's
                   state and adjoint; writes dq, dk, dv, dg, dbeta
                                                  (2K+4V+64) e + 8 + (2K+V) e + 8 + 2 V K e / 64
                   carrying the adjoint it reads neither dDelta nor the adjoints
                                                  (2K+3V+64) e + 8 + (2K+V) e + 8 + V K e / 64
    Flops per chunk of c tokens (C=64; triangular products at half):
      forward   intra: c(c-1)K + c(c-1)(c-2)/3 + c(c-1)(K+V);  recur: 3*2cKV + c(c+1)(K+V)
      backward  the reverse-mode products of the chunk map: dQt, dDelta (both terms), dKt,
                the adjoint update (two terms), dW: 7 * 2cKV; dP, dT, dBk, dBv, the two
                M products, (L.dP)K, (L.dP)^T Q: c^2 (2V + 2(K+V) + K + V + 2K + 2K);
                dA = T^T dT T^T: 2 c^3 / 3
    """
    C = 64
    lens = lengths if lengths is not None else [T] * B
    toks = sum(lens)
    th = toks * H
    chunks = sum((n + C - 1) // C for n in lens)
    st = V * K * esize  # one state in the input precision
    nb = dict(
        intra=th * ((2 * K + 2 * V) * esize + 12),
        recur_out=th * ((3 * K + 2 * V) * esize + 4) + N * H * V * K * 4 * 2 + max(nseg_total - N, 0) * H * V * K * 4,
        recur_states=th * ((2 * K + 2 * V) * esize + 4) + chunks * H * st,
        bwd_reverse=th * ((3 * K + 2 * V) * esize + 4) + chunks * H * st,
        bwd_chunk=(th * ((2 * K + 3 * V + 64) * esize + 8 + (2 * K + V) * esize + 8) + chunks * H * st
                   if carried else
                   th * ((2 * K + 4 * V + 64) * esize + 8 + (2 * K + V) * esize + 8) + 2 * chunks * H * st),
    )
    f_intra = f_recur = f_bwd = 0.0
    for n in lens:
        for j in range((n + C - 1) // C):
            c = min(C, n - j * C)
            f_intra += c * (c - 1) * K + c * (c - 1) * (c - 2) / 3 + c * (c - 1) * (K + V)
            f_recur += 3 * 2 * c * K * V + c * (c + 1) * (K + V)
            f_bwd += 7 * 2 * c * K * V + c * c * (2 * V + 2 * (K + V) + K + V + 4 * K) + 2 * c ** 3 / 3
    # the method's algorithmic bytes: the forward's two kernels as the pages split them (K1 reads
    # k, v, g, beta and writes w, u, gate cumsum; K3 reads q, k, w, u, gate cumsum and writes o),
    # and the backward's minimal I/O (reads q, k, v, dO, g, beta; writes dq, dk, dv, dg, dbeta),
    # which the per-chunk gradient kernel is priced at since it writes every gradient
    # (per token-head at K = V = 128, bf16: intra 1,036 B, recur_out 1,284 B, the forward 2,320 B,
    # the backward 1,808 B; a fully fused forward's floor, q, k, v, g, beta in and o out, 1,032 B)
    alg = dict(
        intra=th * ((2 * K + 2 * V) * esize + 12),
        recur_out=th * ((3 * K + 2 * V) * esize + 4),
        bwd_chunk=th * ((4 * K + 3 * V) * esize + 16),
        fwd=th * ((5 * K + 4 * V) * esize + 16),
        bwd=th * ((4 * K + 3 * V) * esize + 16),
        fused_min=th * ((2 * K + 2 * V) * esize + 8),
    )
    return dict(bytes=nb, alg_bytes=alg, flops=dict(fwd=(f_intra + f_recur) * H, bwd=f_bwd * H), tokens=toks)


# Source files that define each kernel (plus the shared headers): a traffic figure measured
# with hardware counters holds only for the sources it was measured on.
KERNEL_SOURCES = {
    "intra": ["gdn_intra.hip"], "cp_decide": ["gdn_recur.hip"], "cp_prepass": ["gdn_recur.hip"],
    "cp_scan": ["gdn_recur.hip"], "recur_out": ["gdn_recur.hip"], "recur_states": ["gdn_recur.hip"],
    "bwd_cp_prepass": ["gdn_bwd.hip"], "bwd_cp_scan": ["gdn_recur.hip"], "bwd_reverse": ["gdn_bwd.hip"],
    "bwd_chunk": ["gdn_bwd.hip"],
}


def kernel_source_hash(kernel):
    import hashlib
    csrc = os.path.join(ROOT, "gated_deltanet_chunked_04_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel] + ["gdn_common.h", "gdn_kernels.h"]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the counter summary in profiles/, or None.

    profiles/<kernel>_<workload>_traffic.md carries a line
      traffic: kernel=<k> workload=<w> sources=<hash> bytes_per_launch=<n>
    written from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) scaled by a copy of known
    size; it counts only while the kernel's sources hash to the recorded value."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path) or kernel not in KERNEL_SOURCES:
        return None
    with open(path) as fh:
        for line in fh:
            if line.startswith("traffic:"):
                kv = dict(x.split("=", 1) for x in line.split()[1:])
                if kv.get("kernel") == kernel and kv.get("workload") == workload and \
                        kv.get("sources") == kernel_source_hash(kernel):
                    return int(kv["bytes_per_launch"])
    return None


def cpu_baseline(inp, tokens, passes):
    """The fp64 oracle on this host's cores over the whole workload (every head and token)."""
    from oracle import default_threads, ref_bwd, ref_fwd
    threads = default_threads()
    t0 = time.perf_counter()
    if passes in ("both", "fwd"):
        ref_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], 1.0, inp["initial_state"],
                cu_seqlens=inp.get("cu_seqlens"), nthreads=threads)
    if passes in ("both", "bwd"):
        ref_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["d_o"], 1.0, inp["initial_state"],
                inp["d_final_state"], cu_seqlens=inp.get("cu_seqlens"), nthreads=threads)
    dt = time.perf_counter() - t0
    what = {"both": "forward and backward", "fwd": "forward", "bwd": "backward"}[passes]
    return {"value": round(tokens / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"the whole workload's {what} (every head and token) through the fp64 token-by-token "
                      "oracle; forward OpenMP over sequence x head x 32-row value blocks, backward over "
                      "sequence x head"}


def decode_bench(gdn, H, K, V, dtype, reps=50):
    """The recurrent form after a prefill (gdn_recurrent_fwd), one token per call with the state
    updated in place: a batch of 64 sequences (priced against the HBM roofline: the call reads
    and writes every state once, plus q, k, v, g, beta and o) and a single sequence (latency).
    HIP-event timing over `reps` calls on the current stream."""
    import torch
    out = {}
    for B in (64, 1):
        gen = torch.Generator().manual_seed(5)
        q = torch.nn.functional.normalize(torch.randn((B, 1, H, K), generator=gen), dim=-1).to(dtype).cuda()
        k = torch.nn.functional.normalize(torch.randn((B, 1, H, K), generator=gen), dim=-1).to(dtype).cuda()
        v = torch.randn((B, 1, H, V), generator=gen).to(dtype).cuda()
        g = (-torch.nn.functional.softplus(torch.randn((B, 1, H), generator=gen)) * 0.1).cuda()
        beta = torch.sigmoid(torch.randn((B, 1, H), generator=gen)).cuda()
        state = (torch.randn((B, H, V, K), generator=gen) * 0.1).cuda()
        o = torch.empty_like(v)
        for _ in range(5):
            gdn.gdn_recurrent_fwd(q, k, v, g, beta, state, state_out=state, o=o)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            gdn.gdn_recurrent_fwd(q, k, v, g, beta, state, state_out=state, o=o)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        es = q.element_size()
        nbytes = B * H * (2 * V * K * 4 + (2 * K + 2 * V) * es + 8)
        out[f"B{B}"] = {"H": H, "K": K, "V": V, "tokens_per_call": B, "us_per_call": round(us, 2),
                        "tokens_per_s": round(B / (us * 1e-6), 1), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                        "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        if B == 1:
            # the same steps captured in a HIP graph (no host work per token): the GPU-side
            # latency of one decode step
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(reps):
                    gdn.gdn_recurrent_fwd(q, k, v, g, beta, state, state_out=state, o=o)
            graph.replay()
            torch.cuda.synchronize()
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            out["B1"]["graph_us_per_call"] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
            del graph
    return out


def l2norm_leg(gdn, dev, cu, cu_host, cp, timed, steps):
    """The same step with the q/k L2 normalisation inside the library (GDN_FLAG_QK_L2NORM):
    its time, and the reverse-mode kernel against the HBM roofline (it reads the raw q and k
    rows and their gradients and writes the gradients: 6 row passes of q's size). The forward
    normalisation has no kernel of its own: the kernels that stage q and k normalise the rows
    there (the intra-chunk kernel also writes the normalised k rows once)."""
    import torch
    q, k, v, g, beta, s0 = (dev[x] for x in ("q", "k", "v", "g", "beta", "initial_state"))
    kw = dict(cu_seqlens=cu, cu_seqlens_host=cu_host, cp_mode=cp, qk_l2norm=True)
    ws = gdn.gdn_workspace(q, v, **kw)
    o = torch.empty_like(v)
    B, T, H, K = q.shape
    N = B if cu is None else int(cu.numel()) - 1
    sT = torch.empty((N, H, v.shape[-1], K), dtype=torch.float32, device=q.device)
    grads = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                 dg=torch.empty_like(g), dbeta=torch.empty_like(beta),
                 d_initial_state=torch.empty_like(sT))

    def step():
        gdn.gdn_chunk_fwd(q, k, v, g, beta, s0, workspace=ws, o=o, final_state=sT, **kw)
        gdn.gdn_chunk_bwd(q, k, v, g, beta, dev["d_o"], s0, dev["d_final_state"], workspace=ws, out=grads, **kw)

    step()
    ms = timed(step, steps)
    gdn.gdn_profile_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kt = gdn.gdn_profile_read()
    gdn.gdn_profile_enable(False)
    row_bytes = q.numel() * q.element_size()  # all q rows (and as many k rows)
    out = {"ms_per_step": round(ms, 4), "kernels": {}}
    for name, passes in (("qk_l2norm_bwd", 6),):
        n, tot = kt[name]
        us = 1e3 * tot / n
        gbs = passes * row_bytes / (us * 1e-6) / 1e9
        out["kernels"][name] = {"avg_launch_us": round(us, 2), "algorithmic_bytes": passes * row_bytes,
                                "GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def copy_ceiling(buf, reps=10):
    """A plain device-to-device copy through torch (one read and one write of each byte) of half
    of `buf` into its other half, HIP-event timed: the practical streaming rate on this part."""
    import torch
    n = buf.numel() // 2
    src, dst = buf[:n], buf[n:2 * n]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    dst.copy_(src)
    for a, b in ev:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in ev)
    med = ts[reps // 2]
    return {"bytes_copied": int(n), "median_ms": round(med, 4), "GB/s": round(2 * n / (med * 1e-3) / 1e9, 1),
            "frac": round(2 * n / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def fused_leg(gdn, flush, reps=10):
    """The fully fused forward against the two-kernel split (both CP off, bf16, K = V = 128) where
    the plan picks it, a uniform batch of 8 x 4096 tokens and 64 heads (512 sequence-heads: two rounds
    of recurrence workgroups), and on the packed-varlen workload's shape (8 sequences, H = 32, the
    recurrence in one round). Inputs drawn on the device; flushed calls, median ms."""
    import torch
    from gdn_inputs import WORKLOADS, varlen_lengths
    w = WORKLOADS["varlen_packed"]
    lens, _ = varlen_lengths(w.varlen_count, *w.varlen_range, w.varlen_total, 0)
    shapes = {"B8_H64_T4K": dict(B=8, T=4096, H=64, lengths=None),
              "varlen_packed": dict(B=1, T=sum(lens), H=32, lengths=lens)}
    out = {}
    gen = torch.Generator(device="cuda").manual_seed(7)
    for name, sh in shapes.items():
        B, T, H = sh["B"], sh["T"], sh["H"]
        K = V = 128
        q = torch.nn.functional.normalize(torch.randn((B, T, H, K), device="cuda", generator=gen), dim=-1).bfloat16()
        k = torch.nn.functional.normalize(torch.randn((B, T, H, K), device="cuda", generator=gen), dim=-1).bfloat16()
        v = torch.randn((B, T, H, V), device="cuda", generator=gen).bfloat16()
        g = -torch.nn.functional.softplus(torch.randn((B, T, H), device="cuda", generator=gen)) * 0.1
        beta = torch.sigmoid(torch.randn((B, T, H), device="cuda", generator=gen))
        cu = cu_host = None
        if sh["lengths"] is not None:
            import numpy as np
            cu_host = torch.tensor(np.concatenate([[0], np.cumsum(sh["lengths"])]), dtype=torch.int32)
            cu = cu_host.cuda()
        N = B if cu is None else len(sh["lengths"])
        o = torch.empty_like(v)
        sT = torch.empty((N, H, V, K), dtype=torch.float32, device="cuda")
        kw = dict(cu_seqlens=cu, cu_seqlens_host=cu_host, cp_mode="off", o=o, final_state=sT)
        planned = gdn.gdn_plan(gdn.make_desc(q, v, cu_seqlens=cu, cu_seqlens_host=cu_host, cp_mode="off"))
        ws = torch.empty(planned["fwd_workspace_bytes"], dtype=torch.uint8, device="cuda")
        res = {"tokens": int(B * T), "heads": H, "planned_fused": planned["fused_fwd"]}
        th = B * T * H
        for label, fused in (("split", False), ("fused", True)):
            def call():
                gdn.gdn_chunk_fwd(q, k, v, g, beta, None, workspace=ws, fused=fused, **kw)
            call()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for i in range(reps):
                flush(i)
                ev[i][0].record()
                call()
                ev[i][1].record()
            torch.cuda.synchronize()
            ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
            res[label] = {"ms": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
                          # the bytes of that design: 2,320 B per token-head split, 1,032 B fused
                          "GB/s": round(th * (2320 if label == "split" else 1032) / (ms * 1e-3) / 1e9, 1)}
        res["fused_speedup"] = round(res["split"]["ms"] / res["fused"]["ms"], 3)
        out[name] = res
        del q, k, v, g, beta, o, sT, ws
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="edge_prefill")
    ap.add_argument("--pass", dest="passes", default="both", choices=["both", "fwd", "bwd"])
    ap.add_argument("--cp", default=None, help="override the workload's CP mode (auto/off/on/exact/warmup)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fused-leg", action="store_true", help="skip the fused-forward comparison")
    ap.add_argument("--only-step", action="store_true",
                    help="time the step only (no flushed calls, no extra legs, no CPU baseline): for profilers")
    ap.add_argument("--flushed-calls", type=int, default=50,
                    help="calls timed one by one after a 1 GiB cache flush (median and minimum)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run one device-to-device copy of this many MiB (a reference for HBM "
                         "byte counters taken with rocprofv3 --pmc)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the GDN chunked prefill here runs on a single MI355X and has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import dataclasses

    import torch

    import gated_deltanet_chunked_04_amd as gdn
    from gdn_inputs import WORKLOADS, make_inputs

    gdn.load_library()
    w = WORKLOADS[args.workload]
    if args.passes != "fwd" and not w.backward:
        w = dataclasses.replace(w, backward=True)  # draw dO and d(final state) too
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
    do_fwd = args.passes in ("both", "fwd")
    do_bwd = args.passes in ("both", "bwd")
    ws = torch.empty(max(plan["fwd_workspace_bytes"], plan["bwd_workspace_bytes"] if do_bwd else 0),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty((B, T, H, V), dtype=q.dtype, device="cuda")
    sT = torch.empty((N, H, V, K), dtype=torch.float32, device="cuda")
    grads = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v), dg=torch.empty_like(g),
                 dbeta=torch.empty_like(beta), d_initial_state=torch.empty((N, H, V, K), dtype=torch.float32,
                                                                          device="cuda"))

    # the forward's CP decisions and sub-sequence entry states, handed to the backward (None
    # without CP, or when the backward runs without a forward)
    cps = (gdn.gdn_cp_states(q, v, cu_seqlens=cu, cu_seqlens_host=cu_host, cp_mode=cp)
           if do_fwd and do_bwd else None)

    def fwd(carry=False):
        gdn.gdn_chunk_fwd(q, k, v, g, beta, s0, cu_seqlens=cu, cu_seqlens_host=cu_host, cp_mode=cp,
                          workspace=ws, o=o, final_state=sT, cp_states=cps if carry else None)

    def bwd(carry=False):
        gdn.gdn_chunk_bwd(q, k, v, g, beta, dev["d_o"], s0, dev["d_final_state"], cu_seqlens=cu,
                          cu_seqlens_host=cu_host, cp_mode=cp, workspace=ws, out=grads,
                          cp_states=cps if carry else None)

    def step():
        if do_fwd:
            fwd()
        if do_bwd:
            bwd()

    def step_reuse_cp():
        # the backward takes the forward-direction CP results from the forward
        fwd(True)
        bwd(True)

    def step_keep():
        # the opt-in variant: the forward keeps W, U, T, the gate cumsum and the CP entry
        # states in the workspace (which covers both layouts) and the backward starts from them
        gdn.gdn_chunk_fwd(q, k, v, g, beta, s0, cu_seqlens=cu, cu_seqlens_host=cu_host, cp_mode=cp,
                          workspace=ws, o=o, final_state=sT, keep_for_backward=True)
        gdn.gdn_chunk_bwd(q, k, v, g, beta, dev["d_o"], s0, dev["d_final_state"], cu_seqlens=cu,
                          cu_seqlens_host=cu_host, cp_mode=cp, workspace=ws, out=grads, reuse_forward=True)

    def timed(fn, n):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n

    if args.copy_calibration > 0:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE read per dispatch calibrate
        # the same counters for the kernels
        src = torch.empty(args.copy_calibration << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # 1 GiB written between flushed calls evicts the 256 MB Infinity Cache and the L2s, so each
    # flushed call reads its inputs from HBM
    flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")

    def flushed(fn, n):
        """HIP-event durations of n calls on the current stream, each after a flush (the flush
        is outside the events); median and minimum in ms."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            flush_buf.fill_(i & 255)
            ev[i][0].record()
            fn()
            ev[i][1].record()
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in ev)
        return {"median_ms": round(ts[n // 2] if n % 2 else 0.5 * (ts[n // 2 - 1] + ts[n // 2]), 4),
                "min_ms": round(ts[0], 4), "calls": n}

    for _ in range(args.warmup):
        step()
    ms = timed(step, args.steps)
    if args.only_step:
        gdn.gdn_profile_enable(True)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        kt = gdn.gdn_profile_read()
        gdn.gdn_profile_enable(False)
        print(json.dumps({"metric": metric_name(w, B, T, H, lengths), "ms_per_step": round(ms, 4),
                          "steps": args.steps, "warmup": args.warmup, "config": {"workload": w.name},
                          "kernels_us_per_step": {n: round(1e3 * t / args.steps, 2) for n, (c, t) in kt.items()}}),
              flush=True)
        return
    ms_fwd = timed(fwd, args.steps) if do_fwd else None
    ms_bwd = timed(bwd, args.steps) if do_bwd else None
    fl_step = flushed(step, args.flushed_calls)
    fl_fwd = flushed(fwd, args.flushed_calls) if do_fwd else None
    fl_bwd = flushed(bwd, args.flushed_calls) if do_bwd else None
    ms_keep = ms_rcp = None
    if do_fwd and do_bwd:
        step_keep()
        ms_keep = timed(step_keep, args.steps)
        if cps is not None:
            step_reuse_cp()
            ms_rcp = timed(step_reuse_cp, args.steps)
    fused = fused_leg(gdn, lambda i: flush_buf.fill_(i & 255)) if (do_fwd and not args.no_fused_leg) else None
    l2 = l2norm_leg(gdn, dev, cu, cu_host, cp, timed, args.steps) if (do_fwd and do_bwd) else None

    # Per-kernel durations: one more round of steps, each after a flush, with every launch
    # bracketed by HIP events on its launch stream (separate from the timed loops above).
    gdn.gdn_profile_enable(True)
    for i in range(args.steps):
        flush_buf.fill_(i & 255)
        step()
    torch.cuda.synchronize()
    kt = gdn.gdn_profile_read()
    gdn.gdn_profile_enable(False)
    # average duration of one launch, and total per step
    kernels = {name: {"launches": n, "avg_us": 1e3 * tot / n, "per_step_us": 1e3 * tot / args.steps}
               for name, (n, tot) in kt.items()}
    copy = copy_ceiling(flush_buf)
    del flush_buf

    esize = 2 if q.dtype == torch.bfloat16 else 4
    counts = algorithmic_counts(B, T, H, K, V, esize, N, plan["total_segments"], lengths,
                                carried=bool(plan["bwd_carried"]))
    tokens = counts["tokens"]
    alg = counts["alg_bytes"]
    flops_step = (counts["flops"]["fwd"] if do_fwd else 0) + (counts["flops"]["bwd"] if do_bwd else 0)
    # the dominant kernel among those the method's byte accounting prices (each launch covers
    # the whole workload once)
    dominant = max((n for n in kernels if n in alg), key=lambda n: kernels[n]["per_step_us"])
    dur_s = kernels[dominant]["avg_us"] * 1e-6
    achieved = alg[dominant] / dur_s / 1e9
    design = counts["bytes"][dominant]
    roofline = {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(dominant, w.name),
                "algorithmic_bytes_per_launch": int(alg[dominant]), "avg_launch_us": round(dur_s * 1e6, 2),
                # what this design's kernel actually has to move (its intermediates too)
                "design_bytes_per_launch": int(design),
                "design_frac": round(design / dur_s / 1e9 / HBM_PEAK_GBS, 4)}
    peak_mfma = BF16_PEAK_TFLOPS if esize == 2 else FP32_PEAK_TFLOPS
    tflops = flops_step / (ms * 1e-3) / 1e12

    def kroof(n):
        us = kernels[n]["avg_us"]
        r = {"avg_launch_us": round(us, 2)}
        if n in alg:
            r["algorithmic_bytes"] = int(alg[n])
            r["GB/s"] = round(alg[n] / (us * 1e-6) / 1e9, 1)
            r["frac"] = round(alg[n] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        if n in counts["bytes"]:
            r["design_bytes"] = int(counts["bytes"][n])
            r["design_frac"] = round(counts["bytes"][n] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        return r

    def pass_roofline(nbytes, flops, t_ms):
        gbs = nbytes / (t_ms * 1e-3) / 1e9
        return {"bound": "hbm", "algorithmic_bytes": int(nbytes), "GB/s": round(gbs, 1),
                "frac": round(gbs / HBM_PEAK_GBS, 4), "frac_of_copy": round(gbs / copy["GB/s"], 4),
                "mfma_frac": round(flops / (t_ms * 1e-3) / 1e12 / peak_mfma, 4)}

    cp_stats = None
    if plan["cp_on"]:
        # the per-boundary CP decision of this workload: the share of sub-sequence boundaries that
        # take the warmup (forward; reverse for the backward's adjoint pass) and the head summary
        fw, rv = gdn.gdn_cp_windows(k, v, g, beta, cu_seqlens=cu, cu_seqlens_host=cu_host, cp_mode=cp)
        modes = gdn.gdn_cp_modes(k, v, g, beta, cu_seqlens=cu, cu_seqlens_host=cu_host, cp_mode=cp).cpu()
        fw, rv = fw.cpu(), rv.cpu()
        nb = int((fw >= 0).sum())
        cp_stats = {"boundaries": nb,
                    "warmup_frac_fwd": round(float((fw > 0).sum()) / max(nb, 1), 4),
                    "warmup_frac_rev": round(float((rv > 0).sum()) / max(nb, 1), 4),
                    "mean_window_chunks": round(float(fw[fw > 0].float().mean()) if (fw > 0).any() else 0.0, 2),
                    "sequence_heads": {"all_warmup": int((modes == 1).sum()), "mixed": int((modes == 3).sum()),
                                       "all_exact": int((modes == 2).sum())}}
    line = {
        "metric": metric_name(w, B, T, H, lengths),
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
        "config": {"workload": w.name, "pass": args.passes, "B": B, "T": T, "H": H, "K": K, "V": V,
                   "chunk": 64, "cp": cp, "cp_on": plan["cp_on"], "seg_chunks": plan["seg_chunks"],
                   "segments": plan["total_segments"], "tokens": tokens},
        "tflops": round(tflops, 2),
        "mfma_frac": round(tflops / peak_mfma, 4),
        "roofline": roofline,
        "cp": cp_stats,
        # every call after a 1 GiB cache flush, HIP events around the call (median, minimum)
        "flushed": {"step": fl_step, "tokens_per_s_median": round(tokens / (fl_step["median_ms"] * 1e-3), 1)},
        "copy_ceiling": copy,
        "kernels_us_per_step": {n: round(x["per_step_us"], 2) for n, x in kernels.items()},
        # every kernel against the HBM roofline on flushed steps: "frac" on the method's
        # algorithmic bytes where it prices the kernel, "design_frac" on what this design's kernel
        # moves (the backward's reverse chain runs beside its state chain on a second stream, so
        # those durations include shared time; k_intra's average mixes the forward launch with
        # the backward's, which also writes T)
        "kernels_roofline": {n: kroof(n) for n in kernels if n in alg or n in counts["bytes"]},
    }
    if do_fwd:
        line["fwd"] = {"ms": round(ms_fwd, 4), "tokens_per_s": round(tokens / (ms_fwd * 1e-3), 1),
                       "tflops": round(counts["flops"]["fwd"] / (ms_fwd * 1e-3) / 1e12, 2), "flushed": fl_fwd,
                       # the pages' two-kernel method's bytes over the flushed median
                       "roofline": pass_roofline(alg["fwd"], counts["flops"]["fwd"], fl_fwd["median_ms"]),
                       "fused_min_bytes": int(alg["fused_min"])}
    if do_bwd:
        line["bwd"] = {"ms": round(ms_bwd, 4), "tokens_per_s": round(tokens / (ms_bwd * 1e-3), 1),
                       "tflops": round(counts["flops"]["bwd"] / (ms_bwd * 1e-3) / 1e12, 2), "flushed": fl_bwd,
                       "roofline": pass_roofline(alg["bwd"], counts["flops"]["bwd"], fl_bwd["median_ms"])}
    if ms_rcp is not None:
        line["reuse_cp"] = {"ms_per_step": round(ms_rcp, 4),
                                "tokens_per_s": round(tokens / (ms_rcp * 1e-3), 1),
                                "cp_states_bytes": int(cps.numel())}
    if ms_keep is not None:
        line["keep_forward"] = {"ms_per_step": round(ms_keep, 4),
                                "tokens_per_s": round(tokens / (ms_keep * 1e-3), 1)}
    if l2 is not None:
        l2["overhead_ms"] = round(l2["ms_per_step"] - ms, 4)
        line["qk_l2norm"] = l2
    if fused is not None:
        line["fused_forward"] = fused
    line["decode"] = decode_bench(gdn, H, K, V, q.dtype)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, tokens, args.passes)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
