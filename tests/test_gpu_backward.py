"""GPU parity of the backward (gdn_chunk_bwd) against the CPU oracle's reverse mode.

All six gradients (dq, dk, dv, dg, dbeta, d(initial state)) must be within
relative L2 1e-4 in fp32 mode and 1e-2 for bf16 inputs, with CP off, exact,
warmup and gated, ragged tails, packed varlen and dk != dv.
"""
import numpy as np
import pytest
import torch

from gdn_inputs import make_inputs
from gpu_helpers import (check, gpu_fwd, mid_decay_inputs, mixed_decay_inputs, oracle, raw_key_inputs, seq_slices,
                         small_inputs, to_dev, tol_for)
from oracle import ref_bwd

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "d_initial_state")


def with_grads(inp, seed=7):
    gen = torch.Generator().manual_seed(seed)
    B, T, H, V = inp["v"].shape
    N = B if inp.get("cu_seqlens") is None else len(inp["cu_seqlens"]) - 1
    K = inp["q"].shape[-1]
    inp["d_o"] = torch.randn((B, T, H, V), generator=gen).to(inp["q"].dtype)
    inp["d_final_state"] = torch.randn((N, H, V, K), generator=gen) * 0.1
    return inp


def gpu_bwd(d, **kw):
    import gated_deltanet_chunked_04_amd as gdn
    out = gdn.gdn_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["d_o"], d["initial_state"],
                            d["d_final_state"], cu_seqlens=d.get("cu_seqlens"), **kw)
    torch.cuda.synchronize()
    return out


def oracle_bwd(inp, scale=1.0, heads=None):
    x = dict(inp)
    if heads is not None:
        for n in ("q", "k", "v", "g", "beta", "d_o"):
            x[n] = inp[n][:, :, heads]
        for n in ("initial_state", "d_final_state"):
            x[n] = None if inp[n] is None else inp[n][:, heads]
    return ref_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["d_o"], scale, x["initial_state"],
                   x["d_final_state"], cu_seqlens=inp.get("cu_seqlens"))


def compare(out, ref, tol, heads=None):
    errs = {}
    for n in NAMES:
        x = out[n]
        if heads is not None:
            x = x[:, :, heads] if n != "d_initial_state" else x[:, heads]
        errs[n] = check(x, ref[n], tol, n)
    return errs


def test_tiny_workload_fp32(gpu_lib):
    inp = make_inputs("tiny", seed=0)
    out = gpu_bwd(to_dev(inp))
    ref = oracle_bwd(inp)
    print(compare(out, ref, 1e-4))


CASES = [
    (torch.float32, 64, 64, "off", {}),
    (torch.float32, 64, 64, "exact", dict(seg_chunks=3)),
    (torch.float32, 64, 64, "warmup", dict(seg_chunks=4, warmup_chunks=6)),
    (torch.bfloat16, 128, 128, "off", {}),
    (torch.bfloat16, 128, 128, "exact", dict(seg_chunks=3)),
    (torch.bfloat16, 128, 128, "warmup", dict(seg_chunks=4, warmup_chunks=3)),
    (torch.bfloat16, 128, 128, "on", dict(seg_chunks=4)),
    (torch.bfloat16, 64, 128, "exact", dict(seg_chunks=4)),
    (torch.bfloat16, 128, 64, "off", {}),
    (torch.bfloat16, 64, 64, "auto", {}),
    # longer sub-sequences (8 chunks or more), ragged ones included
    (torch.float32, 64, 64, "exact", dict(seg_chunks=8)),
    (torch.float32, 64, 64, "exact", dict(seg_chunks=9)),
    (torch.bfloat16, 128, 128, "exact", dict(seg_chunks=8)),
    (torch.bfloat16, 64, 128, "exact", dict(seg_chunks=11)),
    (torch.bfloat16, 128, 128, "on", dict(seg_chunks=8, warmup_chunks=3)),
]


@pytest.mark.parametrize("dtype,K,V,cp,kw", CASES)
def test_backward_small(gpu_lib, dtype, K, V, cp, kw):
    inp = with_grads(small_inputs(B=2, T=1000, H=2, K=K, V=V, dtype=dtype, seed=11))
    out = gpu_bwd(to_dev(inp), scale=0.9, cp_mode=cp, **kw)
    ref = oracle_bwd(inp, scale=0.9)
    compare(out, ref, tol_for(dtype))


@pytest.mark.parametrize("cp,kw", [("off", {}), ("exact", dict(seg_chunks=2)),
                                   ("warmup", dict(seg_chunks=3, warmup_chunks=2)),
                                   ("exact", dict(seg_chunks=8)), ("on", dict(seg_chunks=9, warmup_chunks=2))])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_backward_varlen(gpu_lib, cp, kw, dtype):
    K = V = 64 if dtype == torch.float32 else 128
    lengths = [1, 63, 64, 65, 0, 700, 1500, 129]
    inp = with_grads(small_inputs(H=3, K=K, V=V, dtype=dtype, lengths=lengths, seed=12))
    out = gpu_bwd(to_dev(inp), cp_mode=cp, **kw)
    ref = oracle_bwd(inp)
    tol = tol_for(dtype)
    compare(out, ref, tol)
    # every sequence on its own: the token gradients of each sequence and its d(initial state)
    for n, a, b in seq_slices(inp["cu_seqlens"]):
        for name in NAMES[:5]:
            check(out[name][:, a:b], ref[name][:, a:b], tol, f"{name} of sequence {n} ({b - a} tokens)")
        check(out["d_initial_state"][n], ref["d_initial_state"][n], tol, f"d_initial_state of sequence {n}")
    # the empty sequence passes d(final state) straight through
    assert torch.equal(out["d_initial_state"][4].cpu(), inp["d_final_state"][4])


def many_lengths(nseq, seed):
    """Packed lengths with many equal chunk counts (ties of the longest-first order), an
    increasing run, a repeated longest length and empty sequences."""
    rng = np.random.default_rng(seed)
    top = 400 if nseq <= 64 else 140
    body = sorted(int(x) for x in rng.integers(1, top, nseq - 8))
    return [top - 100] * 4 + [0, 1, 64, 65] + body


@pytest.mark.parametrize("nseq,cp,kw", [(40, "off", {}), (40, "exact", dict(seg_chunks=2)),
                                        (600, "off", {}), (600, "exact", dict(seg_chunks=1))])
def test_varlen_many_sequences(gpu_lib, nseq, cp, kw):
    """Packed varlen, forward and backward, with the recurrence grids taking the segments in the
    varlen tables' longest-first order (a counting sort over 40 to 955 segments, many of them
    tied); every sequence checked on its own."""
    lengths = many_lengths(nseq, seed=nseq)
    inp = with_grads(small_inputs(H=2, K=128, V=128, dtype=torch.bfloat16, lengths=lengths, seed=33))
    tol = tol_for(torch.bfloat16)
    d = to_dev(inp)
    o, sT = gpu_fwd(d, cp_mode=cp, **kw)
    o_ref, s_ref = oracle(inp)
    check(o, o_ref, tol, "o")
    check(sT, s_ref, tol, "final_state")
    out = gpu_bwd(d, cp_mode=cp, **kw)
    ref = oracle_bwd(inp)
    compare(out, ref, tol)
    oc = o.cpu()
    for n, a, b in seq_slices(inp["cu_seqlens"]):
        if b - a < 64:
            continue  # the short ones weigh little but are covered by the packed checks above
        check(oc[:, a:b], o_ref[:, a:b], tol, f"o of sequence {n}")
        check(out["dk"][:, a:b], ref["dk"][:, a:b], tol, f"dk of sequence {n}")
        check(out["d_initial_state"][n], ref["d_initial_state"][n], tol, f"d_initial_state of sequence {n}")
    assert torch.equal(sT[4].cpu(), inp["initial_state"][4])


def test_varlen_auto_cp_imbalance(gpu_lib):
    """AutoCP's packed-sequence case: 4 sequences x 32 heads fill the recurrence slots, but the
    longest (64 chunks) takes far more than the 12 chunk steps per slot the batch needs, so AUTO
    splits it into 32-chunk sub-sequences; forward and backward against the oracle."""
    import gated_deltanet_chunked_04_amd as gdn
    lengths = [512, 4096, 500, 520]
    inp = with_grads(small_inputs(H=32, K=128, V=128, dtype=torch.bfloat16, lengths=lengths, seed=41))
    d = to_dev(inp)
    p = gdn.gdn_plan(gdn.make_desc(d["q"], d["v"], cu_seqlens=d["cu_seqlens"], cu_seqlens_host=inp["cu_seqlens"],
                                   cp_mode="auto"))
    if p["cp_on"] != 1:
        pytest.skip(f"AutoCP's slot count on this device leaves CP off ({p['seg_chunks']} chunks)")
    assert p["seg_chunks"] == 32 and p["total_segments"] == 5
    tol = tol_for(torch.bfloat16)
    o, sT = gpu_fwd(d, cp_mode="auto")
    o_ref, s_ref = oracle(inp)
    check(o, o_ref, tol, "o")
    check(sT, s_ref, tol, "final_state")
    compare(gpu_bwd(d, cp_mode="auto"), oracle_bwd(inp), tol)


def test_backward_no_initial_state_no_final_grad(gpu_lib):
    inp = with_grads(small_inputs(B=1, T=300, H=2, K=64, V=64, dtype=torch.float32, init_std=None))
    inp["d_final_state"] = None
    out = gpu_bwd(to_dev(inp), cp_mode="off")
    ref = oracle_bwd(inp)
    compare(out, ref, 1e-4)


def test_backward_deterministic(gpu_lib):
    d = to_dev(with_grads(small_inputs(B=1, T=4096, H=4, seed=13)))
    a = gpu_bwd(d, cp_mode="exact", seg_chunks=16)
    b = gpu_bwd(d, cp_mode="exact", seg_chunks=16)
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n


def test_autograd_wrapper(gpu_lib):
    """chunk_gated_delta_rule under torch.autograd returns the library's gradients."""
    inp = with_grads(small_inputs(B=1, T=500, H=2, K=64, V=64, dtype=torch.float32, seed=14))
    d = to_dev(inp)
    leaves = {n: d[n].clone().requires_grad_(True) for n in ("q", "k", "v", "g", "beta", "initial_state")}
    o, sT = gpu_lib.chunk_gated_delta_rule(leaves["q"], leaves["k"], leaves["v"], leaves["g"], leaves["beta"],
                                           initial_state=leaves["initial_state"])
    loss = (o * d["d_o"]).sum() + (sT * d["d_final_state"]).sum()
    loss.backward()
    ref = oracle_bwd(inp)
    pairs = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", initial_state="d_initial_state")
    for n, r in pairs.items():
        check(leaves[n].grad, ref[r], 1e-4, n)


@pytest.mark.parametrize("cp", ["auto", "off"])
def test_backward_workload_16k(gpu_lib, cp):
    """B=2, H=16, T=16384, bf16, dO ~ N(0,1), d(final state) ~ N(0,0.1); sampled heads."""
    inp = make_inputs("backward", seed=0)
    out = gpu_bwd(to_dev(inp), cp_mode=cp)
    heads = [3, 12]
    ref = oracle_bwd(inp, heads=heads)
    errs = compare({n: out[n].cpu() for n in NAMES}, ref, 1e-2, heads=heads)
    print(f"cp={cp} " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)


def test_backward_edge_prefill_32k(gpu_lib):
    """The benchmarked step's backward: B=1, H=16, T=32768, bf16, AutoCP (on: 16 sub-sequences,
    heads in warmup and exact modes), through the same calls bench.py times (the forward keeping
    its workspace, the backward reusing it, and the recomputing backward); sampled heads against
    the oracle, the two backwards bit for bit."""
    import dataclasses
    from gdn_inputs import WORKLOADS
    gdn = gpu_lib
    inp = make_inputs(dataclasses.replace(WORKLOADS["edge_prefill"], backward=True), seed=0)
    d = to_dev(inp)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    modes = gdn.gdn_cp_modes(d["k"], d["v"], d["g"], d["beta"]).cpu()
    assert (modes == 1).any() and (modes >= 2).any(), modes  # both CP kinds at this workload
    ref = gdn.gdn_chunk_bwd(*args, d["d_o"], d["initial_state"], d["d_final_state"])
    ws = gdn.gdn_workspace(d["q"], d["v"])
    gdn.gdn_chunk_fwd(*args, d["initial_state"], workspace=ws, keep_for_backward=True)
    got = gdn.gdn_chunk_bwd(*args, d["d_o"], d["initial_state"], d["d_final_state"], workspace=ws,
                            reuse_forward=True)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(got[n], ref[n]), n
    # the variant whose forward hands its CP results to the backward
    cps = gdn.gdn_cp_states(d["q"], d["v"])
    assert cps is not None
    gdn.gdn_chunk_fwd(*args, d["initial_state"], workspace=ws, cp_states=cps)
    got = gdn.gdn_chunk_bwd(*args, d["d_o"], d["initial_state"], d["d_final_state"], workspace=ws, cp_states=cps)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(got[n], ref[n]), n
    # one warmup head and one exact head
    heads = [int((modes[0] == 1).nonzero()[0]), int((modes[0] >= 2).nonzero()[0])]
    errs = compare({n: ref[n].cpu() for n in NAMES}, oracle_bwd(inp, heads=heads), 1e-2, heads=heads)
    print(f"heads={heads} " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)


REUSE_CASES = [
    (torch.float32, 64, 64, "off", {}, None),
    (torch.float32, 64, 64, "exact", dict(seg_chunks=3), None),
    (torch.bfloat16, 128, 128, "exact", dict(seg_chunks=3), None),
    (torch.bfloat16, 128, 128, "warmup", dict(seg_chunks=4, warmup_chunks=3), None),
    (torch.bfloat16, 128, 128, "auto", {}, None),
    (torch.bfloat16, 128, 128, "exact", dict(seg_chunks=2), [1, 63, 64, 65, 0, 700, 1500, 129]),
    (torch.bfloat16, 64, 128, "off", {}, [300, 0, 1000]),
]


@pytest.mark.parametrize("dtype,K,V,cp,kw,lengths", REUSE_CASES)
def test_backward_reuses_forward(gpu_lib, dtype, K, V, cp, kw, lengths):
    """A backward that starts from a kept forward's workspace gives the recomputing backward's
    gradients bit for bit (same kernels on the same inputs), and keeping changes no forward output."""
    gdn = gpu_lib
    if lengths is None:
        inp = with_grads(small_inputs(B=2, T=1000, H=2, K=K, V=V, dtype=dtype, seed=15))
    else:
        inp = with_grads(small_inputs(H=3, K=K, V=V, dtype=dtype, lengths=lengths, seed=15))
    d = to_dev(inp)
    opts = dict(scale=0.8, cu_seqlens=d.get("cu_seqlens"), cp_mode=cp, **kw)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    o0, s0 = gdn.gdn_chunk_fwd(*args, d["initial_state"], **opts)
    ws = gdn.gdn_workspace(d["q"], d["v"], **{n: x for n, x in opts.items() if n != "scale"})
    ws.fill_(0xA5)  # nothing the backward reads may come from outside what the forward wrote
    o1, s1 = gdn.gdn_chunk_fwd(*args, d["initial_state"], workspace=ws, keep_for_backward=True, **opts)
    assert torch.equal(o0, o1) and torch.equal(s0, s1)
    ref = gdn.gdn_chunk_bwd(*args, d["d_o"], d["initial_state"], d["d_final_state"], **opts)
    got = gdn.gdn_chunk_bwd(*args, d["d_o"], d["initial_state"], d["d_final_state"], workspace=ws,
                            reuse_forward=True, **opts)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(got[n], ref[n]), n
    # and against the oracle
    compare(got, oracle_bwd(inp, scale=0.8), tol_for(dtype))
    # only the CP decisions and sub-sequence entry states handed over (none without CP)
    plain = {n: x for n, x in opts.items() if n != "scale"}
    cps = gdn.gdn_cp_states(d["q"], d["v"], **plain)
    assert (cps is None) == (gdn.gdn_plan(gdn.make_desc(d["q"], d["v"], **plain))["cp_on"] == 0)
    if cps is not None:
        cps.fill_(0xA5)
        ws.fill_(0x5A)
        o2, s2 = gdn.gdn_chunk_fwd(*args, d["initial_state"], workspace=ws, cp_states=cps, **opts)
        ws.fill_(0x5A)  # the backward reads nothing of the forward's workspace
        got = gdn.gdn_chunk_bwd(*args, d["d_o"], d["initial_state"], d["d_final_state"], workspace=ws,
                                cp_states=cps, **opts)
        torch.cuda.synchronize()
        assert torch.equal(o0, o2) and torch.equal(s0, s2)
        for n in NAMES:
            assert torch.equal(got[n], ref[n]), n


def test_autograd_wrapper_carries_cp_states(gpu_lib):
    """The autograd wrapper can hand the forward's CP results to the backward: its gradients equal the
    recomputing backward's bit for bit, with packed sequences and CP on."""
    gdn = gpu_lib
    inp = with_grads(small_inputs(H=3, K=128, V=128, dtype=torch.bfloat16, lengths=[700, 3000, 65, 2500], seed=18))
    d = to_dev(inp)
    opts = dict(cu_seqlens=d["cu_seqlens"], cp_mode="on")
    assert gdn.gdn_cp_states(d["q"], d["v"], seg_chunks=0, **opts) is not None
    leaves = {n: d[n].clone().requires_grad_(True) for n in ("q", "k", "v", "g", "beta", "initial_state")}
    o, sT = gdn.chunk_gated_delta_rule(leaves["q"], leaves["k"], leaves["v"], leaves["g"], leaves["beta"],
                                       initial_state=leaves["initial_state"], carry_cp_states=True, **opts)
    loss = (o.float() * d["d_o"].float()).sum() + (sT * d["d_final_state"]).sum()
    loss.backward()
    ref = gdn.gdn_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["d_o"], d["initial_state"],
                            d["d_final_state"], **opts)
    torch.cuda.synchronize()
    pairs = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", initial_state="d_initial_state")
    for n, r in pairs.items():
        assert torch.equal(leaves[n].grad, ref[r]), n
    compare(ref, oracle_bwd(inp), 1e-2)


def test_autograd_wrapper_keep_intermediates(gpu_lib):
    inp = with_grads(small_inputs(B=1, T=2000, H=3, K=128, V=128, dtype=torch.bfloat16, seed=16))
    d = to_dev(inp)
    grads = []
    for keep in (False, True):
        leaves = {n: d[n].clone().requires_grad_(True) for n in ("q", "k", "v", "g", "beta", "initial_state")}
        o, sT = gpu_lib.chunk_gated_delta_rule(leaves["q"], leaves["k"], leaves["v"], leaves["g"],
                                               leaves["beta"], initial_state=leaves["initial_state"],
                                               cp_mode="exact", keep_intermediates=keep)
        loss = (o.float() * d["d_o"].float()).sum() + (sT * d["d_final_state"]).sum()
        loss.backward()
        grads.append({n: x.grad for n, x in leaves.items()})
    for n in grads[0]:
        assert torch.equal(grads[0][n], grads[1][n]), n


def test_backward_on_side_streams_and_threads(gpu_lib):
    """The backward forks its reverse pass onto a library stream and joins it back to the
    caller's: results on a non-default caller stream, and from two host threads calling at
    once on two streams, equal the serial default-stream results bit for bit."""
    import threading
    gdn = gpu_lib
    inps = [to_dev(with_grads(small_inputs(B=1, T=3000, H=2, K=128, V=128, dtype=torch.bfloat16, seed=s)))
            for s in (21, 22)]
    opts = dict(cp_mode="exact", seg_chunks=8)

    def run(d):
        return gdn.gdn_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["d_o"], d["initial_state"],
                                 d["d_final_state"], **opts)

    ref = [run(d) for d in inps]
    torch.cuda.synchronize()
    # a caller stream other than the default one; outputs read on that stream after the call
    s1 = torch.cuda.Stream()
    with torch.cuda.stream(s1):
        got = run(inps[0])
        copies = {n: got[n].clone() for n in NAMES}
    s1.synchronize()
    for n in NAMES:
        assert torch.equal(copies[n], ref[0][n]), n
    # two host threads, two streams, at once
    outs = [None, None]
    errs = []

    def worker(i):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                o = run(inps[i])
                outs[i] = {n: o[n].clone() for n in NAMES}
            st.synchronize()
        except Exception as e:  # surfaced below
            errs.append(e)

    th = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for x in th:
        x.start()
    for x in th:
        x.join()
    assert not errs, errs
    for i in range(2):
        for n in NAMES:
            assert torch.equal(outs[i][n], ref[i][n]), (i, n)


def test_backward_longer_warmup_window(gpu_lib):
    """The reverse CP on a head that needs a 16-chunk window (constant log-decay of -0.6
    per chunk): with the longer window allowed (warmup) and capped at 8 chunks (exact), all
    six gradients match the oracle."""
    inp = with_grads(mid_decay_inputs())
    d = to_dev(inp)
    ref = oracle_bwd(inp)
    for extra in ({}, dict(warmup_max_chunks=8)):
        out = gpu_bwd(d, cp_mode="on", seg_chunks=32, **extra)
        print(extra, compare(out, ref, 1e-2), flush=True)



def test_backward_autocp_fills_idle_units(gpu_lib):
    """The backward under the default AutoCP at N*H = 48 and 2560 tokens (CP on here, off by the
    pages' thresholds), one slowly decaying head in exact mode; sampled heads against the oracle."""
    gdn = gpu_lib
    inp = with_grads(small_inputs(B=2, T=2560, H=24, seed=19))
    inp["g"][:, :, 5] = -0.3 / 64  # -4.8 over a 16-chunk window: exact
    d = to_dev(inp)
    assert gdn.gdn_plan(gdn.make_desc(d["q"], d["v"]))["cp_on"] == 1
    out = gpu_bwd(d)
    heads = [0, 5, 23]
    compare({n: out[n].cpu() for n in NAMES}, oracle_bwd(inp, heads=heads), 1e-2, heads=heads)


@pytest.mark.parametrize("dtype,K,V", [(torch.float32, 64, 64), (torch.bfloat16, 128, 128)])
def test_backward_raw_keys_exact_correction(gpu_lib, dtype, K, V):
    """Keys with |k|^2 = 3.5 (beta |k|^2 > 2 on part of every window, fast gate decay): both CP
    directions must take the exact correction; all six gradients match the oracle."""
    kw = dict(cp_mode="on", seg_chunks=4, warmup_chunks=2)
    inp = with_grads(raw_key_inputs(K=K, V=V, dtype=dtype))
    d = to_dev(inp)
    _, rev = gpu_lib.gdn_cp_windows(d["k"], d["v"], d["g"], d["beta"], **kw)
    # every boundary whose window does not reach the sequence end: exact (see the forward test)
    assert rev.cpu().view(2, 4, 2).permute(0, 2, 1).tolist() == [[[-1, 0, 0, 4]] * 2] * 2, rev
    errs = compare(gpu_bwd(d, **kw), oracle_bwd(inp), tol_for(dtype))
    print(f"raw keys {dtype} " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)


@pytest.mark.parametrize("dtype,K,V", [(torch.float32, 64, 64), (torch.bfloat16, 128, 128)])
def test_backward_cp_mixed_boundaries(gpu_lib, dtype, K, V):
    """The backward with per-boundary mixing in both CP directions (the head of
    mixed_decay_inputs: exact boundaries where the window lies in the slow half, warmup
    elsewhere): all six gradients against the oracle."""
    inp = with_grads(mixed_decay_inputs(K=K, V=V, dtype=dtype))
    d = to_dev(inp)
    errs = compare(gpu_bwd(d, cp_mode="on", seg_chunks=16), oracle_bwd(inp), tol_for(dtype))
    print(f"mixed {dtype} " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)


@pytest.mark.parametrize("K,cp,kw,lengths", [
    (128, "off", {}, None), (128, "exact", dict(seg_chunks=3), None), (128, "warmup", dict(seg_chunks=4, warmup_chunks=3), None),
    (64, "on", dict(seg_chunks=4), None), (128, "exact", dict(seg_chunks=2), [1, 63, 64, 65, 0, 700, 1500, 129]),
])
def test_backward_carried_adjoint_and_adjoint_pass(gpu_lib, K, cp, kw, lengths):
    """At V = 128 in bf16 the per-chunk kernel carries the adjoint through each sub-sequence
    (default); GDN_FLAG_BWD_ADJOINT_PASS runs the separate adjoint pass instead. Both match the
    oracle on the same inputs, with CP off, exact, warmup, gated and packed sequences."""
    if lengths is None:
        inp = with_grads(small_inputs(B=2, T=1000, H=2, K=K, V=128, seed=23))
    else:
        inp = with_grads(small_inputs(H=3, K=K, V=128, lengths=lengths, seed=23))
    d = to_dev(inp)
    ref = oracle_bwd(inp, scale=0.9)
    carried = gpu_bwd(d, scale=0.9, cp_mode=cp, **kw)
    separate = gpu_bwd(d, scale=0.9, cp_mode=cp, adjoint_pass=True, **kw)
    e1 = compare(carried, ref, 1e-2)
    e2 = compare(separate, ref, 1e-2)
    print("carried " + " ".join(f"{n}={e:.2e}" for n, e in e1.items()), flush=True)
    print("separate " + " ".join(f"{n}={e:.2e}" for n, e in e2.items()), flush=True)
