"""GPU parity of the q/k L2 normalisation ahead of the path (GDN_FLAG_QK_L2NORM) against the
oracle's composition of the normalisation with the fp64 rule (oracle.l2norm).

q and k are raw here: N(0,1) rows times a per-row factor in [0.2, 4], plus an all-zero row
each. The forward must match ref_fwd_l2 and the backward ref_bwd_l2 (gradients with respect
to the raw q and k) within the usual bounds; the normalised k rows the library keeps in its
workspace are checked value by value; a kept forward reused by the backward gives the same
bits as a recomputing backward.
"""
import pytest
import torch

from gdn_inputs import make_inputs
from gpu_helpers import check, small_inputs, to_dev, tol_for
from oracle import ref_bwd_l2, ref_fwd_l2

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "d_initial_state")


def raw_qk(inp, seed=0):
    """Replace the unit-norm q, k by raw rows of varied norms, with one all-zero row each."""
    gen = torch.Generator().manual_seed(1000 + seed)
    for n in ("q", "k"):
        x = inp[n]
        s = 0.2 + 3.8 * torch.rand(x.shape[:-1] + (1,), generator=gen)
        r = torch.randn(x.shape, generator=gen) * s
        r[0, min(5, x.shape[1] - 1), 0] = 0.0
        inp[n] = r.to(x.dtype)
    return inp


def with_grads(inp, seed=7):
    gen = torch.Generator().manual_seed(seed)
    B, T, H, V = inp["v"].shape
    N = B if inp.get("cu_seqlens") is None else len(inp["cu_seqlens"]) - 1
    K = inp["q"].shape[-1]
    inp["d_o"] = torch.randn((B, T, H, V), generator=gen).to(inp["q"].dtype)
    inp["d_final_state"] = torch.randn((N, H, V, K), generator=gen) * 0.1
    return inp


def fwd(gdn, d, **kw):
    o, sT = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"],
                              cu_seqlens=d.get("cu_seqlens"), qk_l2norm=True, **kw)
    torch.cuda.synchronize()
    return o, sT


def bwd(gdn, d, **kw):
    out = gdn.gdn_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["d_o"], d["initial_state"],
                            d["d_final_state"], cu_seqlens=d.get("cu_seqlens"), qk_l2norm=True, **kw)
    torch.cuda.synchronize()
    return out


def oracle_fwd(inp, scale=1.0):
    return ref_fwd_l2(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], scale, inp["initial_state"],
                      cu_seqlens=inp.get("cu_seqlens"))


def oracle_bwd(inp, scale=1.0):
    return ref_bwd_l2(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["d_o"], scale,
                      inp["initial_state"], inp["d_final_state"], cu_seqlens=inp.get("cu_seqlens"))


FWD_CASES = [
    (torch.bfloat16, 128, 128, "off", {}),
    (torch.bfloat16, 128, 128, "exact", dict(seg_chunks=3)),
    (torch.bfloat16, 64, 128, "warmup", dict(seg_chunks=4, warmup_chunks=3)),
    (torch.bfloat16, 128, 64, "auto", {}),
    (torch.float32, 64, 64, "off", {}),
    (torch.float32, 128, 128, "exact", dict(seg_chunks=5)),
    (torch.float32, 64, 128, "warmup", dict(seg_chunks=4, warmup_chunks=3)),
]


@pytest.mark.parametrize("dtype,K,V,cp,kw", FWD_CASES)
def test_l2norm_forward(gpu_lib, dtype, K, V, cp, kw):
    inp = raw_qk(small_inputs(B=2, T=1000, H=2, K=K, V=V, dtype=dtype, seed=31), seed=1)
    o_ref, s_ref = oracle_fwd(inp, scale=0.9)
    o, sT = fwd(gpu_lib, to_dev(inp), scale=0.9, cp_mode=cp, **kw)
    tol = tol_for(dtype)
    check(o, o_ref, tol, "o")
    check(sT, s_ref, tol, "final_state")


def test_l2norm_forward_varlen(gpu_lib):
    lengths = [1, 63, 64, 65, 0, 700, 1500, 129]
    inp = raw_qk(small_inputs(H=3, K=128, V=128, lengths=lengths, seed=32), seed=2)
    o_ref, s_ref = oracle_fwd(inp)
    o, sT = fwd(gpu_lib, to_dev(inp), cp_mode="exact", seg_chunks=2)
    check(o, o_ref, 1e-2, "o")
    for n in range(len(lengths)):
        check(sT[n], s_ref[n], 1e-2, f"sequence {n}")


@pytest.mark.parametrize("dtype,K,V", [(torch.bfloat16, 128, 128), (torch.bfloat16, 64, 128),
                                       (torch.float32, 64, 64), (torch.bfloat16, 128, 64)])
def test_l2norm_rows_in_workspace(gpu_lib, dtype, K, V):
    """The normalised k rows at the start of the workspace (written by the intra-chunk kernel),
    value by value: fp32 arithmetic, rounded once to the input dtype."""
    gdn = gpu_lib
    inp = raw_qk(small_inputs(B=2, T=300, H=3, K=K, V=V, dtype=dtype, seed=33), seed=3)
    d = to_dev(inp)
    ws = gdn.gdn_workspace(d["q"], d["v"], qk_l2norm=True)
    gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], workspace=ws,
                      keep_for_backward=True, qk_l2norm=True)
    torch.cuda.synchronize()
    n = d["k"].numel()
    esize = d["k"].element_size()
    raw = ws.cpu()
    for name, ofs in (("k", 0),):
        got = raw[ofs:ofs + n * esize].view(dtype).view(d[name].shape).double()
        x = inp[name].double()
        want = x / torch.sqrt((x * x).sum(-1, keepdim=True) + 1e-6)
        ulp = 1.01 * 2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -20
        err = ((got - want).abs() / want.abs().clamp_min(1e-30)).masked_fill(want == 0, 0.0)
        assert float(err.max()) <= ulp, (name, float(err.max()))
        assert torch.all(got[want == 0] == 0)


BWD_CASES = [
    (torch.bfloat16, 128, 128, "off", {}),
    (torch.bfloat16, 128, 128, "exact", dict(seg_chunks=3)),
    (torch.bfloat16, 64, 128, "warmup", dict(seg_chunks=4, warmup_chunks=3)),
    (torch.float32, 64, 64, "off", {}),
    (torch.float32, 64, 64, "exact", dict(seg_chunks=3)),
]


@pytest.mark.parametrize("dtype,K,V,cp,kw", BWD_CASES)
def test_l2norm_backward(gpu_lib, dtype, K, V, cp, kw):
    inp = with_grads(raw_qk(small_inputs(B=2, T=1000, H=2, K=K, V=V, dtype=dtype, seed=34), seed=4))
    out = bwd(gpu_lib, to_dev(inp), scale=0.9, cp_mode=cp, **kw)
    ref = oracle_bwd(inp, scale=0.9)
    for n in NAMES:
        check(out[n], ref[n], tol_for(dtype), n)


def test_l2norm_backward_varlen(gpu_lib):
    lengths = [1, 63, 64, 65, 0, 700, 1500, 129]
    inp = with_grads(raw_qk(small_inputs(H=3, K=128, V=128, lengths=lengths, seed=35), seed=5))
    out = bwd(gpu_lib, to_dev(inp), cp_mode="exact", seg_chunks=2)
    ref = oracle_bwd(inp)
    for n in NAMES:
        check(out[n], ref[n], 1e-2, n)


@pytest.mark.parametrize("cp,kw", [("exact", dict(seg_chunks=3)), ("off", {})])
def test_l2norm_keep_and_reuse(gpu_lib, cp, kw):
    """A kept forward (normalised rows included) reused by the backward: the same bits as the
    recomputing backward, and the same forward output as a forward that keeps nothing."""
    gdn = gpu_lib
    inp = with_grads(raw_qk(small_inputs(B=2, T=1000, H=2, seed=36), seed=6))
    d = to_dev(inp)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    o0, s0 = gdn.gdn_chunk_fwd(*args, d["initial_state"], cp_mode=cp, qk_l2norm=True, **kw)
    ref = gdn.gdn_chunk_bwd(*args, d["d_o"], d["initial_state"], d["d_final_state"], cp_mode=cp,
                            qk_l2norm=True, **kw)
    ws = gdn.gdn_workspace(d["q"], d["v"], cp_mode=cp, qk_l2norm=True, **kw)
    o1, s1 = gdn.gdn_chunk_fwd(*args, d["initial_state"], cp_mode=cp, workspace=ws, keep_for_backward=True,
                               qk_l2norm=True, **kw)
    got = gdn.gdn_chunk_bwd(*args, d["d_o"], d["initial_state"], d["d_final_state"], cp_mode=cp,
                            workspace=ws, reuse_forward=True, qk_l2norm=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(s0, s1)
    for n in NAMES:
        assert torch.equal(got[n], ref[n]), n


def test_l2norm_autograd(gpu_lib):
    """chunk_gated_delta_rule(qk_l2norm=True) under autograd returns the oracle's gradients with
    respect to the raw q and k (fp32, 1e-4)."""
    inp = with_grads(raw_qk(small_inputs(B=1, T=300, H=2, K=64, V=64, dtype=torch.float32, seed=37), seed=7))
    d = to_dev(inp)
    leaves = {n: d[n].clone().requires_grad_(True) for n in ("q", "k", "v", "g", "beta", "initial_state")}
    o, sT = gpu_lib.chunk_gated_delta_rule(leaves["q"], leaves["k"], leaves["v"], leaves["g"], leaves["beta"],
                                           initial_state=leaves["initial_state"], qk_l2norm=True,
                                           keep_intermediates=True)
    ((o * d["d_o"]).sum() + (sT * d["d_final_state"]).sum()).backward()
    ref = oracle_bwd(inp)
    pairs = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", initial_state="d_initial_state")
    for n, r in pairs.items():
        check(leaves[n].grad, ref[r], 1e-4, n)


def test_l2norm_intra_and_modes(gpu_lib):
    """gdn_intra_chunk and gdn_cp_modes with the flag see the normalised k: the same results as
    on k normalised beforehand (bf16 rounding of the rows aside, so the WY factors to 1e-2)."""
    gdn = gpu_lib
    inp = raw_qk(small_inputs(B=1, T=4096, H=4, seed=38), seed=8)
    d = to_dev(inp)
    x = inp["k"].double()
    kn = (x / torch.sqrt((x * x).sum(-1, keepdim=True) + 1e-6)).to(torch.bfloat16).cuda()
    g1, w1, u1 = gdn.gdn_intra_chunk(d["k"], d["v"], d["g"], d["beta"], qk_l2norm=True)
    g2, w2, u2 = gdn.gdn_intra_chunk(kn, d["v"], d["g"], d["beta"])
    torch.cuda.synchronize()
    assert torch.equal(g1, g2)
    check(w1, w2.double().cpu(), 1e-2, "w")
    check(u1, u2.double().cpu(), 1e-2, "u")
    m1 = gdn.gdn_cp_modes(d["k"], d["v"], d["g"], d["beta"], cp_mode="on", seg_chunks=16, qk_l2norm=True)
    m2 = gdn.gdn_cp_modes(kn, d["v"], d["g"], d["beta"], cp_mode="on", seg_chunks=16)
    assert torch.equal(m1, m2)


def test_l2norm_edge_prefill_32k(gpu_lib):
    """B=1, H=16, T=32768, bf16 (AutoCP: warmup and exact heads) with raw q and k (unit rows times
    a per-row factor in [0.25, 4]): every head and token on a sample of value rows against the
    oracle (rows of the state evolve independently)."""
    inp = make_inputs("edge_prefill", seed=0)
    gen = torch.Generator().manual_seed(99)
    for n in ("q", "k"):
        x = inp[n].float()
        inp[n] = (x * (0.25 + 3.75 * torch.rand(x.shape[:-1] + (1,), generator=gen))).to(torch.bfloat16)
    o, sT = fwd(gpu_lib, to_dev(inp))
    rows = list(range(0, 8)) + list(range(120, 128))
    s0 = inp["initial_state"]
    o_ref, s_ref = ref_fwd_l2(inp["q"], inp["k"], inp["v"][..., rows], inp["g"], inp["beta"], 1.0,
                              None if s0 is None else s0[:, :, rows])
    e_o = check(o[..., rows], o_ref, 1e-2, "o")
    e_s = check(sT[:, :, rows], s_ref, 1e-2, "final_state")
    print(f"l2norm edge_prefill rel_l2 o={e_o:.2e} final={e_s:.2e}", flush=True)


def test_l2norm_backward_edge_prefill_32k(gpu_lib):
    """The 32K step's backward (B=1, H=16, T=32768, bf16, AutoCP on: warmup and exact heads) with
    raw q and k (unit rows times a per-row factor in [0.25, 4]) and the normalisation inside the
    library; one warmup head and one exact head against the oracle, every token."""
    import dataclasses
    from gdn_inputs import WORKLOADS
    gdn = gpu_lib
    inp = make_inputs(dataclasses.replace(WORKLOADS["edge_prefill"], backward=True), seed=0)
    gen = torch.Generator().manual_seed(98)
    for n in ("q", "k"):
        x = inp[n].float()
        inp[n] = (x * (0.25 + 3.75 * torch.rand(x.shape[:-1] + (1,), generator=gen))).to(torch.bfloat16)
    d = to_dev(inp)
    modes = gdn.gdn_cp_modes(d["k"], d["v"], d["g"], d["beta"], qk_l2norm=True).cpu()
    assert (modes == 1).any() and (modes >= 2).any(), modes
    out = bwd(gdn, d)
    heads = [int((modes[0] == 1).nonzero()[0]), int((modes[0] >= 2).nonzero()[0])]
    x = {n: inp[n][:, :, heads] for n in ("q", "k", "v", "g", "beta", "d_o")}
    ref = ref_bwd_l2(x["q"], x["k"], x["v"], x["g"], x["beta"], x["d_o"], 1.0, inp["initial_state"][:, heads],
                     inp["d_final_state"][:, heads])
    errs = {}
    for n in NAMES:
        got = out[n][:, heads] if n == "d_initial_state" else out[n][:, :, heads]
        errs[n] = check(got, ref[n], 1e-2, n)
    print(f"l2norm backward heads={heads} " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)


@pytest.mark.parametrize("l2", [False, True])
def test_no_tokens(gpu_lib, l2):
    """T = 0: the forward returns the initial state as the final state, the backward passes
    d(final state) through to d(initial state) and every other output is empty."""
    gdn = gpu_lib
    inp = with_grads(small_inputs(B=2, T=0, H=2, K=128, V=64, seed=39))
    d = to_dev(inp)
    o, sT = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], qk_l2norm=l2)
    out = gdn.gdn_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["d_o"], d["initial_state"],
                            d["d_final_state"], qk_l2norm=l2)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 2, 64) and torch.equal(sT, d["initial_state"])
    assert torch.equal(out["d_initial_state"], d["d_final_state"])
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        assert out[n].numel() == 0, n
