"""GPU parity of the forward path against the CPU oracle (needs an MI355X).

Bounds: relative L2 <= 1e-2 for bf16 inputs with fp32 accumulation and
<= 1e-4 in fp32 mode, on O and on the final state, for every CP mode (off,
exact correction, warmup), with ragged tails, dk != dv and packed varlen.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import (BF16_TOL, MIXED_FWD_HEAD1, MIXED_REV_HEAD1, check, gpu_fwd, mid_decay_inputs,  # noqa: F401
                         mixed_decay_inputs, oracle, raw_key_inputs, rel_l2, seq_slices, small_inputs, to_dev,
                         tol_for)
from oracle.chunked import chunked_fwd

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("KV", [(64, 64), (128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("varlen", [False, True])
def test_intra_chunk_factors(gpu_lib, dtype, KV, varlen):
    """gam, w, u of the intra-chunk kernel vs the chunked (WY) reformulation."""
    K, V = KV
    lengths = [1, 64, 130, 0, 77] if varlen else None
    inp = small_inputs(B=2, T=200, H=3, K=K, V=V, dtype=dtype, lengths=lengths, init_std=None)
    d = to_dev(inp)
    gam, w, u = gpu_lib.gdn_intra_chunk(d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    _, _, it = chunked_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], 1.0, None,
                           cu_seqlens=inp["cu_seqlens"], return_intermediates=True)
    tol = tol_for(dtype)
    check(gam, it["gam"], 1e-5, "gam")
    check(w, it["w"], tol, "w")
    check(u, it["u"], tol, "u")


CASES = [
    # dtype, K, V, cp_mode, extra kwargs
    (torch.float32, 64, 64, "off", {}),
    (torch.float32, 64, 64, "exact", dict(seg_chunks=3)),
    (torch.float32, 64, 64, "warmup", dict(seg_chunks=4, warmup_chunks=6)),
    (torch.float32, 128, 128, "exact", dict(seg_chunks=5)),
    (torch.float32, 128, 64, "exact", dict(seg_chunks=3)),
    (torch.float32, 64, 128, "warmup", dict(seg_chunks=4, warmup_chunks=3)),
    (torch.bfloat16, 128, 128, "off", {}),
    (torch.bfloat16, 128, 128, "exact", dict(seg_chunks=3)),
    (torch.bfloat16, 128, 128, "warmup", dict(seg_chunks=4, warmup_chunks=3)),
    (torch.bfloat16, 128, 128, "on", dict(seg_chunks=4)),
    (torch.bfloat16, 64, 128, "exact", dict(seg_chunks=4)),
    (torch.bfloat16, 128, 64, "warmup", dict(seg_chunks=4)),
    (torch.bfloat16, 64, 64, "auto", {}),
    # longer sub-sequences (8 chunks or more), ragged ones included
    (torch.float32, 64, 64, "exact", dict(seg_chunks=8)),
    (torch.float32, 128, 128, "exact", dict(seg_chunks=9)),
    (torch.bfloat16, 128, 128, "exact", dict(seg_chunks=8)),
    (torch.bfloat16, 64, 128, "exact", dict(seg_chunks=11)),
    (torch.bfloat16, 128, 128, "on", dict(seg_chunks=8, warmup_chunks=3)),
]


@pytest.mark.parametrize("dtype,K,V,cp,kw", CASES)
def test_forward_small(gpu_lib, dtype, K, V, cp, kw):
    inp = small_inputs(B=2, T=1000, H=2, K=K, V=V, dtype=dtype, seed=1)
    o_ref, s_ref = oracle(inp, scale=0.9)
    o, sT = gpu_fwd(to_dev(inp), scale=0.9, cp_mode=cp, **kw)
    tol = tol_for(dtype)
    check(o, o_ref, tol, "o")
    check(sT, s_ref, tol, "final_state")


@pytest.mark.parametrize("cp,kw", [("off", {}), ("exact", dict(seg_chunks=2)),
                                   ("warmup", dict(seg_chunks=3, warmup_chunks=2)),
                                   ("exact", dict(seg_chunks=8)), ("on", dict(seg_chunks=9, warmup_chunks=2))])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_forward_varlen(gpu_lib, cp, kw, dtype):
    lengths = [1, 63, 64, 65, 0, 700, 1500, 129]
    inp = small_inputs(H=3, K=128, V=128, dtype=dtype, lengths=lengths, seed=2)
    o_ref, s_ref = oracle(inp)
    o, sT = gpu_fwd(to_dev(inp), cp_mode=cp, **kw)
    tol = tol_for(dtype)
    check(o, o_ref, tol)
    # every sequence on its own: a wrong 1- or 63-token sequence weighs little in the packed O
    oc = o.cpu()
    for n, a, b in seq_slices(inp["cu_seqlens"]):
        check(oc[:, a:b], o_ref[:, a:b], tol, f"o of sequence {n} ({b - a} tokens)")
    for n in range(len(lengths)):
        check(sT[n], s_ref[n], tol, f"sequence {n}")
    # the empty sequence returns its initial state
    assert torch.equal(sT[4].cpu(), inp["initial_state"][4])


def test_forward_zero_initial_state_and_no_final(gpu_lib):
    inp = small_inputs(B=1, T=300, H=2, K=64, V=64, dtype=torch.float32, init_std=None)
    o_ref, s_ref = oracle(inp)
    o, sT = gpu_fwd(to_dev(inp), cp_mode="off")
    check(o, o_ref, 1e-4)
    check(sT, s_ref, 1e-4)
    o2, s2 = gpu_fwd(to_dev(inp), cp_mode="off", output_final_state=False)
    assert s2 is None and torch.equal(o2, o)


def test_tiny_workload_fp32(gpu_lib):
    """The tiny fp32 workload: B=1, H=2, T=256, dk=dv=64, zero initial state, seed 0."""
    from gdn_inputs import make_inputs
    inp = make_inputs("tiny", seed=0)
    o_ref, s_ref = oracle(inp)
    o, sT = gpu_fwd(to_dev(inp))
    check(o, o_ref, 1e-4)
    check(sT, s_ref, 1e-4)


def test_deterministic(gpu_lib):
    inp = to_dev(small_inputs(B=1, T=4096, H=4, seed=3))
    a = gpu_fwd(inp, cp_mode="exact", seg_chunks=16)
    b = gpu_fwd(inp, cp_mode="exact", seg_chunks=16)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_cp_modes_decision(gpu_lib):
    """Fast-decaying heads take the warmup, slow ones the exact correction."""
    inp = small_inputs(B=1, T=8192, H=4, seed=4)
    # head 0, 1: fast decay; head 2, 3: almost none
    inp["g"][:, :, 2:] *= 0.001
    d = to_dev(inp)
    modes = gpu_lib.gdn_cp_modes(d["k"], d["v"], d["g"], d["beta"], cp_mode="on", seg_chunks=32)
    torch.cuda.synchronize()
    # heads 2, 3: exact at every boundary but the first, whose 32-chunk window reaches the
    # sequence start (it runs from the known state there): mixed
    assert modes.cpu().tolist() == [[1, 1, 3, 3]]
    o_ref, s_ref = oracle(inp)
    o, sT = gpu_fwd(d, cp_mode="on", seg_chunks=32)
    check(o, o_ref, 1e-2)
    check(sT, s_ref, 1e-2)


def test_cp_longer_warmup_window(gpu_lib):
    """A head that fails the warmup bound over 8 chunks takes a longer window that meets
    it (here 16 chunks) when allowed, the exact correction when the cap is below that; every
    variant matches the oracle."""
    inp = mid_decay_inputs()
    d = to_dev(inp)
    kw = dict(cp_mode="on", seg_chunks=32)

    def modes(**extra):
        m = gpu_lib.gdn_cp_modes(d["k"], d["v"], d["g"], d["beta"], **kw, **extra)
        torch.cuda.synchronize()
        return m.cpu().tolist()

    assert modes() == [[1, 1]]
    assert modes(warmup_max_chunks=16) == [[1, 1]]
    assert modes(warmup_max_chunks=15) == [[1, 2]]
    assert modes(warmup_max_chunks=8) == [[1, 2]]
    o_ref, s_ref = oracle(inp)
    for extra in ({}, dict(warmup_max_chunks=15), dict(warmup_chunks=6, warmup_max_chunks=69)):
        o, sT = gpu_fwd(d, **kw, **extra)
        e_o = check(o, o_ref, 1e-2, f"o {extra}")
        e_s = check(sT, s_ref, 1e-2, f"final_state {extra}")
        print(f"{extra} rel_l2 o={e_o:.2e} final={e_s:.2e}", flush=True)



def test_autocp_fills_idle_units(gpu_lib):
    """Default AutoCP at a shape the pages' thresholds leave serial: N*H = 48 (> 40) at 2560
    tokens fills 48 of the 256 recurrence slots, so CP is on; one head decays slowly enough to
    take the exact correction. Sampled heads against the oracle, all heads against CP off."""
    gdn = gpu_lib
    inp = small_inputs(B=2, T=2560, H=24, seed=9)
    inp["g"][:, :, 5] = -0.3 / 64  # -4.8 over a 16-chunk window: exact
    d = to_dev(inp)
    assert gdn.gdn_plan(gdn.make_desc(d["q"], d["v"]))["cp_on"] == 1
    assert gdn.gdn_plan(gdn.make_desc(d["q"], d["v"], cp_mode="pages"))["cp_on"] == 0
    modes = gdn.gdn_cp_modes(d["k"], d["v"], d["g"], d["beta"]).cpu()
    # head 5's first boundary (chunk 16) takes a window that reaches the sequence start, its
    # second the exact correction: mixed; every other head takes the warmup everywhere
    assert modes[:, 5].tolist() == [3, 3] and set(modes.flatten().tolist()) == {1, 3}, modes
    o, sT = gpu_fwd(d)
    heads = [0, 5, 23]
    o_ref, s_ref = oracle(inp, heads=heads)
    check(o[:, :, heads], o_ref, BF16_TOL, "o")
    check(sT[:, heads], s_ref, BF16_TOL, "final_state")
    o2, s2 = gpu_fwd(d, cp_mode="pages")
    check(o, o2.double().cpu(), BF16_TOL, "o vs serial")
    check(sT, s2.double().cpu(), BF16_TOL, "final_state vs serial")


@pytest.mark.parametrize("dtype,K,V", [(torch.float32, 64, 64), (torch.bfloat16, 128, 128)])
def test_raw_keys_take_the_exact_correction(gpu_lib, dtype, K, V):
    """Keys with |k|^2 = 3.5 (not normalised, no qk_l2norm): beta |k|^2 > 2 on part of every
    window, so the warmup's error bound does not hold and every sequence-head takes the exact
    correction although the gates decay fast; the same gates with unit-norm keys take the
    warmup. O and the final state match the oracle."""
    kw = dict(cp_mode="on", seg_chunks=4, warmup_chunks=2)
    inp = raw_key_inputs(K=K, V=V, dtype=dtype)
    bk = inp["beta"] * inp["k"].float().pow(2).sum(-1)
    assert float((bk > 2).float().mean()) > 0.2
    d = to_dev(inp)
    # 16 chunks in sub-sequences of 4: boundaries at chunks 4, 8, 12; windows of 2..4 chunks. Only
    # the first boundary's 4-chunk window reaches the sequence start (runs from the known state),
    # and only the last one's reaches its end in the reverse direction: every other boundary
    # must take the exact correction.
    fwd, rev = gpu_lib.gdn_cp_windows(d["k"], d["v"], d["g"], d["beta"], **kw)
    for b in range(2):
        assert fwd.cpu()[4 * b:4 * b + 4].T.tolist() == [[-1, 4, 0, 0]] * 2, fwd
        assert rev.cpu()[4 * b:4 * b + 4].T.tolist() == [[-1, 0, 0, 4]] * 2, rev
    unit = to_dev(small_inputs(K=K, V=V, dtype=dtype, seed=21))  # same seed: same gates and beta
    assert torch.equal(unit["g"], d["g"]) and torch.equal(unit["beta"], d["beta"])
    m1 = gpu_lib.gdn_cp_modes(unit["k"], unit["v"], unit["g"], unit["beta"], **kw).cpu()
    assert (m1 == 1).all(), m1
    o_ref, s_ref = oracle(inp)
    o, sT = gpu_fwd(d, **kw)
    tol = tol_for(dtype)
    e_o = check(o, o_ref, tol, "o")
    e_s = check(sT, s_ref, tol, "final_state")
    print(f"raw keys {dtype} rel_l2 o={e_o:.2e} final={e_s:.2e}", flush=True)


def test_binding_rejects_bad_buffers(gpu_lib):
    """Caller-supplied outputs, upstream gradients and workspaces are checked in the binding
    (device, shape, dtype, contiguity, alignment) before any pointer reaches the library."""
    gdn = gpu_lib
    d = to_dev(small_inputs(B=1, T=200, H=2, K=64, V=64, dtype=torch.float32))
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"])
    B, T, H, K = d["q"].shape
    with pytest.raises(ValueError, match="^o"):
        gdn.gdn_chunk_fwd(*args, o=torch.empty((B, T, H, K)))  # host tensor
    with pytest.raises(ValueError, match="^o"):
        gdn.gdn_chunk_fwd(*args, o=torch.empty((B, T, H, K + 1), device="cuda"))
    with pytest.raises(ValueError, match="^o"):
        gdn.gdn_chunk_fwd(*args, o=torch.empty((B, T, K, H), device="cuda").transpose(2, 3))
    with pytest.raises(ValueError, match="^final_state"):
        gdn.gdn_chunk_fwd(*args, final_state=torch.empty((1, H, K, K), device="cuda", dtype=torch.bfloat16))
    ws = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="aligned"):
        gdn.gdn_chunk_fwd(*args, workspace=ws[1:])
    with pytest.raises(ValueError, match="too small"):
        gdn.gdn_chunk_fwd(*args, workspace=ws[:256])
    # a workspace of another element type is sized in bytes
    o_ref, _ = gdn.gdn_chunk_fwd(*args)
    o_ws, _ = gdn.gdn_chunk_fwd(*args, workspace=torch.empty(1 << 20, dtype=torch.float32, device="cuda"))
    assert torch.equal(o_ref, o_ws)
    d_o = torch.randn((B, T, H, K), device="cuda")
    with pytest.raises(ValueError, match="^d_o"):
        gdn.gdn_chunk_bwd(*args[:5], d_o.cpu(), d["initial_state"])
    with pytest.raises(ValueError, match="d_final_state"):
        gdn.gdn_chunk_bwd(*args[:5], d_o, d["initial_state"], torch.zeros((1, H, K, K)))
    out = dict(dq=torch.empty_like(d["q"]), dk=torch.empty_like(d["k"]), dv=torch.empty_like(d["v"]),
               dg=torch.empty_like(d["g"]), dbeta=torch.empty_like(d["beta"]),
               d_initial_state=torch.empty((1, H, K, K), device="cuda"))
    bad = dict(out, dg=torch.empty((B, T, H + 1), device="cuda"))
    with pytest.raises(ValueError, match="dg"):
        gdn.gdn_chunk_bwd(*args[:5], d_o, d["initial_state"], out=bad)
    bad = dict(out, dk=out["dk"].cpu())
    with pytest.raises(ValueError, match="dk"):
        gdn.gdn_chunk_bwd(*args[:5], d_o, d["initial_state"], out=bad)
    with pytest.raises(ValueError, match="^o"):
        gdn.gdn_recurrent_fwd(d["q"][:, :3], d["k"][:, :3], d["v"][:, :3], d["g"][:, :3].contiguous(),
                              d["beta"][:, :3].contiguous(), d["initial_state"], o=torch.empty((B, 3, H, K)))


@pytest.mark.parametrize("dtype,K,V", [(torch.float32, 64, 64), (torch.bfloat16, 128, 128)])
def test_cp_mixed_boundaries(gpu_lib, dtype, K, V):
    """Per-boundary warmup/exact mixing: a head whose gates decay slowly over the first half of
    the sequence and fast over the second takes the exact correction at the boundaries whose
    window lies in the slow half and the warmup elsewhere (both directions); the forward
    matches the oracle with the exact maps and the scan running across the exact boundaries
    only."""
    gdn = gpu_lib
    inp = mixed_decay_inputs(K=K, V=V, dtype=dtype)
    d = to_dev(inp)
    kw = dict(cp_mode="on", seg_chunks=16)
    fwd, rev = gdn.gdn_cp_windows(d["k"], d["v"], d["g"], d["beta"], **kw)
    fwd, rev = fwd.cpu(), rev.cpu()
    assert fwd[:, 1].tolist() == MIXED_FWD_HEAD1, fwd[:, 1]
    assert rev[:, 1].tolist() == MIXED_REV_HEAD1, rev[:, 1]
    assert fwd[0, 0] == -1 and (fwd[1:, 0] == 8).all() and rev[0, 0] == -1 and (rev[1:, 0] == 8).all()
    modes = gdn.gdn_cp_modes(d["k"], d["v"], d["g"], d["beta"], **kw).cpu()
    assert modes.tolist() == [[1, 3]], modes
    o_ref, s_ref = oracle(inp)
    o, sT = gpu_fwd(d, **kw)
    tol = tol_for(dtype)
    e_o = check(o, o_ref, tol, "o")
    e_s = check(sT, s_ref, tol, "final_state")
    # the mixed head alone, and against every boundary exact
    check(o[:, :, 1], o_ref[:, :, 1], tol, "o of the mixed head")
    o2, s2 = gpu_fwd(d, cp_mode="exact", seg_chunks=16)
    check(o, o2.double().cpu(), tol, "o vs all exact")
    print(f"mixed {dtype} rel_l2 o={e_o:.2e} final={e_s:.2e}", flush=True)
