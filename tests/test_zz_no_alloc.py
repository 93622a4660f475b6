"""The forward entry point that allocates nothing (gdn_chunk_fwd_noalloc), for callers that
cannot allocate device memory: its workspace is the library's fixed per-GPU scratch array.
Called through the C ABI (the binding only marshals pointers) and compared with gdn_chunk_fwd,
which runs the same kernels on a caller workspace, on two calls in a row, the second smaller
and of another layout (so stale contents of the first call's scratch must not matter); the
second also against the oracle. Run last: a failure here hides no other test.
"""
import pytest
import torch

from gpu_helpers import check, oracle, small_inputs, to_dev

pytestmark = pytest.mark.gpu


def _both(gdn, d, **kw):
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"])
    ref = gdn.gdn_chunk_fwd(*args, cu_seqlens=d.get("cu_seqlens"), **kw)
    got = gdn.gdn_chunk_fwd_noalloc(*args, cu_seqlens=d.get("cu_seqlens"), **kw)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_forward_matches_the_workspace_forward(gpu_lib):
    gdn = gpu_lib
    # 1: B=1, H=16, T=8192, K=V=128, bf16, AutoCP (CP on: warmup and exact sub-sequences)
    big = small_inputs(B=1, T=8192, H=16, seed=31)
    big["g"][:, :, 3] = -0.3 / 64  # one slowly decaying head: the exact correction
    d = to_dev(big)
    plan = gdn.gdn_plan(gdn.make_desc(d["q"], d["v"]))
    assert plan["cp_on"] == 1 and 0 < plan["fwd_workspace_bytes"] <= gdn.GDN_NOALLOC_SCRATCH_BYTES
    (o0, s0), (o1, s1) = _both(gdn, d)
    assert torch.equal(o0, o1) and torch.equal(s0, s1)
    # 2: smaller, fp32, K=V=64, packed sequences with CP forced exact
    lengths = [1, 63, 0, 700, 129]
    small = small_inputs(H=3, K=64, V=64, dtype=torch.float32, lengths=lengths, seed=32)
    d = to_dev(small)
    (o0, s0), (o1, s1) = _both(gdn, d, cp_mode="exact", seg_chunks=2, scale=0.9)
    assert torch.equal(o0, o1) and torch.equal(s0, s1)
    # with the outputs preallocated, a call allocates no device memory at all
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    gdn.gdn_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"],
                              cu_seqlens=d["cu_seqlens"], cu_seqlens_host=small["cu_seqlens"], cp_mode="exact",
                              seg_chunks=2, scale=0.9, o=o1, final_state=s1)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.equal(o0, o1) and torch.equal(s0, s1)
    o_ref, s_ref = oracle(small, scale=0.9)
    check(o1, o_ref, 1e-4, "o")
    check(s1, s_ref, 1e-4, "final_state")


def test_noalloc_refuses_what_it_cannot_hold(gpu_lib):
    gdn = gpu_lib
    d = to_dev(small_inputs(B=1, T=40960, H=16, seed=33, init_std=None))
    assert gdn.gdn_plan(gdn.make_desc(d["q"], d["v"]))["fwd_workspace_bytes"] > gdn.GDN_NOALLOC_SCRATCH_BYTES
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"])
    assert e.value.status == 3  # GDN_ERR_WORKSPACE, before any launch
