"""GPU parity of the recurrent form (gdn_recurrent_fwd): the gated delta rule token by token
from a given state, as a decoder runs it after a prefill. Checked against the CPU oracle's
token-by-token recurrence on the same bytes (relative L2 1e-4 fp32, 1e-2 bf16), and as the
continuation of the chunked forward: prefill T0 tokens with gdn_chunk_fwd, decode T1 more
from its final state, compare with the oracle over all T0 + T1 tokens."""
import pytest
import torch

from gpu_helpers import check, oracle, small_inputs, to_dev, tol_for

pytestmark = pytest.mark.gpu


def slice_tokens(inp, t0, t1):
    out = dict(inp)
    for n in ("q", "k", "v", "g", "beta"):
        out[n] = inp[n][:, t0:t1].contiguous()
    return out


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("KV", [(64, 64), (128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("T", [1, 5])
@pytest.mark.parametrize("with_state", [True, False])
def test_recurrent_parity(gpu_lib, dtype, KV, T, with_state):
    K, V = KV
    inp = small_inputs(B=3, T=T, H=2, K=K, V=V, dtype=dtype, seed=21, init_std=0.1 if with_state else None)
    d = to_dev(inp)
    o, sT = gpu_lib.gdn_recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], scale=0.8)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle(inp, scale=0.8)
    tol = tol_for(dtype)
    check(o, o_ref, tol, "o")
    check(sT, s_ref, tol, "state")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_continues_chunked_prefill(gpu_lib, dtype):
    """Prefill 1000 tokens (chunked, CP on), then decode 16 more one call per token and as
    one call of 16: both match the oracle over the 1016 tokens."""
    T0, T1 = 1000, 16
    inp = small_inputs(B=2, T=T0 + T1, H=2, K=128, V=128, dtype=dtype, seed=22)
    d = to_dev(inp)
    pre = slice_tokens(d, 0, T0)
    o_pre, s_pre = gpu_lib.gdn_chunk_fwd(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], d["initial_state"],
                                         cp_mode="on", seg_chunks=4)
    o_ref, s_ref = oracle(inp)
    tol = tol_for(dtype)
    # one call of T1 tokens
    dec = slice_tokens(d, T0, T0 + T1)
    o_dec, s_dec = gpu_lib.gdn_recurrent_fwd(dec["q"], dec["k"], dec["v"], dec["g"], dec["beta"], s_pre)
    # T1 calls of one token, the state updated in place
    state = s_pre.clone()
    outs = []
    for t in range(T0, T0 + T1):
        step = slice_tokens(d, t, t + 1)
        o1, _ = gpu_lib.gdn_recurrent_fwd(step["q"], step["k"], step["v"], step["g"], step["beta"], state,
                                          state_out=state)
        outs.append(o1)
    torch.cuda.synchronize()
    check(o_pre, o_ref[:, :T0], tol, "prefill o")
    check(o_dec, o_ref[:, T0:], tol, "decode o")
    check(s_dec, s_ref, tol, "decode state")
    check(torch.cat(outs, dim=1), o_ref[:, T0:], tol, "token-by-token o")
    check(state, s_ref, tol, "token-by-token state")
    # one call of T1 tokens and T1 calls of one token run the same arithmetic
    assert torch.equal(torch.cat(outs, dim=1), o_dec) and torch.equal(state, s_dec)


def test_recurrent_in_place_and_empty(gpu_lib):
    inp = small_inputs(B=2, T=3, H=3, K=128, V=64, dtype=torch.bfloat16, seed=23)
    d = to_dev(inp)
    o_a, s_a = gpu_lib.gdn_recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"])
    st = d["initial_state"].clone()
    o_b, s_b = gpu_lib.gdn_recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], st, state_out=st)
    torch.cuda.synchronize()
    assert s_b.data_ptr() == st.data_ptr()
    assert torch.equal(o_a, o_b) and torch.equal(s_a, s_b)
    # zero tokens: the state passes through (zeros without one)
    e = {n: d[n][:, :0].contiguous() for n in ("q", "k", "v", "g", "beta")}
    _, s_e = gpu_lib.gdn_recurrent_fwd(e["q"], e["k"], e["v"], e["g"], e["beta"], d["initial_state"])
    _, s_z = gpu_lib.gdn_recurrent_fwd(e["q"], e["k"], e["v"], e["g"], e["beta"], None)
    torch.cuda.synchronize()
    assert torch.equal(s_e, d["initial_state"])
    assert torch.count_nonzero(s_z) == 0


def test_batch_decode_step(gpu_lib):
    """One token for each of 64 sequences, H=16, K=V=128, bf16 (the batched decode the
    benchmark times), every output and state against the oracle."""
    inp = small_inputs(B=64, T=1, H=16, K=128, V=128, dtype=torch.bfloat16, seed=24)
    d = to_dev(inp)
    o, sT = gpu_lib.gdn_recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"])
    torch.cuda.synchronize()
    o_ref, s_ref = oracle(inp)
    check(o, o_ref, 1e-2, "o")
    check(sT, s_ref, 1e-2, "state")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("KV", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_recurrent_qk_l2norm(gpu_lib, dtype, KV):
    """Raw q and k (rows of norms 0.2-4, one all-zero row) normalised inside the decode kernel:
    against the oracle's composition of the normalisation with the rule."""
    from oracle import ref_fwd_l2
    K, V = KV
    inp = small_inputs(B=3, T=5, H=2, K=K, V=V, dtype=dtype, seed=24)
    gen = torch.Generator().manual_seed(25)
    for n in ("q", "k"):
        x = torch.randn(inp[n].shape, generator=gen) * (0.2 + 3.8 * torch.rand(inp[n].shape[:-1] + (1,), generator=gen))
        x[1, 2, 0] = 0.0
        inp[n] = x.to(dtype)
    d = to_dev(inp)
    o, sT = gpu_lib.gdn_recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], scale=0.8,
                                      qk_l2norm=True)
    torch.cuda.synchronize()
    o_ref, s_ref = ref_fwd_l2(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], 0.8, inp["initial_state"])
    tol = tol_for(dtype)
    check(o, o_ref, tol, "o")
    check(sT, s_ref, tol, "state")


def test_decode_continues_l2norm_prefill(gpu_lib):
    """A prefill with the q/k normalisation inside the library, continued token by token with it:
    the oracle over all tokens."""
    from oracle import ref_fwd_l2
    T0, T1 = 700, 8
    inp = small_inputs(B=2, T=T0 + T1, H=2, K=128, V=128, seed=26)
    gen = torch.Generator().manual_seed(27)
    for n in ("q", "k"):
        x = torch.randn(inp[n].shape, generator=gen) * (0.2 + 3.8 * torch.rand(inp[n].shape[:-1] + (1,), generator=gen))
        inp[n] = x.to(torch.bfloat16)
    d = to_dev(inp)
    pre = slice_tokens(d, 0, T0)
    o_pre, s_pre = gpu_lib.gdn_chunk_fwd(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], d["initial_state"],
                                         qk_l2norm=True)
    dec = slice_tokens(d, T0, T0 + T1)
    o_dec, s_dec = gpu_lib.gdn_recurrent_fwd(dec["q"], dec["k"], dec["v"], dec["g"], dec["beta"], s_pre,
                                             qk_l2norm=True)
    torch.cuda.synchronize()
    o_ref, s_ref = ref_fwd_l2(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], 1.0, inp["initial_state"])
    check(o_pre, o_ref[:, :T0], 1e-2, "prefill o")
    check(o_dec, o_ref[:, T0:], 1e-2, "decode o")
    check(s_dec, s_ref, 1e-2, "decode state")


def test_decode_in_hip_graph(gpu_lib):
    """Eight in-place decode steps captured in a HIP graph (launches only, no memsets): every
    replay, with eager work and synchronisations between replays, matches the same eight steps
    run eagerly from the same state, bit for bit."""
    inp = small_inputs(B=1, T=8, H=4, K=128, V=128, seed=28)
    d = to_dev(inp)
    steps = [slice_tokens(d, t, t + 1) for t in range(8)]
    state = d["initial_state"].clone()
    o = torch.empty((1, 1, 4, 128), dtype=torch.bfloat16, device="cuda")
    outs = [torch.empty_like(o) for _ in range(8)]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t, x in enumerate(steps):
            gpu_lib.gdn_recurrent_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], state, state_out=state, o=outs[t])
    ref_state = d["initial_state"].clone()
    for rep in range(3):
        start = ref_state.clone()
        state.copy_(start)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        # the same steps eagerly, from the same start
        s_e = start.clone()
        for t, x in enumerate(steps):
            o_e, _ = gpu_lib.gdn_recurrent_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], s_e, state_out=s_e)
            torch.cuda.synchronize()
            assert torch.equal(outs[t], o_e), (rep, t)
        assert torch.equal(state, s_e), rep
        ref_state = s_e * 0.5  # a different start for the next replay
    del graph
