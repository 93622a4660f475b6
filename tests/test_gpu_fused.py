"""GPU parity of the fully fused forward (the intra-chunk step and the recurrence in one kernel,
no CP, bf16) against the CPU oracle, and against the two-kernel split on the same inputs.

Bound: relative L2 <= 1e-2 (bf16 inputs, fp32 accumulation) on O and the final state, for
every K/V combination, ragged tails, packed sequences (empty, one-token, partial chunks), with
and without an initial state, and with the q/k L2 normalisation inside.
"""
import pytest
import torch

from gpu_helpers import BF16_TOL, check, oracle, seq_slices, small_inputs, to_dev
from oracle import ref_fwd_l2

pytestmark = pytest.mark.gpu


def run(gdn, d, fused, **kw):
    o, sT = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"],
                              cu_seqlens=d.get("cu_seqlens"), cp_mode="off", fused=fused, **kw)
    torch.cuda.synchronize()
    return o, sT


@pytest.mark.parametrize("K,V", [(64, 64), (128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("init", [0.1, None])
def test_fused_forward(gpu_lib, K, V, init):
    gdn = gpu_lib
    inp = small_inputs(B=2, T=1000, H=3, K=K, V=V, seed=41, init_std=init)
    d = to_dev(inp)
    assert gdn.gdn_plan(gdn.make_desc(d["q"], d["v"], cp_mode="off", flags=gdn.GDN_FLAG_FWD_FUSED))["fused_fwd"] == 1
    o_ref, s_ref = oracle(inp, scale=0.9)
    o, sT = run(gdn, d, True, scale=0.9)
    e_o = check(o, o_ref, BF16_TOL, "o")
    e_s = check(sT, s_ref, BF16_TOL, "final_state")
    o2, s2 = run(gdn, d, False, scale=0.9)
    check(o, o2.double().cpu(), BF16_TOL, "o vs split")
    print(f"fused K={K} V={V} rel_l2 o={e_o:.2e} final={e_s:.2e}", flush=True)


def test_fused_forward_varlen(gpu_lib):
    gdn = gpu_lib
    lengths = [1, 63, 64, 65, 0, 700, 1500, 129]
    inp = small_inputs(H=3, K=128, V=128, lengths=lengths, seed=42)
    d = to_dev(inp)
    o_ref, s_ref = oracle(inp)
    o, sT = run(gdn, d, True)
    check(o, o_ref, BF16_TOL, "o")
    oc = o.cpu()
    for n, a, b in seq_slices(inp["cu_seqlens"]):
        check(oc[:, a:b], o_ref[:, a:b], BF16_TOL, f"o of sequence {n} ({b - a} tokens)")
        check(sT[n], s_ref[n], BF16_TOL, f"final state of sequence {n}")
    assert torch.equal(sT[4].cpu(), inp["initial_state"][4])  # the empty sequence


def test_fused_forward_l2norm(gpu_lib):
    """Raw q and k rows, normalised inside the fused kernel as they are staged."""
    gdn = gpu_lib
    inp = small_inputs(B=2, T=700, H=2, K=128, V=128, seed=43)
    gen = torch.Generator().manual_seed(44)
    for n in ("q", "k"):
        x = inp[n].float()
        inp[n] = (x * (0.25 + 3.75 * torch.rand(x.shape[:-1] + (1,), generator=gen))).to(torch.bfloat16)
    d = to_dev(inp)
    o_ref, s_ref = ref_fwd_l2(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], 1.0, inp["initial_state"])
    o, sT = run(gdn, d, True, qk_l2norm=True)
    check(o, o_ref, BF16_TOL, "o")
    check(sT, s_ref, BF16_TOL, "final_state")


def test_fused_forward_large_batch_planned(gpu_lib):
    """Where the plan picks the fused forward by itself (two rounds of sequence-heads on the chip),
    sampled heads against the oracle and the whole output against the split."""
    gdn = gpu_lib
    inp = small_inputs(B=8, T=320, H=64, K=128, V=128, seed=45)
    d = to_dev(inp)
    assert gdn.gdn_plan(gdn.make_desc(d["q"], d["v"]))["fused_fwd"] == 1
    o, sT = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"])
    torch.cuda.synchronize()
    heads = [0, 31, 63]
    o_ref, s_ref = oracle(inp, heads=heads)
    check(o[:, :, heads], o_ref, BF16_TOL, "o")
    check(sT[:, heads], s_ref, BF16_TOL, "final_state")
    o2, s2 = run(gdn, d, False)
    check(o, o2.double().cpu(), BF16_TOL, "o vs split")
    check(sT, s2.double().cpu(), BF16_TOL, "final state vs split")
