"""Full-size forward parity on the workloads' real shapes, in the launch
configuration the benchmark times (AutoCP on its own unless stated).

The oracle runs on a sample of outputs it computes exactly: every head and
token, restricted to a subset of value rows (rows of the state evolve
independently, so the oracle given only those rows of v and of the initial
state returns exactly those rows of O and of the final state).
"""
import numpy as np
import pytest
import torch

from gdn_inputs import make_inputs
from gpu_helpers import check, gpu_fwd, oracle, to_dev

pytestmark = pytest.mark.gpu

# Four rows of every 16-row block: the output pass gives each wave of its workgroup one block
# of 16 state rows, so every wave's rows (first, last and two inside) are compared.
ROWS = sorted(16 * w + i for w in range(8) for i in (0, 5, 10, 15))


def _sampled(inp, o, sT, rows=ROWS, tol=1e-2):
    o_ref, s_ref = oracle(inp, rows=rows)
    e_o = check(o[..., rows], o_ref, tol, "o")
    e_s = check(sT[:, :, rows], s_ref, tol, "final_state")
    return e_o, e_s


@pytest.mark.parametrize("cp", ["auto", "off", "exact"])
def test_edge_prefill_32k(gpu_lib, cp):
    """B=1, H=16, T=32768, bf16, per-head decay scale in [0.01, 1], fp32 initial state."""
    inp = make_inputs("edge_prefill", seed=0)
    d = to_dev(inp)
    modes = gpu_lib.gdn_cp_modes(d["k"], d["v"], d["g"], d["beta"], cp_mode=cp).cpu().numpy()
    o, sT = gpu_fwd(d, cp_mode=cp)
    e_o, e_s = _sampled(inp, o.cpu(), sT.cpu())
    print(f"cp={cp} modes={modes.tolist()} warmup_frac={(modes == 1).mean():.2f} "
          f"rel_l2 o={e_o:.2e} final={e_s:.2e}", flush=True)
    if cp == "auto":
        # the per-head decay scales straddle the warmup threshold: both paths are used
        assert (modes == 1).any() and (modes >= 2).any()
        fwd, rev = gpu_lib.gdn_cp_windows(d["k"], d["v"], d["g"], d["beta"], cp_mode=cp)
        b = fwd.cpu()[fwd.cpu() >= 0]
        print(f"boundaries taking the warmup: {float((b > 0).float().mean()):.2f}", flush=True)


def test_tp8_long_256k(gpu_lib):
    """B=1, H=8, T=262144 (one TP8 shard of a 256K prompt), bf16, zero initial state."""
    inp = make_inputs("tp8_long", seed=0)
    o, sT = gpu_fwd(to_dev(inp))
    e_o, e_s = _sampled(inp, o.cpu(), sT.cpu())
    print(f"tp8_long rel_l2 o={e_o:.2e} final={e_s:.2e}", flush=True)


def test_varlen_packed(gpu_lib):
    """8 packed sequences of 1K-16K tokens (~64K total), H=32, bf16, no CP."""
    inp = make_inputs("varlen_packed", seed=0)
    lengths = inp["meta"]["lengths"]
    assert abs(sum(lengths) - 65536) <= 6554
    o, sT = gpu_fwd(to_dev(inp), cp_mode="off")
    e_o, e_s = _sampled(inp, o.cpu(), sT.cpu())
    print(f"varlen lengths={lengths} rel_l2 o={e_o:.2e} final={e_s:.2e}", flush=True)
    # and the same batch with CP forced on over the packed sequences
    o2, s2 = gpu_fwd(to_dev(inp), cp_mode="on")
    _sampled(inp, o2.cpu(), s2.cpu())
