"""Pins of the comparator that decides every GPU parity test (no GPU).

rel_l2(x, ref) = ||x - ref||_2 / ||ref||_2 over the whole tensor, the relative L2 error the
parity bounds are stated in (1e-2 for bf16 inputs with fp32 accumulation, 1e-4 in fp32
mode). Hand values fix the numerator, the denominator (the reference's norm, not the
candidate's) and the flattening over every element; planted mismatches just above each
bound must fail the same assertion the GPU tests use.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import BF16_TOL, FP32_TOL, check
from oracle import rel_l2


def test_hand_values():
    assert rel_l2([1.0, 0.0], [1.0, 0.0]) == 0.0
    # a zero reference: the absolute error ||(3, 4)|| is returned
    assert rel_l2([3.0, 4.0], [0.0, 0.0]) == 5.0
    # ||(2,0) - (1,0)|| / ||(1,0)|| = 1
    assert rel_l2([2.0, 0.0], [1.0, 0.0]) == 1.0
    # the denominator is the reference's norm: swapping the arguments halves the value
    assert rel_l2([1.0, 0.0], [2.0, 0.0]) == 0.5
    # (3,4) + (0.03, 0.04): ||diff|| = 0.05, ||ref|| = 5 -> 0.01
    assert rel_l2([3.03, 4.04], [3.0, 4.0]) == pytest.approx(0.01, rel=1e-12)
    # an error perpendicular to the reference counts in full: ||(0, 1)|| / ||(1, 0)|| = 1
    assert rel_l2([1.0, 1.0], [1.0, 0.0]) == 1.0


def test_whole_tensor_not_per_row():
    # two rows: one exact, one off by its own size; per-row errors would be 0 and 1, the
    # whole-tensor value is ||(0,0,1,0)|| / ||(10,0,1,0)|| = 1 / sqrt(101)
    ref = np.array([[10.0, 0.0], [1.0, 0.0]])
    x = np.array([[10.0, 0.0], [2.0, 0.0]])
    assert rel_l2(x, ref) == pytest.approx(1.0 / np.sqrt(101.0), rel=1e-14)
    # shape does not matter, only the elements
    assert rel_l2(x.T.copy().T, ref) == rel_l2(x.ravel(), ref.ravel())


def test_torch_and_bf16_inputs_upcast_exactly():
    ref = torch.tensor([1.0, 2.0, 3.0], dtype=torch.float64)
    x = ref.to(torch.bfloat16)  # 1, 2, 3 are exact in bf16
    assert rel_l2(x, ref) == 0.0
    y = torch.tensor([1.0, 2.0, 3.0 + 2.0 ** -6], dtype=torch.float32)  # exact in fp32
    assert rel_l2(y, ref) == pytest.approx(2.0 ** -6 / np.sqrt(14.0), rel=1e-14)


@pytest.mark.parametrize("tol", [BF16_TOL, FP32_TOL])
def test_planted_mismatch_fails_the_bound(tol):
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((4, 64, 8))
    noise = rng.standard_normal(ref.shape)
    noise *= np.linalg.norm(ref) / np.linalg.norm(noise)
    # 1.5x the bound: must fail; 0.5x: must pass
    bad = torch.from_numpy(ref + 1.5 * tol * noise)
    good = torch.from_numpy(ref + 0.5 * tol * noise)
    assert rel_l2(bad, ref) == pytest.approx(1.5 * tol, rel=1e-9)
    with pytest.raises(AssertionError):
        check(bad, ref, tol, "planted")
    assert check(good, ref, tol, "clean") == pytest.approx(0.5 * tol, rel=1e-9)


def test_one_sign_flip_is_caught():
    # a sign flip of one element of many is caught at the bf16 bound
    ref = np.ones(1000)
    x = ref.copy()
    x[17] = -1.0
    assert rel_l2(x, ref) == pytest.approx(2.0 / np.sqrt(1000.0), rel=1e-14)
    with pytest.raises(AssertionError):
        check(torch.from_numpy(x), ref, BF16_TOL)
