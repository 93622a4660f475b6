"""Pins of the CPU oracle's forward pass (no GPU).

The pages print no formula or worked example for the gated delta rule
(FlashQLA: ollai.cn article, "main features"), so the oracle is pinned to
things other than itself:
  * an independent chunked (WY) reformulation at several chunk sizes,
  * the recurrence evaluated literally with explicit (I - b k k^T) matrices,
  * a hand-worked two-token example (tests/golden/hand_example.txt),
  * closed forms and invariants (identity update, pure decay, delta-rule
    write with orthonormal keys, masked matmul with orthogonal keys,
    split continuation, varlen packing, linearity).
Each case uses dk != dv somewhere so a transposed state fails.
"""
import os

import numpy as np
import pytest

from oracle import ref_fwd, rel_l2
from oracle.chunked import chunked_fwd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(rng, B=1, T=37, H=2, K=6, V=5, init=True, decay=0.3, normalise=True):
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    if normalise:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, V))
    g = -decay * np.log1p(np.exp(rng.standard_normal((B, T, H))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    s0 = 0.3 * rng.standard_normal((B, H, V, K)) if init else None
    return q, k, v, g, beta, s0


def literal_recurrence(q, k, v, g, beta, scale, s0):
    """S_t = e^{g_t} S_{t-1} (I - b k k^T) + b v k^T with explicit matrices (one sequence, one head)."""
    T, K = k.shape
    V = v.shape[1]
    S = np.zeros((V, K)) if s0 is None else s0.copy()
    o = np.zeros((T, V))
    for t in range(T):
        M = np.eye(K) - beta[t] * np.outer(k[t], k[t])
        S = np.exp(g[t]) * S @ M + beta[t] * np.outer(v[t], k[t])
        o[t] = scale * S @ q[t]
    return o, S


@pytest.mark.parametrize("C", [1, 4, 16, 64])
def test_chunked_reformulation_matches(C):
    rng = np.random.default_rng(1)
    q, k, v, g, beta, s0 = rand_case(rng, B=2, T=150, H=2, K=12, V=20)
    o, sT = ref_fwd(q, k, v, g, beta, 0.75, s0)
    o2, sT2 = chunked_fwd(q, k, v, g, beta, 0.75, s0, chunk=C)
    assert rel_l2(o2, o) < 1e-12
    assert rel_l2(sT2, sT) < 1e-12


def test_chunked_varlen_partial_chunks():
    rng = np.random.default_rng(2)
    lens = [70, 1, 0, 130, 64]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta, _ = rand_case(rng, B=1, T=int(cu[-1]), H=3, K=8, V=4, init=False)
    s0 = 0.2 * rng.standard_normal((len(lens), 3, 4, 8))
    o, sT = ref_fwd(q, k, v, g, beta, 1.0, s0, cu_seqlens=cu)
    o2, sT2 = chunked_fwd(q, k, v, g, beta, 1.0, s0, cu_seqlens=cu, chunk=64)
    assert rel_l2(o2, o) < 1e-12
    assert rel_l2(sT2, sT) < 1e-12
    # the empty sequence returns its initial state unchanged
    np.testing.assert_array_equal(sT[2], s0[2])


def test_literal_matrix_recurrence():
    rng = np.random.default_rng(3)
    q, k, v, g, beta, s0 = rand_case(rng, B=1, T=23, H=2, K=3, V=7, normalise=False)
    o, sT = ref_fwd(q, k, v, g, beta, 1.3, s0)
    for h in range(2):
        ol, Sl = literal_recurrence(q[0, :, h], k[0, :, h], v[0, :, h], g[0, :, h],
                                    beta[0, :, h], 1.3, s0[0, h])
        np.testing.assert_allclose(o[0, :, h], ol, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(sT[0, h], Sl, rtol=1e-12, atol=1e-12)


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *nums = line.split()
            vals[key] = np.array([float(x) for x in nums])
    return vals


def test_hand_worked_example():
    gv = _read_golden("hand_example.txt")
    T, K, V = 2, 2, 2
    q = gv["q"].reshape(1, T, 1, K)
    k = gv["k"].reshape(1, T, 1, K)
    v = gv["v"].reshape(1, T, 1, V)
    g = gv["g"].reshape(1, T, 1)
    beta = gv["beta"].reshape(1, T, 1)
    o, sT = ref_fwd(q, k, v, g, beta, 1.0, None)
    np.testing.assert_allclose(o.ravel(), gv["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(sT.ravel(), gv["final_state"], rtol=0, atol=1e-14)


def test_identity_update_keeps_state():
    """g = 0 and beta = 0: S_T = S_0 and O = scale Q S_0^T."""
    rng = np.random.default_rng(4)
    q, k, v, g, beta, s0 = rand_case(rng, B=2, T=40, H=2, K=5, V=9)
    o, sT = ref_fwd(q, k, v, 0 * g, 0 * beta, 0.5, s0)
    np.testing.assert_array_equal(sT, s0)
    expect = 0.5 * np.einsum("bthk,bhvk->bthv", q, s0)
    np.testing.assert_allclose(o, expect, rtol=1e-13, atol=1e-14)


def test_pure_decay_closed_form():
    """beta = 0: S_t = exp(sum_{s<=t} g_s) S_0."""
    rng = np.random.default_rng(5)
    q, k, v, g, beta, s0 = rand_case(rng, B=1, T=50, H=2, K=4, V=6)
    o, sT = ref_fwd(q, k, v, g, 0 * beta, 1.0, s0)
    cg = np.cumsum(g[0], axis=0)  # [T,H]
    np.testing.assert_allclose(sT[0], np.exp(cg[-1])[:, None, None] * s0[0], rtol=1e-12)
    expect = np.exp(cg)[:, :, None] * np.einsum("thk,hvk->thv", q[0], s0[0])
    np.testing.assert_allclose(o[0], expect, rtol=1e-11, atol=1e-14)


def test_delta_rule_write_orthonormal_keys():
    """Orthonormal keys, beta = 1, g = 0, S_0 = 0: the state maps k_j to v_j exactly."""
    rng = np.random.default_rng(6)
    K, V, T = 8, 3, 8
    Qm, _ = np.linalg.qr(rng.standard_normal((K, K)))
    k = Qm.T[:T].reshape(1, T, 1, K)
    v = rng.standard_normal((1, T, 1, V))
    q = rng.standard_normal((1, T, 1, K))
    _, sT = ref_fwd(q, k, v, np.zeros((1, T, 1)), np.ones((1, T, 1)), 1.0, None)
    np.testing.assert_allclose(sT[0, 0] @ k[0, :, 0].T, v[0, :, 0].T, atol=1e-13)


def test_orthogonal_keys_masked_matmul():
    """Mutually orthogonal (not unit) keys, g = 0, S_0 = 0: O = tril(Q K^T) diag(beta) V."""
    rng = np.random.default_rng(7)
    K, V, T = 10, 4, 10
    Qm, _ = np.linalg.qr(rng.standard_normal((K, K)))
    kk = Qm.T * rng.uniform(0.5, 2.0, size=(K, 1))
    k = kk.reshape(1, T, 1, K)
    q = rng.standard_normal((1, T, 1, K))
    v = rng.standard_normal((1, T, 1, V))
    beta = rng.uniform(0.1, 0.9, size=(1, T, 1))
    o, _ = ref_fwd(q, k, v, np.zeros((1, T, 1)), beta, 1.0, None)
    expect = np.tril(q[0, :, 0] @ kk.T) @ (beta[0, :, 0][:, None] * v[0, :, 0])
    np.testing.assert_allclose(o[0, :, 0], expect, rtol=1e-12, atol=1e-13)


def test_split_continuation():
    """Running [0, m) then [m, T) from the state at m equals one run."""
    rng = np.random.default_rng(8)
    q, k, v, g, beta, s0 = rand_case(rng, B=1, T=91, H=2, K=7, V=5)
    o, sT = ref_fwd(q, k, v, g, beta, 1.0, s0)
    m = 38
    oa, sa = ref_fwd(q[:, :m], k[:, :m], v[:, :m], g[:, :m], beta[:, :m], 1.0, s0)
    ob, sb = ref_fwd(q[:, m:], k[:, m:], v[:, m:], g[:, m:], beta[:, m:], 1.0, sa)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(sb, sT, rtol=1e-13, atol=1e-14)


def test_varlen_equals_separate_runs():
    rng = np.random.default_rng(9)
    lens = [17, 64, 3, 90]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta, _ = rand_case(rng, B=1, T=int(cu[-1]), H=2, K=6, V=3, init=False)
    s0 = rng.standard_normal((4, 2, 3, 6))
    o, sT = ref_fwd(q, k, v, g, beta, 1.0, s0, cu_seqlens=cu)
    for n in range(4):
        a, b = cu[n], cu[n + 1]
        on, sn = ref_fwd(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b], 1.0, s0[n:n + 1])
        np.testing.assert_allclose(o[:, a:b], on, rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(sT[n], sn[0], rtol=1e-14, atol=1e-15)


def test_linear_in_values_and_initial_state():
    rng = np.random.default_rng(10)
    q, k, v, g, beta, s0 = rand_case(rng, B=1, T=45, H=1, K=4, V=6)
    v2 = rng.standard_normal(v.shape)
    s02 = rng.standard_normal(s0.shape)
    a, b = 0.7, -1.9
    o1, s1 = ref_fwd(q, k, v, g, beta, 1.0, s0)
    o2, s2 = ref_fwd(q, k, v2, g, beta, 1.0, s02)
    o3, s3 = ref_fwd(q, k, a * v + b * v2, g, beta, 1.0, a * s0 + b * s02)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s3, a * s1 + b * s2, rtol=1e-11, atol=1e-12)


def test_batch_rows_independent_and_threads_deterministic():
    rng = np.random.default_rng(11)
    q, k, v, g, beta, s0 = rand_case(rng, B=3, T=33, H=2, K=40, V=70)
    o1, s1 = ref_fwd(q, k, v, g, beta, 1.0, s0, nthreads=1)
    o4, s4 = ref_fwd(q, k, v, g, beta, 1.0, s0, nthreads=4)
    np.testing.assert_array_equal(o1, o4)
    np.testing.assert_array_equal(s1, s4)
    ob, sb = ref_fwd(q[1:2], k[1:2], v[1:2], g[1:2], beta[1:2], 1.0, s0[1:2])
    np.testing.assert_array_equal(o1[1:2], ob)
    # value rows evolve independently: a subset of rows gives the same rows
    rows = [3, 40, 69]
    orow, srow = ref_fwd(q, k, v[..., rows], g, beta, 1.0, s0[:, :, rows])
    np.testing.assert_array_equal(orow, o1[..., rows])
    np.testing.assert_array_equal(srow, s1[:, :, rows])


def test_rejects_bad_offsets():
    rng = np.random.default_rng(12)
    q, k, v, g, beta, _ = rand_case(rng, B=1, T=10, H=1, K=2, V=2, init=False)
    with pytest.raises(ValueError):
        ref_fwd(q, k, v, g, beta, 1.0, None, cu_seqlens=[0, 6, 4, 10])
    with pytest.raises(ValueError):
        ref_fwd(q, k, v, g, beta, 1.0, None, cu_seqlens=[0, 9])
