"""Pins of the oracle's q/k L2 normalisation (no GPU).

The pages print no formula for the normalisation ahead of the path; the reading is
x / sqrt(sum x^2 + eps), eps = 1e-6. It is pinned by
  * closed forms on hand rows (3-4-5, all ones, all zero),
  * unit norm and direction against numpy's own vector norm (eps = 0),
  * central finite differences of the normalisation and of the whole path with it,
  * orthogonality of the raw-row gradient to the row and its 1/c scaling (eps = 0),
  * invariance of the whole path under positive per-row scaling of q and k (eps = 0).
"""
import numpy as np
import pytest

from oracle import l2norm, l2norm_bwd, ref_bwd_l2, ref_fwd, ref_fwd_l2, L2_EPS

from test_oracle_forward import rand_case


def test_hand_rows():
    x = np.array([[3.0, 4.0, 0.0, 0.0], [1.0, 1.0, 1.0, 1.0], [0.0, 0.0, 0.0, 0.0]])
    y = l2norm(x[:2], eps=0.0)
    assert np.allclose(y[0], [0.6, 0.8, 0.0, 0.0], rtol=0, atol=1e-16)
    assert np.allclose(y[1], [0.5, 0.5, 0.5, 0.5], rtol=0, atol=1e-16)
    y = l2norm(x)
    assert L2_EPS == 1e-6
    assert np.allclose(y[0, :2], np.array([3.0, 4.0]) / np.sqrt(25.000001), rtol=1e-15, atol=0)
    assert np.all(y[2] == 0.0)  # an all-zero row stays zero (and finite)


def test_unit_norm_and_direction():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 7, 3, 16)) * rng.uniform(0.1, 10, (5, 7, 3, 1))
    y = l2norm(x, eps=0.0)
    assert np.allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=0, atol=1e-14)
    assert np.allclose(y, x / np.linalg.norm(x, axis=-1, keepdims=True), rtol=0, atol=1e-15)
    # eps shrinks every row a little, more for short rows
    n = np.linalg.norm(l2norm(x), axis=-1)
    assert np.all(n < 1.0) and np.allclose(n, np.sqrt(np.sum(x * x, -1) / (np.sum(x * x, -1) + 1e-6)))


def test_bwd_finite_differences():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 5)) * 0.7
    c = rng.standard_normal((3, 5))
    for eps in (0.0, L2_EPS, 0.3):
        dx = l2norm_bwd(x, c, eps)
        h = 1e-6
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            fd[idx] = (np.sum(c * l2norm(xp, eps)) - np.sum(c * l2norm(xm, eps))) / (2 * h)
        assert np.allclose(dx, fd, rtol=1e-7, atol=1e-8), eps


def test_bwd_orthogonal_and_scaling():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 6, 32))
    dy = rng.standard_normal((4, 6, 32))
    dx = l2norm_bwd(x, dy, eps=0.0)
    assert np.allclose(np.sum(dx * x, -1), 0.0, atol=1e-12)
    assert np.allclose(l2norm_bwd(2.5 * x, dy, eps=0.0), dx / 2.5, rtol=1e-13, atol=1e-14)


def _loss(q, k, v, g, beta, s0, d_o, dsT, scale):
    o, sT = ref_fwd_l2(q, k, v, g, beta, scale, s0)
    return float(np.sum(o * d_o) + np.sum(sT * dsT))


def test_path_finite_differences():
    rng = np.random.default_rng(4)
    q, k, v, g, beta, s0 = rand_case(rng, B=1, T=7, H=1, K=3, V=2, normalise=False)
    q *= rng.uniform(0.3, 3.0, (1, 7, 1, 1))
    k *= rng.uniform(0.3, 3.0, (1, 7, 1, 1))
    d_o = rng.standard_normal(v.shape)
    dsT = rng.standard_normal(s0.shape)
    scale = 0.7
    out = ref_bwd_l2(q, k, v, g, beta, d_o, scale, s0, dsT)
    h = 1e-6
    for name, x in (("dq", q), ("dk", k)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = (xp, k) if name == "dq" else (q, xp)
            args_m = (xm, k) if name == "dq" else (q, xm)
            fd[idx] = (_loss(*args_p, v, g, beta, s0, d_o, dsT, scale)
                       - _loss(*args_m, v, g, beta, s0, d_o, dsT, scale)) / (2 * h)
        assert np.allclose(out[name], fd, rtol=1e-6, atol=1e-8), name


def test_path_scale_invariance():
    rng = np.random.default_rng(5)
    q, k, v, g, beta, s0 = rand_case(rng, B=2, T=40, H=2, K=8, V=4, normalise=False)
    a = rng.uniform(0.05, 20.0, (2, 40, 2, 1))
    b = rng.uniform(0.05, 20.0, (2, 40, 2, 1))
    o1, s1 = ref_fwd_l2(q, k, v, g, beta, 1.0, s0, eps=0.0)
    o2, s2 = ref_fwd_l2(a * q, b * k, v, g, beta, 1.0, s0, eps=0.0)
    o3, s3 = ref_fwd(q / np.linalg.norm(q, axis=-1, keepdims=True),
                     k / np.linalg.norm(k, axis=-1, keepdims=True), v, g, beta, 1.0, s0)
    for x, y in ((o1, o2), (s1, s2), (o1, o3), (s1, s3)):
        assert np.allclose(x, y, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("flip", ["sign", "drop_projection"])
def test_planted_mistakes_fail(flip):
    """A wrong sign or a dropped projection term in the reverse mode is caught by the pins."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((2, 4))
    c = rng.standard_normal((2, 4))
    r = 1.0 / np.sqrt(np.sum(x * x, -1, keepdims=True) + L2_EPS)
    xh = x * r
    bad = r * (c + xh * np.sum(xh * c, -1, keepdims=True)) if flip == "sign" else r * c
    h = 1e-6
    fd = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fd[idx] = (np.sum(c * l2norm(xp)) - np.sum(c * l2norm(xm))) / (2 * h)
    assert not np.allclose(bad, fd, rtol=1e-6, atol=1e-8)
    assert np.allclose(l2norm_bwd(x, c), fd, rtol=1e-6, atol=1e-8)
