"""Pins of the CPU oracle's reverse mode (no GPU).

The pages ask for dq, dk, dv, dg, dbeta and d(initial_state) but give no
formula for them (FlashQLA announcement: the backward was "the hardest
part"). The oracle's hand-derived reverse mode is pinned by
  * central finite differences of the oracle forward (fp64, tiny sizes),
  * torch.autograd through the literal matrix recurrence (fp64),
  * the chunked (WY) reverse mode, an independent derivation,
  * Euler homogeneity identities, exact up to rounding at any size,
  * closed forms at g = 0, beta = 0.
"""
import numpy as np
import pytest
import torch

from oracle import ref_bwd, ref_fwd, rel_l2
from oracle.chunked import chunked_bwd

from test_oracle_forward import rand_case


def loss(o, sT, d_o, dsT):
    return float(np.sum(o * d_o) + np.sum(sT * dsT))


@pytest.mark.parametrize("varlen", [False, True])
def test_finite_differences(varlen):
    rng = np.random.default_rng(20)
    K, V, H = 3, 5, 1
    if varlen:
        cu = np.array([0, 5, 5, 12])
        B, T, N = 1, 12, 3
    else:
        cu = None
        B, T, N = 2, 9, 2
    q, k, v, g, beta, _ = rand_case(rng, B=B, T=T, H=H, K=K, V=V, init=False, normalise=False)
    s0 = 0.5 * rng.standard_normal((N, H, V, K))
    d_o = rng.standard_normal((B, T, H, V))
    dsT = rng.standard_normal((N, H, V, K))
    scale = 0.8
    grads = ref_bwd(q, k, v, g, beta, d_o, scale, s0, dsT, cu_seqlens=cu)
    args = dict(q=q, k=k, v=v, g=g, beta=beta, s0=s0)
    names = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", s0="d_initial_state")
    h = 1e-6
    for name, arr in args.items():
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            saved = arr[idx]
            vals = []
            for sgn in (1, -1):
                arr[idx] = saved + sgn * h
                o, sT = ref_fwd(args["q"], args["k"], args["v"], args["g"], args["beta"],
                                scale, args["s0"], cu_seqlens=cu)
                vals.append(loss(o, sT, d_o, dsT))
            arr[idx] = saved
            fd[idx] = (vals[0] - vals[1]) / (2 * h)
        err = rel_l2(grads[names[name]], fd)
        assert err < 1e-7, (name, err)


def test_torch_autograd_literal_recurrence():
    rng = np.random.default_rng(21)
    B, T, H, K, V = 1, 14, 2, 4, 6
    q, k, v, g, beta, s0 = rand_case(rng, B=B, T=T, H=H, K=K, V=V, normalise=False)
    d_o = rng.standard_normal((B, T, H, V))
    dsT = rng.standard_normal((B, H, V, K))
    scale = 1.1
    tt = {n: torch.tensor(x, dtype=torch.float64, requires_grad=True)
          for n, x in dict(q=q, k=k, v=v, g=g, beta=beta, s0=s0).items()}
    total = torch.zeros((), dtype=torch.float64)
    for h in range(H):
        S = tt["s0"][0, h]
        for t in range(T):
            kt = tt["k"][0, t, h]
            M = torch.eye(K, dtype=torch.float64) - tt["beta"][0, t, h] * torch.outer(kt, kt)
            S = torch.exp(tt["g"][0, t, h]) * (S @ M) + tt["beta"][0, t, h] * torch.outer(tt["v"][0, t, h], kt)
            o = scale * (S @ tt["q"][0, t, h])
            total = total + (o * torch.tensor(d_o[0, t, h])).sum()
        total = total + (S * torch.tensor(dsT[0, h])).sum()
    total.backward()
    grads = ref_bwd(q, k, v, g, beta, d_o, scale, s0, dsT)
    pairs = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", s0="d_initial_state")
    for n, gname in pairs.items():
        np.testing.assert_allclose(grads[gname], tt[n].grad.numpy(), rtol=1e-10, atol=1e-12,
                                   err_msg=gname)


@pytest.mark.parametrize("C", [1, 16, 64])
def test_chunked_reverse_mode_matches(C):
    rng = np.random.default_rng(22)
    lens = [100, 7, 64, 0, 129]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta, _ = rand_case(rng, B=1, T=int(cu[-1]), H=2, K=10, V=14, init=False)
    s0 = 0.3 * rng.standard_normal((5, 2, 14, 10))
    d_o = rng.standard_normal(v.shape)
    dsT = 0.1 * rng.standard_normal(s0.shape)
    a = ref_bwd(q, k, v, g, beta, d_o, 0.9, s0, dsT, cu_seqlens=cu)
    b = chunked_bwd(q, k, v, g, beta, d_o, 0.9, s0, dsT, cu_seqlens=cu, chunk=C)
    for key in a:
        assert rel_l2(b[key], a[key]) < 1e-11, key


def test_euler_homogeneity():
    """<dq, q> = <dO, O>;  <dv, v> + <dS0, S0> = <dO, O> + <dS_T, S_T>."""
    rng = np.random.default_rng(23)
    q, k, v, g, beta, s0 = rand_case(rng, B=2, T=130, H=2, K=16, V=24)
    d_o = rng.standard_normal(v.shape)
    dsT = rng.standard_normal(s0.shape)
    o, sT = ref_fwd(q, k, v, g, beta, 1.0, s0)
    gr = ref_bwd(q, k, v, g, beta, d_o, 1.0, s0, dsT)
    lo = np.sum(d_o * o)
    ls = np.sum(dsT * sT)
    assert np.isclose(np.sum(gr["dq"] * q), lo, rtol=1e-11)
    assert np.isclose(np.sum(gr["dv"] * v) + np.sum(gr["d_initial_state"] * s0), lo + ls, rtol=1e-11)


def test_closed_forms_identity_update():
    """g = 0, beta = 0: dv = 0, dk = 0, dq = scale S0^T do, dS0 = dS_T + scale dO^T Q,
    dg_t = <dS_T, S0> + scale sum_{s>=t} do_s^T S0 q_s,
    dbeta_t = (G_t k_t).(v_t - S0 k_t) with G_t = dS_T + scale sum_{s>=t} do_s q_s^T."""
    rng = np.random.default_rng(24)
    B, T, H, K, V = 1, 20, 1, 5, 3
    q, k, v, g, beta, s0 = rand_case(rng, B=B, T=T, H=H, K=K, V=V)
    d_o = rng.standard_normal(v.shape)
    dsT = rng.standard_normal(s0.shape)
    sc = 0.6
    gr = ref_bwd(q, k, v, 0 * g, 0 * beta, d_o, sc, s0, dsT)
    S0, dS = s0[0, 0], dsT[0, 0]
    Q, Kk, Vv, dO = q[0, :, 0], k[0, :, 0], v[0, :, 0], d_o[0, :, 0]
    np.testing.assert_array_equal(gr["dv"], 0)
    np.testing.assert_allclose(gr["dk"], 0, atol=1e-14)
    np.testing.assert_allclose(gr["dq"][0, :, 0], sc * dO @ S0, rtol=1e-12)
    np.testing.assert_allclose(gr["d_initial_state"][0, 0], dS + sc * dO.T @ Q, rtol=1e-12)
    per_tok = sc * np.einsum("tv,vk,tk->t", dO, S0, Q)
    dg_expect = np.sum(dS * S0) + np.cumsum(per_tok[::-1])[::-1]
    np.testing.assert_allclose(gr["dg"][0, :, 0], dg_expect, rtol=1e-11)
    dbeta_expect = np.zeros(T)
    for t in range(T):
        Gt = dS + sc * dO[t:].T @ Q[t:]
        dbeta_expect[t] = (Gt @ Kk[t]) @ (Vv[t] - S0 @ Kk[t])
    np.testing.assert_allclose(gr["dbeta"][0, :, 0], dbeta_expect, rtol=1e-11)


def test_empty_sequence_gradients():
    rng = np.random.default_rng(25)
    cu = np.array([0, 0, 6])
    q, k, v, g, beta, _ = rand_case(rng, B=1, T=6, H=1, K=2, V=3, init=False)
    s0 = rng.standard_normal((2, 1, 3, 2))
    dsT = rng.standard_normal((2, 1, 3, 2))
    gr = ref_bwd(q, k, v, g, beta, rng.standard_normal(v.shape), 1.0, s0, dsT, cu_seqlens=cu)
    np.testing.assert_array_equal(gr["d_initial_state"][0], dsT[0])
