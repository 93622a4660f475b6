"""Chunked (WY-form) fp64 reformulation of the gated delta rule -- TEST INFRASTRUCTURE ONLY.

An independent rewrite of the same recurrence in numpy, used to pin the
token-by-token oracle (gdn_oracle.c) and to provide per-chunk intermediates
(chunk-local gate cumsum, w, u) for kernel-level checks. It shares no code
with the token oracle or with the GPU library.

The FlashQLA pages name the chunked prefill and its split into an intra-chunk
kernel and an inter-chunk kernel (ollai.cn article, "technical principles" and
"core advantages"), but print no algebra. The algebra below is derived from
the recurrence S_t = e^{g_t} S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T,
o_t = scale S_t q_t. For one chunk of c tokens entering with state S:

  gam_r = sum_{j<=r} g_j                 (chunk-local cumsum, Gam = gam_c)
  D_rj  = exp(gam_r - gam_j)
  A     = strict_lower(diag(b) (D * K K^T)),   T = (I + A)^{-1}
  W     = T diag(b e^gam) K,             U = T diag(b) V
  Delta = U - W S^T                      (row r: b_r (v_r - S'_r k_r))
  O     = diag(e^gam) Qs S^T + (tril(D) * Qs K^T) Delta,   Qs = scale Q
  S_new = e^Gam S + Delta^T diag(e^{Gam - gam}) K

The triangular solve is a library call; nothing else is fused or reordered.
The backward is reverse mode through exactly these chunk formulas.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular

from .oracle import to_f64


def _segments(B, T, cu_seqlens):
    if cu_seqlens is None:
        return [(b, b * T, (b + 1) * T) for b in range(B)], B
    cu = np.asarray(to_f64(cu_seqlens), dtype=np.int64)
    return [(n, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)], len(cu) - 1


def chunk_forward(Qs, Kc, Vc, gc, bc, S):
    """One chunk of the WY-form forward. Returns (O, S_new, intermediates)."""
    c = Kc.shape[0]
    gam = np.cumsum(gc)
    Gam = gam[-1]
    D = np.exp(gam[:, None] - gam[None, :])
    A = np.tril(bc[:, None] * D * (Kc @ Kc.T), -1)
    I = np.eye(c)
    T = solve_triangular(I + A, I, lower=True, unit_diagonal=True)
    Bk = (bc * np.exp(gam))[:, None] * Kc
    Bv = bc[:, None] * Vc
    W = T @ Bk
    U = T @ Bv
    Delta = U - W @ S.T
    L = np.tril(D)
    P = L * (Qs @ Kc.T)
    Qt = np.exp(gam)[:, None] * Qs
    O = Qt @ S.T + P @ Delta
    Kt = np.exp(Gam - gam)[:, None] * Kc
    S_new = np.exp(Gam) * S + Delta.T @ Kt
    inter = dict(gam=gam, Gam=Gam, D=D, A=A, T=T, Bk=Bk, Bv=Bv, W=W, U=U, Delta=Delta,
                 L=L, P=P, Qt=Qt, Kt=Kt, S=S)
    return O, S_new, inter


def chunked_fwd(q, k, v, g, beta, scale=1.0, initial_state=None, cu_seqlens=None,
                chunk=64, return_intermediates=False):
    """Forward in WY form. Same shapes and returns as oracle.ref_fwd.

    With return_intermediates, also returns dict(gam [B,T,H], w [B,T,H,K],
    u [B,T,H,V], chunk_states [list per (seq, head) of entering states]).
    """
    q, k, v, g, beta = (to_f64(x) for x in (q, k, v, g, beta))
    B, T, H, K = q.shape
    V = v.shape[-1]
    segs, N = _segments(B, T, cu_seqlens)
    s0 = to_f64(initial_state)
    qf, kf, vf = q.reshape(B * T, H, K), k.reshape(B * T, H, K), v.reshape(B * T, H, V)
    gf, bf = g.reshape(B * T, H), beta.reshape(B * T, H)
    o = np.zeros((B * T, H, V))
    sT = np.zeros((N, H, V, K))
    gam_all = np.zeros((B * T, H))
    w_all = np.zeros((B * T, H, K))
    u_all = np.zeros((B * T, H, V))
    states = {}
    for n, bos, eos in segs:
        for h in range(H):
            S = np.zeros((V, K)) if s0 is None else s0[n, h].copy()
            st = []
            for t0 in range(bos, eos, chunk):
                t1 = min(t0 + chunk, eos)
                st.append(S.copy())
                O, S, it = chunk_forward(scale * qf[t0:t1, h], kf[t0:t1, h], vf[t0:t1, h],
                                         gf[t0:t1, h], bf[t0:t1, h], S)
                o[t0:t1, h] = O
                gam_all[t0:t1, h] = it["gam"]
                w_all[t0:t1, h] = it["W"]
                u_all[t0:t1, h] = it["U"]
            sT[n, h] = S
            states[(n, h)] = st
    o = o.reshape(B, T, H, V)
    if not return_intermediates:
        return o, sT
    return o, sT, dict(gam=gam_all.reshape(B, T, H), w=w_all.reshape(B, T, H, K),
                       u=u_all.reshape(B, T, H, V), chunk_states=states)


def chunk_backward(it, Qs, Kc, Vc, bc, dO, G):
    """Reverse mode of chunk_forward for one chunk.

    `it` holds the chunk's forward intermediates (entering state S included),
    dO the output gradient and G = dL/dS_new. Returns (dQs, dK, dV, dbeta,
    dg, G_prev) with G_prev = dL/dS for the entering state.
    """
    gam, Gam, D, A, T = it["gam"], it["Gam"], it["D"], it["A"], it["T"]
    Bk, Bv, W, Delta, L, P, Qt, Kt, S = (it[x] for x in
                                         ("Bk", "Bv", "W", "Delta", "L", "P", "Qt", "Kt", "S"))
    c = Kc.shape[0]
    # O = Qt S^T + P Delta ; S_new = e^Gam S + Delta^T Kt
    dQt = dO @ S
    dP = dO @ Delta.T
    dDelta = P.T @ dO + Kt @ G.T
    dKt = Delta @ G
    G_prev = np.exp(Gam) * G + dO.T @ Qt - dDelta.T @ W
    # Delta = U - W S^T
    dW = -dDelta @ S
    dU = dDelta
    # W = T Bk, U = T Bv
    dT = dW @ Bk.T + dU @ Bv.T
    dBk = T.T @ dW
    dBv = T.T @ dU
    # T = (I + A)^{-1}; A strictly lower
    dA = np.tril(-T.T @ dT @ T.T, -1)
    dgam = np.zeros(c)
    dK = np.zeros_like(Kc)
    dbeta = np.zeros(c)
    # A = strict_lower(diag(b) (D * K K^T))
    KK = Kc @ Kc.T
    Mx = dA * bc[:, None] * D
    dK += Mx @ Kc + Mx.T @ Kc
    dbeta += np.sum(dA * D * KK, axis=1)
    dAA = dA * A
    dgam += dAA.sum(axis=1) - dAA.sum(axis=0)
    # Bk = diag(b e^gam) K ; Bv = diag(b) V
    eg = np.exp(gam)
    dK += (bc * eg)[:, None] * dBk
    dbeta += eg * np.sum(dBk * Kc, axis=1)
    dgam += np.sum(dBk * Bk, axis=1)
    dV = bc[:, None] * dBv
    dbeta += np.sum(dBv * Vc, axis=1)
    # Qt = diag(e^gam) Qs
    dQs = eg[:, None] * dQt
    dgam += np.sum(dQt * Qt, axis=1)
    # Kt = diag(e^{Gam - gam}) K
    eK = np.exp(Gam - gam)
    dK += eK[:, None] * dKt
    dKtKt = np.sum(dKt * Kt, axis=1)
    dgam -= dKtKt
    dGam = dKtKt.sum()
    # P = L * (Qs K^T)
    LdP = L * dP
    dQs += LdP @ Kc
    dK += LdP.T @ Qs
    dPP = dP * P
    dgam += dPP.sum(axis=1) - dPP.sum(axis=0)
    # S_new = e^Gam S + ...
    dGam += np.exp(Gam) * np.sum(G * S)
    dgam[-1] += dGam
    # gam = cumsum(g)
    dg = np.cumsum(dgam[::-1])[::-1]
    return dQs, dK, dV, dbeta, dg, G_prev


def chunked_bwd(q, k, v, g, beta, d_o, scale=1.0, initial_state=None, d_final_state=None,
                cu_seqlens=None, chunk=64):
    """Backward in WY form. Same returns as oracle.ref_bwd."""
    q, k, v, g, beta, d_o = (to_f64(x) for x in (q, k, v, g, beta, d_o))
    B, T, H, K = q.shape
    V = v.shape[-1]
    segs, N = _segments(B, T, cu_seqlens)
    s0 = to_f64(initial_state)
    dsT = to_f64(d_final_state)
    R = lambda x, d: x.reshape(B * T, H, d) if d else x.reshape(B * T, H)  # noqa: E731
    qf, kf, vf, dof = R(q, K), R(k, K), R(v, V), R(d_o, V)
    gf, bf = R(g, 0), R(beta, 0)
    dq, dk, dv = np.zeros_like(qf), np.zeros_like(kf), np.zeros_like(vf)
    dg, dbeta = np.zeros_like(gf), np.zeros_like(bf)
    ds0 = np.zeros((N, H, V, K))
    for n, bos, eos in segs:
        for h in range(H):
            S = np.zeros((V, K)) if s0 is None else s0[n, h].copy()
            its = []
            for t0 in range(bos, eos, chunk):
                t1 = min(t0 + chunk, eos)
                _, S, it = chunk_forward(scale * qf[t0:t1, h], kf[t0:t1, h], vf[t0:t1, h],
                                         gf[t0:t1, h], bf[t0:t1, h], S)
                its.append((t0, t1, it))
            G = np.zeros((V, K)) if dsT is None else dsT[n, h].copy()
            for t0, t1, it in reversed(its):
                dQs, dK, dV, dB, dG, G = chunk_backward(
                    it, scale * qf[t0:t1, h], kf[t0:t1, h], vf[t0:t1, h], bf[t0:t1, h],
                    dof[t0:t1, h], G)
                dq[t0:t1, h] = scale * dQs
                dk[t0:t1, h] = dK
                dv[t0:t1, h] = dV
                dbeta[t0:t1, h] = dB
                dg[t0:t1, h] = dG
            ds0[n, h] = G
    return dict(dq=dq.reshape(B, T, H, K), dk=dk.reshape(B, T, H, K), dv=dv.reshape(B, T, H, V),
                dg=dg.reshape(B, T, H), dbeta=dbeta.reshape(B, T, H), d_initial_state=ds0)
