"""CPU oracle for Gated DeltaNet chunked prefill -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module. The GPU library never calls it and shares no code with it.

`ref_fwd` / `ref_bwd` wrap the fp64 C token loop in gdn_oracle.c: the gated
delta rule S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
o_t = scale S_t q_t, and its hand-derived reverse mode. The pages that name
the method (FlashQLA: ollai.cn article, sections "main features" and
"how to use") state the inputs q, k, v, g, beta, the outputs O and the final
state, and the optional initial_state and cu_seqlens; they print no formula.

Inputs may be numpy arrays or torch tensors of any float dtype; they are
upcast exactly to fp64 (bf16 and fp32 values are representable in fp64), so
input quantisation is never counted as error.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int64)


def _lib():
    global _LIB
    if _LIB is None:
        path = _build.ensure_built()
        lib = ctypes.CDLL(path)
        lib.gdn_oracle_fwd.restype = ctypes.c_int
        lib.gdn_oracle_fwd.argtypes = [ctypes.c_int64, _ip, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, _dp, _dp, _dp, _dp, _dp, ctypes.c_double,
                                       _dp, _dp, _dp, ctypes.c_int]
        lib.gdn_oracle_bwd.restype = ctypes.c_int
        lib.gdn_oracle_bwd.argtypes = [ctypes.c_int64, _ip, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, _dp, _dp, _dp, _dp, _dp, ctypes.c_double,
                                       _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int]
        lib.gdn_oracle_num_threads.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def default_threads() -> int:
    """Threads the oracle uses: the CPUs this process may run on, capped by OMP_NUM_THREADS."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def to_f64(x):
    """Exact upcast of a numpy array or torch tensor to a C-contiguous fp64 array."""
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def _offsets(B, T, cu_seqlens):
    if cu_seqlens is None:
        return np.arange(B + 1, dtype=np.int64) * T
    if B != 1:
        raise ValueError("cu_seqlens requires B == 1")
    if hasattr(cu_seqlens, "detach"):
        cu_seqlens = cu_seqlens.detach().cpu().numpy()
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, end at T and not decrease")
    return cu


def ref_fwd(q, k, v, g, beta, scale=1.0, initial_state=None, cu_seqlens=None,
            nthreads=None):
    """Forward oracle. q, k: [B,T,H,K]; v: [B,T,H,V]; g, beta: [B,T,H];
    initial_state: [N,H,V,K] or None (zeros); cu_seqlens: [N+1] or None.

    Returns (o [B,T,H,V], final_state [N,H,V,K]) in fp64.
    """
    q, k, v, g, beta = (to_f64(x) for x in (q, k, v, g, beta))
    B, T, H, K = q.shape
    V = v.shape[-1]
    cu = _offsets(B, T, cu_seqlens)
    N = len(cu) - 1
    s0 = to_f64(initial_state)
    if s0 is not None and s0.shape != (N, H, V, K):
        raise ValueError(f"initial_state shape {s0.shape} != {(N, H, V, K)}")
    o = np.zeros((B, T, H, V))
    sT = np.zeros((N, H, V, K))
    rc = _lib().gdn_oracle_fwd(N, cu.ctypes.data_as(_ip), H, K, V, _ptr(q), _ptr(k), _ptr(v),
                               _ptr(g), _ptr(beta), float(scale), _ptr(s0), _ptr(o), _ptr(sT),
                               nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"gdn_oracle_fwd failed ({rc})")
    return o, sT


def ref_bwd(q, k, v, g, beta, d_o, scale=1.0, initial_state=None, d_final_state=None,
            cu_seqlens=None, nthreads=None):
    """Reverse-mode oracle for L = <dO, O> + <dS_T, S_T>.

    Returns a dict of fp64 arrays: dq, dk [B,T,H,K]; dv [B,T,H,V];
    dg, dbeta [B,T,H]; d_initial_state [N,H,V,K].
    """
    q, k, v, g, beta, d_o = (to_f64(x) for x in (q, k, v, g, beta, d_o))
    B, T, H, K = q.shape
    V = v.shape[-1]
    cu = _offsets(B, T, cu_seqlens)
    N = len(cu) - 1
    s0 = to_f64(initial_state)
    dsT = to_f64(d_final_state)
    out = dict(dq=np.zeros((B, T, H, K)), dk=np.zeros((B, T, H, K)), dv=np.zeros((B, T, H, V)),
               dg=np.zeros((B, T, H)), dbeta=np.zeros((B, T, H)),
               d_initial_state=np.zeros((N, H, V, K)))
    rc = _lib().gdn_oracle_bwd(N, cu.ctypes.data_as(_ip), H, K, V, _ptr(q), _ptr(k), _ptr(v),
                               _ptr(g), _ptr(beta), float(scale), _ptr(s0), _ptr(d_o), _ptr(dsT),
                               _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
                               _ptr(out["dbeta"]), _ptr(out["d_initial_state"]),
                               nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"gdn_oracle_bwd failed ({rc})")
    return out


def rel_l2(x, ref) -> float:
    """||x - ref||_2 / ||ref||_2 over the whole tensor (0 if both are zero)."""
    x = to_f64(x)
    ref = to_f64(ref)
    den = float(np.linalg.norm(ref.ravel()))
    num = float(np.linalg.norm((x - ref).ravel()))
    if den == 0.0:
        return num
    return num / den
