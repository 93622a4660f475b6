"""q/k L2 normalisation over the key dimension, the optional step ahead of the path --
TEST INFRASTRUCTURE ONLY (imported by the tests, the smoke check and the benchmark's
CPU-baseline leg; the GPU library never calls it).

The pages place preprocessing ahead of the fused kernels (edge.aivizor.me community post,
its account of the FLA chunked-prefill pipeline: gate preprocessing comes first) and
their workloads use unit-norm query and key rows; they print no formula for the
normalisation. Reading taken: each row x of q and of k (one token, one head, K values)
becomes x / sqrt(sum_i x_i^2 + eps) with eps = 1e-6, the eps keeping an all-zero row
finite. Its reverse mode follows from d(x r) with r = (sum x^2 + eps)^(-1/2):
dx = r (dy - xhat (xhat . dy)), xhat = x r.

ref_fwd_l2 / ref_bwd_l2 compose it with the fp64 oracle of the gated delta rule.
"""
from __future__ import annotations

import numpy as np

from .oracle import ref_bwd, ref_fwd, to_f64

L2_EPS = 1e-6


def l2norm(x, eps=L2_EPS):
    """Rows over the last axis scaled to (nearly) unit L2 norm, fp64."""
    x = to_f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def l2norm_bwd(x, dy, eps=L2_EPS):
    """Gradient with respect to the raw rows x, given dy = dL/d(l2norm(x)), fp64."""
    x, dy = to_f64(x), to_f64(dy)
    r = 1.0 / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)
    xh = x * r
    return r * (dy - xh * np.sum(xh * dy, axis=-1, keepdims=True))


def ref_fwd_l2(q, k, v, g, beta, scale=1.0, initial_state=None, cu_seqlens=None, eps=L2_EPS,
               nthreads=None):
    """Forward oracle on raw q, k: the gated delta rule on l2norm(q), l2norm(k)."""
    return ref_fwd(l2norm(q, eps), l2norm(k, eps), v, g, beta, scale, initial_state, cu_seqlens,
                   nthreads=nthreads)


def ref_bwd_l2(q, k, v, g, beta, d_o, scale=1.0, initial_state=None, d_final_state=None,
               cu_seqlens=None, eps=L2_EPS, nthreads=None):
    """Reverse mode of ref_fwd_l2: the oracle's gradients on the normalised rows, with dq and
    dk taken back through the normalisation to the raw q and k."""
    out = ref_bwd(l2norm(q, eps), l2norm(k, eps), v, g, beta, d_o, scale, initial_state,
                  d_final_state, cu_seqlens, nthreads=nthreads)
    out["dq"] = l2norm_bwd(q, out["dq"], eps)
    out["dk"] = l2norm_bwd(k, out["dk"], eps)
    return out
