"""Gated DeltaNet chunked prefill on AMD MI355X (gfx950): Python binding of libgdn.

The functions below carry the C ABI's names (include/gdn.h) and only marshal
torch tensors into it: device pointers, sizes and the current HIP stream.
Every step of the computation runs in the HIP library; if libgdn.so is
missing they raise instead of computing anything elsewhere.

  gdn_plan(...)               host-side plan (AutoCP decision, sub-sequence length, workspace)
  gdn_chunk_fwd(...)          O and the final state
  gdn_chunk_fwd_noalloc(...)  the same on the library's fixed scratch array (no allocation)
  gdn_chunk_bwd(...)          gradients of <dO, O> + <dS_T, S_T>
  gdn_workspace(...)          one buffer that serves a forward that keeps its intermediates
                              and the backward that reuses them
  gdn_cp_states(...)          the small buffer that carries the forward's CP decisions and
                              sub-sequence entry states to the backward
  gdn_intra_chunk(...)        the intra-chunk kernel alone (gate cumsum, w, u)
  gdn_cp_modes(...)           per sequence-head CP decision (0 none, 1 warmup, 2 exact, 3 mixed)
  gdn_cp_windows(...)         per-boundary CP decision (warmup window, or 0 for exact)
  gdn_recurrent_fwd(...)      token-by-token form from a given state (decoding after a prefill)
  chunk_gated_delta_rule(...) autograd wrapper over gdn_chunk_fwd / gdn_chunk_bwd
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np
import torch

from ._abi import (CP_MODES, EXPORTS, GDN_DTYPE_BF16, GDN_DTYPE_FP32, GDN_FLAG_BWD_ADJOINT_PASS,  # noqa: F401
                   GDN_FLAG_FWD_FUSED, GDN_FLAG_FWD_SPLIT, GDN_FLAG_KEEP_FORWARD, GDN_FLAG_QK_L2NORM, GDN_NOALLOC_SCRATCH_BYTES, GDN_FLAG_REUSE_FORWARD, GDN_FLAG_REUSE_CP, GdnDesc, GdnError, GdnKernelTime, GdnPlanInfo, check,
                   load_library, status_string)

__all__ = ["gdn_plan", "gdn_chunk_fwd", "gdn_chunk_fwd_noalloc", "gdn_chunk_bwd", "gdn_workspace", "gdn_cp_states", "gdn_intra_chunk", "gdn_cp_modes",
           "gdn_cp_windows", "gdn_recurrent_fwd", "gdn_profile_enable", "gdn_profile_read", "chunk_gated_delta_rule", "load_library",
           "make_desc", "GdnError"]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Desc:
    """A gdn_desc plus the host objects its pointers refer to."""

    def __init__(self, B, T, H, K, V, dtype, *, scale=1.0, cu_seqlens=None, cu_seqlens_host=None,
                 cp_mode="auto", warmup_chunks=0, seg_chunks=0, warmup_eps=0.0, num_cus=0, flags=0,
                 warmup_max_chunks=0, qk_l2norm=False, cp_states=None):
        d = GdnDesc()
        d.B, d.T, d.H, d.K, d.V = int(B), int(T), int(H), int(K), int(V)
        d.chunk = 64
        if dtype == torch.bfloat16:
            d.dtype = GDN_DTYPE_BF16
        elif dtype == torch.float32:
            d.dtype = GDN_DTYPE_FP32
        else:
            raise TypeError(f"unsupported input dtype {dtype} (bf16 or fp32)")
        d.scale = float(scale)
        self._host_cu = None
        self._dev_cu = None
        if cu_seqlens is not None:
            if cu_seqlens_host is None:
                cu_seqlens_host = cu_seqlens.detach().cpu()
            hc = np.ascontiguousarray(np.asarray(
                cu_seqlens_host.numpy() if hasattr(cu_seqlens_host, "numpy") else cu_seqlens_host,
                dtype=np.int32))
            self._host_cu = hc
            if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda:
                raise TypeError("cu_seqlens must be an int32 device tensor")
            self._dev_cu = cu_seqlens.contiguous()
            d.num_seqs = len(hc) - 1
            d.cu_seqlens = self._dev_cu.data_ptr()
            d.cu_seqlens_host = hc.ctypes.data
        d.cp_mode = CP_MODES[cp_mode] if isinstance(cp_mode, str) else int(cp_mode)
        d.warmup_chunks = int(warmup_chunks)
        d.warmup_max_chunks = int(warmup_max_chunks)
        d.seg_chunks = int(seg_chunks)
        d.warmup_eps = float(warmup_eps)
        d.num_cus = int(num_cus)
        d.flags = int(flags) | (GDN_FLAG_QK_L2NORM if qk_l2norm else 0)
        self._cp = cp_states
        if cp_states is not None:
            d.cp_states = cp_states.data_ptr()
        self.c = d

    @property
    def ref(self):
        return ctypes.byref(self.c)


def make_desc(q, v, **kw) -> Desc:
    B, T, H, K = q.shape
    return Desc(B, T, H, K, v.shape[-1], q.dtype, **kw)


def gdn_plan(desc: Desc) -> dict:
    info = GdnPlanInfo()
    check(load_library().gdn_plan(desc.ref, ctypes.byref(info)), "gdn_plan")
    return {f: getattr(info, f) for f, _ in GdnPlanInfo._fields_ if f != "reserved_out"}


def gdn_workspace(q, v, *, cu_seqlens=None, cu_seqlens_host=None, cp_mode="auto", warmup_chunks=0,
                  seg_chunks=0, warmup_eps=0.0, warmup_max_chunks=0, qk_l2norm=False):
    """A workspace large enough for gdn_chunk_fwd(keep_for_backward=True) and for
    gdn_chunk_bwd(reuse_forward=True) with the same shapes and options."""
    kw = dict(cu_seqlens=cu_seqlens, cu_seqlens_host=cu_seqlens_host, cp_mode=cp_mode,
              warmup_chunks=warmup_chunks, seg_chunks=seg_chunks, warmup_eps=warmup_eps,
              warmup_max_chunks=warmup_max_chunks, qk_l2norm=qk_l2norm)
    lib = load_library()
    f, b = ctypes.c_size_t(), ctypes.c_size_t()
    # the descriptors stay referenced through the calls: they own the host copy of cu_seqlens
    dk = make_desc(q, v, flags=GDN_FLAG_KEEP_FORWARD, **kw)
    dr = make_desc(q, v, flags=GDN_FLAG_REUSE_FORWARD, **kw)
    check(lib.gdn_chunk_fwd_workspace_size(dk.ref, ctypes.byref(f)), "gdn_chunk_fwd_workspace_size")
    check(lib.gdn_chunk_bwd_workspace_size(dr.ref, ctypes.byref(b)), "gdn_chunk_bwd_workspace_size")
    return torch.empty(max(f.value, b.value, 256), dtype=torch.uint8, device=q.device)


def gdn_cp_states(q, v, *, cu_seqlens=None, cu_seqlens_host=None, cp_mode="auto", warmup_chunks=0,
                  seg_chunks=0, warmup_eps=0.0, warmup_max_chunks=0, qk_l2norm=False):
    """The buffer (uint8 device tensor) in which gdn_chunk_fwd(cp_states=...) leaves its CP
    decisions and sub-sequence entry states for gdn_chunk_bwd(cp_states=...) on the same inputs and
    options; None when the plan has CP off (nothing to carry)."""
    desc = make_desc(q, v, cu_seqlens=cu_seqlens, cu_seqlens_host=cu_seqlens_host, cp_mode=cp_mode,
                     warmup_chunks=warmup_chunks, seg_chunks=seg_chunks, warmup_eps=warmup_eps,
                     warmup_max_chunks=warmup_max_chunks, qk_l2norm=qk_l2norm)
    nbytes = gdn_plan(desc)["cp_states_bytes"]
    return torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None


def _check_cp_states(cp_states, desc, device):
    """A caller's CP-state buffer: contiguous, on the inputs' device, 256-byte aligned and at least
    the plan's cp_states_bytes."""
    if cp_states is None:
        return
    if not isinstance(cp_states, torch.Tensor) or cp_states.device != torch.device(device):
        raise ValueError(f"cp_states must be a tensor on {device}")
    if not cp_states.is_contiguous() or cp_states.data_ptr() % 256:
        raise ValueError("cp_states must be contiguous and start at a 256-byte aligned address")
    need = gdn_plan(desc)["cp_states_bytes"]
    if cp_states.numel() * cp_states.element_size() < need:
        raise ValueError(f"cp_states too small: {need} bytes needed (gdn_cp_states)")


def _workspace(nbytes: int, device, workspace=None):
    """(workspace tensor, its size in bytes). A caller's workspace must be a contiguous tensor on
    the inputs' device whose first byte is 256-byte aligned; any element type (its size in bytes
    is what the library is told)."""
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.device != torch.device(device):
            raise ValueError(f"workspace must be a tensor on {device}")
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        if workspace.data_ptr() % 256:
            raise ValueError("workspace must start at a 256-byte aligned address")
        size = workspace.numel() * workspace.element_size()
        if size < nbytes:
            raise ValueError(f"workspace too small: {size} bytes, {nbytes} needed")
        return workspace, size
    ws = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    return ws, ws.numel()


def _check_buffer(name, t, shape, dtype, device):
    """A caller-supplied output (or upstream gradient) must be a contiguous tensor of exactly
    this shape and dtype on the inputs' device: the library writes through its pointer."""
    if t is None:
        return
    if (not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(shape) or t.dtype != dtype
            or t.device != device or not t.is_contiguous()):
        raise ValueError(f"{name}: expected a contiguous {tuple(shape)} {dtype} tensor on {device}")


def _check_inputs(q, k, v, g, beta, initial_state, N):
    B, T, H, K = q.shape
    V = v.shape[-1]
    dev = q.device
    if not q.is_cuda:
        raise ValueError("inputs must be device tensors")
    for name, t, shape in (("k", k, (B, T, H, K)), ("v", v, (B, T, H, V))):
        if tuple(t.shape) != shape or t.dtype != q.dtype or t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name}: expected contiguous {shape} {q.dtype} on {dev}")
    for name, t in (("g", g), ("beta", beta)):
        if tuple(t.shape) != (B, T, H) or t.dtype != torch.float32 or t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name}: expected contiguous fp32 {(B, T, H)} on {dev}")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if initial_state is not None:
        if (tuple(initial_state.shape) != (N, H, V, K) or initial_state.dtype != torch.float32
                or not initial_state.is_contiguous() or initial_state.device != dev):
            raise ValueError(f"initial_state: expected contiguous fp32 {(N, H, V, K)} on {dev}")


def _fused_flag(fused):
    return 0 if fused is None else (GDN_FLAG_FWD_FUSED if fused else GDN_FLAG_FWD_SPLIT)


def _num_seqs(q, cu_seqlens):
    return q.shape[0] if cu_seqlens is None else int(cu_seqlens.numel()) - 1


def gdn_chunk_fwd(q, k, v, g, beta, initial_state=None, *, scale=1.0, cu_seqlens=None,
                  cu_seqlens_host=None, output_final_state=True, cp_mode="auto", warmup_chunks=0,
                  seg_chunks=0, warmup_eps=0.0, warmup_max_chunks=0, workspace=None, o=None, final_state=None,
                  keep_for_backward=False, qk_l2norm=False, fused=None, cp_states=None):
    """Forward. Returns (o, final_state or None). Runs on the current stream.

    fused=None lets the plan choose between the two-kernel split and the fully fused forward;
    True asks for the fused one where it is supported (CP off, bf16, no kept intermediates), False
    for the split.

    qk_l2norm=True takes raw q and k and runs the path on their rows scaled to
    x / sqrt(sum x^2 + 1e-6) (normalised inside the kernels as they stage the rows).

    keep_for_backward=True leaves the intra-chunk results (gate cumsum, W, U, T), the CP
    decisions, the sub-sequence entry states, every chunk's entry state and Delta in `workspace`
    (required; see gdn_workspace), so that gdn_chunk_bwd(reuse_forward=True) on the same inputs
    and options skips recomputing them.

    cp_states (see gdn_cp_states): the forward writes its CP decisions and sub-sequence entry
    states there, for gdn_chunk_bwd(cp_states=...) to skip the forward CP preprocessing.
    """
    N = _num_seqs(q, cu_seqlens)
    _check_inputs(q, k, v, g, beta, initial_state, N)
    if keep_for_backward and workspace is None:
        raise ValueError("keep_for_backward needs a caller-owned workspace (gdn_workspace)")
    desc = make_desc(q, v, scale=scale, cu_seqlens=cu_seqlens, cu_seqlens_host=cu_seqlens_host,
                     cp_mode=cp_mode, warmup_chunks=warmup_chunks, seg_chunks=seg_chunks,
                     warmup_eps=warmup_eps, warmup_max_chunks=warmup_max_chunks, qk_l2norm=qk_l2norm,
                     flags=(GDN_FLAG_KEEP_FORWARD if keep_for_backward else 0) | _fused_flag(fused),
                     cp_states=cp_states)
    _check_cp_states(cp_states, desc, q.device)
    lib = load_library()
    nbytes = ctypes.c_size_t()
    check(lib.gdn_chunk_fwd_workspace_size(desc.ref, ctypes.byref(nbytes)), "gdn_chunk_fwd_workspace_size")
    ws, ws_bytes = _workspace(nbytes.value, q.device, workspace)
    B, T, H, K = q.shape
    V = v.shape[-1]
    if o is None:
        o = torch.empty((B, T, H, V), dtype=q.dtype, device=q.device)
    _check_buffer("o", o, (B, T, H, V), q.dtype, q.device)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, V, K), dtype=torch.float32, device=q.device)
    if not output_final_state:
        final_state = None
    _check_buffer("final_state", final_state, (N, H, V, K), torch.float32, q.device)
    check(lib.gdn_chunk_fwd(desc.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                            _ptr(o), _ptr(final_state), _ptr(ws), ctypes.c_size_t(ws_bytes), _stream()),
          "gdn_chunk_fwd")
    return o, final_state


def gdn_chunk_fwd_noalloc(q, k, v, g, beta, initial_state=None, *, scale=1.0, cu_seqlens=None,
                          cu_seqlens_host=None, output_final_state=True, cp_mode="auto", warmup_chunks=0,
                          seg_chunks=0, warmup_eps=0.0, warmup_max_chunks=0, o=None, final_state=None,
                          qk_l2norm=False):
    """Forward on the library's fixed per-GPU scratch array instead of a workspace (for callers
    that cannot allocate: pass `o` and `final_state` preallocated). Returns (o, final_state or None).
    Problems whose forward workspace exceeds GDN_NOALLOC_SCRATCH_BYTES raise GdnError (workspace).
    Calls that overlap on one GPU race on the shared array."""
    N = _num_seqs(q, cu_seqlens)
    _check_inputs(q, k, v, g, beta, initial_state, N)
    desc = make_desc(q, v, scale=scale, cu_seqlens=cu_seqlens, cu_seqlens_host=cu_seqlens_host,
                     cp_mode=cp_mode, warmup_chunks=warmup_chunks, seg_chunks=seg_chunks,
                     warmup_eps=warmup_eps, warmup_max_chunks=warmup_max_chunks, qk_l2norm=qk_l2norm)
    B, T, H, K = q.shape
    V = v.shape[-1]
    if o is None:
        o = torch.empty((B, T, H, V), dtype=q.dtype, device=q.device)
    _check_buffer("o", o, (B, T, H, V), q.dtype, q.device)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, V, K), dtype=torch.float32, device=q.device)
    if not output_final_state:
        final_state = None
    _check_buffer("final_state", final_state, (N, H, V, K), torch.float32, q.device)
    check(load_library().gdn_chunk_fwd_noalloc(desc.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                               _ptr(initial_state), _ptr(o), _ptr(final_state), _stream()),
          "gdn_chunk_fwd_noalloc")
    return o, final_state


def gdn_chunk_bwd(q, k, v, g, beta, d_o, initial_state=None, d_final_state=None, *, scale=1.0,
                  cu_seqlens=None, cu_seqlens_host=None, cp_mode="auto", warmup_chunks=0, seg_chunks=0,
                  warmup_eps=0.0, warmup_max_chunks=0, workspace=None, need_d_initial_state=True, out=None,
                  reuse_forward=False, qk_l2norm=False, adjoint_pass=False, cp_states=None):
    """Backward. Returns dict(dq, dk, dv, dg, dbeta, d_initial_state); `out` may hold them preallocated.

    qk_l2norm=True: the forward normalised q and k (see gdn_chunk_fwd); dq and dk are with respect
    to the raw q and k.

    reuse_forward=True takes the forward's intermediates from `workspace`, which must be the buffer a
    gdn_chunk_fwd(keep_for_backward=True) call on the same inputs and options wrote, untouched since.

    adjoint_pass=True runs the reverse adjoint recurrence as a separate pass (GDN_FLAG_BWD_ADJOINT_PASS)
    where the per-chunk kernel would otherwise carry the adjoint itself (for comparison).

    cp_states: the buffer a gdn_chunk_fwd(cp_states=...) on the same inputs and options filled; the
    backward takes the forward CP decisions and sub-sequence entry states from it (GDN_FLAG_REUSE_CP)
    instead of recomputing them.
    """
    N = _num_seqs(q, cu_seqlens)
    _check_inputs(q, k, v, g, beta, initial_state, N)
    B, T, H, K = q.shape
    V = v.shape[-1]
    if d_o is None:
        raise ValueError("d_o is required")
    _check_buffer("d_o", d_o, (B, T, H, V), q.dtype, q.device)
    _check_buffer("d_final_state", d_final_state, (N, H, V, K), torch.float32, q.device)
    if reuse_forward and workspace is None:
        raise ValueError("reuse_forward needs the forward's workspace")
    desc = make_desc(q, v, scale=scale, cu_seqlens=cu_seqlens, cu_seqlens_host=cu_seqlens_host,
                     cp_mode=cp_mode, warmup_chunks=warmup_chunks, seg_chunks=seg_chunks,
                     warmup_eps=warmup_eps, warmup_max_chunks=warmup_max_chunks, qk_l2norm=qk_l2norm,
                     flags=(GDN_FLAG_REUSE_FORWARD if reuse_forward else 0)
                     | (GDN_FLAG_BWD_ADJOINT_PASS if adjoint_pass else 0)
                     | (GDN_FLAG_REUSE_CP if cp_states is not None else 0),
                     cp_states=cp_states)
    _check_cp_states(cp_states, desc, q.device)
    lib = load_library()
    nbytes = ctypes.c_size_t()
    check(lib.gdn_chunk_bwd_workspace_size(desc.ref, ctypes.byref(nbytes)), "gdn_chunk_bwd_workspace_size")
    ws, ws_bytes = _workspace(nbytes.value, q.device, workspace)
    if out is None:
        out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                   dg=torch.empty_like(g), dbeta=torch.empty_like(beta),
                   d_initial_state=(torch.empty((N, H, V, K), dtype=torch.float32, device=q.device)
                                    if need_d_initial_state else None))
    shapes = dict(dq=((B, T, H, K), q.dtype), dk=((B, T, H, K), q.dtype), dv=((B, T, H, V), q.dtype),
                  dg=((B, T, H), torch.float32), dbeta=((B, T, H), torch.float32),
                  d_initial_state=((N, H, V, K), torch.float32))
    for name, (shape, dt) in shapes.items():
        if name not in out or (out[name] is None and name != "d_initial_state"):
            raise ValueError(f"out[{name!r}] is required")
        _check_buffer(f"out[{name!r}]", out[name], shape, dt, q.device)
    check(lib.gdn_chunk_bwd(desc.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                            _ptr(d_o), _ptr(d_final_state), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                            _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["d_initial_state"]),
                            _ptr(ws), ctypes.c_size_t(ws_bytes), _stream()),
          "gdn_chunk_bwd")
    return out


def gdn_intra_chunk(k, v, g, beta, *, cu_seqlens=None, cu_seqlens_host=None, qk_l2norm=False):
    """The intra-chunk kernel alone: returns (gam [B,T,H] fp32, w [B,T,H,K], u [B,T,H,V]).
    qk_l2norm=True normalises the k rows first."""
    B, T, H, K = k.shape
    desc = make_desc(k, v, cu_seqlens=cu_seqlens, cu_seqlens_host=cu_seqlens_host, qk_l2norm=qk_l2norm)
    lib = load_library()
    nbytes = ctypes.c_size_t()
    check(lib.gdn_chunk_fwd_workspace_size(desc.ref, ctypes.byref(nbytes)), "gdn_chunk_fwd_workspace_size")
    ws, ws_bytes = _workspace(nbytes.value, k.device)
    gam = torch.empty((B, T, H), dtype=torch.float32, device=k.device)
    w = torch.empty_like(k)
    u = torch.empty_like(v)
    check(lib.gdn_intra_chunk(desc.ref, _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(gam), _ptr(w), _ptr(u),
                              _ptr(ws), ctypes.c_size_t(ws_bytes), _stream()), "gdn_intra_chunk")
    return gam, w, u


def gdn_cp_modes(k, v, g, beta, *, cu_seqlens=None, cu_seqlens_host=None, cp_mode="auto",
                 warmup_chunks=0, seg_chunks=0, warmup_eps=0.0, warmup_max_chunks=0, qk_l2norm=False):
    """Per sequence-head CP decision [N, H] int32: 0 no split, 1 every boundary warmup, 2 every
    boundary exact, 3 mixed."""
    N = _num_seqs(k, cu_seqlens)
    desc = make_desc(k, v, cu_seqlens=cu_seqlens, cu_seqlens_host=cu_seqlens_host, cp_mode=cp_mode,
                     warmup_chunks=warmup_chunks, seg_chunks=seg_chunks, warmup_eps=warmup_eps,
                     warmup_max_chunks=warmup_max_chunks, qk_l2norm=qk_l2norm)
    lib = load_library()
    nbytes = ctypes.c_size_t()
    check(lib.gdn_chunk_fwd_workspace_size(desc.ref, ctypes.byref(nbytes)), "gdn_chunk_fwd_workspace_size")
    ws, ws_bytes = _workspace(nbytes.value, k.device)
    modes = torch.empty((N, k.shape[2]), dtype=torch.int32, device=k.device)
    check(lib.gdn_cp_modes(desc.ref, _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(modes), _ptr(ws),
                           ctypes.c_size_t(ws_bytes), _stream()), "gdn_cp_modes")
    return modes


def gdn_cp_windows(k, v, g, beta, *, cu_seqlens=None, cu_seqlens_host=None, cp_mode="auto", warmup_chunks=0,
                   seg_chunks=0, warmup_eps=0.0, warmup_max_chunks=0, qk_l2norm=False, reverse=True):
    """Per-boundary CP decision: (fwd, rev) int32 [total_segments, H] device tensors, row gs for the
    boundary at the start of sub-sequence gs: the warmup window in chunks, 0 = exact, -1 = no
    boundary (a sequence's first sub-sequence). rev (the backward's adjoint pass) is None unless
    reverse=True."""
    desc = make_desc(k, v, cu_seqlens=cu_seqlens, cu_seqlens_host=cu_seqlens_host, cp_mode=cp_mode,
                     warmup_chunks=warmup_chunks, seg_chunks=seg_chunks, warmup_eps=warmup_eps,
                     warmup_max_chunks=warmup_max_chunks, qk_l2norm=qk_l2norm)
    lib = load_library()
    plan = gdn_plan(desc)
    ws, ws_bytes = _workspace(plan["fwd_workspace_bytes"], k.device)
    shape = (plan["total_segments"], k.shape[2])
    fwd = torch.empty(shape, dtype=torch.int32, device=k.device)
    rev = torch.empty(shape, dtype=torch.int32, device=k.device) if reverse else None
    check(lib.gdn_cp_windows(desc.ref, _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(fwd), _ptr(rev), _ptr(ws),
                             ctypes.c_size_t(ws_bytes), _stream()), "gdn_cp_windows")
    return fwd, rev


def gdn_recurrent_fwd(q, k, v, g, beta, state=None, *, scale=1.0, state_out=None, o=None, qk_l2norm=False):
    """Recurrent form (decode): the gated delta rule token by token from `state`.

    q, k [B,T,H,K], v [B,T,H,V], g, beta [B,T,H] as in gdn_chunk_fwd (no cu_seqlens); state
    [B,H,V,K] fp32 or None (zeros), e.g. the final state of gdn_chunk_fwd. Returns (o,
    state_out); state_out may be `state` itself (updated in place). Runs on the current stream.
    qk_l2norm=True takes raw q and k rows and normalises them as gdn_chunk_fwd(qk_l2norm=True) does.
    """
    B, T, H, K = q.shape
    V = v.shape[-1]
    _check_inputs(q, k, v, g, beta, state, B)
    if state_out is None:
        state_out = torch.empty((B, H, V, K), dtype=torch.float32, device=q.device)
    elif (tuple(state_out.shape) != (B, H, V, K) or state_out.dtype != torch.float32
          or not state_out.is_contiguous() or state_out.device != q.device):
        raise ValueError(f"state_out: expected contiguous fp32 {(B, H, V, K)} on {q.device}")
    if o is None:
        o = torch.empty((B, T, H, V), dtype=q.dtype, device=q.device)
    _check_buffer("o", o, (B, T, H, V), q.dtype, q.device)
    desc = make_desc(q, v, scale=scale, qk_l2norm=qk_l2norm)
    check(load_library().gdn_recurrent_fwd(desc.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                           _ptr(state), _ptr(state_out), _ptr(o), _stream()),
          "gdn_recurrent_fwd")
    return o, state_out


def gdn_profile_enable(enable: bool = True) -> None:
    """Bracket every kernel launch with HIP events (see gdn_profile_read)."""
    check(load_library().gdn_profile_enable(int(bool(enable))), "gdn_profile_enable")


def gdn_profile_read() -> dict:
    """Wait for the recorded events; return {kernel: (launches, total_ms)} and clear the totals."""
    buf = (GdnKernelTime * 32)()
    n = load_library().gdn_profile_read(buf, 32)
    if n < 0:
        raise GdnError(4, "gdn_profile_read")
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(n)}


class _GDNFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, g, beta, initial_state, scale, cu_seqlens, cu_host, cp_mode, keep, l2, carry_cp):
        # one host copy of cu_seqlens for every call of the step (planning reads the host copy;
        # taking it from the device would synchronise once per call)
        if cu_seqlens is not None and cu_host is None:
            cu_host = cu_seqlens.detach().cpu()
        cu = dict(cu_seqlens=cu_seqlens, cu_seqlens_host=cu_host)
        ws = gdn_workspace(q, v, cp_mode=cp_mode, qk_l2norm=l2, **cu) if keep else None
        # with carry_cp the CP decisions and sub-sequence entry states (a few MB) go to the
        # backward, which then skips the forward CP preprocessing; with keep, the workspace
        # carries them already
        cps = gdn_cp_states(q, v, cp_mode=cp_mode, qk_l2norm=l2, **cu) if carry_cp and not keep else None
        o, sT = gdn_chunk_fwd(q, k, v, g, beta, initial_state, scale=scale, cp_mode=cp_mode, workspace=ws,
                              keep_for_backward=keep, qk_l2norm=l2, cp_states=cps, **cu)
        ctx.save_for_backward(q, k, v, g, beta, initial_state, cu_seqlens)
        ctx.cu_host = cu_host
        ctx.scale = scale
        ctx.cp_mode = cp_mode
        ctx.l2 = l2
        ctx.ws = ws
        ctx.cps = cps
        return o, sT

    @staticmethod
    def backward(ctx, d_o, d_sT):
        q, k, v, g, beta, s0, cu = ctx.saved_tensors
        ws, ctx.ws = ctx.ws, None
        cps, ctx.cps = ctx.cps, None
        gr = gdn_chunk_bwd(q, k, v, g, beta, d_o.contiguous(), s0,
                           None if d_sT is None else d_sT.contiguous(), scale=ctx.scale,
                           cu_seqlens=cu, cu_seqlens_host=ctx.cu_host, cp_mode=ctx.cp_mode,
                           need_d_initial_state=s0 is not None, workspace=ws, reuse_forward=ws is not None,
                           qk_l2norm=ctx.l2, cp_states=cps)
        return (gr["dq"], gr["dk"], gr["dv"], gr["dg"], gr["dbeta"], gr["d_initial_state"],
                None, None, None, None, None, None, None)


def chunk_gated_delta_rule(q, k, v, g, beta, scale: float = 1.0, initial_state=None,
                           output_final_state: bool = True, cu_seqlens=None, cp_mode: str = "auto",
                           keep_intermediates: bool = False, qk_l2norm: bool = False, cu_seqlens_host=None,
                           carry_cp_states: bool = False):
    """High-level call: (o, final_state) with autograd through gdn_chunk_bwd.

    q, k: [B,T,H,K]; v: [B,T,H,V] (bf16 or fp32); g (natural-log decay) and beta: [B,T,H] fp32;
    initial_state: [N,H,V,K] fp32 or None; cu_seqlens: int32 [N+1] device tensor (B must be 1), with
    cu_seqlens_host its host copy if the caller has one (else one device-to-host copy per forward,
    kept for the backward).
    keep_intermediates=True holds the forward's workspace (W, U, T, gate cumsum, CP entry states,
    chunk states and Delta) until the backward, which then skips recomputing them: more memory,
    less backward time. carry_cp_states=True keeps only the forward's CP decisions and sub-sequence
    entry states (gdn_cp_states: fp32 [segments, H, V, K], 16 MB at B=1 H=16 T=32K) for the
    backward, which then skips the forward CP preprocessing and recomputes the rest. qk_l2norm=True normalises q and k rows inside the library
    (x / sqrt(sum x^2 + 1e-6)); gradients flow to the raw q and k.
    """
    grad = torch.is_grad_enabled() and any(x is not None and x.requires_grad
                                           for x in (q, k, v, g, beta, initial_state))
    o, sT = _GDNFunction.apply(q, k, v, g, beta, initial_state, scale, cu_seqlens, cu_seqlens_host, cp_mode,
                               bool(keep_intermediates and grad), bool(qk_l2norm), bool(carry_cp_states and grad))
    return (o, sT) if output_final_state else (o, None)
