"""libgdn: the gated delta rule on AMD MI355X (gfx950), called through its C ABI.

The three entry points mirror ``include/gdn.h``:

  chunk_fwd(q, k, v, beta, log_alpha, s0=None, chunk=64, cu_seqlens=None)
      -> (o, s_final)
  chunk_bwd(q, k, v, beta, log_alpha, s0, d_o, ds_final=None, chunk=64,
            cu_seqlens=None) -> (dq, dk, dv, dbeta, dlog_alpha, ds0)
  decode_step(q, k, v, beta, log_alpha, state) -> o   (state updated in place)

Tensors are torch CUDA tensors (HIP device memory); torch is used only to
allocate outputs / workspaces and to name the current stream.  The gate mode
follows ``log_alpha``: None = no decay (delta rule), one value per
(token, head) = scalar gate, one value per key channel = per-channel gate.
"""

from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import GdnError  # noqa: F401

__all__ = ["chunk_fwd", "chunk_bwd", "decode_step", "decode_step_product",
           "chunk_fwd_product", "tree_verify",
           "tree_commit", "FwdPlan", "GdnError", "set_segment_chunks",
           "abi_version", "stage_times"]

_DT = {torch.float32: _lib.GDN_F32, torch.bfloat16: _lib.GDN_BF16}


def abi_version() -> int:
    return _lib.load().gdn_abi_version()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("libgdn takes contiguous tensors")
    return t.data_ptr() or None


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _gate_of(log_alpha, token_dims: int) -> int:
    if log_alpha is None:
        return _lib.GDN_GATE_NONE
    return _lib.GDN_GATE_CHANNEL if log_alpha.dim() == token_dims + 1 else _lib.GDN_GATE_SCALAR


def _problem(q, v, beta, log_alpha, chunk, cu_seqlens, gate=None):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    nseq = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    p = _lib.GdnProblem()
    p.B, p.T, p.H, p.dk, p.dv, p.chunk = B, T, H, dk, dv, chunk
    p.nseq = nseq
    p.cu_seqlens = None if cu_seqlens is None else cu_seqlens.data_ptr()
    p.io_dtype = _dtype_code(q)
    p.gate_dtype = _dtype_code(beta)
    p.gate = _gate_of(log_alpha, 3) if gate is None else gate
    return p


def _check_cu(cu_seqlens, q):
    if cu_seqlens is None:
        return
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != q.device:
        raise ValueError("cu_seqlens must be an int32 tensor on the inputs' device")


def chunk_fwd(q, k, v, beta, log_alpha=None, s0=None, chunk: int = 64,
              cu_seqlens=None, output_final_state: bool = True,
              workspace: Optional[torch.Tensor] = None, qk_l2norm: bool = False):
    """Chunkwise forward.  Returns (o, s_final or None).  qk_l2norm: q and k
    rows are L2-normalised inside the kernels (gdn_chunk_fwd_qknorm)."""
    lib = _lib.load()
    _check_cu(cu_seqlens, q)
    p = _problem(q, v, beta, log_alpha, chunk, cu_seqlens)
    nseq = q.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1
    H, dk, dv = q.shape[2], q.shape[3], v.shape[3]
    o = torch.empty(v.shape, dtype=q.dtype, device=q.device)
    sf = (torch.empty((nseq, H, dk, dv), dtype=torch.float32, device=q.device)
          if output_final_state else None)
    need = ctypes.c_size_t(0)
    _lib.check(lib.gdn_chunk_fwd_workspace(ctypes.byref(p), ctypes.byref(need)),
               "gdn_chunk_fwd_workspace")
    ws = workspace
    if ws is None or ws.numel() < need.value:
        ws = torch.empty(max(need.value, 1), dtype=torch.uint8, device=q.device)
    fn, name = ((lib.gdn_chunk_fwd_qknorm, "gdn_chunk_fwd_qknorm") if qk_l2norm
                else (lib.gdn_chunk_fwd, "gdn_chunk_fwd"))
    st = fn(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
            _ptr(log_alpha), _ptr(s0), _ptr(o), _ptr(sf),
            _ptr(ws), ws.numel(), _stream(q.device))
    _lib.check(st, name)
    return o, sf


def chunk_fwd_product(q, k, v, beta, log_alpha=None, s0=None, chunk: int = 64,
                      cu_seqlens=None, output_final_state: bool = True):
    """Householder-product forward (gdn_chunk_fwd_product): k [B,T,nh,H,dk],
    v [B,T,nh,H,dv], beta [B,T,nh,H], q [B,T,H,dk], log_alpha [B,T,H] or None.
    Returns (o [B,T,H,dv], s_final or None)."""
    lib = _lib.load()
    _check_cu(cu_seqlens, q)
    nh = k.shape[2]
    H, dk, dv = q.shape[2], q.shape[3], v.shape[-1]
    p = _problem(q, v, beta, log_alpha, chunk, cu_seqlens)
    nseq = q.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1
    o = torch.empty(q.shape[:3] + (dv,), dtype=q.dtype, device=q.device)
    sf = (torch.empty((nseq, H, dk, dv), dtype=torch.float32, device=q.device)
          if output_final_state else None)
    need = ctypes.c_size_t(0)
    _lib.check(lib.gdn_chunk_fwd_product_workspace(ctypes.byref(p), nh, ctypes.byref(need)),
               "gdn_chunk_fwd_product_workspace")
    ws = torch.empty(max(need.value, 1), dtype=torch.uint8, device=q.device)
    st = lib.gdn_chunk_fwd_product(ctypes.byref(p), nh, _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                   _ptr(log_alpha), _ptr(s0), _ptr(o), _ptr(sf),
                                   _ptr(ws), ws.numel(), _stream(q.device))
    _lib.check(st, "gdn_chunk_fwd_product")
    return o, sf


def _check_tree_index(t, name, q):
    if t.dtype != torch.int32 or t.device != q.device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor on the inputs' device")


def decode_step_product(q, k, v, beta, log_alpha, state):
    """One token per sequence with nh delta steps (gdn_decode_step_product):
    q [N, H, dk], k [N, nh, H, dk], v [N, nh, H, dv], beta [N, nh, H],
    log_alpha [N, H] or None; ``state`` [N, H, dk, dv] fp32 is updated in
    place.  Returns o [N, H, dv]."""
    lib = _lib.load()
    N, H, dk = q.shape
    nh, dv = k.shape[1], v.shape[-1]
    p = _lib.GdnProblem()
    p.B, p.T, p.H, p.dk, p.dv, p.chunk, p.nseq = N, 1, H, dk, dv, 0, 0
    p.cu_seqlens = None
    p.io_dtype = _dtype_code(q)
    p.gate_dtype = _dtype_code(beta)
    p.gate = _gate_of(log_alpha, 2)
    if state.dtype != torch.float32:
        raise TypeError("state must be fp32")
    o = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    st = lib.gdn_decode_step_product(ctypes.byref(p), nh, _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(beta), _ptr(log_alpha), _ptr(state), _ptr(o),
                                     _stream(q.device))
    _lib.check(st, "gdn_decode_step_product")
    return o


def tree_verify_workspace(q, v, beta, log_alpha=None, chunk: int = 64,
                          cu_seqlens=None) -> int:
    """Workspace bytes of tree_verify for these inputs."""
    lib = _lib.load()
    p = _problem(q, v, beta, log_alpha, chunk, cu_seqlens)
    need = ctypes.c_size_t(0)
    _lib.check(lib.gdn_tree_verify_workspace(ctypes.byref(p), ctypes.byref(need)),
               "gdn_tree_verify_workspace")
    return need.value


def tree_verify(q, k, v, beta, log_alpha, parent, state=None, chunk: int = 64,
                cu_seqlens=None, workspace: Optional[torch.Tensor] = None):
    """Outputs of every node of draft trees (gdn_tree_verify).  q, k [B,n,H,dk],
    v [B,n,H,dv], beta [B,n,H], log_alpha [B,n,H] or None; parent int32
    [B,n] (or [total] with cu_seqlens), parents inside each tree, -1 = the
    committed state; state [ntrees,H,dk,dv] fp32 (read only) or None.
    Returns o [B,n,H,dv]."""
    lib = _lib.load()
    _check_cu(cu_seqlens, q)
    _check_tree_index(parent, "parent", q)
    p = _problem(q, v, beta, log_alpha, chunk, cu_seqlens)
    o = torch.empty(v.shape, dtype=q.dtype, device=q.device)
    need = ctypes.c_size_t(0)
    _lib.check(lib.gdn_tree_verify_workspace(ctypes.byref(p), ctypes.byref(need)),
               "gdn_tree_verify_workspace")
    ws = workspace
    if ws is None or ws.numel() < need.value:
        ws = torch.empty(max(need.value, 1), dtype=torch.uint8, device=q.device)
    st = lib.gdn_tree_verify(ctypes.byref(p), _ptr(parent), _ptr(q), _ptr(k), _ptr(v),
                             _ptr(beta), _ptr(log_alpha), _ptr(state), _ptr(o),
                             _ptr(ws), ws.numel(), _stream(q.device))
    _lib.check(st, "gdn_tree_verify")
    return o


def tree_commit(k, v, beta, log_alpha, parent, accepted, state, chunk: int = 64,
                cu_seqlens=None):
    """In place: state[m] becomes the state of node accepted[m] of tree m
    (gdn_tree_commit); accepted[m] = -1 keeps it.  Shapes as tree_verify;
    accepted int32 [ntrees].  Returns state."""
    lib = _lib.load()
    _check_cu(cu_seqlens, k)
    _check_tree_index(parent, "parent", k)
    _check_tree_index(accepted, "accepted", k)
    p = _problem(k, v, beta, log_alpha, chunk, cu_seqlens)
    st = lib.gdn_tree_commit(ctypes.byref(p), _ptr(parent), _ptr(accepted), _ptr(k),
                             _ptr(v), _ptr(beta), _ptr(log_alpha), _ptr(state),
                             _stream(k.device))
    _lib.check(st, "gdn_tree_commit")
    return state


class FwdPlan:
    """A forward call with its outputs and workspace allocated once.

    ``run()`` enqueues gdn_chunk_fwd on the stream that was current when the
    plan was made, with cached pointers: the input tensors may be refilled in
    place between runs, and ``o`` / ``s_final`` are overwritten each time.
    This keeps the host cost of a call to one ctypes call."""

    def __init__(self, q, k, v, beta, log_alpha=None, s0=None, chunk: int = 64,
                 cu_seqlens=None, output_final_state: bool = True,
                 qk_l2norm: bool = False):
        lib = _lib.load()
        _check_cu(cu_seqlens, q)
        self._keep = (q, k, v, beta, log_alpha, s0, cu_seqlens)
        self.problem = _problem(q, v, beta, log_alpha, chunk, cu_seqlens)
        nseq = q.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1
        H, dk, dv = q.shape[2], q.shape[3], v.shape[3]
        self.o = torch.empty(v.shape, dtype=q.dtype, device=q.device)
        self.s_final = (torch.empty((nseq, H, dk, dv), dtype=torch.float32,
                                    device=q.device) if output_final_state else None)
        need = ctypes.c_size_t(0)
        _lib.check(lib.gdn_chunk_fwd_workspace(ctypes.byref(self.problem),
                                               ctypes.byref(need)),
                   "gdn_chunk_fwd_workspace")
        self.workspace = torch.empty(max(need.value, 1), dtype=torch.uint8,
                                     device=q.device)
        self._name = "gdn_chunk_fwd_qknorm" if qk_l2norm else "gdn_chunk_fwd"
        self._fn = getattr(lib, self._name)
        self._args = (ctypes.byref(self.problem), _ptr(q), _ptr(k), _ptr(v),
                      _ptr(beta), _ptr(log_alpha), _ptr(s0), _ptr(self.o),
                      _ptr(self.s_final), _ptr(self.workspace),
                      self.workspace.numel(), _stream(q.device))

    def run(self):
        st = self._fn(*self._args)
        if st != _lib.GDN_OK:
            _lib.check(st, self._name)
        return self.o, self.s_final


def stage_times(enable: Optional[bool] = None):
    """Stage timing hook of the library.  ``stage_times(True)`` starts
    recording HIP events around every kernel launch, ``stage_times(False)``
    stops; ``stage_times()`` waits for the recorded events and returns
    {stage: (total_ms, launches)} for the stages that ran, then clears."""
    lib = _lib.load()
    if enable is not None:
        lib.gdn_profile_enable(1 if enable else 0)
        return None
    ms = (ctypes.c_double * _lib.STAGE_COUNT)()
    cnt = (ctypes.c_int32 * _lib.STAGE_COUNT)()
    _lib.check(lib.gdn_profile_read(ms, cnt), "gdn_profile_read")
    return {_lib.STAGES[i]: (ms[i], cnt[i]) for i in range(_lib.STAGE_COUNT)
            if cnt[i] > 0}


def set_segment_chunks(n: int) -> None:
    """Segment length of the forward state pass, process-wide: 0 automatic
    (default), n > 0 segments of n chunks, n < 0 never split sequences.  A
    FwdPlan sizes its workspace when it is built, so build plans after
    changing this."""
    _lib.load().gdn_set_segment_chunks(int(n))


def fwd_workspace_bytes(q, v, beta, log_alpha=None, chunk=64, cu_seqlens=None) -> int:
    lib = _lib.load()
    p = _problem(q, v, beta, log_alpha, chunk, cu_seqlens)
    need = ctypes.c_size_t(0)
    _lib.check(lib.gdn_chunk_fwd_workspace(ctypes.byref(p), ctypes.byref(need)),
               "gdn_chunk_fwd_workspace")
    return need.value


def chunk_bwd(q, k, v, beta, log_alpha, s0, d_o, ds_final=None,
              chunk: int = 64, cu_seqlens=None, need_ds0: bool = True,
              workspace: Optional[torch.Tensor] = None):
    """Chunkwise backward.  Returns (dq, dk, dv, dbeta, dlog_alpha, ds0)."""
    lib = _lib.load()
    _check_cu(cu_seqlens, q)
    p = _problem(q, v, beta, log_alpha, chunk, cu_seqlens)
    nseq = q.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1
    H, dk, dv = q.shape[2], q.shape[3], v.shape[3]
    dq = torch.empty_like(q)
    dk_ = torch.empty_like(k)
    dv_ = torch.empty_like(v)
    dbeta = torch.empty(beta.shape, dtype=torch.float32, device=q.device)
    dla = (None if log_alpha is None else
           torch.empty(log_alpha.shape, dtype=torch.float32, device=q.device))
    ds0 = (torch.empty((nseq, H, dk, dv), dtype=torch.float32, device=q.device)
           if need_ds0 else None)
    need = ctypes.c_size_t(0)
    _lib.check(lib.gdn_chunk_bwd_workspace(ctypes.byref(p), ctypes.byref(need)),
               "gdn_chunk_bwd_workspace")
    ws = workspace
    if ws is None or ws.numel() < need.value:
        ws = torch.empty(max(need.value, 1), dtype=torch.uint8, device=q.device)
    st = lib.gdn_chunk_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                           _ptr(log_alpha), _ptr(s0), _ptr(d_o), _ptr(ds_final),
                           _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dbeta), _ptr(dla),
                           _ptr(ds0), _ptr(ws), ws.numel(), _stream(q.device))
    _lib.check(st, "gdn_chunk_bwd")
    return dq, dk_, dv_, dbeta, dla, ds0


def decode_step(q, k, v, beta, log_alpha, state):
    """One token per sequence; ``state`` [N, H, dk, dv] fp32 is updated in
    place.  q, k [N, H, dk]; v [N, H, dv]; beta [N, H]; log_alpha [N, H],
    [N, H, dk] or None.  Returns o [N, H, dv]."""
    lib = _lib.load()
    N, H, dk = q.shape
    dv = v.shape[-1]
    p = _lib.GdnProblem()
    p.B, p.T, p.H, p.dk, p.dv, p.chunk, p.nseq = N, 1, H, dk, dv, 0, 0
    p.cu_seqlens = None
    p.io_dtype = _dtype_code(q)
    p.gate_dtype = _dtype_code(beta)
    p.gate = _gate_of(log_alpha, 2)
    if state.dtype != torch.float32:
        raise TypeError("state must be fp32")
    o = torch.empty(v.shape, dtype=q.dtype, device=q.device)
    st = lib.gdn_decode_step(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                             _ptr(log_alpha), _ptr(state), _ptr(o),
                             _stream(q.device))
    _lib.check(st, "gdn_decode_step")
    return o
