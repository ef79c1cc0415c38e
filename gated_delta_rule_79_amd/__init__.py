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

__all__ = ["chunk_fwd", "chunk_fwd_noalloc", "chunk_fwd_conv", "gdn2_chunk_fwd",
           "gdn2_decode_step",
           "chunk_bwd", "decode_step", "decode_step_product",
           "chunk_fwd_product", "tree_verify",
           "tree_commit", "FwdPlan", "GdnError",
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


def _problem(q, v, beta, log_alpha, chunk, cu_seqlens, gate=None, seg_chunks=0):
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
    p.seg_chunks = int(seg_chunks)
    return p


def _check_cu(cu_seqlens, q):
    if cu_seqlens is None:
        return
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != q.device:
        raise ValueError("cu_seqlens must be an int32 tensor on the inputs' device")


def _out(t, shape, dtype, device):
    """A caller's preallocated output, checked, or a new tensor."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"output must be a contiguous {dtype} tensor of shape {tuple(shape)}")
    return t


def chunk_fwd(q, k, v, beta, log_alpha=None, s0=None, chunk: int = 64,
              cu_seqlens=None, output_final_state: bool = True,
              workspace: Optional[torch.Tensor] = None, qk_l2norm: bool = False,
              seg_chunks: int = 0, o=None, s_final=None):
    """Chunkwise forward.  Returns (o, s_final or None).  qk_l2norm: q and k
    rows are L2-normalised inside the kernels (gdn_chunk_fwd_qknorm).
    seg_chunks: state-pass segment length (0 automatic, > 0 chunks per
    segment, < 0 never split).  o / s_final: optional preallocated outputs."""
    lib = _lib.load()
    _check_cu(cu_seqlens, q)
    p = _problem(q, v, beta, log_alpha, chunk, cu_seqlens, seg_chunks=seg_chunks)
    nseq = q.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1
    H, dk, dv = q.shape[2], q.shape[3], v.shape[3]
    o = _out(o, v.shape, q.dtype, q.device)
    sf = (_out(s_final, (nseq, H, dk, dv), torch.float32, q.device)
          if output_final_state else None)
    need = ctypes.c_size_t(0)
    wsq = lib.gdn_chunk_fwd_qknorm_workspace if qk_l2norm else lib.gdn_chunk_fwd_workspace
    _lib.check(wsq(ctypes.byref(p), ctypes.byref(need)), "workspace query")
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


def chunk_fwd_noalloc(q, k, v, beta, log_alpha=None, s0=None, chunk: int = 64,
                      cu_seqlens=None, o=None, s_final=None, seg_chunks: int = 0):
    """gdn_chunk_fwd_noalloc: the forward with the library's static scratch
    buffer as its workspace (no workspace argument).  ``o`` / ``s_final`` may
    be preallocated outputs (then nothing at all is allocated here);
    otherwise they are created.  Returns (o, s_final)."""
    lib = _lib.load()
    _check_cu(cu_seqlens, q)
    p = _problem(q, v, beta, log_alpha, chunk, cu_seqlens, seg_chunks=seg_chunks)
    nseq = q.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1
    H, dk, dv = q.shape[2], q.shape[3], v.shape[3]
    if o is None:
        o = torch.empty(v.shape, dtype=q.dtype, device=q.device)
    if s_final is None:
        s_final = torch.empty((nseq, H, dk, dv), dtype=torch.float32, device=q.device)
    st = lib.gdn_chunk_fwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                   _ptr(log_alpha), _ptr(s0), _ptr(o), _ptr(s_final),
                                   _stream(q.device))
    _lib.check(st, "gdn_chunk_fwd_noalloc")
    return o, s_final


def chunk_fwd_conv(xq, xk, xv, wq, wk, wv, beta, log_alpha=None, s0=None, chunk: int = 64,
                   cu_seqlens=None, output_final_state: bool = True, seg_chunks: int = 0):
    """The forward behind the block's q, k, v paths (gdn_chunk_fwd_conv):
    xq, xk [B,T,H,dk], xv [B,T,H,dv] projections; wq, wk [H,dk,W], wv
    [H,dv,W] fp32 convolution taps (W in 1..8).  q = l2(silu(conv(xq))),
    k = l2(silu(conv(xk))), v = silu(conv(xv)), then the forward.
    Returns (o, s_final or None)."""
    lib = _lib.load()
    _check_cu(cu_seqlens, xq)
    width = wq.shape[-1]
    for w in (wq, wk, wv):
        if w.dtype != torch.float32 or w.shape[-1] != width:
            raise ValueError("taps must be fp32 with one width")
    p = _problem(xq, xv, beta, log_alpha, chunk, cu_seqlens, seg_chunks=seg_chunks)
    nseq = xq.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1
    H, dk, dv = xq.shape[2], xq.shape[3], xv.shape[3]
    o = torch.empty(xv.shape, dtype=xq.dtype, device=xq.device)
    sf = (torch.empty((nseq, H, dk, dv), dtype=torch.float32, device=xq.device)
          if output_final_state else None)
    need = ctypes.c_size_t(0)
    _lib.check(lib.gdn_chunk_fwd_conv_workspace(ctypes.byref(p), width, ctypes.byref(need)),
               "gdn_chunk_fwd_conv_workspace")
    ws = torch.empty(max(need.value, 1), dtype=torch.uint8, device=xq.device)
    st = lib.gdn_chunk_fwd_conv(ctypes.byref(p), width, _ptr(xq), _ptr(xk), _ptr(xv), _ptr(wq),
                                _ptr(wk), _ptr(wv), _ptr(beta), _ptr(log_alpha), _ptr(s0),
                                _ptr(o), _ptr(sf), _ptr(ws), ws.numel(), _stream(xq.device))
    _lib.check(st, "gdn_chunk_fwd_conv")
    return o, sf


def _prologue_problem(x, cu_seqlens):
    """A problem whose dk or dv is x's channel count (the prologue entry
    points read B, T, H, the dtype and the packing; dk, dv name d)."""
    d = x.shape[-1]
    dk = d if d in (16, 32, 64, 128) else 16
    p = _lib.GdnProblem()
    B, T, H = x.shape[:3]
    nseq = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    for name, val in dict(B=B, T=T, H=H, dk=dk, dv=d, chunk=64, nseq=nseq,
                          cu_seqlens=_ptr(cu_seqlens), io_dtype=_dtype_code(x),
                          gate_dtype=_lib.GDN_F32, gate=_lib.GDN_GATE_NONE,
                          seg_chunks=0).items():
        setattr(p, name, val)
    return p


def prologue_fwd(x, taps, normalize: bool, cu_seqlens=None):
    """One projection's prologue (gdn_prologue_fwd): silu(conv(x)) and, with
    normalize, its rows over |.|.  x [B,T,H,d]; taps [H,d,W] fp32."""
    lib = _lib.load()
    _check_cu(cu_seqlens, x)
    if taps.dtype != torch.float32:
        raise ValueError("taps must be fp32")
    p = _prologue_problem(x, cu_seqlens)
    y = torch.empty_like(x)
    st = lib.gdn_prologue_fwd(ctypes.byref(p), x.shape[-1], taps.shape[-1], int(normalize),
                              _ptr(x), _ptr(taps), _ptr(y), _stream(x.device))
    _lib.check(st, "gdn_prologue_fwd")
    return y


def prologue_bwd(x, taps, dy, normalize: bool, cu_seqlens=None):
    """Backward of :func:`prologue_fwd` (gdn_prologue_bwd): returns
    (dx [B,T,H,d] in x's dtype, dtaps [H,d,W] fp32)."""
    lib = _lib.load()
    _check_cu(cu_seqlens, x)
    if dy.shape != x.shape or dy.dtype != x.dtype:
        raise ValueError("dy must match x")
    if taps.dtype != torch.float32:
        raise ValueError("taps must be fp32")
    p = _prologue_problem(x, cu_seqlens)
    d, w = x.shape[-1], taps.shape[-1]
    need = ctypes.c_size_t(0)
    _lib.check(lib.gdn_prologue_bwd_workspace(ctypes.byref(p), d, w, ctypes.byref(need)),
               "gdn_prologue_bwd_workspace")
    ws = torch.empty(max(need.value, 1), dtype=torch.uint8, device=x.device)
    dx = torch.empty_like(x)
    dtaps = torch.empty(taps.shape, dtype=torch.float32, device=x.device)
    st = lib.gdn_prologue_bwd(ctypes.byref(p), d, w, int(normalize), _ptr(x), _ptr(taps),
                              _ptr(dy), _ptr(dx), _ptr(dtaps), _ptr(ws), ws.numel(),
                              _stream(x.device))
    _lib.check(st, "gdn_prologue_bwd")
    return dx, dtaps


def chunk_bwd_conv(xq, xk, xv, wq, wk, wv, beta, log_alpha, s0, do, ds_final=None,
                   chunk: int = 64, cu_seqlens=None, need_ds0: bool = True):
    """Backward of :func:`chunk_fwd_conv`: the three prologues again
    (gdn_prologue_fwd), gdn_chunk_bwd on their outputs, then each path's
    gdn_prologue_bwd.  Returns (dxq, dxk, dxv, dwq, dwk, dwv, dbeta,
    dlog_alpha, ds0)."""
    q = prologue_fwd(xq, wq, True, cu_seqlens)
    k = prologue_fwd(xk, wk, True, cu_seqlens)
    v = prologue_fwd(xv, wv, False, cu_seqlens)
    dq, dk, dv, dbeta, dla, ds0 = chunk_bwd(q, k, v, beta, log_alpha, s0, do, ds_final,
                                            chunk=chunk, cu_seqlens=cu_seqlens,
                                            need_ds0=need_ds0)
    dxq, dwq = prologue_bwd(xq, wq, dq, True, cu_seqlens)
    dxk, dwk = prologue_bwd(xk, wk, dk, True, cu_seqlens)
    dxv, dwv = prologue_bwd(xv, wv, dv, False, cu_seqlens)
    return dxq, dxk, dxv, dwq, dwk, dwv, dbeta, dla, ds0


def gdn2_chunk_fwd(q, k, v, erase, write, log_alpha=None, s0=None, chunk: int = 64,
                   cu_seqlens=None, output_final_state: bool = True,
                   workspace: Optional[torch.Tensor] = None, seg_chunks: int = 0):
    """Gated DeltaNet-2 forward (gdn2_chunk_fwd): separate erase and write
    strengths [B,T,H] in place of beta.  Returns (o, s_final or None)."""
    lib = _lib.load()
    _check_cu(cu_seqlens, q)
    if write.shape != erase.shape or write.dtype != erase.dtype:
        raise ValueError("erase and write must have the same shape and dtype")
    p = _problem(q, v, erase, log_alpha, chunk, cu_seqlens, seg_chunks=seg_chunks)
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
    st = lib.gdn2_chunk_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(erase),
                            _ptr(write), _ptr(log_alpha), _ptr(s0), _ptr(o), _ptr(sf),
                            _ptr(ws), ws.numel(), _stream(q.device))
    _lib.check(st, "gdn2_chunk_fwd")
    return o, sf


def gdn2_decode_step(q, k, v, erase, write, log_alpha, state):
    """Gated DeltaNet-2 decode step (gdn2_decode_step); ``state`` is updated
    in place.  erase, write [N, H].  Returns o [N, H, dv]."""
    lib = _lib.load()
    N, H, dk = q.shape
    dv = v.shape[-1]
    if write.shape != erase.shape or write.dtype != erase.dtype:
        raise ValueError("erase and write must have the same shape and dtype")
    p = _lib.GdnProblem()
    p.B, p.T, p.H, p.dk, p.dv, p.chunk, p.nseq = N, 1, H, dk, dv, 0, 0
    p.cu_seqlens = None
    p.io_dtype = _dtype_code(q)
    p.gate_dtype = _dtype_code(erase)
    p.gate = _gate_of(log_alpha, 2)
    if state.dtype != torch.float32:
        raise TypeError("state must be fp32")
    o = torch.empty(v.shape, dtype=q.dtype, device=q.device)
    st = lib.gdn2_decode_step(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(erase),
                              _ptr(write), _ptr(log_alpha), _ptr(state), _ptr(o),
                              _stream(q.device))
    _lib.check(st, "gdn2_decode_step")
    return o


def chunk_fwd_product(q, k, v, beta, log_alpha=None, s0=None, chunk: int = 64,
                      cu_seqlens=None, output_final_state: bool = True,
                      seg_chunks: int = 0):
    """Householder-product forward (gdn_chunk_fwd_product): k [B,T,nh,H,dk],
    v [B,T,nh,H,dv], beta [B,T,nh,H], q [B,T,H,dk], log_alpha [B,T,H] or None.
    Returns (o [B,T,H,dv], s_final or None)."""
    lib = _lib.load()
    _check_cu(cu_seqlens, q)
    nh = k.shape[2]
    H, dk, dv = q.shape[2], q.shape[3], v.shape[-1]
    p = _problem(q, v, beta, log_alpha, chunk, cu_seqlens, seg_chunks=seg_chunks)
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
                 qk_l2norm: bool = False, seg_chunks: int = 0, conv_taps=None):
        # conv_taps = (wq, wk, wv): q, k, v are the projections of
        # gdn_chunk_fwd_conv (short convolution, SiLU, L2 norm of q and k)
        lib = _lib.load()
        _check_cu(cu_seqlens, q)
        self._keep = (q, k, v, beta, log_alpha, s0, cu_seqlens, conv_taps)
        self.problem = _problem(q, v, beta, log_alpha, chunk, cu_seqlens,
                                seg_chunks=seg_chunks)
        nseq = q.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1
        H, dk, dv = q.shape[2], q.shape[3], v.shape[3]
        self.o = torch.empty(v.shape, dtype=q.dtype, device=q.device)
        self.s_final = (torch.empty((nseq, H, dk, dv), dtype=torch.float32,
                                    device=q.device) if output_final_state else None)
        need = ctypes.c_size_t(0)
        if conv_taps is not None:
            width = conv_taps[0].shape[-1]
            _lib.check(lib.gdn_chunk_fwd_conv_workspace(ctypes.byref(self.problem), width,
                                                        ctypes.byref(need)), "workspace query")
        else:
            wsq = (lib.gdn_chunk_fwd_qknorm_workspace if qk_l2norm
                   else lib.gdn_chunk_fwd_workspace)
            _lib.check(wsq(ctypes.byref(self.problem), ctypes.byref(need)), "workspace query")
        self.workspace = torch.empty(max(need.value, 1), dtype=torch.uint8,
                                     device=q.device)
        tail = (_ptr(beta), _ptr(log_alpha), _ptr(s0), _ptr(self.o), _ptr(self.s_final),
                _ptr(self.workspace), self.workspace.numel(), _stream(q.device))
        if conv_taps is not None:
            self._name = "gdn_chunk_fwd_conv"
            self._args = (ctypes.byref(self.problem), width, _ptr(q), _ptr(k), _ptr(v),
                          *(_ptr(w) for w in conv_taps)) + tail
        else:
            self._name = "gdn_chunk_fwd_qknorm" if qk_l2norm else "gdn_chunk_fwd"
            self._args = (ctypes.byref(self.problem), _ptr(q), _ptr(k), _ptr(v)) + tail
        self._fn = getattr(lib, self._name)

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


def fwd_workspace_bytes(q, v, beta, log_alpha=None, chunk=64, cu_seqlens=None,
                        seg_chunks: int = 0) -> int:
    lib = _lib.load()
    p = _problem(q, v, beta, log_alpha, chunk, cu_seqlens, seg_chunks=seg_chunks)
    need = ctypes.c_size_t(0)
    _lib.check(lib.gdn_chunk_fwd_workspace(ctypes.byref(p), ctypes.byref(need)),
               "gdn_chunk_fwd_workspace")
    return need.value


def chunk_bwd(q, k, v, beta, log_alpha, s0, d_o, ds_final=None,
              chunk: int = 64, cu_seqlens=None, need_ds0: bool = True,
              workspace: Optional[torch.Tensor] = None, seg_chunks: int = 0,
              out=None):
    """Chunkwise backward.  Returns (dq, dk, dv, dbeta, dlog_alpha, ds0).
    seg_chunks as in chunk_fwd (the state recompute's segments).  out:
    optional preallocated (dq, dk, dv, dbeta, dlog_alpha, ds0), entries may
    be None."""
    lib = _lib.load()
    _check_cu(cu_seqlens, q)
    p = _problem(q, v, beta, log_alpha, chunk, cu_seqlens, seg_chunks=seg_chunks)
    nseq = q.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1
    H, dk, dv = q.shape[2], q.shape[3], v.shape[3]
    out = (None,) * 6 if out is None else tuple(out)
    dq = _out(out[0], q.shape, q.dtype, q.device)
    dk_ = _out(out[1], k.shape, k.dtype, k.device)
    dv_ = _out(out[2], v.shape, v.dtype, v.device)
    dbeta = _out(out[3], beta.shape, torch.float32, q.device)
    dla = (None if log_alpha is None else
           _out(out[4], log_alpha.shape, torch.float32, q.device))
    ds0 = (_out(out[5], (nseq, H, dk, dv), torch.float32, q.device)
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
