"""Helpers shared by the GPU parity tests: device transfer, the oracle call
on exactly the values handed to the GPU, and the normwise error measure.

Error measure: for every (sequence, head) slice of an output, max|x - y| /
max|y| over the slice; the worst slice is reported.  A slice whose reference
is below 1e-30 (fully decayed) is judged by absolute error relative to the
tensor's global max |y|.  Tolerances: 1e-4 when every operand is fp32, 2e-2
when bf16 operands enter the matrix cores (fp32 accumulation)."""

import sys

import numpy as np
import torch

import oracle

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(inp):
    return inp.to("cuda")


def _slices(x, cu):
    """Yield per-(sequence, head) 2-D slices of a [B, T, H, D] array."""
    B, T, H = x.shape[:3]
    if cu is None:
        for b in range(B):
            for h in range(H):
                yield x[b, :, h]
    else:
        cu = np.asarray(cu)
        for n in range(len(cu) - 1):
            for h in range(H):
                yield x[0, cu[n]:cu[n + 1], h]


def slice_err(x, y, cu=None):
    """Normwise error of token outputs [B, T, H, D] per (sequence, head)."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    assert x.shape == y.shape
    if x.size == 0:
        return 0.0
    if not np.all(np.isfinite(x)):
        return float("inf")
    gmax = float(np.max(np.abs(y)))
    worst = 0.0
    for xs, ys in zip(_slices(x, cu), _slices(y, cu)):
        if xs.size == 0:
            continue
        ref = float(np.max(np.abs(ys)))
        diff = float(np.max(np.abs(xs - ys)))
        worst = max(worst, diff / ref if ref >= 1e-30 else diff / max(gmax, 1e-30))
    return worst


def state_err(x, y):
    """Normwise error of states [N, H, dk, dv] per (sequence, head)."""
    return oracle.normwise_rel_err(np.asarray(x, dtype=np.float64), y)


def np64(t):
    return t.detach().float().cpu().double().numpy()


def oracle_fwd(inp, s0=True):
    f = inp.f64
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.cpu().numpy()
    return oracle.gdn_fwd(f["q"], f["k"], f["v"], f["beta"], f["log_alpha"],
                          f["s0"] if s0 else None, inp.gate, cu_seqlens=cu)


def row_err(x, y, floor=1e-3):
    """Diagnostic only: worst per-(token, head) row error max|x-y| / max|y|
    over rows whose reference is at least ``floor`` times the max of their
    (sequence, head) slice (tiny rows are all rounding)."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    if x.size == 0:
        return 0.0
    ref = np.max(np.abs(y), axis=-1)
    diff = np.max(np.abs(x - y), axis=-1)
    smax = np.max(ref, axis=1, keepdims=True)
    ok = ref >= floor * np.maximum(smax, 1e-30)
    if not np.any(ok):
        return 0.0
    return float(np.max(diff[ok] / ref[ok]))


# ---- parallel oracle: independent (sequence, head) chains in forked CPU workers

_POOL_JOB = None


def _pool_call(item):
    return _POOL_JOB(item)


def par_map(job, items, workers=None):
    """job(item) for every item, in forked worker processes that only run
    numpy (the oracle); results in order.  Everything a job reads must be a
    host array prepared before the call: the workers never touch the GPU."""
    global _POOL_JOB
    import multiprocessing as mp
    import os
    items = list(items)
    n = workers or min(len(items), 16, len(os.sched_getaffinity(0)))
    if n <= 1:
        return [job(i) for i in items]
    _POOL_JOB = job
    try:
        with mp.get_context("fork").Pool(n) as pool:
            return pool.map(_pool_call, items, chunksize=1)
    finally:
        _POOL_JOB = None


def fwd_errors_per_head(inp, o, sf, heads=None, s0=True):
    """Compare GPU outputs (o, s_final) with the oracle head by head in
    parallel workers.  Returns [(head, err_o, err_s, row_err_o), ...]."""
    f = inp.f64
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.numpy()
    xo, xs = np64(o), np64(sf)
    H = xo.shape[2]
    heads = range(H) if heads is None else heads

    def job(h):
        hs = slice(h, h + 1)
        sub = lambda a: None if a is None else a[:, :, hs]
        o_ref, s_ref = oracle.gdn_fwd(sub(f["q"]), sub(f["k"]), sub(f["v"]), sub(f["beta"]),
                                      sub(f["log_alpha"]),
                                      None if (f["s0"] is None or not s0) else f["s0"][:, hs],
                                      inp.gate, cu_seqlens=cu)
        return (h, slice_err(xo[:, :, hs], o_ref, cu), state_err(xs[:, hs], s_ref),
                row_err(xo[:, :, hs], o_ref))

    return par_map(job, heads)


def bwd_errors_per_head(inp, got, heads=None):
    """Compare GPU gradients with the oracle's adjoint head by head in
    parallel workers.  Returns [(head, {name: err}), ...]."""
    f = inp.f64
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.numpy()
    xs = [None if g is None else np64(g) for g in got]
    H = xs[0].shape[2]
    heads = range(H) if heads is None else heads

    def job(h):
        hs = slice(h, h + 1)
        sub = lambda a: None if a is None else a[:, :, hs]
        ref = oracle.gdn_bwd(sub(f["q"]), sub(f["k"]), sub(f["v"]), sub(f["beta"]),
                             sub(f["log_alpha"]),
                             None if f["s0"] is None else f["s0"][:, hs],
                             sub(f["do"]),
                             None if f["ds_final"] is None else f["ds_final"][:, hs],
                             inp.gate, cu_seqlens=cu)
        errs = {}
        for nm, x, y in zip(("dq", "dk", "dv", "dbeta", "dlog_alpha"), xs[:5], ref[:5]):
            if y is None:
                continue
            xa = x[:, :, hs]
            if y.ndim == 3:
                xa, y = xa[..., None], y[..., None]
            errs[nm] = slice_err(xa, y, cu)
        if xs[5] is not None:
            errs["ds0"] = state_err(xs[5][:, hs], ref[5])
        return h, errs

    return par_map(job, heads)


# ---- canary-padded outputs: every kernel write outside its output is caught

CANARY_BYTES = 4096
CANARY = 0x5A


class Padded:
    """An output tensor inside a larger byte buffer whose CANARY_BYTES before
    and after hold a fixed byte pattern; check() asserts they are intact."""

    def __init__(self, shape, dtype, device="cuda"):
        n = 1
        for x in shape:
            n *= int(x)
        nbytes = n * torch.tensor([], dtype=dtype).element_size()
        self.raw = torch.full((CANARY_BYTES * 2 + nbytes,), CANARY, dtype=torch.uint8,
                              device=device)
        self.nbytes = nbytes
        self.t = self.raw[CANARY_BYTES:CANARY_BYTES + nbytes].view(dtype).view(*shape)

    def check(self, what=""):
        head = self.raw[:CANARY_BYTES]
        tail = self.raw[CANARY_BYTES + self.nbytes:]
        bad = int((head != CANARY).sum()) + int((tail != CANARY).sum())
        assert bad == 0, f"{what}: {bad} canary bytes overwritten around the output"


def padded_like(shape, dtype):
    return Padded(shape, dtype)
