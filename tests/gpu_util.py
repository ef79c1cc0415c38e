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
