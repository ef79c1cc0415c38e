"""Seeded synthetic inputs for the gated delta rule workloads.

This module holds no arithmetic of the method itself: it only draws random
arrays with the value distributions of the workloads and rounds them to the
dtype handed to the GPU.  Both the HIP path (tests, benchmark) and the fp64
oracle receive the same rounded values: the oracle through the exact fp64
upcast in ``Inputs.f64``.

Distributions (the language-model block of "Gated Delta Networks: Improving
Mamba2 with Delta Rule", section "Method": q and k are L2-normalised, v is
not; alpha is a Mamba2-style decay in (0,1), beta a writing strength):
    q, k  ~ N(0, 1), L2-normalised per (token, head) in fp64
    v, dO ~ N(0, 1)
    beta  = sigmoid(N(0, 1))
    log alpha = -softplus(N(-2, 1))     (per head, or per channel)
    S0    ~ N(0, std^2) when requested
Draw order from one numpy PCG64 stream: lengths -> q -> k -> v -> beta
logits -> alpha logits -> S0 -> dO -> dS.

Inputs for the forward that normalises q and k itself (``raw_qk``): the
unit rows above are multiplied by log-uniform row scales in [lo, hi] (q's,
then k's, drawn after everything else), and a fraction of the rows is set
to zero (q's, then k's uniform draws).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

__all__ = ["Inputs", "make_inputs", "make_gdn2_inputs", "make_product_inputs",
           "make_tree_inputs",
           "random_parents", "varlen_lengths",
           "WORKLOADS", "workload"]


@dataclass
class Inputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    beta: torch.Tensor
    log_alpha: Optional[torch.Tensor]
    s0: Optional[torch.Tensor]
    do: Optional[torch.Tensor]
    cu_seqlens: Optional[torch.Tensor]
    ds_final: Optional[torch.Tensor]
    gate: str
    chunk: int
    seed: int
    f64: dict = field(default_factory=dict)
    write: Optional[torch.Tensor] = None   # decoupled rule: write strength

    def to(self, device):
        """Copy every tensor to ``device`` (fp64 views stay on the host)."""
        out = Inputs(**{k: (v.to(device) if isinstance(v, torch.Tensor) else v)
                        for k, v in self.__dict__.items()})
        out.f64 = self.f64
        return out


def _round(x64: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """Round fp64 values to ``dtype`` (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x64)).to(dtype)


def _l2norm(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def varlen_lengths(rng: np.random.Generator, total: int, lo: int, hi: int):
    """Integer lengths uniform in [lo, hi] drawn until they reach ``total``;
    the last length is ``total`` minus the others, and if that falls below
    ``lo`` the whole list is drawn again from the same stream."""
    while True:
        out = []
        s = 0
        while s < total:
            L = int(rng.integers(lo, hi + 1))
            if s + L >= total:
                L = total - s
            out.append(L)
            s += L
        if out[-1] >= lo or len(out) == 1:
            return out


def make_inputs(B: int, T: int, H: int, dk: int, dv: int, *,
                dtype: torch.dtype = torch.bfloat16,
                gate: str = "scalar",
                gate_dtype: Optional[torch.dtype] = None,
                chunk: int = 64,
                seed: int = 0,
                s0_std: Optional[float] = None,
                with_do: bool = False,
                with_ds: bool = False,
                lengths=None,
                varlen: Optional[tuple] = None,
                raw_qk: Optional[tuple] = None) -> Inputs:
    """Draw one problem.  ``lengths`` (explicit list) or ``varlen`` =
    (total, lo, hi) packs sequences into B = 1 with ``cu_seqlens``.
    ``raw_qk`` = (lo, hi, zero_frac): q and k rows not normalised (see the
    module docstring)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if gate_dtype is None:
        gate_dtype = dtype
    if varlen is not None:
        lengths = varlen_lengths(rng, *varlen)
    cu = None
    nseq = B
    if lengths is not None:
        assert B == 1
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        T = int(cu[-1])
        nseq = len(lengths)
    q = _l2norm(rng.standard_normal((B, T, H, dk)))
    k = _l2norm(rng.standard_normal((B, T, H, dk)))
    v = rng.standard_normal((B, T, H, dv))
    beta = _sigmoid(rng.standard_normal((B, T, H)))
    gshape = (B, T, H, dk) if gate == "channel" else (B, T, H)
    la = -_softplus(rng.standard_normal(gshape) - 2.0)
    s0 = None
    if s0_std is not None:
        s0 = rng.standard_normal((nseq, H, dk, dv)) * s0_std
    do = rng.standard_normal((B, T, H, dv)) if with_do else None
    ds = rng.standard_normal((nseq, H, dk, dv)) if with_ds else None
    if raw_qk is not None:
        lo, hi, zf = raw_qk
        q = q * np.exp(rng.uniform(np.log(lo), np.log(hi), (B, T, H, 1)))
        k = k * np.exp(rng.uniform(np.log(lo), np.log(hi), (B, T, H, 1)))
        q = np.where(rng.uniform(size=(B, T, H, 1)) < zf, 0.0, q)
        k = np.where(rng.uniform(size=(B, T, H, 1)) < zf, 0.0, k)

    inp = Inputs(
        q=_round(q, dtype), k=_round(k, dtype), v=_round(v, dtype),
        beta=_round(beta, gate_dtype),
        log_alpha=None if gate == "none" else _round(la, gate_dtype),
        s0=None if s0 is None else _round(s0, torch.float32),
        do=None if do is None else _round(do, dtype),
        cu_seqlens=None if cu is None else torch.from_numpy(cu),
        ds_final=None if ds is None else _round(ds, torch.float32),
        gate=gate, chunk=chunk, seed=seed)
    f = {}
    for name in ("q", "k", "v", "beta", "log_alpha", "s0", "do"):
        t = getattr(inp, name)
        f[name] = None if t is None else t.double().numpy()
    for name in ("ds_final",):
        t = getattr(inp, name)
        f[name] = None if t is None else t.double().numpy()
    inp.f64 = f
    return inp


def make_gdn2_inputs(*args, seed: int = 0, **kw) -> Inputs:
    """make_inputs' problem for the decoupled erase / write rule: ``beta``
    serves as the erase strength and ``write`` (same shape and dtype) is drawn
    from the same distribution, sigmoid(N(0, 1)), from a second PCG64 stream
    seeded seed + 4099.  The pages give no distribution for either strength;
    beta's is reused for both."""
    inp = make_inputs(*args, seed=seed, **kw)
    rng = np.random.Generator(np.random.PCG64(seed + 4099))
    w = _sigmoid(rng.standard_normal(tuple(inp.beta.shape)))
    inp.write = _round(w, inp.beta.dtype)
    inp.f64["write"] = inp.write.double().numpy()
    return inp


def make_product_inputs(B: int, T: int, H: int, dk: int, dv: int, nh: int, *,
                        dtype: torch.dtype = torch.bfloat16,
                        gate: str = "scalar",
                        chunk: int = 64,
                        seed: int = 0,
                        s0_std: Optional[float] = None,
                        lengths=None) -> Inputs:
    """Draw one problem with nh (key, value, beta) triples per token, the
    inputs of the Householder-product forward: k [B,T,nh,H,dk],
    v [B,T,nh,H,dv], beta [B,T,nh,H]; q [B,T,H,dk] and log alpha [B,T,H]
    per token.  Same distributions as make_inputs."""
    assert gate in ("none", "scalar")
    rng = np.random.Generator(np.random.PCG64(seed))
    cu = None
    nseq = B
    if lengths is not None:
        assert B == 1
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        T = int(cu[-1])
        nseq = len(lengths)
    q = _l2norm(rng.standard_normal((B, T, H, dk)))
    k = _l2norm(rng.standard_normal((B, T, nh, H, dk)))
    v = rng.standard_normal((B, T, nh, H, dv))
    beta = _sigmoid(rng.standard_normal((B, T, nh, H)))
    la = -_softplus(rng.standard_normal((B, T, H)) - 2.0)
    s0 = None
    if s0_std is not None:
        s0 = rng.standard_normal((nseq, H, dk, dv)) * s0_std
    inp = Inputs(
        q=_round(q, dtype), k=_round(k, dtype), v=_round(v, dtype),
        beta=_round(beta, dtype),
        log_alpha=None if gate == "none" else _round(la, dtype),
        s0=None if s0 is None else _round(s0, torch.float32),
        do=None, cu_seqlens=None if cu is None else torch.from_numpy(cu),
        ds_final=None, gate=gate, chunk=chunk, seed=seed)
    inp.f64 = {name: (None if getattr(inp, name) is None
                      else getattr(inp, name).double().numpy())
               for name in ("q", "k", "v", "beta", "log_alpha", "s0")}
    return inp


def random_parents(rng: np.random.Generator, n: int) -> np.ndarray:
    """A random recursive tree of n nodes: node i's parent is uniform over
    the earlier nodes and the root (-1)."""
    return np.array([int(rng.integers(-1, i)) for i in range(n)], dtype=np.int32)


def make_tree_inputs(B: int, n: int, H: int, dk: int, dv: int, *,
                     dtype: torch.dtype = torch.bfloat16,
                     gate: str = "scalar",
                     chunk: int = 64,
                     seed: int = 0,
                     s0_std: Optional[float] = 0.02,
                     lengths=None,
                     shape: str = "random"):
    """Draw B draft trees of n nodes (or trees of the given ``lengths``
    packed with cu_seqlens), one token per node, with the distributions of
    make_inputs and the committed states ~ N(0, s0_std^2).  ``shape``:
    "random" (random recursive trees), "chain" (parent i - 1) or "star"
    (every parent -1).  The tensors are make_inputs' draws; the parents and
    one accepted node per tree (uniform over its nodes, -1 for an empty
    tree) come from a second PCG64 stream seeded seed + 7919.  Returns (Inputs, parent int32 tensor [B, n] or
    [total], accepted int32 tensor [ntrees])."""
    inp = make_inputs(B, n, H, dk, dv, dtype=dtype, gate=gate, chunk=chunk, seed=seed,
                      s0_std=s0_std, lengths=lengths)
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    sizes = [n] * B if lengths is None else list(lengths)
    par, acc = [], []
    for L in sizes:
        if shape == "chain":
            par.append(np.arange(L, dtype=np.int32) - 1)
        elif shape == "star":
            par.append(np.full(L, -1, dtype=np.int32))
        else:
            par.append(random_parents(rng, L))
        acc.append(int(rng.integers(0, L)) if L > 0 else -1)
    parent = (np.stack(par) if lengths is None else np.concatenate(par + [np.zeros(0, np.int32)]))
    return (inp, torch.from_numpy(parent.astype(np.int32)),
            torch.tensor(acc, dtype=torch.int32))


# Named workloads.  Sizes follow the configurations the method is measured on.
WORKLOADS = {
    # tiny fp32 forward, 4 chunks of 16
    "tiny_fp32": dict(B=1, T=64, H=2, dk=16, dv=16, dtype=torch.float32,
                      chunk=16, seed=1001),
    # 350M-scale layer forward
    "layer_b8_t2048": dict(B=8, T=2048, H=8, dk=128, dv=128, chunk=64, seed=1002),
    # decode: 256 sequences x 32 heads, state ~ N(0, 0.02^2)
    "decode_n256_h32": dict(B=256, T=1, H=32, dk=128, dv=128, chunk=64,
                            seed=1003, s0_std=0.02),
    # long context with initial state
    "long_t65536": dict(B=1, T=65536, H=16, dk=128, dv=128, chunk=64,
                        seed=1004, s0_std=0.02),
    # varlen training batch (scalar gate); per-channel variant below
    "varlen_16k_dv256": dict(B=1, T=16384, H=16, dk=128, dv=256, chunk=64,
                             seed=1005, varlen=(16384, 512, 8192), with_do=True),
    "varlen_16k_dv256_channel": dict(B=1, T=16384, H=16, dk=128, dv=256,
                                     chunk=64, seed=1005, gate="channel",
                                     varlen=(16384, 512, 8192), with_do=True),
    # headline forward: T=4096, H=16, d=128, bf16, B=1
    "fwd_t4096_h16": dict(B=1, T=4096, H=16, dk=128, dv=128, chunk=64,
                          seed=1000),
}


def conv_taps(H: int, dk: int, dv: int, W: int, seed: int):
    """Short-convolution taps (q, k, v) for gdn_chunk_fwd_conv: fp32 [H, d, W]
    drawn from N(0, 1 / W) on a stream of their own (PCG64(seed + 6007))."""
    r = np.random.Generator(np.random.PCG64(seed + 6007))
    mk = lambda d: torch.from_numpy(r.standard_normal((H, d, W)) / np.sqrt(W)).float()
    return mk(dk), mk(dk), mk(dv)


def workload(name: str, **overrides) -> Inputs:
    kw = dict(WORKLOADS[name])
    kw.update(overrides)
    return make_inputs(**kw)
