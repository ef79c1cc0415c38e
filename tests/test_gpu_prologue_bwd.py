"""GPU parity of the prologue entry points (gdn_prologue_fwd, gdn_prologue_bwd)
and of the block backward built on them, against the fp64 oracle's
conv_prologue / conv_prologue_bwd (the latter pinned by finite differences)
and gdn_bwd ("Gated Delta Networks: Improving Mamba2 with Delta Rule",
"Method": the q, k, v paths of the block).

Inputs: projections ~ N(0, 1) (scaled by 2, so SiLU sees both signs), taps
~ N(0, 1/W) from their own stream, upstream gradients ~ N(0, 1); both
dtypes, widths 1 to 8, normalised (d a power of two) and plain paths (also
d = 48 and 256), packed sequences with empty ones and ones shorter than the
convolution, and an empty batch."""

import numpy as np
import pytest
import torch

import gated_delta_rule_79_amd as gdn
import oracle
from gated_delta_rule_79_amd import synth
from gpu_util import TOL, log, np64, par_map, slice_err, state_err

pytestmark = pytest.mark.gpu


def draw(B, T, H, d, W, seed, dtype, lengths=None):
    r = np.random.Generator(np.random.PCG64(seed))
    cu = None
    if lengths is not None:
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        B, T = 1, int(cu[-1])
    x = torch.from_numpy(2.0 * r.standard_normal((B, T, H, d))).to(dtype)
    dy = torch.from_numpy(r.standard_normal((B, T, H, d))).to(dtype)
    taps = synth.conv_taps(H, d, d, W, seed)[0]
    return x, dy, taps, cu


def taps_err(got, ref):
    """Normwise error of a tap gradient [H, d, W], per head."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    if not np.all(np.isfinite(got)):
        return float("inf")
    return max(float(np.max(np.abs(got[h] - ref[h])) / max(np.max(np.abs(ref[h])), 1e-30))
               for h in range(ref.shape[0]))


def run(x, dy, taps, cu, normalize):
    xc, dyc, tc = x.cuda(), dy.cuda(), taps.cuda()
    cuc = None if cu is None else torch.from_numpy(cu).cuda()
    y = gdn.prologue_fwd(xc, tc, normalize, cuc)
    dx, dw = gdn.prologue_bwd(xc, tc, dyc, normalize, cuc)
    torch.cuda.synchronize()
    return y, dx, dw


def check(x, dy, taps, cu, normalize, name):
    log(f"[prologue] {name} x={tuple(x.shape)} {x.dtype} W={taps.shape[-1]} norm={normalize}")
    y, dx, dw = run(x, dy, taps, cu, normalize)
    xf, dyf, tf = x.double().numpy(), dy.double().numpy(), taps.double().numpy()
    y_ref = oracle.conv_prologue(xf, tf, normalize, cu)
    dx_ref, dw_ref = oracle.conv_prologue_bwd(xf, tf, normalize, dyf, cu)
    ey, ex, ew = slice_err(np64(y), y_ref, cu), slice_err(np64(dx), dx_ref, cu), \
        taps_err(np64(dw), dw_ref)
    tol = TOL[x.dtype]
    log(f"    err y={ey:.2e} dx={ex:.2e} dtaps={ew:.2e} tol={tol}")
    assert ey < tol and ex < tol and ew < tol, (ey, ex, ew)


@pytest.mark.parametrize("W", [1, 4, 8])
@pytest.mark.parametrize("d,normalize", [(16, True), (64, True), (128, True), (48, False),
                                         (256, False), (128, False)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_prologue_dense(gpu_lib, W, d, normalize, dtype):
    x, dy, taps, cu = draw(2, 150, 2, d, W, seed=300 + W + d, dtype=dtype)
    check(x, dy, taps, cu, normalize, "dense")


@pytest.mark.parametrize("normalize", [True, False])
def test_prologue_packed_short_sequences(gpu_lib, normalize):
    # empty sequences, sequences shorter than the convolution, and runs of
    # the tap pass that cross sequence starts
    x, dy, taps, cu = draw(0, 0, 3, 64, 4, seed=311, dtype=torch.float32,
                           lengths=[3, 0, 1, 70, 2, 200, 33, 0, 5])
    check(x, dy, taps, cu, normalize, "packed")


def test_prologue_bwd_is_deterministic(gpu_lib):
    x, dy, taps, cu = draw(1, 3000, 4, 128, 4, seed=312, dtype=torch.bfloat16)
    a = run(x, dy, taps, cu, True)
    b = run(x, dy, taps, cu, True)
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])


def test_prologue_empty_batch_has_zero_tap_gradient(gpu_lib):
    x, dy, taps, _ = draw(1, 0, 2, 32, 3, seed=313, dtype=torch.float32)
    y, dx, dw = run(x, dy, taps, None, True)
    assert y.numel() == 0 and dx.numel() == 0 and torch.all(dw == 0)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_block_backward_through_the_prologues(gpu_lib, gate, dtype):
    # dL/d(projections, taps, beta, log alpha, s0) of the block forward
    # gdn_chunk_fwd_conv, against the oracle's adjoints composed
    B, T, H, dk, dv, W = 1, 150, 2, 64, 32, 4
    C = 32 if (gate == "channel" and dtype == torch.float32) else 64
    inp = synth.make_inputs(B, T, H, dk, dv, dtype=dtype, gate=gate, chunk=C, seed=314,
                            s0_std=0.1, with_do=True, with_ds=True)
    r = np.random.Generator(np.random.PCG64(315))
    xs = [torch.from_numpy(2.0 * r.standard_normal((B, T, H, d))).to(dtype)
          for d in (dk, dk, dv)]
    wq, wk, wv = synth.conv_taps(H, dk, dv, W, 316)
    log(f"[prologue] block backward gate={gate} {dtype} C={C}")
    d = inp.to("cuda")
    got = gdn.chunk_bwd_conv(*(x.cuda() for x in xs), wq.cuda(), wk.cuda(), wv.cuda(),
                             d.beta, d.log_alpha, d.s0, d.do, d.ds_final, chunk=C)
    torch.cuda.synchronize()
    f = inp.f64
    xf = [x.double().numpy() for x in xs]
    tf = [w.double().numpy() for w in (wq, wk, wv)]
    q = oracle.conv_prologue(xf[0], tf[0], True)
    k = oracle.conv_prologue(xf[1], tf[1], True)
    v = oracle.conv_prologue(xf[2], tf[2], False)
    dq, dkk, dvv, db, dla, ds0 = oracle.gdn_bwd(q, k, v, f["beta"], f["log_alpha"], f["s0"],
                                                f["do"], f["ds_final"], gate)
    dxq, dwq = oracle.conv_prologue_bwd(xf[0], tf[0], True, dq)
    dxk, dwk = oracle.conv_prologue_bwd(xf[1], tf[1], True, dkk)
    dxv, dwv = oracle.conv_prologue_bwd(xf[2], tf[2], False, dvv)
    errs = {"dxq": slice_err(np64(got[0]), dxq), "dxk": slice_err(np64(got[1]), dxk),
            "dxv": slice_err(np64(got[2]), dxv), "dwq": taps_err(np64(got[3]), dwq),
            "dwk": taps_err(np64(got[4]), dwk), "dwv": taps_err(np64(got[5]), dwv),
            "dbeta": slice_err(np64(got[6])[..., None], db[..., None]),
            "ds0": state_err(np64(got[8]), ds0)}
    la = np64(got[7])
    errs["dlog_alpha"] = slice_err(la if la.ndim == 4 else la[..., None],
                                   dla if dla.ndim == 4 else dla[..., None])
    log("    " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()))
    for k_, v_ in errs.items():
        assert v_ < TOL[dtype], (k_, v_)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_block_backward_training_batch_all_heads(gpu_lib, gate):
    # the packed training batch (16384 tokens in sequences of 512 to 8192,
    # H16, dk128, dv256, bf16) through the block backward: every head's
    # projection and tap gradients and the gate and state gradients against
    # the oracle's composed adjoints (run head by head in forked workers)
    H, dk, dv, W = 16, 128, 256, 4
    inp = synth.make_inputs(1, 16384, H, dk, dv, dtype=torch.bfloat16, gate=gate, chunk=64,
                            seed=317, varlen=(16384, 512, 8192), s0_std=0.05, with_do=True,
                            with_ds=True)
    cu = inp.cu_seqlens.numpy()
    r = np.random.Generator(np.random.PCG64(318))
    T = inp.q.shape[1]
    xs = [torch.from_numpy(2.0 * r.standard_normal((1, T, H, d))).to(torch.bfloat16)
          for d in (dk, dk, dv)]
    wq, wk, wv = synth.conv_taps(H, dk, dv, W, 319)
    log(f"[prologue] block backward, packed training batch, gate={gate}, lengths="
        f"{np.diff(cu).tolist()}")
    d = inp.to("cuda")
    got = gdn.chunk_bwd_conv(*(x.cuda() for x in xs), wq.cuda(), wk.cuda(), wv.cuda(),
                             d.beta, d.log_alpha, d.s0, d.do, d.ds_final, chunk=64,
                             cu_seqlens=d.cu_seqlens)
    torch.cuda.synchronize()
    g = [None if x is None else np64(x) for x in got]
    f = inp.f64
    xf = [x.double().numpy() for x in xs]
    tf = [w.double().numpy() for w in (wq, wk, wv)]

    def job(h):
        hs = slice(h, h + 1)
        sub = lambda a: a[:, :, hs]
        q = oracle.conv_prologue(sub(xf[0]), tf[0][hs], True, cu)
        k = oracle.conv_prologue(sub(xf[1]), tf[1][hs], True, cu)
        v = oracle.conv_prologue(sub(xf[2]), tf[2][hs], False, cu)
        dq, dkk, dvv, db, dla, ds0 = oracle.gdn_bwd(
            q, k, v, sub(f["beta"]), sub(f["log_alpha"]), f["s0"][:, hs], sub(f["do"]),
            f["ds_final"][:, hs], gate, cu_seqlens=cu)
        dxq, dwq = oracle.conv_prologue_bwd(sub(xf[0]), tf[0][hs], True, dq, cu)
        dxk, dwk = oracle.conv_prologue_bwd(sub(xf[1]), tf[1][hs], True, dkk, cu)
        dxv, dwv = oracle.conv_prologue_bwd(sub(xf[2]), tf[2][hs], False, dvv, cu)
        la = sub(g[7])
        errs = {"dxq": slice_err(sub(g[0]), dxq, cu), "dxk": slice_err(sub(g[1]), dxk, cu),
                "dxv": slice_err(sub(g[2]), dxv, cu), "dwq": taps_err(g[3][hs], dwq),
                "dwk": taps_err(g[4][hs], dwk), "dwv": taps_err(g[5][hs], dwv),
                "dbeta": slice_err(sub(g[6])[..., None], db[..., None], cu),
                "dlog_alpha": slice_err(la if la.ndim == 4 else la[..., None],
                                        dla if dla.ndim == 4 else dla[..., None], cu),
                "ds0": state_err(g[8][:, hs], ds0)}
        return h, errs

    for h, errs in par_map(job, range(H)):
        log(f"    head {h}: " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()))
        for k_, v_ in errs.items():
            assert v_ < TOL[torch.bfloat16], (h, k_, v_)
