"""GPU parity of gdn_chunk_bwd against the fp64 oracle's adjoint (MI355X).

The oracle's adjoint is itself pinned by central finite differences
(tests/test_oracle_pins.py).  Gradients are compared per (sequence, head)
slice with the normwise error of the forward tests."""

import numpy as np
import pytest
import torch

import gated_delta_rule_79_amd as gdn
import oracle
from gated_delta_rule_79_amd import synth
from gpu_util import TOL, Padded, bwd_errors_per_head, log, np64, slice_err, state_err

pytestmark = pytest.mark.gpu


def run_bwd(inp, need_ds0=True, **kw):
    # every gradient inside a canary-padded buffer: a write past either end
    # fails
    d = inp.to("cuda")
    nseq = inp.q.shape[0] if inp.cu_seqlens is None else inp.cu_seqlens.numel() - 1
    H, dk, dv = inp.q.shape[2], inp.q.shape[3], inp.v.shape[3]
    pads = [Padded(tuple(inp.q.shape), inp.q.dtype), Padded(tuple(inp.k.shape), inp.k.dtype),
            Padded(tuple(inp.v.shape), inp.v.dtype),
            Padded(tuple(inp.beta.shape), torch.float32),
            None if inp.log_alpha is None else Padded(tuple(inp.log_alpha.shape), torch.float32),
            Padded((nseq, H, dk, dv), torch.float32) if need_ds0 else None]
    g = gdn.chunk_bwd(d.q, d.k, d.v, d.beta, d.log_alpha, d.s0, d.do, d.ds_final,
                      chunk=inp.chunk, cu_seqlens=d.cu_seqlens, need_ds0=need_ds0,
                      out=[None if x is None else x.t for x in pads], **kw)
    torch.cuda.synchronize()
    for nm, x in zip(("dq", "dk", "dv", "dbeta", "dlog_alpha", "ds0"), pads):
        if x is not None:
            x.check(nm)
    return g


def ref_bwd(inp):
    f = inp.f64
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.numpy()
    return oracle.gdn_bwd(f["q"], f["k"], f["v"], f["beta"], f["log_alpha"], f["s0"],
                          f["do"], f["ds_final"], inp.gate, cu_seqlens=cu)


def check(inp, name="", tol=None, **kw):
    log(f"[bwd] {name} q={tuple(inp.q.shape)} {inp.q.dtype} gate={inp.gate} "
        f"C={inp.chunk} seed={inp.seed} {kw}")
    got = run_bwd(inp, **kw)
    ref = ref_bwd(inp)
    tol = tol or TOL[inp.q.dtype]
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.numpy()
    errs = {}
    for nm, x, y in zip(("dq", "dk", "dv", "dbeta", "dlog_alpha"), got[:5], ref[:5]):
        if y is None:
            assert x is None
            continue
        xa, ya = np64(x), y
        if ya.ndim == 3:
            xa, ya = xa[..., None], ya[..., None]
        errs[nm] = slice_err(xa, ya, cu)
    errs["ds0"] = state_err(np64(got[5]), ref[5])
    log("    " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) + f" tol={tol}")
    for k, v in errs.items():
        assert v < tol, (k, v)
    return got


@pytest.mark.parametrize("gate", ["scalar", "none", "channel"])
def test_tiny_fp32(gpu_lib, gate):
    inp = synth.make_inputs(1, 64, 2, 16, 16, dtype=torch.float32, gate=gate,
                            chunk=16, seed=1001, s0_std=0.1, with_do=True, with_ds=True)
    check(inp, "tiny")


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("gate", ["scalar", "none", "channel"])
def test_fp32_ragged(gpu_lib, C, gate):
    inp = synth.make_inputs(2, 90, 2, 32, 48, dtype=torch.float32, gate=gate, chunk=C,
                            seed=31, s0_std=0.3, with_do=True, with_ds=True)
    check(inp, "fp32_ragged")


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 48), (64, 32), (128, 128), (128, 256)])
@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_bf16_shapes(gpu_lib, dk, dv, gate):
    inp = synth.make_inputs(1, 150, 2, dk, dv, dtype=torch.bfloat16, gate=gate,
                            seed=32, s0_std=0.05, with_do=True, with_ds=True)
    check(inp, "bf16_shapes")


def test_fp32_dk128_channel_small_chunk(gpu_lib):
    inp = synth.make_inputs(1, 70, 2, 128, 64, dtype=torch.float32, gate="channel",
                            chunk=32, seed=33, s0_std=0.1, with_do=True, with_ds=True)
    check(inp, "fp32_dk128_channel_C32")


@pytest.mark.parametrize("seg", [0, 1])
def test_fp32_dk128_channel_c64(gpu_lib, seg):
    # the library runs this case on 32-token chunks (the 64-token LDS plan
    # does not fit for fp32 rows); varlen with a ragged tail, and a fixed
    # segment length that it rescales to the same number of tokens
    inp = synth.make_inputs(1, 0, 2, 128, 64, dtype=torch.float32, gate="channel",
                            chunk=64, seed=33, lengths=[150, 0, 70], s0_std=0.1,
                            with_do=True, with_ds=True)
    check(inp, "fp32_dk128_channel_C64", seg_chunks=seg)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_varlen(gpu_lib, gate):
    inp = synth.make_inputs(1, 0, 2, 64, 64, dtype=torch.bfloat16, gate=gate, seed=34,
                            lengths=[5, 0, 130, 64, 1, 77], s0_std=0.1, with_do=True,
                            with_ds=True)
    check(inp, "varlen")


def test_beta_to_two_and_alpha_to_zero(gpu_lib):
    inp = synth.make_inputs(1, 80, 2, 32, 32, dtype=torch.float32, gate="scalar",
                            seed=35, s0_std=0.5, with_do=True, with_ds=True)
    inp.beta.mul_(2.0)
    inp.f64["beta"] = inp.beta.double().numpy()
    inp.log_alpha[:, 40:] = -30.0
    inp.f64["log_alpha"] = inp.log_alpha.double().numpy()
    check(inp, "beta2_alpha0")


def test_no_initial_state_no_final_grad(gpu_lib):
    inp = synth.make_inputs(2, 100, 2, 64, 64, dtype=torch.float32, gate="scalar",
                            seed=36, with_do=True)
    check(inp, "no_s0")


@pytest.mark.parametrize("gate", ["scalar", "none"])
def test_empty_sequences(gpu_lib, gate):
    # T = 0: no step of the recurrence, so S_final = S0 and the gradient of
    # <dS_final, S_final> w.r.t. S0 is dS_final itself; without dS_final it is 0
    for with_ds in (True, False):
        inp = synth.make_inputs(2, 0, 2, 64, 32, dtype=torch.bfloat16, gate=gate,
                                seed=38, s0_std=0.1, with_do=True, with_ds=with_ds)
        log(f"[bwd] empty gate={gate} with_ds={with_ds}")
        dq, dk, dv, db, dla, ds0 = run_bwd(inp)
        assert dq.shape == (2, 0, 2, 64) and dv.shape == (2, 0, 2, 32) and db.numel() == 0
        want = inp.ds_final if with_ds else torch.zeros(2, 2, 64, 32)
        assert torch.equal(ds0.cpu(), want)


def test_deterministic(gpu_lib):
    inp = synth.make_inputs(1, 200, 2, 128, 128, dtype=torch.bfloat16, gate="channel",
                            seed=37, s0_std=0.05, with_do=True, with_ds=True)
    a = run_bwd(inp)
    b = run_bwd(inp)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name", ["varlen_16k_dv256", "varlen_16k_dv256_channel"])
def test_varlen_training_batch_all_heads(gpu_lib, name):
    # 16384 packed tokens, H=16, dk=128, dv=256: every head of every sequence
    inp = synth.workload(name)
    log(f"[bwd] {name} lengths={np.diff(inp.cu_seqlens.numpy()).tolist()}")
    got = run_bwd(inp, need_ds0=False)
    for h, errs in bwd_errors_per_head(inp, got):
        log(f"    head {h} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
        for k, v in errs.items():
            assert v < TOL[torch.bfloat16], (name, h, k, v)


def test_long_context_two_heads(gpu_lib):
    # T=65536 (1024 chunks per chain, the split reverse pass) with an initial
    # state and a final-state gradient: both heads compared in full
    inp = synth.make_inputs(1, 65536, 2, 128, 128, dtype=torch.bfloat16, gate="scalar",
                            seed=1014, s0_std=0.02, with_do=True, with_ds=True)
    log("[bwd] T=65536 H=2")
    got = run_bwd(inp)
    for h, errs in bwd_errors_per_head(inp, got):
        log(f"    head {h} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
        for k, v in errs.items():
            assert v < TOL[torch.bfloat16], (h, k, v)


@pytest.mark.parametrize("side", [0.95, 1.05])
@pytest.mark.parametrize("C", [32, 64])
def test_channel_gate_near_factored_limit(gpu_lib, side, C):
    # the per-channel backward's factored products near their e^+-80 limit
    # (see the forward test of the same name)
    inp = synth.make_inputs(1, 3 * C + 13, 2, 128, 64, dtype=torch.bfloat16,
                            gate="channel", chunk=C, seed=60 + C, s0_std=0.1,
                            with_do=True, with_ds=True)
    inp.log_alpha[..., [0, 5, 77, 127]] = -side * 160.0 / (C - 1)
    inp.f64["log_alpha"] = inp.log_alpha.double().numpy()
    check(inp, f"channel_near_limit C={C} side={side}")


@pytest.mark.parametrize("C,dtype,dk", [(16, torch.float32, 64), (32, torch.float32, 64),
                                         (64, torch.float32, 64), (64, torch.bfloat16, 128)])
@pytest.mark.parametrize("which", ["all", "some"])
def test_channel_gate_exact_path(gpu_lib, C, dtype, dk, which):
    # log alpha = -60 on every channel (erasure) or on four of them: the
    # chunk's channel span is far beyond the factored products' range, so
    # the per-element path runs in every product of the gradient kernel
    inp = synth.make_inputs(1, 2 * C + 9, 2, dk, 64, dtype=dtype, gate="channel", chunk=C,
                            seed=70 + C, s0_std=0.5, with_do=True, with_ds=True)
    if which == "some":
        inp.log_alpha[..., [1, 6, 30, dk - 1]] = -60.0
        inp.f64["log_alpha"] = inp.log_alpha.double().numpy()
        check(inp, f"channel_exact C={C} some")
        return
    inp.log_alpha.fill_(-60.0)
    inp.f64["log_alpha"] = inp.log_alpha.double().numpy()
    log(f"[bwd] channel_exact C={C} all q={tuple(inp.q.shape)} {inp.q.dtype}")
    got, ref = run_bwd(inp), ref_bwd(inp)
    tol = TOL[inp.q.dtype]
    errs = {nm: slice_err(np64(x), y) for nm, x, y in
            zip(("dq", "dk", "dv"), got[:3], ref[:3])}
    errs["dbeta"] = slice_err(np64(got[3])[..., None], ref[3][..., None])
    errs["ds0"] = state_err(np64(got[5]), ref[5])
    # every decay across tokens is e^-60, so the true d log alpha is ~1e-26:
    # its error is measured against the size of the terms whose rounding it
    # carries, the products dq (.) q and dk (.) k of each slice
    f = inp.f64
    scale = max(np.abs(ref[0] * f["q"]).max(), np.abs(ref[1] * f["k"]).max())
    errs["dlog_alpha_abs"] = float(np.abs(np64(got[4]) - ref[4]).max() / scale)
    log("    " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) + f" tol={tol}")
    for k, v in errs.items():
        assert v < tol, (k, v)


@pytest.mark.parametrize("L", [1, 3])
@pytest.mark.parametrize("gate", ["scalar", "none", "channel"])
def test_segmented_state_recompute(gpu_lib, L, gate):
    # the chunk-start states recomputed by the split state pass (per-segment
    # maps, their chain, every segment from its entering state)
    inp = synth.make_inputs(2, 300, 2, 64, 32, dtype=torch.float32, gate=gate, chunk=32,
                            seed=41, s0_std=0.2, with_do=True, with_ds=True)
    check(inp, name=f"segmented L={L}", seg_chunks=L)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_segmented_phi_halves_from_different_workgroups(gpu_lib, dtype):
    # dv = 144, dk = 128: the transition pass's first slab group ends inside
    # Phi, so two workgroups write the halves of its last fragment column;
    # the split reverse pass applies every segment's Phi^T
    inp = synth.make_inputs(1, 400, 2, 128, 144, dtype=dtype, gate="scalar", chunk=32,
                            seed=47, s0_std=0.1, with_do=True, with_ds=True)
    check(inp, name="segmented phi halves", seg_chunks=2)


def test_segmented_state_recompute_varlen_bf16(gpu_lib):
    inp = synth.make_inputs(1, 0, 2, 128, 128, dtype=torch.bfloat16, gate="scalar",
                            chunk=64, seed=42, s0_std=0.05, with_do=True, with_ds=True,
                            lengths=[130, 0, 700, 64, 1])
    check(inp, name="segmented varlen", seg_chunks=2)
