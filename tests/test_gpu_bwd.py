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
from gpu_util import TOL, log, np64, slice_err, state_err

pytestmark = pytest.mark.gpu


def run_bwd(inp, need_ds0=True):
    d = inp.to("cuda")
    g = gdn.chunk_bwd(d.q, d.k, d.v, d.beta, d.log_alpha, d.s0, d.do, d.ds_final,
                      chunk=inp.chunk, cu_seqlens=d.cu_seqlens, need_ds0=need_ds0)
    torch.cuda.synchronize()
    return g


def ref_bwd(inp):
    f = inp.f64
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.numpy()
    return oracle.gdn_bwd(f["q"], f["k"], f["v"], f["beta"], f["log_alpha"], f["s0"],
                          f["do"], f["ds_final"], inp.gate, cu_seqlens=cu)


def check(inp, name="", tol=None):
    log(f"[bwd] {name} q={tuple(inp.q.shape)} {inp.q.dtype} gate={inp.gate} "
        f"C={inp.chunk} seed={inp.seed}")
    got = run_bwd(inp)
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


@pytest.mark.parametrize("dk,dv", [(64, 32), (128, 128), (128, 256)])
@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_bf16_shapes(gpu_lib, dk, dv, gate):
    inp = synth.make_inputs(1, 150, 2, dk, dv, dtype=torch.bfloat16, gate=gate,
                            seed=32, s0_std=0.05, with_do=True, with_ds=True)
    check(inp, "bf16_shapes")


def test_fp32_dk128_channel_small_chunk(gpu_lib):
    inp = synth.make_inputs(1, 70, 2, 128, 64, dtype=torch.float32, gate="channel",
                            chunk=32, seed=33, s0_std=0.1, with_do=True, with_ds=True)
    check(inp, "fp32_dk128_channel_C32")


def test_fp32_dk128_channel_c64_unsupported(gpu_lib):
    inp = synth.make_inputs(1, 70, 2, 128, 64, dtype=torch.float32, gate="channel",
                            chunk=64, seed=33, with_do=True)
    with pytest.raises(gdn.GdnError) as e:
        run_bwd(inp)
    assert e.value.status == 4  # GDN_ERR_UNSUPPORTED


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


def test_varlen_training_batch_sampled(gpu_lib):
    # 16384 packed tokens, H=16, dk=128, dv=256, both gate modes: all heads run,
    # two heads of every sequence are compared with the oracle
    for name in ("varlen_16k_dv256", "varlen_16k_dv256_channel"):
        inp = synth.workload(name)
        log(f"[bwd] {name} lengths={np.diff(inp.cu_seqlens.numpy()).tolist()}")
        got = run_bwd(inp, need_ds0=False)
        f = inp.f64
        cu = inp.cu_seqlens.numpy()
        for h in (0, 11):
            hs = slice(h, h + 1)
            sub = lambda x: None if x is None else x[:, :, hs]
            ref = oracle.gdn_bwd(sub(f["q"]), sub(f["k"]), sub(f["v"]), sub(f["beta"]),
                                 sub(f["log_alpha"]), None, sub(f["do"]), None, inp.gate,
                                 cu_seqlens=cu)
            for nm, x, y in zip(("dq", "dk", "dv", "dbeta", "dlog_alpha"), got[:5], ref[:5]):
                xa = np64(x)[:, :, hs]
                ya = y
                if ya.ndim == 3:
                    xa, ya = xa[..., None], ya[..., None]
                e = slice_err(xa, ya, cu)
                log(f"    head {h} {nm} err={e:.2e}")
                assert e < TOL[torch.bfloat16], (name, h, nm, e)


@pytest.fixture
def seg_chunks(gpu_lib):
    yield gdn.set_segment_chunks
    gdn.set_segment_chunks(0)


@pytest.mark.parametrize("L", [1, 3])
@pytest.mark.parametrize("gate", ["scalar", "none", "channel"])
def test_segmented_state_recompute(seg_chunks, L, gate):
    # the chunk-start states recomputed by the split state pass (per-segment
    # maps, their chain, every segment from its entering state)
    inp = synth.make_inputs(2, 300, 2, 64, 32, dtype=torch.float32, gate=gate, chunk=32,
                            seed=41, s0_std=0.2, with_do=True, with_ds=True)
    seg_chunks(L)
    check(inp, name=f"segmented L={L}")


def test_segmented_state_recompute_varlen_bf16(seg_chunks):
    inp = synth.make_inputs(1, 0, 2, 128, 128, dtype=torch.bfloat16, gate="scalar",
                            chunk=64, seed=42, s0_std=0.05, with_do=True, with_ds=True,
                            lengths=[130, 0, 700, 64, 1])
    seg_chunks(2)
    check(inp, name="segmented varlen")
