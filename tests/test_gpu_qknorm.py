"""GPU parity of gdn_chunk_fwd_qknorm (the forward that L2-normalises q and
k per token and head itself) against the fp64 oracle (MI355X only).

Inputs: the usual unit rows times log-uniform row scales in [0.05, 20], with
about one row in ten set to zero (zero rows must stay zero), so that a kernel
that skipped or misplaced a normalisation fails by a wide margin.  Covers both
per-token gate modes, both dtypes, every chunk size, ragged tails, varlen
packing with empty sequences, initial states, split state passes and the
headline size."""

import numpy as np
import pytest
import torch

import gated_delta_rule_79_amd as gdn
import oracle
from gated_delta_rule_79_amd import _lib, synth
from gpu_util import TOL, dev, log, np64, par_map, slice_err, state_err

pytestmark = pytest.mark.gpu

RAW = (0.05, 20.0, 0.1)


def check(inp, name="", **kw):
    log(f"[qknorm] {name} q={tuple(inp.q.shape)} v={tuple(inp.v.shape)} "
        f"dtype={inp.q.dtype} gate={inp.gate} C={inp.chunk} seed={inp.seed}")
    d = dev(inp)
    o, sf = gdn.chunk_fwd(d.q, d.k, d.v, d.beta, d.log_alpha, d.s0, chunk=inp.chunk,
                          cu_seqlens=d.cu_seqlens, qk_l2norm=True, **kw)
    torch.cuda.synchronize()
    f = inp.f64
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.numpy()
    o_ref, sf_ref = oracle.gdn_fwd_qknorm(f["q"], f["k"], f["v"], f["beta"],
                                          f["log_alpha"], f["s0"], inp.gate,
                                          cu_seqlens=cu)
    tol = TOL[inp.q.dtype]
    eo = slice_err(np64(o), o_ref, cu)
    es = state_err(np64(sf), sf_ref)
    log(f"    err o={eo:.3e} s_final={es:.3e} tol={tol}")
    assert eo < tol and es < tol, (eo, es)
    return o, sf


@pytest.mark.parametrize("gate", ["scalar", "none"])
@pytest.mark.parametrize("C", [16, 32, 64])
def test_qknorm_fp32(gpu_lib, gate, C):
    inp = synth.make_inputs(2, 77, 3, 32, 48, dtype=torch.float32, gate=gate,
                            chunk=C, seed=71, s0_std=0.3, raw_qk=RAW)
    check(inp, name="fp32")


@pytest.mark.parametrize("dk", [16, 64, 128])
def test_qknorm_fp32_dk(gpu_lib, dk):
    inp = synth.make_inputs(1, 130, 2, dk, 32, dtype=torch.float32, gate="scalar",
                            chunk=64, seed=72, s0_std=0.2, raw_qk=RAW)
    check(inp, name="fp32 dk")


@pytest.mark.parametrize("dk,dv", [(16, 16), (128, 128), (128, 256)])
@pytest.mark.parametrize("gate", ["scalar", "none"])
def test_qknorm_bf16(gpu_lib, dk, dv, gate):
    inp = synth.make_inputs(1, 200, 2, dk, dv, dtype=torch.bfloat16, gate=gate,
                            chunk=64, seed=73, s0_std=0.05, raw_qk=RAW)
    check(inp, name="bf16")


def test_qknorm_varlen(gpu_lib):
    inp = synth.make_inputs(1, 0, 2, 64, 32, dtype=torch.float32, gate="scalar",
                            chunk=32, seed=74, lengths=[5, 0, 41, 16, 1, 70],
                            s0_std=0.2, raw_qk=RAW)
    check(inp, name="varlen")


@pytest.mark.parametrize("L", [1, 3])
def test_qknorm_segmented(gpu_lib, L):
    inp = synth.make_inputs(1, 600, 2, 128, 64, dtype=torch.bfloat16, gate="scalar",
                            chunk=64, seed=75, s0_std=0.05, raw_qk=RAW)
    check(inp, name=f"segmented L={L}", seg_chunks=L)


def test_qknorm_headline_full_size(gpu_lib):
    # T=4096, H=16, d=128, bf16, B=1, raw rows: every head against the oracle
    inp = synth.make_inputs(1, 4096, 16, 128, 128, dtype=torch.bfloat16,
                            gate="scalar", chunk=64, seed=76, raw_qk=RAW)
    check(inp, name="t4096_h16")


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_qknorm_training_batch_all_heads(gpu_lib, gate):
    # the packed training batch (16384 tokens in sequences of 512 to 8192,
    # H16, dk128, dv256, bf16) with raw q, k rows: the scalar gate
    # normalises inside the prep, the per-channel gate through the prologue
    # pass; every head against the oracle
    inp = synth.make_inputs(1, 16384, 16, 128, 256, dtype=torch.bfloat16, gate=gate,
                            chunk=64, seed=79, varlen=(16384, 512, 8192), s0_std=0.05,
                            raw_qk=RAW)
    cu = inp.cu_seqlens.numpy()
    log(f"[qknorm] packed training batch gate={gate} lengths={np.diff(cu).tolist()}")
    d = dev(inp)
    o, sf = gdn.chunk_fwd(d.q, d.k, d.v, d.beta, d.log_alpha, d.s0, chunk=64,
                          cu_seqlens=d.cu_seqlens, qk_l2norm=True)
    torch.cuda.synchronize()
    f = inp.f64
    xo, xs = np64(o), np64(sf)

    def job(h):
        hs = slice(h, h + 1)
        sub = lambda a: a[:, :, hs]
        o_ref, s_ref = oracle.gdn_fwd_qknorm(sub(f["q"]), sub(f["k"]), sub(f["v"]),
                                             sub(f["beta"]), sub(f["log_alpha"]),
                                             f["s0"][:, hs], gate, cu_seqlens=cu)
        return h, slice_err(xo[:, :, hs], o_ref, cu), state_err(xs[:, hs], s_ref)

    for h, eo, es in par_map(job, range(16)):
        log(f"    head {h}: err o={eo:.3e} s={es:.3e}")
        assert eo < TOL[torch.bfloat16] and es < TOL[torch.bfloat16], (h, eo, es)


def test_qknorm_of_unit_rows_is_the_plain_forward(gpu_lib):
    # rows that are already unit vectors: the same result as gdn_chunk_fwd up
    # to the rounding of the norm
    inp = synth.make_inputs(1, 300, 4, 128, 128, dtype=torch.float32, gate="scalar",
                            chunk=64, seed=77, s0_std=0.1)
    d = dev(inp)
    o1, s1 = gdn.chunk_fwd(d.q, d.k, d.v, d.beta, d.log_alpha, d.s0)
    o2, s2 = gdn.chunk_fwd(d.q, d.k, d.v, d.beta, d.log_alpha, d.s0, qk_l2norm=True)
    torch.cuda.synchronize()
    e = max(slice_err(np64(o2), np64(o1)), state_err(np64(s2), np64(s1)))
    log(f"[qknorm] unit rows vs plain forward: {e:.3e}")
    assert e < 2e-5


def test_qknorm_scale_invariance(gpu_lib):
    # q and k rows times powers of two (exact in every dtype) give the same
    # result
    inp = synth.make_inputs(1, 257, 2, 128, 128, dtype=torch.bfloat16, gate="scalar",
                            chunk=64, seed=78, s0_std=0.05, raw_qk=RAW)
    d = dev(inp)
    g = torch.Generator().manual_seed(5)
    sq = (2.0 ** torch.randint(-6, 7, d.q.shape[:3] + (1,), generator=g)).to(d.q)
    sk = (2.0 ** torch.randint(-6, 7, d.k.shape[:3] + (1,), generator=g)).to(d.k)
    o1, s1 = gdn.chunk_fwd(d.q, d.k, d.v, d.beta, d.log_alpha, d.s0, qk_l2norm=True)
    o2, s2 = gdn.chunk_fwd((d.q * sq).contiguous(), (d.k * sk).contiguous(), d.v,
                           d.beta, d.log_alpha, d.s0, qk_l2norm=True)
    torch.cuda.synchronize()
    e = max(slice_err(np64(o2), np64(o1)), state_err(np64(s2), np64(s1)))
    log(f"[qknorm] power-of-two rescaled rows: {e:.3e}")
    # a bf16 rounding of a normalised k element may land on the other side
    # when the norm's last bit differs; a missed normalisation is off by O(1)
    assert e < 2e-3


def test_qknorm_plan_matches_call(gpu_lib):
    inp = synth.make_inputs(1, 100, 2, 64, 64, dtype=torch.bfloat16, gate="scalar",
                            chunk=64, seed=79, raw_qk=RAW)
    d = dev(inp)
    plan = gdn.FwdPlan(d.q, d.k, d.v, d.beta, d.log_alpha, qk_l2norm=True)
    o1, _ = plan.run()
    o2, _ = gdn.chunk_fwd(d.q, d.k, d.v, d.beta, d.log_alpha, qk_l2norm=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    # the per-channel gate: normalised rows from the prologue pass
    ch = synth.make_inputs(1, 40, 2, 64, 64, dtype=torch.float32, gate="channel",
                           chunk=64, seed=80, raw_qk=RAW)
    dc = dev(ch)
    plan = gdn.FwdPlan(dc.q, dc.k, dc.v, dc.beta, dc.log_alpha, qk_l2norm=True)
    o1, _ = plan.run()
    o2, _ = gdn.chunk_fwd(dc.q, dc.k, dc.v, dc.beta, dc.log_alpha, qk_l2norm=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_qknorm_channel_gate(gpu_lib, C, dtype):
    inp = synth.make_inputs(2, 150, 2, 128, 64, dtype=dtype, gate="channel", chunk=C,
                            seed=81, s0_std=0.1, raw_qk=RAW)
    check(inp, name="channel")


def test_qknorm_channel_gate_varlen_full_size(gpu_lib):
    # the per-channel training batch's shapes (16384 packed tokens, H16,
    # dk128, dv256) with rows that are not unit vectors
    inp = synth.make_inputs(1, 16384, 16, 128, 256, dtype=torch.bfloat16, gate="channel",
                            chunk=64, seed=82, varlen=(16384, 512, 8192), raw_qk=RAW)
    log(f"[qknorm] channel varlen lengths={np.diff(inp.cu_seqlens.numpy()).tolist()}")
    d = dev(inp)
    o, sf = gdn.chunk_fwd(d.q, d.k, d.v, d.beta, d.log_alpha, None, chunk=64,
                          cu_seqlens=d.cu_seqlens, qk_l2norm=True)
    torch.cuda.synchronize()
    f = inp.f64
    cu = inp.cu_seqlens.numpy()
    xo, xs = np64(o), np64(sf)

    def job(h):
        hs = slice(h, h + 1)
        o_ref, s_ref = oracle.gdn_fwd_qknorm(f["q"][:, :, hs], f["k"][:, :, hs],
                                             f["v"][:, :, hs], f["beta"][:, :, hs],
                                             f["log_alpha"][:, :, hs], None, "channel",
                                             cu_seqlens=cu)
        return h, slice_err(xo[:, :, hs], o_ref, cu), state_err(xs[:, hs], s_ref)

    for h, eo, es in par_map(job, range(16)):
        log(f"    head {h}: err o={eo:.3e} s={es:.3e}")
        assert eo < TOL[torch.bfloat16] and es < TOL[torch.bfloat16], (h, eo, es)


def test_qknorm_empty_sequences_copy_state(gpu_lib):
    inp = synth.make_inputs(2, 0, 2, 64, 32, dtype=torch.bfloat16, seed=1011, s0_std=1.0,
                            raw_qk=(0.1, 10.0, 0.0))
    log("[qknorm] empty")
    d = inp.to("cuda")
    o, sf = gdn.chunk_fwd(d.q, d.k, d.v, d.beta, d.log_alpha, d.s0, qk_l2norm=True)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 2, 32)
    assert torch.equal(sf.cpu(), inp.s0)
