"""GPU parity of gdn_chunk_fwd against the fp64 oracle (MI355X only).

Sizes span several chunks and 16-wide tiles and include ragged tails
(T not a multiple of the chunk), every supported chunk size, key sizes,
both dtypes, all gate modes, initial states and varlen packing with empty
sequences.  The headline shapes run at full size."""

import numpy as np
import pytest
import torch

import gated_delta_rule_79_amd as gdn
from gated_delta_rule_79_amd import synth
import oracle
from gpu_util import (TOL, Padded, dev, fwd_errors_per_head, log, np64, oracle_fwd,
                      par_map, slice_err, state_err)

pytestmark = pytest.mark.gpu


def run(inp, **kw):
    # outputs inside canary-padded buffers: a write past either end fails
    d = dev(inp)
    nseq = inp.q.shape[0] if inp.cu_seqlens is None else inp.cu_seqlens.numel() - 1
    H, dk, dv = inp.q.shape[2], inp.q.shape[3], inp.v.shape[3]
    po = Padded(tuple(inp.v.shape), inp.q.dtype)
    ps = Padded((nseq, H, dk, dv), torch.float32)
    o, sf = gdn.chunk_fwd(d.q, d.k, d.v, d.beta, d.log_alpha, d.s0,
                          chunk=inp.chunk, cu_seqlens=d.cu_seqlens, o=po.t, s_final=ps.t,
                          **kw)
    torch.cuda.synchronize()
    po.check("o")
    ps.check("s_final")
    return o, sf


def check(inp, tol=None, name="", **kw):
    log(f"[fwd] {name} q={tuple(inp.q.shape)} dtype={inp.q.dtype} gate={inp.gate} "
        f"C={inp.chunk} seed={inp.seed} {kw}")
    o, sf = run(inp, **kw)
    o_ref, sf_ref = oracle_fwd(inp)
    tol = tol or TOL[inp.q.dtype]
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.numpy()
    eo = slice_err(np64(o), o_ref, cu)
    es = state_err(np64(sf), sf_ref)
    log(f"    err o={eo:.3e} s_final={es:.3e} tol={tol}")
    assert eo < tol and es < tol, (eo, es)
    return o, sf


@pytest.mark.parametrize("gate", ["scalar", "none", "channel"])
def test_tiny_fp32(gpu_lib, gate):
    inp = synth.workload("tiny_fp32", gate=gate)
    check(inp, name="tiny_fp32")


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("gate", ["scalar", "none", "channel"])
def test_fp32_ragged(gpu_lib, C, gate):
    inp = synth.make_inputs(2, 100, 3, 32, 48, dtype=torch.float32, gate=gate,
                            chunk=C, seed=7, s0_std=0.3)
    check(inp, name="fp32_ragged")


@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 32), (128, 128), (128, 256)])
@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_bf16_shapes(gpu_lib, dk, dv, gate):
    inp = synth.make_inputs(2, 200, 2, dk, dv, dtype=torch.bfloat16, gate=gate,
                            chunk=64, seed=11, s0_std=0.05)
    check(inp, name="bf16_shapes")


@pytest.mark.parametrize("C", [16, 32])
def test_bf16_small_chunks(gpu_lib, C):
    inp = synth.make_inputs(1, 173, 4, 128, 64, dtype=torch.bfloat16, gate="scalar",
                            chunk=C, seed=12)
    check(inp, name="bf16_small_chunks")


def test_gate_dtype_fp32_with_bf16_io(gpu_lib):
    inp = synth.make_inputs(1, 130, 2, 128, 128, dtype=torch.bfloat16,
                            gate_dtype=torch.float32, gate="scalar", seed=13)
    check(inp, name="gate_fp32")


@pytest.mark.parametrize("gate", ["scalar", "channel", "none"])
def test_varlen(gpu_lib, gate):
    inp = synth.make_inputs(1, 0, 2, 128, 64, dtype=torch.bfloat16, gate=gate,
                            seed=14, lengths=[5, 0, 130, 64, 1, 77], s0_std=0.1)
    check(inp, name="varlen")


def test_varlen_fp32_chunk16(gpu_lib):
    inp = synth.make_inputs(1, 0, 3, 32, 32, dtype=torch.float32, gate="channel",
                            chunk=16, seed=15, lengths=[17, 0, 0, 33, 2])
    check(inp, name="varlen_fp32")


def test_alpha_to_zero_channel_exact_path(gpu_lib):
    # log alpha = -60 everywhere: erasure; the per-channel span is far beyond
    # the factored products' range, so the exact per-element path runs
    inp = synth.make_inputs(1, 70, 2, 64, 32, dtype=torch.float32, gate="channel",
                            seed=16, s0_std=1.0)
    inp.log_alpha.fill_(-60.0)
    inp.f64["log_alpha"][:] = -60.0
    check(inp, name="alpha0_channel")


def test_alpha_to_zero_scalar(gpu_lib):
    inp = synth.make_inputs(1, 70, 2, 64, 32, dtype=torch.float32, gate="scalar",
                            seed=17, s0_std=1.0)
    inp.log_alpha.fill_(-60.0)
    inp.f64["log_alpha"][:] = -60.0
    check(inp, name="alpha0_scalar")


def test_beta_up_to_two(gpu_lib):
    inp = synth.make_inputs(2, 150, 2, 64, 64, dtype=torch.float32, gate="scalar",
                            seed=18)
    inp.beta.mul_(2.0)
    inp.f64["beta"] = inp.beta.double().numpy()
    check(inp, name="beta_2")


def test_gate_none_equals_scalar_zero(gpu_lib):
    inp = synth.make_inputs(1, 140, 2, 128, 128, dtype=torch.bfloat16, gate="scalar",
                            seed=19, s0_std=0.02)
    d = dev(inp)
    o1, s1 = gdn.chunk_fwd(d.q, d.k, d.v, d.beta, torch.zeros_like(d.log_alpha), d.s0)
    o2, s2 = gdn.chunk_fwd(d.q, d.k, d.v, d.beta, None, d.s0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_chunk_size_invariance_and_determinism(gpu_lib):
    inp = synth.make_inputs(1, 250, 2, 64, 64, dtype=torch.float32, gate="channel",
                            seed=20, s0_std=0.1)
    outs = []
    for C in (16, 32, 64):
        inp.chunk = C
        outs.append(run(inp))
    for o, s in outs[1:]:
        assert slice_err(np64(o), np64(outs[0][0])) < 1e-5
        assert state_err(np64(s), np64(outs[0][1])) < 1e-5
    a = run(inp)
    b = run(inp)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_split_and_resume(gpu_lib):
    inp = synth.make_inputs(1, 300, 2, 128, 128, dtype=torch.float32, gate="scalar",
                            seed=21, s0_std=0.1)
    d = dev(inp)
    o, s = gdn.chunk_fwd(d.q, d.k, d.v, d.beta, d.log_alpha, d.s0)
    cut = 110
    oa, sa = gdn.chunk_fwd(d.q[:, :cut].contiguous(), d.k[:, :cut].contiguous(),
                           d.v[:, :cut].contiguous(), d.beta[:, :cut].contiguous(),
                           d.log_alpha[:, :cut].contiguous(), d.s0)
    ob, sb = gdn.chunk_fwd(d.q[:, cut:].contiguous(), d.k[:, cut:].contiguous(),
                           d.v[:, cut:].contiguous(), d.beta[:, cut:].contiguous(),
                           d.log_alpha[:, cut:].contiguous(), sa)
    torch.cuda.synchronize()
    assert slice_err(np64(torch.cat([oa, ob], 1)), np64(o)) < 1e-5
    assert state_err(np64(sb), np64(s)) < 1e-5


def test_empty_sequence_copies_state(gpu_lib):
    inp = synth.make_inputs(2, 0, 2, 64, 32, dtype=torch.bfloat16, seed=22,
                            s0_std=1.0)
    o, sf = run(inp)
    assert o.shape == (2, 0, 2, 32)
    assert torch.equal(sf.cpu(), inp.s0)


def test_headline_full_size(gpu_lib):
    # T=4096, H=16, d=128, bf16, B=1: every head against the oracle
    inp = synth.workload("fwd_t4096_h16")
    check(inp, name="fwd_t4096_h16")


def _check_heads(inp, o, sf, name, tol=None, heads=None):
    tol = tol or TOL[inp.q.dtype]
    for h, eo, es, er in fwd_errors_per_head(inp, o, sf, heads=heads):
        log(f"    {name} head {h}: err o={eo:.3e} s={es:.3e} (worst token row {er:.2e})")
        assert eo < tol and es < tol, (name, h, eo, es)


def test_layer_b8_all_rows(gpu_lib):
    # B=8, T=2048, H=8, d=128: every batch row and head against the oracle
    inp = synth.workload("layer_b8_t2048")
    log("[fwd] layer_b8_t2048")
    o, sf = run(inp)
    f = inp.f64
    xo, xs = np64(o), np64(sf)

    def job(b):
        sl = slice(b, b + 1)
        o_ref, s_ref = oracle.gdn_fwd(f["q"][sl], f["k"][sl], f["v"][sl], f["beta"][sl],
                                      f["log_alpha"][sl], None, "scalar")
        return b, slice_err(xo[sl], o_ref), state_err(xs[sl], s_ref)

    for b, eo, es in par_map(job, range(8)):
        log(f"    batch {b}: err o={eo:.3e} s={es:.3e}")
        assert eo < TOL[torch.bfloat16] and es < TOL[torch.bfloat16], (b, eo, es)


def test_long_context_all_heads(gpu_lib):
    # B=1, T=65536, H=16, d=128, initial and final state (64-chunk segments):
    # every head compared with the oracle over the whole sequence
    inp = synth.workload("long_t65536")
    log("[fwd] long_t65536")
    o, sf = run(inp)
    _check_heads(inp, o, sf, "long_t65536")


def test_gate_none_long_context(gpu_lib):
    # alpha = 1 (the plain delta rule) over 65536 tokens with an initial
    # state: nothing decays the rounding of the segment transitions away
    inp = synth.workload("long_t65536", gate="none")
    log("[fwd] long_t65536 gate=none")
    o, sf = run(inp)
    _check_heads(inp, o, sf, "long_t65536_none")


@pytest.mark.parametrize("name", ["varlen_16k_dv256", "varlen_16k_dv256_channel"])
def test_varlen_training_forward_all_heads(gpu_lib, name):
    # 16384 packed tokens, H=16, dk=128, dv=256: every head of every sequence
    inp = synth.workload(name)
    log(f"[fwd] {name} lengths={np.diff(inp.cu_seqlens.numpy()).tolist()}")
    o, sf = run(inp)
    _check_heads(inp, o, sf, name)


def _channel_threshold(C):
    # per-token log alpha at which a chunk's per-channel log-gate half-span
    # (C - 1) |log alpha| / 2 reaches the factored products' limit of 80
    return 160.0 / (C - 1)


@pytest.mark.parametrize("side", [0.95, 1.05])
@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_channel_gate_near_factored_limit(gpu_lib, side, C, dtype):
    # a few key channels decay at a constant rate whose half-span inside a
    # chunk sits just below (factored products, factors near e^+-76) or just
    # above (exact per-element path) the switch; the others follow the usual
    # distribution
    inp = synth.make_inputs(1, 3 * C + 13, 2, 128, 64, dtype=dtype, gate="channel",
                            chunk=C, seed=50 + C, s0_std=0.1)
    la = -side * _channel_threshold(C)
    chans = [0, 5, 77, 127]
    inp.log_alpha[..., chans] = la
    inp.f64["log_alpha"] = inp.log_alpha.double().numpy()
    check(inp, name=f"channel_near_limit C={C} log_alpha={la:.3f}")


# ---------------------------------------------------- segmented state pass ---
# The state pass can split each sequence into segments of L chunks: segment
# maps [M0 | Phi] in parallel, a sequential combine, then the segments from
# their entering states.  Forced segment lengths cover one-chunk segments,
# ragged last segments, single-segment sequences, empty sequences in varlen
# batches and every dtype / gate / key size.

@pytest.mark.parametrize("L", [1, 2, 3, 5])
@pytest.mark.parametrize("gate", ["scalar", "none", "channel"])
def test_segmented_fp32(gpu_lib, L, gate):
    inp = synth.make_inputs(2, 150, 3, 32, 48, dtype=torch.float32, gate=gate,
                            chunk=16, seed=41, s0_std=0.3)
    check(inp, name=f"segmented_fp32 L={L}", seg_chunks=L)


@pytest.mark.parametrize("C", [16, 32, 64])
def test_segmented_fp32_dk128(gpu_lib, C):
    inp = synth.make_inputs(1, 333, 2, 128, 64, dtype=torch.float32, gate="channel",
                            chunk=C, seed=42, s0_std=0.1)
    check(inp, name=f"segmented_fp32_dk128 C={C}", seg_chunks=2)


@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 32), (128, 128), (128, 256)])
@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_segmented_bf16(gpu_lib, dk, dv, gate):
    inp = synth.make_inputs(1, 700, 2, dk, dv, dtype=torch.bfloat16, gate=gate,
                            chunk=64, seed=43, s0_std=0.05)
    check(inp, name="segmented_bf16", seg_chunks=3)


# The transition pass writes a segment's map Phi as operand fragments, one
# 8-byte half of a fragment lane per 16-column slab; with dv / 16 + dk / 16
# slabs per (segment, head) in groups of 16, a fragment's two halves can come
# from different waves (odd dv / 16) or different workgroups (dv = 144,
# dk = 128: group 0 ends inside Phi).
@pytest.mark.parametrize("dk,dv,dtype,C", [(128, 144, torch.bfloat16, 64),
                                           (64, 208, torch.bfloat16, 32),
                                           (64, 48, torch.bfloat16, 64),
                                           (128, 144, torch.float32, 32)])
def test_segmented_phi_halves_from_different_slabs(gpu_lib, dk, dv, dtype, C):
    inp = synth.make_inputs(1, 400, 2, dk, dv, dtype=dtype, gate="scalar", chunk=C,
                            seed=46, s0_std=0.1)
    check(inp, name=f"segmented_phi_halves dk={dk} dv={dv}", seg_chunks=2)


@pytest.mark.parametrize("gate", ["scalar", "none", "channel"])
def test_segmented_varlen(gpu_lib, gate):
    inp = synth.make_inputs(1, 0, 2, 128, 64, dtype=torch.bfloat16, gate=gate,
                            seed=44, lengths=[5, 0, 300, 64, 1, 177, 129, 0],
                            s0_std=0.1)
    check(inp, name="segmented_varlen", seg_chunks=2)


def test_segmented_varlen_fp32_no_s0(gpu_lib):
    inp = synth.make_inputs(1, 0, 3, 64, 32, dtype=torch.float32, gate="scalar",
                            chunk=16, seed=45, lengths=[40, 0, 97, 16, 33])
    check(inp, name="segmented_varlen_fp32", seg_chunks=1)


def test_segmented_deterministic_and_unsplit_agree(gpu_lib):
    inp = synth.make_inputs(1, 1000, 2, 128, 128, dtype=torch.float32, gate="scalar",
                            seed=46, s0_std=0.1)
    o0, s0 = run(inp, seg_chunks=-1)
    o1, s1 = run(inp, seg_chunks=4)
    o2, s2 = run(inp, seg_chunks=4)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert slice_err(np64(o1), np64(o0)) < 1e-5
    assert state_err(np64(s1), np64(s0)) < 1e-5


def test_segmented_empty_batch_keeps_state(gpu_lib):
    inp = synth.make_inputs(2, 0, 2, 64, 32, dtype=torch.bfloat16, seed=47,
                            s0_std=1.0)
    o, sf = run(inp, seg_chunks=2)
    assert torch.equal(sf.cpu(), inp.s0)
