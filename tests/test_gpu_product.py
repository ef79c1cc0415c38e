"""GPU parity of gdn_chunk_fwd_product (Householder-product transitions:
nh delta steps per token after one decay) against the fp64 oracle
(MI355X only).  Covers nh = 1, 2, 4, both per-token gate modes, both
dtypes, ragged tails (steps and tokens), every chunk size, varlen packing
with empty sequences, initial states and split state passes."""

import numpy as np
import pytest
import torch

import gated_delta_rule_79_amd as gdn
import oracle
from gated_delta_rule_79_amd import _lib, synth
from gpu_util import TOL, dev, log, np64, slice_err, state_err

pytestmark = pytest.mark.gpu


def check(inp, name="", **kw):
    nh = inp.k.shape[2]
    log(f"[product] {name} q={tuple(inp.q.shape)} nh={nh} dtype={inp.q.dtype} "
        f"gate={inp.gate} C={inp.chunk} seed={inp.seed}")
    d = dev(inp)
    o, sf = gdn.chunk_fwd_product(d.q, d.k, d.v, d.beta, d.log_alpha, d.s0,
                                  chunk=inp.chunk, cu_seqlens=d.cu_seqlens, **kw)
    torch.cuda.synchronize()
    f = inp.f64
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.numpy()
    o_ref, sf_ref = oracle.deltaproduct_fwd(f["q"], f["k"], f["v"], f["beta"],
                                            f["log_alpha"], f["s0"], inp.gate,
                                            cu_seqlens=cu)
    tol = TOL[inp.q.dtype]
    eo = slice_err(np64(o), o_ref, cu)
    es = state_err(np64(sf), sf_ref)
    log(f"    err o={eo:.3e} s_final={es:.3e} tol={tol}")
    assert eo < tol and es < tol, (eo, es)
    return o, sf


@pytest.mark.parametrize("nh", [1, 2, 4])
@pytest.mark.parametrize("gate", ["scalar", "none"])
@pytest.mark.parametrize("C", [16, 64])
def test_product_fp32(gpu_lib, nh, gate, C):
    inp = synth.make_product_inputs(2, 37, 3, 32, 48, nh, dtype=torch.float32,
                                    gate=gate, chunk=C, seed=61, s0_std=0.3)
    check(inp, name="fp32")


@pytest.mark.parametrize("nh", [2, 4])
@pytest.mark.parametrize("dk,dv", [(16, 16), (128, 128), (128, 256)])
def test_product_bf16(gpu_lib, nh, dk, dv):
    inp = synth.make_product_inputs(1, 150, 2, dk, dv, nh, dtype=torch.bfloat16,
                                    gate="scalar", chunk=64, seed=62, s0_std=0.05)
    check(inp, name="bf16")


@pytest.mark.parametrize("nh", [2, 4])
def test_product_varlen(gpu_lib, nh):
    inp = synth.make_product_inputs(1, 0, 2, 64, 32, nh, dtype=torch.float32,
                                    gate="scalar", chunk=32, seed=63,
                                    lengths=[5, 0, 41, 16, 1, 27], s0_std=0.2)
    check(inp, name="varlen")


@pytest.mark.parametrize("L", [1, 3])
def test_product_segmented(gpu_lib, L):
    inp = synth.make_product_inputs(1, 300, 2, 128, 64, 2, dtype=torch.bfloat16,
                                    gate="scalar", chunk=64, seed=64, s0_std=0.05)
    check(inp, name=f"segmented L={L}", seg_chunks=L)


def test_product_nh1_equals_chunk_fwd(gpu_lib):
    inp = synth.make_product_inputs(1, 200, 2, 128, 128, 1, dtype=torch.bfloat16,
                                    gate="scalar", seed=65, s0_std=0.05)
    d = dev(inp)
    o1, s1 = gdn.chunk_fwd_product(d.q, d.k, d.v, d.beta, d.log_alpha, d.s0)
    o2, s2 = gdn.chunk_fwd(d.q, d.k[:, :, 0].contiguous(), d.v[:, :, 0].contiguous(),
                           d.beta[:, :, 0].contiguous(), d.log_alpha, d.s0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_product_rejects(gpu_lib):
    inp = synth.make_product_inputs(1, 8, 1, 16, 16, 3, dtype=torch.float32,
                                    gate="scalar", seed=66)
    d = dev(inp)
    with pytest.raises(_lib.GdnError) as e:
        gdn.chunk_fwd_product(d.q, d.k, d.v, d.beta, d.log_alpha)
    assert e.value.status == _lib.GDN_ERR_UNSUPPORTED


# ------------------------------------------------------------ decode step ---

def _decode_inputs(N, H, dk, dv, nh, dtype, gate, seed, beta_scale=1.0):
    inp = synth.make_product_inputs(N, 1, H, dk, dv, nh, dtype=dtype, gate=gate,
                                    chunk=16, seed=seed, s0_std=0.3)
    if beta_scale != 1.0:       # beta in (0, beta_scale): negative eigenvalues
        inp.beta = (inp.beta.double() * beta_scale).to(inp.beta.dtype)
        inp.f64["beta"] = inp.beta.double().numpy()
    return inp


@pytest.mark.parametrize("nh", [1, 2, 4])
@pytest.mark.parametrize("gate", ["scalar", "none"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_product_decode(gpu_lib, nh, gate, dtype):
    inp = _decode_inputs(5, 3, 128, 96, nh, dtype, gate, seed=65, beta_scale=2.0)
    log(f"[product decode] nh={nh} gate={gate} dtype={dtype}")
    d = dev(inp)
    state = d.s0.clone()
    la = None if d.log_alpha is None else d.log_alpha[:, 0].contiguous()
    o = gdn.decode_step_product(d.q[:, 0].contiguous(), d.k[:, 0].contiguous(),
                                d.v[:, 0].contiguous(), d.beta[:, 0].contiguous(), la, state)
    torch.cuda.synchronize()
    f = inp.f64
    o_ref, s_ref = oracle.deltaproduct_fwd(f["q"], f["k"], f["v"], f["beta"], f["log_alpha"],
                                           f["s0"], gate)
    eo = np.max(np.abs(np64(o) - o_ref[:, 0])) / np.max(np.abs(o_ref))
    es = state_err(np64(state), s_ref)
    log(f"    err o={eo:.3e} state={es:.3e}")
    # the step runs in fp32 on the stored values: only the output's rounding
    # to the input dtype separates it from the oracle
    assert eo < (1e-5 if dtype == torch.float32 else 1e-2) and es < 1e-5, (eo, es)


def test_product_decode_steps_equal_the_chunked_forward(gpu_lib):
    # T decode steps from S0 give the chunked forward's outputs and state
    T, nh = 23, 2
    inp = synth.make_product_inputs(2, T, 2, 64, 64, nh, dtype=torch.float32,
                                    gate="scalar", chunk=16, seed=66, s0_std=0.2)
    d = dev(inp)
    o_ref, s_ref = gdn.chunk_fwd_product(d.q, d.k, d.v, d.beta, d.log_alpha, d.s0, chunk=16)
    state = d.s0.clone()
    outs = []
    for t in range(T):
        outs.append(gdn.decode_step_product(
            d.q[:, t].contiguous(), d.k[:, t].contiguous(), d.v[:, t].contiguous(),
            d.beta[:, t].contiguous(), d.log_alpha[:, t].contiguous(), state))
    torch.cuda.synchronize()
    o = torch.stack(outs, dim=1)
    e = max(slice_err(np64(o), np64(o_ref)), state_err(np64(state), np64(s_ref)))
    log(f"[product decode] {T} steps vs chunked forward: {e:.3e}")
    assert e < 1e-4


@pytest.mark.parametrize("nh", [2, 4])
def test_product_forward_beta_up_to_two(gpu_lib, nh):
    # beta in (0, 2): each factor I - beta k k^T may have a negative eigenvalue
    inp = synth.make_product_inputs(1, 130, 2, 64, 64, nh, dtype=torch.float32,
                                    gate="scalar", chunk=64, seed=67, s0_std=0.2)
    inp.beta = inp.beta * 2.0
    inp.f64["beta"] = inp.beta.double().numpy()
    check(inp, name="beta in (0, 2)")


def test_product_headline_size(gpu_lib):
    # the benchmark's workload: T=4096, H=16, d=128, 2 steps per token, bf16;
    # every head against the oracle
    inp = synth.make_product_inputs(1, 4096, 16, 128, 128, 2, dtype=torch.bfloat16,
                                    gate="scalar", chunk=64, seed=1006)
    check(inp, name="t4096_h16_nh2")


def test_product_decode_batch_sampled(gpu_lib):
    # the benchmark's decode batch (N256 H32 d128, 2 steps), sampled sequences
    inp = synth.make_product_inputs(256, 1, 32, 128, 128, 2, dtype=torch.bfloat16,
                                    gate="scalar", chunk=16, seed=1008, s0_std=0.02)
    d = dev(inp)
    state = d.s0.clone()
    o = gdn.decode_step_product(d.q[:, 0].contiguous(), d.k[:, 0].contiguous(),
                                d.v[:, 0].contiguous(), d.beta[:, 0].contiguous(),
                                d.log_alpha[:, 0].contiguous(), state)
    torch.cuda.synchronize()
    f = inp.f64
    for n in (0, 1, 100, 255):
        sl = slice(n, n + 1)
        o_ref, s_ref = oracle.deltaproduct_fwd(f["q"][sl], f["k"][sl], f["v"][sl],
                                               f["beta"][sl], f["log_alpha"][sl], f["s0"][sl],
                                               "scalar")
        eo = np.max(np.abs(np64(o[sl]) - o_ref[:, 0])) / np.max(np.abs(o_ref))
        es = state_err(np64(state[sl]), s_ref)
        log(f"[product decode] batch seq {n}: err o={eo:.3e} state={es:.3e}")
        assert eo < 1e-2 and es < 1e-5


@pytest.mark.parametrize("nh", [2, 4])
def test_product_empty_sequences_copy_state(gpu_lib, nh):
    # T = 0: no transition, the final state is the initial one bit for bit
    inp = synth.make_product_inputs(2, 0, 2, 64, 32, nh, dtype=torch.bfloat16, seed=1010,
                                    s0_std=1.0)
    log(f"[product] empty nh={nh}")
    d = inp.to("cuda")
    o, sf = gdn.chunk_fwd_product(d.q, d.k, d.v, d.beta, d.log_alpha, d.s0)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 2, 32)
    assert torch.equal(sf.cpu(), inp.s0)
