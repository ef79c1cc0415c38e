"""GPU parity of gdn_decode_step against the fp64 oracle (MI355X only)."""

import numpy as np
import pytest
import torch

import gated_delta_rule_79_amd as gdn
import oracle
from gated_delta_rule_79_amd import synth
from gpu_util import TOL, log, np64, state_err

pytestmark = pytest.mark.gpu


def decode_inputs(N, H, dk, dv, dtype, gate, seed, s0_std=0.02):
    inp = synth.make_inputs(N, 1, H, dk, dv, dtype=dtype, gate=gate, seed=seed,
                            s0_std=s0_std)
    sq = lambda t: None if t is None else t[:, 0].contiguous()
    f = {k: (None if v is None else (v[:, 0] if k not in ("s0",) else v))
         for k, v in inp.f64.items() if k in ("q", "k", "v", "beta", "log_alpha", "s0")}
    return (sq(inp.q), sq(inp.k), sq(inp.v), sq(inp.beta), sq(inp.log_alpha),
            inp.s0.clone()), f


def check(N, H, dk, dv, dtype, gate, seed, s0_std=0.02):
    log(f"[decode] N={N} H={H} dk={dk} dv={dv} {dtype} gate={gate} seed={seed}")
    (q, k, v, b, la, s0), f = decode_inputs(N, H, dk, dv, dtype, gate, seed, s0_std)
    state = s0.cuda()
    o = gdn.decode_step(q.cuda(), k.cuda(), v.cuda(), b.cuda(),
                        None if la is None else la.cuda(), state)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.gdn_decode(f["q"], f["k"], f["v"], f["beta"],
                                     f["log_alpha"], f["s0"], gate)
    eo = oracle.normwise_rel_err(np64(o)[:, :, None, :], o_ref[:, :, None, :])
    es = state_err(np64(state), s_ref)
    tol = TOL[dtype]
    log(f"    err o={eo:.3e} state={es:.3e} tol={tol}")
    assert eo < tol and es < tol
    return eo, es


@pytest.mark.parametrize("gate", ["scalar", "channel", "none"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_full_size(gpu_lib, gate, dtype):
    # 256 sequences x 32 heads x 128 x 128 fp32 state, updated in place
    eo, es = check(256, 32, 128, 128, dtype, gate, 1003)
    if dtype == torch.bfloat16:
        # the arithmetic is fp32; only the bf16 output rounding remains
        assert es < 1e-5 and eo < 1e-2


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 48), (64, 80), (128, 256)])
def test_decode_shapes(gpu_lib, dk, dv):
    check(7, 3, dk, dv, torch.float32, "channel", 5, s0_std=1.0)


def test_decode_after_fwd_equals_longer_fwd(gpu_lib):
    inp = synth.make_inputs(2, 97, 3, 64, 64, dtype=torch.float32, gate="scalar",
                            seed=23, s0_std=0.1)
    d = inp.to("cuda")
    o_all, s_all = gdn.chunk_fwd(d.q, d.k, d.v, d.beta, d.log_alpha, d.s0)
    o_a, s_a = gdn.chunk_fwd(d.q[:, :96].contiguous(), d.k[:, :96].contiguous(),
                             d.v[:, :96].contiguous(), d.beta[:, :96].contiguous(),
                             d.log_alpha[:, :96].contiguous(), d.s0)
    o_d = gdn.decode_step(d.q[:, 96].contiguous(), d.k[:, 96].contiguous(),
                          d.v[:, 96].contiguous(), d.beta[:, 96].contiguous(),
                          d.log_alpha[:, 96].contiguous(), s_a)
    torch.cuda.synchronize()
    assert np.max(np.abs(np64(o_d) - np64(o_all[:, 96]))) < 1e-5
    assert state_err(np64(s_a), np64(s_all)) < 1e-5


def test_decode_repeated_steps(gpu_lib):
    # 20 steps in place equal the oracle recurrence over 20 tokens
    inp = synth.make_inputs(4, 20, 2, 128, 128, dtype=torch.float32, gate="channel",
                            seed=24, s0_std=0.02)
    d = inp.to("cuda")
    state = d.s0.clone()
    outs = []
    for t in range(20):
        outs.append(gdn.decode_step(d.q[:, t].contiguous(), d.k[:, t].contiguous(),
                                    d.v[:, t].contiguous(), d.beta[:, t].contiguous(),
                                    d.log_alpha[:, t].contiguous(), state))
    torch.cuda.synchronize()
    f = inp.f64
    o_ref, s_ref = oracle.gdn_fwd(f["q"], f["k"], f["v"], f["beta"], f["log_alpha"],
                                  f["s0"], "channel")
    o = torch.stack(outs, 1)
    assert oracle.normwise_rel_err(np64(o), o_ref) < 1e-4
    assert state_err(np64(state), s_ref) < 1e-4
