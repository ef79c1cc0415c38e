"""GPU parity of draft-tree verification and commit (gdn_tree_verify,
gdn_tree_commit) against the fp64 oracle (MI355X only).

Random recursive trees (parent uniform over the earlier nodes and the root),
chains and stars; both per-token gate modes, both dtypes, every chunk size,
trees that fill the chunk and trees with a ragged tail, varlen packing with
empty and one-node trees, out-of-range parents and accepted indices, a
verify -> commit -> verify round, and the decode-sized batch."""

import numpy as np
import pytest
import torch

import gated_delta_rule_79_amd as gdn
import oracle
from gated_delta_rule_79_amd import _lib, synth
from gpu_util import TOL, log, np64, slice_err, state_err

pytestmark = pytest.mark.gpu


def _cu(inp):
    return None if inp.cu_seqlens is None else inp.cu_seqlens.numpy()


def verify(inp, parent, name=""):
    log(f"[tree] verify {name} q={tuple(inp.q.shape)} v={tuple(inp.v.shape)} "
        f"dtype={inp.q.dtype} gate={inp.gate} C={inp.chunk} seed={inp.seed}")
    d = inp.to("cuda")
    o = gdn.tree_verify(d.q, d.k, d.v, d.beta, d.log_alpha, parent.cuda(), d.s0,
                        chunk=inp.chunk, cu_seqlens=d.cu_seqlens)
    torch.cuda.synchronize()
    f = inp.f64
    o_ref, _ = oracle.tree_fwd(f["q"], f["k"], f["v"], f["beta"], f["log_alpha"],
                               parent.numpy(), f["s0"], inp.gate, cu_seqlens=_cu(inp))
    tol = TOL[inp.q.dtype]
    e = slice_err(np64(o), o_ref, _cu(inp))
    log(f"    err o={e:.3e} tol={tol}")
    assert e < tol, e
    return o


def commit(inp, parent, accepted, name=""):
    log(f"[tree] commit {name} k={tuple(inp.k.shape)} dtype={inp.q.dtype} "
        f"gate={inp.gate} accepted={accepted.tolist()[:8]}")
    d = inp.to("cuda")
    st = d.s0.clone()
    gdn.tree_commit(d.k, d.v, d.beta, d.log_alpha, parent.cuda(), accepted.cuda(), st,
                    chunk=inp.chunk, cu_seqlens=d.cu_seqlens)
    torch.cuda.synchronize()
    f = inp.f64
    # an accepted index outside the tree leaves the state: -1 for the oracle
    cu = _cu(inp)
    sizes = np.diff(cu) if cu is not None else np.full(len(accepted), inp.k.shape[1])
    acc = accepted.numpy()
    acc = np.where((acc < 0) | (acc >= sizes), -1, acc)
    ref = oracle.tree_commit(f["k"], f["v"], f["beta"], f["log_alpha"], parent.numpy(),
                             acc, f["s0"], inp.gate, cu_seqlens=cu)
    e = state_err(np64(st), ref)
    log(f"    err state={e:.3e}")
    assert e < 1e-5, e
    return st


@pytest.mark.parametrize("gate", ["scalar", "none"])
@pytest.mark.parametrize("C,n", [(16, 16), (32, 23), (64, 64), (64, 41)])
def test_verify_fp32(gpu_lib, gate, C, n):
    inp, par, _ = synth.make_tree_inputs(3, n, 2, 32, 48, dtype=torch.float32, gate=gate,
                                         chunk=C, seed=81, s0_std=0.3)
    verify(inp, par, name="fp32")


@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 64), (128, 128), (128, 256)])
def test_verify_bf16(gpu_lib, dk, dv):
    inp, par, _ = synth.make_tree_inputs(4, 64, 2, dk, dv, dtype=torch.bfloat16,
                                         gate="scalar", chunk=64, seed=82, s0_std=0.05)
    verify(inp, par, name="bf16")


@pytest.mark.parametrize("shape", ["chain", "star"])
def test_verify_chain_and_star(gpu_lib, shape):
    inp, par, _ = synth.make_tree_inputs(2, 37, 2, 64, 32, dtype=torch.float32,
                                         gate="scalar", chunk=64, seed=83, s0_std=0.2,
                                         shape=shape)
    verify(inp, par, name=shape)


def test_chain_tree_is_the_forward(gpu_lib):
    # a chain is one sequence: the verification equals gdn_chunk_fwd
    inp, par, _ = synth.make_tree_inputs(3, 64, 2, 128, 128, dtype=torch.float32,
                                         gate="scalar", chunk=64, seed=84, s0_std=0.1,
                                         shape="chain")
    d = inp.to("cuda")
    o1 = gdn.tree_verify(d.q, d.k, d.v, d.beta, d.log_alpha, par.cuda(), d.s0)
    o2, _ = gdn.chunk_fwd(d.q, d.k, d.v, d.beta, d.log_alpha, d.s0)
    torch.cuda.synchronize()
    e = slice_err(np64(o1), np64(o2))
    log(f"[tree] chain vs forward: {e:.3e}")
    assert e < 1e-5


def test_verify_varlen(gpu_lib):
    inp, par, _ = synth.make_tree_inputs(1, 0, 2, 64, 32, dtype=torch.float32,
                                         gate="scalar", chunk=32, seed=85, s0_std=0.2,
                                         lengths=[5, 0, 32, 1, 17, 9])
    verify(inp, par, name="varlen")


def test_verify_out_of_range_parents_read_as_root(gpu_lib):
    inp, par, _ = synth.make_tree_inputs(2, 20, 2, 32, 32, dtype=torch.float32,
                                         gate="scalar", chunk=32, seed=86, s0_std=0.2)
    bad = par.clone()
    bad[0, 3], bad[0, 7], bad[1, 5], bad[1, 19] = 3, 12, -5, 100
    fixed = bad.clone()
    fixed[0, 3], fixed[0, 7], fixed[1, 5], fixed[1, 19] = -1, -1, -1, -1
    d = inp.to("cuda")
    o1 = gdn.tree_verify(d.q, d.k, d.v, d.beta, d.log_alpha, bad.cuda(), d.s0, chunk=32)
    o2 = gdn.tree_verify(d.q, d.k, d.v, d.beta, d.log_alpha, fixed.cuda(), d.s0, chunk=32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    verify(inp, fixed, name="fixed parents")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("gate", ["scalar", "none"])
def test_commit(gpu_lib, dtype, gate):
    inp, par, acc = synth.make_tree_inputs(6, 64, 2, 128, 128, dtype=dtype, gate=gate,
                                           chunk=64, seed=87, s0_std=0.1)
    acc[1] = -1       # nothing accepted
    acc[2] = 0        # the first node
    acc[3] = 64       # outside the tree: unchanged
    st = commit(inp, par, acc, name=str(dtype))
    assert torch.equal(st[1].cpu(), inp.s0[1]) and torch.equal(st[3].cpu(), inp.s0[3])


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 80), (64, 256)])
def test_commit_shapes(gpu_lib, dk, dv):
    inp, par, acc = synth.make_tree_inputs(3, 30, 3, dk, dv, dtype=torch.float32,
                                           gate="scalar", chunk=32, seed=88, s0_std=0.3)
    commit(inp, par, acc, name=f"dk{dk} dv{dv}")


def test_commit_varlen(gpu_lib):
    inp, par, acc = synth.make_tree_inputs(1, 0, 2, 64, 64, dtype=torch.float32,
                                           gate="scalar", chunk=64, seed=89, s0_std=0.2,
                                           lengths=[7, 0, 64, 1, 33])
    commit(inp, par, acc, name="varlen")


def test_verify_commit_verify(gpu_lib):
    # one speculative step and the next: verify, accept a node, commit,
    # verify a new tree from the committed state
    inp, par, acc = synth.make_tree_inputs(4, 32, 2, 128, 128, dtype=torch.bfloat16,
                                           gate="scalar", chunk=32, seed=90, s0_std=0.05)
    verify(inp, par, name="first verify")
    st = commit(inp, par, acc, name="first commit")
    nxt, par2, _ = synth.make_tree_inputs(4, 32, 2, 128, 128, dtype=torch.bfloat16,
                                          gate="scalar", chunk=32, seed=91, s0_std=0.05)
    nxt.s0 = st.cpu()
    nxt.f64["s0"] = nxt.s0.double().numpy()
    verify(nxt, par2, name="second verify")


def test_decode_sized_batch_sampled(gpu_lib):
    # 256 trees of 16 nodes, 32 heads, d = 128 (the decode batch): the oracle
    # on 6 of the trees, every head
    inp, par, acc = synth.make_tree_inputs(256, 16, 32, 128, 128, dtype=torch.bfloat16,
                                           gate="scalar", chunk=16, seed=92, s0_std=0.02)
    d = inp.to("cuda")
    o = gdn.tree_verify(d.q, d.k, d.v, d.beta, d.log_alpha, par.cuda(), d.s0, chunk=16)
    st = d.s0.clone()
    gdn.tree_commit(d.k, d.v, d.beta, d.log_alpha, par.cuda(), acc.cuda(), st, chunk=16)
    torch.cuda.synchronize()
    f = inp.f64
    for m in (0, 1, 77, 128, 200, 255):
        sl = slice(m, m + 1)
        la = None if f["log_alpha"] is None else f["log_alpha"][sl]
        o_ref, _ = oracle.tree_fwd(f["q"][sl], f["k"][sl], f["v"][sl], f["beta"][sl], la,
                                   par.numpy()[sl], f["s0"][sl], "scalar")
        s_ref = oracle.tree_commit(f["k"][sl], f["v"][sl], f["beta"][sl], la,
                                   par.numpy()[sl], acc.numpy()[sl], f["s0"][sl], "scalar")
        eo = slice_err(np64(o[sl]), o_ref)
        es = state_err(np64(st[sl]), s_ref)
        log(f"[tree] batch tree {m}: err o={eo:.3e} state={es:.3e}")
        assert eo < TOL[torch.bfloat16] and es < 1e-5


def test_tree_rejections(gpu_lib):
    inp, par, acc = synth.make_tree_inputs(2, 40, 2, 32, 32, dtype=torch.float32,
                                           gate="scalar", chunk=32, seed=93)
    d = inp.to("cuda")
    with pytest.raises(_lib.GdnError) as ei:       # 40 nodes > chunk 32
        gdn.tree_verify(d.q, d.k, d.v, d.beta, d.log_alpha, par.cuda(), d.s0, chunk=32)
    assert ei.value.status == _lib.GDN_ERR_SHAPE
    ch, par2, _ = synth.make_tree_inputs(2, 16, 2, 32, 32, dtype=torch.float32,
                                         gate="channel", chunk=16, seed=94)
    dc = ch.to("cuda")
    with pytest.raises(_lib.GdnError) as ei:
        gdn.tree_verify(dc.q, dc.k, dc.v, dc.beta, dc.log_alpha, par2.cuda(), dc.s0, chunk=16)
    assert ei.value.status == _lib.GDN_ERR_UNSUPPORTED
