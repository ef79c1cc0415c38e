"""Pins of the fp64 oracle against facts fixed by the pages and by
mathematics (CPU only).  Pages: "Gated Delta Networks: Improving Mamba2 with
Delta Rule" (paper review), sections "Method", "Key idea", "Background"."""

import os

import numpy as np
import pytest

import oracle
import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_problem(r, B, T, H, dk, dv, gate, s0=True, beta_scale=1.0,
                  la_scale=1.0):
    q = pins.unit(r.standard_normal((B, T, H, dk)))
    k = pins.unit(r.standard_normal((B, T, H, dk)))
    v = r.standard_normal((B, T, H, dv))
    beta = beta_scale * r.random((B, T, H))
    if gate == "scalar":
        la = -la_scale * r.random((B, T, H))
    elif gate == "channel":
        la = -la_scale * r.random((B, T, H, dk))
    else:
        la = None
    m0 = r.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, beta, la, m0


# ---------------------------------------------------------------- golden ---

def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(":", 1)
            vals[key.strip()] = np.array([float(x) for x in rest.split()])
    return vals


def test_golden_hand_worked():
    g = _read_golden("hand_worked_t2.txt")
    dk, dv = int(g["dk"][0]), int(g["dv"][0])
    T = len(g["beta"])
    o, M = oracle.gdn_fwd_chain(g["q"].reshape(T, dk), g["k"].reshape(T, dk),
                                g["v"].reshape(T, dv), g["beta"],
                                g["log_alpha"], np.zeros((dk, dv)), "scalar")
    np.testing.assert_allclose(o.reshape(-1), g["o"], atol=1e-14)
    np.testing.assert_allclose(M.reshape(-1), g["M_final"], atol=1e-14)


# -------------------------------------------------------------- P1 chunks ---

@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("C,T", [(1, 5), (4, 23), (16, 37), (64, 70)])
def test_p1_chunked_form_equals_recurrence(gate, C, T):
    r = pins.rng(100 + C)
    q, k, v, beta, la, m0 = _rand_problem(r, 1, T, 1, 8, 6, gate,
                                          beta_scale=1.9, la_scale=0.6)
    la0 = None if la is None else la[0, :, 0]
    o1, M1 = oracle.gdn_fwd_chain(q[0, :, 0], k[0, :, 0], v[0, :, 0],
                                  beta[0, :, 0], la0, m0[0, 0], gate)
    o2, M2 = oracle.gdn_chunked_bruteforce(q[0, :, 0], k[0, :, 0], v[0, :, 0],
                                           beta[0, :, 0], la0, m0[0, 0], gate, C)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    assert np.max(np.abs(M1 - M2)) < 1e-12


# ------------------------------------------------------------ P2 .. P10 ---

@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_p2_orthonormal_retrieval(gate):
    assert pins.p2_orthonormal_retrieval(oracle.gdn_fwd_chain, gate=gate) < 1e-13


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_p3_beta_zero_gate_product(gate):
    assert pins.p3_gate_product(oracle.gdn_fwd_chain, gate=gate) < 1e-13


def test_p4_deltanet_limit():
    r = pins.rng(4)
    q, k, v, beta, la, m0 = _rand_problem(r, 1, 30, 1, 7, 5, "scalar",
                                          beta_scale=1.5)
    args = (q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0])
    o_ref, M_ref = oracle.delta_rule_ungated(*args, m0[0, 0])
    for gate, la0 in (("scalar", np.zeros(30)), ("channel", np.zeros((30, 7))),
                      ("none", None)):
        o, M = oracle.gdn_fwd_chain(*args, la0, m0[0, 0], gate)
        assert np.max(np.abs(o - o_ref)) < 1e-13
        assert np.max(np.abs(M - M_ref)) < 1e-13


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_p5_norm_bound(gate):
    assert pins.p5_norm_bound(oracle.gdn_fwd_chain, gate=gate) <= 1 + 1e-12
    assert pins.p5_norm_bound(oracle.gdn_fwd_chain, zero_v=True,
                              gate=gate) <= 1 + 1e-12


def test_p5_norm_bound_has_teeth():
    # beta beyond 2 leaves the contraction regime: the bound must fail
    assert pins.p5_norm_bound(oracle.gdn_fwd_chain, beta_max=3.0,
                              zero_v=True) > 1.2


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_p6_erasure(gate):
    assert pins.p6_erasure(oracle.gdn_fwd_chain, gate=gate) < 1e-13


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_p7_gated_linear_attention_limit(gate):
    assert pins.p7_gla_limit(oracle.gdn_fwd_chain, gate=gate) < 1e-13


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_p8_sgd_reading(gate):
    r = pins.rng(8)
    q, k, v, beta, la, m0 = _rand_problem(r, 1, 25, 1, 6, 4, gate,
                                          beta_scale=1.8)
    la0 = None if la is None else la[0, :, 0]
    a = (q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0], la0, m0[0, 0], gate)
    o1, M1 = oracle.gdn_fwd_chain(*a)
    o2, M2 = oracle.gdn_sgd_form(*a)
    assert np.max(np.abs(o1 - o2)) < 1e-13 and np.max(np.abs(M1 - M2)) < 1e-13


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_p9_single_token(gate):
    assert pins.p9_single_token(oracle.gdn_fwd_chain, gate=gate) < 1e-14


def test_p10_equal_channels_equal_scalar():
    r = pins.rng(10)
    q, k, v, beta, la, m0 = _rand_problem(r, 2, 19, 3, 8, 5, "scalar")
    la_c = np.repeat(la[..., None], 8, axis=-1)
    o1, s1 = oracle.gdn_fwd(q, k, v, beta, la, m0, "scalar")
    o2, s2 = oracle.gdn_fwd(q, k, v, beta, la_c, m0, "channel")
    assert np.max(np.abs(o1 - o2)) < 1e-13 and np.max(np.abs(s1 - s2)) < 1e-13


# ------------------------------------------------------ P11 boundaries ---

@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_p11_varlen_equals_separate(gate):
    r = pins.rng(11)
    lens = [5, 0, 17, 1, 9]
    T = sum(lens)
    q, k, v, beta, la, _ = _rand_problem(r, 1, T, 2, 6, 4, gate)
    m0 = r.standard_normal((len(lens), 2, 6, 4))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, sf = oracle.gdn_fwd(q, k, v, beta, la, m0, gate, cu_seqlens=cu)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        o_n, s_n = oracle.gdn_fwd(q[:, a:b], k[:, a:b], v[:, a:b], beta[:, a:b],
                                  la[:, a:b], m0[n:n + 1], gate)
        assert np.array_equal(o[:, a:b], o_n)
        assert np.array_equal(sf[n:n + 1], s_n)
    assert np.array_equal(sf[1], m0[1])          # empty sequence: S_final = S0


def test_p11_split_and_resume_and_decode():
    r = pins.rng(12)
    q, k, v, beta, la, m0 = _rand_problem(r, 2, 31, 2, 6, 5, "scalar")
    o, sf = oracle.gdn_fwd(q, k, v, beta, la, m0, "scalar")
    oa, sa = oracle.gdn_fwd(q[:, :13], k[:, :13], v[:, :13], beta[:, :13],
                            la[:, :13], m0, "scalar")
    ob, sb = oracle.gdn_fwd(q[:, 13:], k[:, 13:], v[:, 13:], beta[:, 13:],
                            la[:, 13:], sa, "scalar")
    assert np.max(np.abs(np.concatenate([oa, ob], 1) - o)) < 1e-13
    assert np.max(np.abs(sb - sf)) < 1e-13
    # decode after fwd(T-1) equals fwd(T)
    o1, s1 = oracle.gdn_fwd(q[:, :30], k[:, :30], v[:, :30], beta[:, :30],
                            la[:, :30], m0, "scalar")
    od, sd = oracle.gdn_decode(q[:, 30], k[:, 30], v[:, 30], beta[:, 30],
                               la[:, 30], s1, "scalar")
    assert np.max(np.abs(od - o[:, 30])) < 1e-13
    assert np.max(np.abs(sd - sf)) < 1e-13


def test_p11_permutation_equivariance():
    r = pins.rng(13)
    q, k, v, beta, la, m0 = _rand_problem(r, 3, 11, 4, 5, 3, "channel")
    o, sf = oracle.gdn_fwd(q, k, v, beta, la, m0, "channel")
    pb, ph = [2, 0, 1], [3, 1, 0, 2]
    perm = lambda x: x[pb][:, :, ph]
    o2, sf2 = oracle.gdn_fwd(perm(q), perm(k), perm(v), perm(beta), perm(la),
                             m0[pb][:, ph], "channel")
    assert np.array_equal(o2, perm(o)) and np.array_equal(sf2, sf[pb][:, ph])


def test_chunk_size_invariance_of_chunked_form():
    r = pins.rng(14)
    q, k, v, beta, la, m0 = _rand_problem(r, 1, 50, 1, 6, 4, "channel")
    args = (q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0], la[0, :, 0],
            m0[0, 0], "channel")
    outs = [oracle.gdn_chunked_bruteforce(*args, C) for C in (3, 16, 32, 64)]
    for o, M in outs[1:]:
        assert np.max(np.abs(o - outs[0][0])) < 1e-12
        assert np.max(np.abs(M - outs[0][1])) < 1e-12


def test_empty_and_single():
    r = pins.rng(15)
    q, k, v, beta, la, m0 = _rand_problem(r, 1, 0, 2, 4, 3, "scalar")
    o, sf = oracle.gdn_fwd(q, k, v, beta, la, m0, "scalar")
    assert o.shape == (1, 0, 2, 3) and np.array_equal(sf, m0)


# ---------------------------------------------------- P12 the adjoint ---

def _loss(q, k, v, beta, la, m0, do, dS, gate):
    o, sf = oracle.gdn_fwd(q, k, v, beta, la, m0, gate)
    return np.sum(do * o) + np.sum(dS * sf)


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_p12_adjoint_vs_finite_differences(gate):
    r = pins.rng(16)
    B, T, H, dk, dv = 1, 7, 1, 4, 3
    q, k, v, beta, la, m0 = _rand_problem(r, B, T, H, dk, dv, gate,
                                          beta_scale=1.9, la_scale=0.8)
    do = r.standard_normal((B, T, H, dv))
    dS = r.standard_normal((B, H, dk, dv))
    grads = oracle.gdn_bwd(q, k, v, beta, la, m0, do, dS, gate)
    names = ["q", "k", "v", "beta", "la", "m0"]
    vals = dict(q=q, k=k, v=v, beta=beta, la=la, m0=m0)
    got = dict(q=grads[0], k=grads[1], v=grads[2], beta=grads[3], la=grads[4],
               m0=grads[5])
    h = 1e-6
    for name in names:
        x = vals[name]
        if x is None:
            assert got[name] is None
            continue
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            a = dict(vals); a[name] = xp
            b = dict(vals); b[name] = xm
            fd[idx] = (_loss(a["q"], a["k"], a["v"], a["beta"], a["la"], a["m0"],
                             do, dS, gate)
                       - _loss(b["q"], b["k"], b["v"], b["beta"], b["la"], b["m0"],
                               do, dS, gate)) / (2 * h)
        err = np.max(np.abs(fd - got[name])) / max(np.max(np.abs(fd)), 1e-30)
        assert err < 1e-7, (name, err)


def test_p12_adjoint_checkpoint_segments():
    # the segment-wise recomputation must not depend on the checkpoint stride
    r = pins.rng(17)
    q, k, v, beta, la, m0 = _rand_problem(r, 1, 45, 1, 5, 4, "channel")
    do = r.standard_normal((45, 4))
    a = (q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0], la[0, :, 0],
         m0[0, 0], do, None, "channel")
    g1 = oracle.gdn_bwd_chain(*a, ckpt=64)
    g2 = oracle.gdn_bwd_chain(*a, ckpt=4)
    for x, y in zip(g1, g2):
        assert np.max(np.abs(x - y)) < 1e-12


# ------------------------------------------- Householder-product transitions ---

def test_dp_single_step_is_gdn():
    assert pins.dp_single_step_is_gdn(oracle.deltaproduct_fwd, oracle.gdn_fwd) < 1e-14


def test_dp_reflections():
    assert pins.dp_reflections(oracle.deltaproduct_fwd) < 1e-12


def test_dp_two_step_closed_form():
    assert pins.dp_two_step_closed_form(oracle.deltaproduct_fwd) < 1e-13


def test_dp_gate_once_per_token():
    assert pins.dp_gate_once_per_token(oracle.deltaproduct_fwd, oracle.gdn_fwd) < 1e-13


# ------------------------------------------------ normalised q and k ---

def test_l2_normalize_rows_are_unit_and_parallel():
    r = pins.rng(21)
    x = r.standard_normal((3, 5, 2, 7)) * r.random((3, 5, 2, 1)) * 10
    y = oracle.l2_normalize(x)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), 1.0, atol=1e-15)
    # y is a positive multiple of x: cosine 1 row by row
    cos = np.sum(x * y, axis=-1) / np.linalg.norm(x, axis=-1)
    np.testing.assert_allclose(cos, 1.0, atol=1e-15)
    z = np.zeros((2, 3))
    assert np.all(oracle.l2_normalize(z) == 0)


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_qknorm_is_scale_invariant(gate):
    """Positive per-row scales of q and k do not change the outputs, and
    already-unit rows give the plain forward."""
    r = pins.rng(22)
    q, k, v, beta, la, m0 = _rand_problem(r, 1, 9, 2, 6, 4, gate)
    o1, s1 = oracle.gdn_fwd(q, k, v, beta, la, m0, gate)
    o2, s2 = oracle.gdn_fwd_qknorm(q, k, v, beta, la, m0, gate)
    sq = np.exp(r.standard_normal(q.shape[:-1] + (1,)))
    sk = np.exp(r.standard_normal(k.shape[:-1] + (1,)))
    o3, s3 = oracle.gdn_fwd_qknorm(q * sq, k * sk, v, beta, la, m0, gate)
    for a, b in ((o1, o2), (s1, s2), (o1, o3), (s1, s3)):
        assert np.max(np.abs(a - b)) < 1e-12


# ------------------------------------------------------------- draft trees ---

@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_tree_reductions_to_sequences(gate):
    assert pins.tree_chain_is_sequence(oracle.tree_fwd, oracle.gdn_fwd, gate) < 1e-13
    assert pins.tree_star_is_single_steps(oracle.tree_fwd, oracle.gdn_decode, gate) < 1e-13
    assert pins.tree_paths_are_sequences(oracle.tree_fwd, oracle.gdn_fwd, gate) < 1e-13


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_tree_commit_and_wy_form(gate):
    assert pins.tree_commit_is_node_state(oracle.tree_commit, oracle.tree_fwd, gate) < 1e-13
    assert pins.tree_wy_matches_recurrence(oracle.tree_wy_bruteforce, oracle.tree_fwd,
                                           gate) < 1e-12


def test_tree_relabelling():
    """Another topological numbering of the same tree permutes the outputs."""
    r = pins.rng(26)
    n = 10
    q, k, v, beta, la, s0 = pins._tree_problem(r, 1, n, 2, 4, 3, "scalar")
    par = pins.random_tree(r, n)
    # children of the root first, then by depth (a breadth-first numbering)
    depth = np.zeros(n, dtype=int)
    for i in range(n):
        depth[i] = 0 if par[i] < 0 else depth[par[i]] + 1
    perm = np.argsort(depth, kind="stable")        # new node j is old perm[j]
    inv = np.argsort(perm)
    par2 = np.array([-1 if par[perm[j]] < 0 else inv[par[perm[j]]] for j in range(n)])
    o1, _ = oracle.tree_fwd(q, k, v, beta, la, par[None], s0, "scalar")
    o2, _ = oracle.tree_fwd(q[:, perm], k[:, perm], v[:, perm], beta[:, perm], la[:, perm],
                            par2[None], s0, "scalar")
    assert np.max(np.abs(o2 - o1[:, perm])) < 1e-14


def test_tree_rejects_parent_after_child():
    with pytest.raises(AssertionError):
        oracle.tree_path([-1, 2, 0], 1)


# ------------------------------------------------ Gated DeltaNet-2 ---

@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_g2_equal_strengths_is_gdn(gate):
    assert pins.g2_equal_strengths_is_gdn(oracle.gdn2_fwd_chain, oracle.gdn_fwd_chain,
                                          gate) < 1e-13


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_g2_no_erase_is_linear_attention(gate):
    assert pins.g2_no_erase_is_linear_attention(oracle.gdn2_fwd_chain, gate) < 1e-12


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_g2_no_write_is_erasure(gate):
    assert pins.g2_no_write_is_erasure(oracle.gdn2_fwd_chain, gate) < 1e-12


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_g2_full_erase_stores_write(gate):
    assert pins.g2_full_erase_stores_write(oracle.gdn2_fwd_chain, gate) < 1e-12


@pytest.mark.parametrize("C", [1, 4, 16])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_g2_chunked_form(gate, C):
    assert pins.g2_chunked_equals_recurrence(oracle.gdn2_fwd_chain,
                                             oracle.gdn2_chunked_bruteforce, gate, C) < 1e-11


def test_g2_batch_and_decode_wrap_the_chain():
    r = pins.rng(36)
    B, T, H, dk, dv = 2, 9, 3, 6, 4
    q = pins.unit(r.standard_normal((B, T, H, dk)))
    k = pins.unit(r.standard_normal((B, T, H, dk)))
    v = r.standard_normal((B, T, H, dv))
    er, wr = r.random((B, T, H)), r.random((B, T, H)) * 2
    la = -r.random((B, T, H, dk))
    s0 = r.standard_normal((B, H, dk, dv))
    o, sf = oracle.gdn2_fwd(q, k, v, er, wr, la, s0, "channel")
    for b in range(B):
        for h in range(H):
            oc, mc = oracle.gdn2_fwd_chain(q[b, :, h], k[b, :, h], v[b, :, h], er[b, :, h],
                                           wr[b, :, h], la[b, :, h], s0[b, h], "channel")
            assert np.max(np.abs(o[b, :, h] - oc)) < 1e-14
            assert np.max(np.abs(sf[b, h] - mc)) < 1e-14
    # decode of the next token continues the forward
    od, st = oracle.gdn2_decode(q[:, 0], k[:, 0], v[:, 0], er[:, 0], wr[:, 0], la[:, 0],
                                s0, "channel")
    o1, s1 = oracle.gdn2_fwd(q[:, :1], k[:, :1], v[:, :1], er[:, :1], wr[:, :1], la[:, :1],
                             s0, "channel")
    assert np.max(np.abs(od - o1[:, 0])) < 1e-14 and np.max(np.abs(st - s1)) < 1e-14


# ------------------------------------ short convolution + SiLU prologue ---

def test_conv_equals_numpy_convolve():
    assert pins.conv_equals_numpy_convolve(oracle.short_conv) < 1e-13


@pytest.mark.parametrize("W,t0", [(1, 0), (3, 4), (4, 10), (4, 0)])
def test_conv_impulse_response(W, t0):
    assert pins.conv_impulse_response(oracle.short_conv, W=W, t0=t0) < 1e-15


def test_conv_isolates_sequences():
    assert pins.conv_isolates_sequences(oracle.short_conv) < 1e-15


def test_silu_identities():
    assert pins.silu_identities(oracle.silu) < 1e-12


def test_conv_prologue_paths():
    # q and k rows come out unit (or zero), v rows are not normalised; with
    # width-1 unit taps the convolution is the identity
    r = pins.rng(44)
    x = r.standard_normal((1, 7, 2, 5))
    w1 = np.ones((2, 5, 1))
    qk = oracle.conv_prologue(x, w1, True)
    n = np.linalg.norm(qk, axis=-1)
    assert np.max(np.abs(n - 1.0)) < 1e-14
    vv = oracle.conv_prologue(x, w1, False)
    assert np.max(np.abs(vv - x / (1 + np.exp(-x)))) < 1e-15
    z = oracle.conv_prologue(x, np.zeros((2, 5, 3)), True)
    assert np.all(z == 0.0)


def test_conv_forward_composes_the_paths():
    # the block forward is the pinned forward on the three prologue outputs,
    # each built here from numpy's convolution
    r = pins.rng(45)
    B, T, H, dk, dv, W = 1, 20, 2, 6, 4, 4
    xq, xk = r.standard_normal((B, T, H, dk)), r.standard_normal((B, T, H, dk))
    xv = r.standard_normal((B, T, H, dv))
    wq, wk = r.standard_normal((H, dk, W)), r.standard_normal((H, dk, W))
    wv = r.standard_normal((H, dv, W))
    beta, la = r.random((B, T, H)), -r.random((B, T, H))

    def path(x, w, norm):
        y = np.zeros_like(x)
        for h in range(x.shape[2]):
            for c in range(x.shape[3]):
                y[0, :, h, c] = np.convolve(x[0, :, h, c], w[h, c])[:T]
        y = y / (1.0 + np.exp(-y))
        return pins.unit(y) if norm else y

    o, s = oracle.gdn_fwd_conv(xq, xk, xv, wq, wk, wv, beta, la, None, "scalar")
    o2, s2 = oracle.gdn_fwd(path(xq, wq, True), path(xk, wk, True), path(xv, wv, False),
                            beta, la, None, "scalar")
    assert np.max(np.abs(o - o2)) < 1e-12 and np.max(np.abs(s - s2)) < 1e-12


# ------------------------------------- adjoint of the prologue path ---

@pytest.mark.parametrize("normalize", [True, False])
@pytest.mark.parametrize("varlen", [False, True])
def test_prologue_bwd_matches_finite_differences(normalize, varlen):
    assert pins.prologue_bwd_fd(oracle.conv_prologue_bwd, oracle.conv_prologue,
                                normalize, varlen) < 1e-7


def test_prologue_bwd_width_one_closed_form():
    assert pins.prologue_bwd_width_one(oracle.conv_prologue_bwd) < 1e-14


def test_prologue_bwd_zero_row_has_zero_gradient():
    # zero taps make every row zero; the normalised path's rows stay zero and
    # their gradient reaching x is zero; dtaps still sees dy through SiLU'(0)
    r = pins.rng(48)
    x, dy = r.standard_normal((1, 5, 1, 3)), r.standard_normal((1, 5, 1, 3))
    dx, dw = oracle.conv_prologue_bwd(x, np.zeros((1, 3, 2)), True, dy)
    assert np.all(dx == 0.0) and np.all(dw == 0.0)
