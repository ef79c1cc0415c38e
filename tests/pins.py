"""Pin checks for the oracle, written against a ``chain`` callable with the
signature of ``oracle.gdn_fwd_chain(q, k, v, beta, log_alpha, m0, gate)``.

Each check returns the worst error it saw; the tests assert it is below a
bound.  They take the implementation as an argument so that the same checks
can be run on deliberately broken copies (tests/test_oracle_teeth.py) to
show that each pin catches the mistake it is meant to catch.

Everything the checks compare against is fixed by the pages or by
mathematics, never by the oracle itself:
  "Gated Delta Networks: Improving Mamba2 with Delta Rule" (paper review),
  sections "Method" (recurrence, SGD reading), "Key idea" (alpha -> 0 erases,
  alpha -> 1 is the pure delta rule), "Background" (associative memory of
  outer products: exact retrieval for orthogonal keys).
"""

import numpy as np

RNG_SEED = 12345


def rng(seed=RNG_SEED):
    return np.random.Generator(np.random.PCG64(seed))


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def orthonormal_keys(r, T, dk):
    Qm, _ = np.linalg.qr(r.standard_normal((dk, dk)))
    return Qm[:, :T].T.copy()           # T mutually orthonormal rows


def p2_orthonormal_retrieval(chain, dk=8, dv=5, T=6, gate="scalar"):
    """alpha = 1, beta = 1, orthonormal keys, any S0: the final state returns
    every stored value exactly (M_T^T k_i = v_i) and o_t = v_t when q_t = k_t.
    (Associative memory of outer products, "Background"; delta rule writes
    replace the value under a key, "Method".)"""
    r = rng(2)
    k = orthonormal_keys(r, T, dk)
    v = r.standard_normal((T, dv))
    q = k.copy()
    beta = np.ones(T)
    la = None if gate == "none" else (np.zeros(T) if gate == "scalar"
                                      else np.zeros((T, dk)))
    m0 = r.standard_normal((dk, dv))
    o, M = chain(q, k, v, beta, la, m0, gate)
    err = np.max(np.abs(M.T @ k.T - v.T))
    err = max(err, np.max(np.abs(o - v)))
    return err


def p3_gate_product(chain, dk=6, dv=4, T=9, gate="scalar"):
    """beta = 0: no writes, the state only decays: M_T = (prod alpha) M_0 and
    o_t = (prod_{s<=t} alpha_s) M_0^T q_t (per channel for the channel gate)."""
    r = rng(3)
    q = unit(r.standard_normal((T, dk)))
    k = unit(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    beta = np.zeros(T)
    m0 = r.standard_normal((dk, dv))
    if gate == "scalar":
        la = -0.02 * r.random(T)
        cum = np.exp(np.cumsum(la))[:, None] * np.ones((T, dk))
    else:
        la = -0.02 * r.random((T, dk))
        cum = np.exp(np.cumsum(la, axis=0))
    o, M = chain(q, k, v, beta, la, m0, gate)
    ref_o = np.stack([(cum[t][:, None] * m0).T @ q[t] for t in range(T)])
    ref_M = cum[-1][:, None] * m0
    return max(np.max(np.abs(o - ref_o)), np.max(np.abs(M - ref_M)))


def p6_erasure(chain, dk=6, dv=4, T=7, gate="scalar"):
    """log alpha = -60 (alpha -> 0, "Key idea": rapid erasure): each token
    sees an empty memory, so o_t = beta_t (k_t.q_t) v_t and
    M_T = beta_T k_T v_T^T (the fresh write is not decayed)."""
    r = rng(6)
    q = unit(r.standard_normal((T, dk)))
    k = unit(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    beta = r.random(T)
    la = np.full(T, -60.0) if gate == "scalar" else np.full((T, dk), -60.0)
    m0 = r.standard_normal((dk, dv))
    o, M = chain(q, k, v, beta, la, m0, gate)
    ref_o = (beta * np.sum(k * q, axis=1))[:, None] * v
    ref_M = beta[-1] * np.outer(k[-1], v[-1])
    return max(np.max(np.abs(o - ref_o)), np.max(np.abs(M - ref_M)))


def p7_gla_limit(chain, dk=10, dv=4, T=8, gate="scalar"):
    """Mutually orthogonal keys (coordinate axes for the channel gate) and
    S0 = 0: the delta correction never sees an earlier key, so the layer reduces to gated linear attention,
    o_t = sum_{s<=t} exp(G_t - G_s) beta_s (k_s.q_t) v_s, G the cumulative
    log-gate (per channel: the decay sits inside the k_s.q_t sum)."""
    r = rng(7)
    if gate == "scalar":
        k = orthonormal_keys(r, T, dk)
    else:
        # a per-channel decay rescales key directions; distinct coordinate
        # axes stay orthogonal under any diagonal scaling
        k = np.eye(dk)[r.permutation(dk)[:T]]
    q = unit(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    beta = r.random(T) * 1.5
    if gate == "scalar":
        la = -0.5 * r.random(T)
        G = np.cumsum(la)[:, None] * np.ones((T, dk))
    else:
        la = -0.5 * r.random((T, dk))
        G = np.cumsum(la, axis=0)
    o, M = chain(q, k, v, beta, la, np.zeros((dk, dv)), gate)
    ref = np.zeros((T, dv))
    for t in range(T):
        for s in range(t + 1):
            ref[t] += beta[s] * np.sum(np.exp(G[t] - G[s]) * k[s] * q[t]) * v[s]
    return np.max(np.abs(o - ref))


def p9_single_token(chain, dk=5, dv=3, gate="scalar"):
    """T = 1 written out from the page's equation in the stored orientation:
    S_1 = S_0 alpha (I - beta k k^T) + beta v k^T, o = S_1 q, M = S^T."""
    r = rng(9)
    q = unit(r.standard_normal(dk))
    k = unit(r.standard_normal(dk))
    v = r.standard_normal(dv)
    beta = 0.7
    S0 = r.standard_normal((dv, dk))
    if gate == "scalar":
        la = -0.3
        A = np.exp(la) * np.eye(dk)
        lat = np.array([la])
    else:
        la = -0.3 * r.random(dk)
        A = np.diag(np.exp(la))
        lat = la[None]
    S1 = S0 @ A @ (np.eye(dk) - beta * np.outer(k, k)) + beta * np.outer(v, k)
    o, M = chain(q[None], k[None], v[None], np.array([beta]), lat, S0.T.copy(),
                 gate)
    return max(np.max(np.abs(o[0] - S1 @ q)), np.max(np.abs(M - S1.T)))


def p5_norm_bound(chain, dk=8, dv=6, T=40, beta_max=2.0, zero_v=False,
                  gate="scalar"):
    """Unit keys, beta in [0, beta_max]: ||I - beta k k^T||_2 = max(1,|1-beta|)
    is 1 for beta in [0, 2], so ||M_t||_F <= alpha_t ||M_{t-1}||_F +
    beta_t ||v_t|| at every step; with v = 0 the norm never grows.
    Returns the largest violation ratio (<= 1 means the bound holds)."""
    r = rng(5)
    q = unit(r.standard_normal((T, dk)))
    k = unit(r.standard_normal((T, dk)))
    v = np.zeros((T, dv)) if zero_v else r.standard_normal((T, dv))
    beta = beta_max * r.random(T)
    beta[::7] = beta_max
    la = -0.05 * r.random(T) if gate == "scalar" else -0.05 * r.random((T, dk))
    M = r.standard_normal((dk, dv))
    worst = 0.0
    for t in range(T):
        _, Mn = chain(q[t:t + 1], k[t:t + 1], v[t:t + 1], beta[t:t + 1],
                      la[t:t + 1], M, gate)
        amax = np.max(np.exp(np.atleast_1d(la[t])))
        bound = amax * np.linalg.norm(M) + beta[t] * np.linalg.norm(v[t])
        worst = max(worst, np.linalg.norm(Mn) / bound)
        M = Mn
    return worst


# ------------------------------------------------ Householder products ---
# Checks of ``dp_fwd`` (signature of oracle.deltaproduct_fwd) for the
# Householder-product reading: nh delta steps per token after one decay.

def _dp_problem(r, T, H, nh, dk, dv):
    q = unit(r.standard_normal((1, T, H, dk)))
    k = unit(r.standard_normal((1, T, nh, H, dk)))
    v = r.standard_normal((1, T, nh, H, dv))
    beta = r.random((1, T, nh, H))
    la = -r.random((1, T, H))
    s0 = r.standard_normal((1, H, dk, dv))
    return q, k, v, beta, la, s0


def dp_single_step_is_gdn(dp_fwd, gdn_fwd, seed=7):
    """nh = 1 is the gated delta rule itself."""
    r = rng(seed)
    q, k, v, beta, la, s0 = _dp_problem(r, 9, 2, 1, 6, 5)
    o1, s1 = dp_fwd(q, k, v, beta, la, s0, "scalar")
    o2, s2 = gdn_fwd(q, k[:, :, 0], v[:, :, 0], beta[:, :, 0], la, s0, "scalar")
    return max(np.max(np.abs(o1 - o2)), np.max(np.abs(s1 - s2)))


def dp_reflections(dp_fwd, seed=8):
    """beta = 2 with unit keys and no write makes every factor a reflection:
    the Frobenius norm of the state is preserved, and the same key twice in
    one token cancels (H H = I).  Returns the worst deviation."""
    r = rng(seed)
    dk, dv, T = 5, 4, 6
    q, k, v, beta, la, s0 = _dp_problem(r, T, 1, 3, dk, dv)
    v[:] = 0.0
    beta[:] = 2.0
    _, s = dp_fwd(q, k, v, beta, None, s0, "none")
    worst = abs(np.linalg.norm(s[0, 0]) - np.linalg.norm(s0[0, 0]))
    k2 = np.repeat(k[:, :, :1], 2, axis=2)           # k_t1 = k_t2
    _, s = dp_fwd(q, k2, v[:, :, :2], beta[:, :, :2], None, s0, "none")
    return max(worst, np.max(np.abs(s - s0)))


def dp_two_step_closed_form(dp_fwd, seed=9):
    """One token, nh = 2, written with explicit Householder matrices:
    M_1 = H_2 (H_1 a M_0 + b_1 k_1 v_1^T) + b_2 k_2 v_2^T, H_j = I - b_j k_j k_j^T,
    o = M_1^T q.  Returns the worst deviation."""
    r = rng(seed)
    dk, dv = 4, 3
    q, k, v, beta, la, s0 = _dp_problem(r, 1, 1, 2, dk, dv)
    a = np.exp(la[0, 0, 0])
    k1, k2 = k[0, 0, 0, 0], k[0, 0, 1, 0]
    v1, v2 = v[0, 0, 0, 0], v[0, 0, 1, 0]
    b1, b2 = beta[0, 0, 0, 0], beta[0, 0, 1, 0]
    H1 = np.eye(dk) - b1 * np.outer(k1, k1)
    H2 = np.eye(dk) - b2 * np.outer(k2, k2)
    M = H2 @ (H1 @ (a * s0[0, 0]) + b1 * np.outer(k1, v1)) + b2 * np.outer(k2, v2)
    o, s = dp_fwd(q, k, v, beta, la, s0, "scalar")
    return max(np.max(np.abs(s[0, 0] - M)), np.max(np.abs(o[0, 0, 0] - M.T @ q[0, 0, 0])))


def dp_gate_once_per_token(dp_fwd, gdn_fwd, seed=10):
    """With beta = 0 on one of the two steps the token is a single gated
    delta step: the decay is applied once, before the steps.  Returns the
    worst deviation over both choices of the silent step."""
    r = rng(seed)
    q, k, v, beta, la, s0 = _dp_problem(r, 7, 2, 2, 5, 4)
    worst = 0.0
    for live in (0, 1):
        b = beta.copy()
        b[:, :, 1 - live] = 0.0
        o1, s1 = dp_fwd(q, k, v, b, la, s0, "scalar")
        o2, s2 = gdn_fwd(q, k[:, :, live], v[:, :, live], b[:, :, live], la, s0, "scalar")
        worst = max(worst, np.max(np.abs(o1 - o2)), np.max(np.abs(s1 - s2)))
    return worst


# ------------------------------------------------------------- draft trees ---
# Checks of oracle.tree_fwd / tree_commit / tree_wy_bruteforce (draft-tree
# verification): a node continues its parent's state with one step on its own
# token.  Each check reduces a tree to sequences of the pinned recurrence.

def _tree_problem(r, B, n, H, dk, dv, gate):
    q = unit(r.standard_normal((B, n, H, dk)))
    k = unit(r.standard_normal((B, n, H, dk)))
    v = r.standard_normal((B, n, H, dv))
    beta = r.random((B, n, H))
    if gate == "channel":
        la = -r.random((B, n, H, dk))
    elif gate == "scalar":
        la = -r.random((B, n, H))
    else:
        la = None
    s0 = r.standard_normal((B, H, dk, dv))
    return q, k, v, beta, la, s0


def random_tree(r, n):
    """Parents drawn uniformly from the earlier nodes and the root (-1)."""
    return np.array([int(r.integers(-1, i)) for i in range(n)], dtype=np.int64)


def _sel(la, b, idx, h):
    return None if la is None else la[b, idx, h][None, :, None]


def tree_chain_is_sequence(tree_fwd, gdn_fwd, gate, seed=21):
    """parent[i] = i - 1: the tree is one sequence."""
    r = rng(seed)
    q, k, v, beta, la, s0 = _tree_problem(r, 2, 9, 2, 5, 4, gate)
    par = np.tile(np.arange(9) - 1, (2, 1))
    o1, st = tree_fwd(q, k, v, beta, la, par, s0, gate)
    o2, sf = gdn_fwd(q, k, v, beta, la, s0, gate)
    return max(np.max(np.abs(o1 - o2)), np.max(np.abs(st[:, -1] - sf)))


def tree_star_is_single_steps(tree_fwd, gdn_decode, gate, seed=22):
    """All parents -1: every node is one decode step from the committed
    state."""
    r = rng(seed)
    n = 7
    q, k, v, beta, la, s0 = _tree_problem(r, 1, n, 2, 5, 4, gate)
    o1, st = tree_fwd(q, k, v, beta, la, np.full((1, n), -1), s0, gate)
    worst = 0.0
    for i in range(n):
        lai = None if la is None else la[:, i]
        o2, s2 = gdn_decode(q[:, i], k[:, i], v[:, i], beta[:, i], lai, s0, gate)
        worst = max(worst, np.max(np.abs(o1[:, i] - o2)), np.max(np.abs(st[:, i] - s2)))
    return worst


def tree_paths_are_sequences(tree_fwd, gdn_fwd, gate, seed=23):
    """Every node's output and state are those of the sequence of tokens on
    its root path."""
    r = rng(seed)
    n = 12
    q, k, v, beta, la, s0 = _tree_problem(r, 1, n, 2, 5, 4, gate)
    par = random_tree(r, n)
    o1, st = tree_fwd(q, k, v, beta, la, par[None], s0, gate)
    worst = 0.0
    for node in range(n):
        path, a = [], node
        while a >= 0:
            path.append(a)
            a = par[a]
        path = path[::-1]
        for h in range(2):
            lap = None if la is None else la[0, path, h][None, :, None]
            o2, s2 = gdn_fwd(q[0, path, h][None, :, None], k[0, path, h][None, :, None],
                             v[0, path, h][None, :, None], beta[0, path, h][None, :, None],
                             lap, s0[:, h:h + 1], gate)
            worst = max(worst, np.max(np.abs(o1[0, node, h] - o2[0, -1, 0])),
                        np.max(np.abs(st[0, node, h] - s2[0, 0])))
    return worst


def tree_commit_is_node_state(tree_commit, tree_fwd, gate, seed=24):
    """The commit of node a equals the verification's state after a (the
    two are computed along different routes); a = -1 keeps the committed
    state.  Trees packed by cu_seqlens."""
    r = rng(seed)
    lens = [6, 1, 9, 4]
    n = sum(lens)
    q, k, v, beta, la, _ = _tree_problem(r, 1, n, 2, 5, 4, gate)
    s0 = r.standard_normal((len(lens), 2, 5, 4))
    cu = np.concatenate([[0], np.cumsum(lens)])
    par = np.concatenate([random_tree(r, L) for L in lens])
    acc = np.array([3, -1, 8, 2])
    _, st = tree_fwd(q, k, v, beta, la, par, s0, gate, cu_seqlens=cu)
    new = tree_commit(k, v, beta, la, par, acc, s0, gate, cu_seqlens=cu)
    worst = 0.0
    for m, a in enumerate(acc):
        ref = s0[m] if a < 0 else st[0, cu[m] + a]
        worst = max(worst, np.max(np.abs(new[m] - ref)))
    return worst


def tree_wy_matches_recurrence(tree_wy, tree_fwd, gate, seed=25):
    """The tree WY form (one triangular solve over ancestors) gives every
    node's output."""
    r = rng(seed)
    n = 14
    q, k, v, beta, la, s0 = _tree_problem(r, 1, n, 1, 6, 3, gate)
    par = random_tree(r, n)
    o1, _ = tree_fwd(q, k, v, beta, la, par[None], s0, gate)
    lah = None if la is None else la[0, :, 0]
    o2 = tree_wy(q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0], lah, par, s0[0, 0], gate)
    return np.max(np.abs(o1[0, :, 0] - o2))


# ------------------------------------------------ Gated DeltaNet-2 ---
# Checks of the decoupled erase/write reading, written against a callable
# with the signature of oracle.gdn2_fwd_chain(q, k, v, erase, write,
# log_alpha, m0, gate).  Everything compared against is fixed without the
# decoupled oracle: the pinned gated delta rule, explicit sums and explicit
# matrix products.

def _g2_problem(r, T, dk, dv, gate, s0_std=0.5):
    q = unit(r.standard_normal((T, dk)))
    k = unit(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    er = 1.0 / (1.0 + np.exp(-r.standard_normal(T)))
    wr = 1.0 / (1.0 + np.exp(-r.standard_normal(T)))
    if gate == "none":
        la = None
    elif gate == "scalar":
        la = -np.logaddexp(0.0, r.standard_normal(T) - 2.0)
    else:
        la = -np.logaddexp(0.0, r.standard_normal((T, dk)) - 2.0)
    m0 = r.standard_normal((dk, dv)) * s0_std
    return q, k, v, er, wr, la, m0


def _decay_rows(la, t, gate, dk):
    """Per-row decay of token t (vector of dk)."""
    if gate == "none":
        return np.ones(dk)
    if gate == "scalar":
        return np.full(dk, np.exp(la[t]))
    return np.exp(la[t])


def g2_equal_strengths_is_gdn(g2, gdn_chain, gate, T=23, dk=8, dv=5, seed=31):
    """erase = write = beta: the gated delta rule (per-channel gate: the
    per-channel reading), i.e. the pinned gdn_fwd_chain."""
    r = rng(seed)
    q, k, v, er, _, la, m0 = _g2_problem(r, T, dk, dv, gate)
    o1, m1 = g2(q, k, v, er, er, la, m0, gate)
    o2, m2 = gdn_chain(q, k, v, er, la, m0, gate)
    return max(np.max(np.abs(o1 - o2)), np.max(np.abs(m1 - m2)))


def g2_no_erase_is_linear_attention(g2, gate, T=17, dk=7, dv=4, seed=32):
    """erase = 0: nothing is erased, every token only adds write_s v_s k_s^T
    to the decayed state, so o_t is the gated-linear-attention sum
        o_t = (D_t..D_1 M0)^T q_t + sum_{s<=t} write_s (q_t . (d_ts * k_s)) v_s
    with d_ts the product of the decays of tokens s+1..t (per channel),
    for any keys."""
    r = rng(seed)
    q, k, v, _, wr, la, m0 = _g2_problem(r, T, dk, dv, gate)
    o, m = g2(q, k, v, np.zeros(T), wr, la, m0, gate)
    worst = 0.0
    for t in range(T):
        dec0 = np.ones(dk)
        for u in range(t + 1):
            dec0 = dec0 * _decay_rows(la, u, gate, dk)
        want = (dec0[:, None] * m0).T @ q[t]
        for s in range(t + 1):
            d = np.ones(dk)
            for u in range(s + 1, t + 1):
                d = d * _decay_rows(la, u, gate, dk)
            want = want + wr[s] * np.dot(q[t], d * k[s]) * v[s]
        worst = max(worst, np.max(np.abs(o[t] - want)))
    return worst


def g2_no_write_is_erasure(g2, gate, T=11, dk=6, dv=4, seed=33):
    """write = 0: the state only decays and is projected away from each key,
    M_t = (I - erase_t k_t k_t^T) D_t M_{t-1} as explicit dk x dk matrices,
    and o_t = M_t^T q_t."""
    r = rng(seed)
    q, k, v, er, _, la, m0 = _g2_problem(r, T, dk, dv, gate)
    o, m = g2(q, k, v, er, np.zeros(T), la, m0, gate)
    M = m0.copy()
    worst = 0.0
    for t in range(T):
        Pm = np.eye(dk) - er[t] * np.outer(k[t], k[t])
        M = Pm @ np.diag(_decay_rows(la, t, gate, dk)) @ M
        worst = max(worst, np.max(np.abs(o[t] - M.T @ q[t])))
    return max(worst, np.max(np.abs(m - M)))


def g2_full_erase_stores_write(g2, gate, T=13, dk=8, dv=5, seed=34):
    """erase = 1 with unit keys: the old value under k_t is removed entirely
    and write_t v_t stored in its place, whatever the history and gate:
    M_t^T k_t = write_t v_t (read with q_t = k_t)."""
    r = rng(seed)
    q, k, v, _, wr, la, m0 = _g2_problem(r, T, dk, dv, gate, s0_std=1.0)
    o, _ = g2(q, k, v, np.ones(T), wr * 3.0, la, m0, gate)
    o2, _ = g2(k, k, v, np.ones(T), wr * 3.0, la, m0, gate)
    return max(np.max(np.abs(o2[t] - 3.0 * wr[t] * v[t])) for t in range(T))


def g2_chunked_equals_recurrence(g2, g2_chunked, gate, C, T=37, dk=8, dv=5, seed=35):
    """The decoupled chunk equations (erase in A and W, write in U) give the
    recurrence's outputs and final state for any chunk size."""
    r = rng(seed + C)
    q, k, v, er, wr, la, m0 = _g2_problem(r, T, dk, dv, gate)
    o1, m1 = g2(q, k, v, er, wr, la, m0, gate)
    o2, m2 = g2_chunked(q, k, v, er, wr, la, m0, gate, C)
    return max(np.max(np.abs(o1 - o2)), np.max(np.abs(m1 - m2)))


# ------------------------------------ short convolution + SiLU prologue ---
# Checks written against callables with the signatures of
# oracle.short_conv(x, taps, cu_seqlens) and oracle.silu(x); references are
# numpy's own convolution and closed forms.

def conv_equals_numpy_convolve(conv, seed=41, B=2, T=19, H=2, D=3, W=4):
    """Each channel of each row is numpy's full convolution of the inputs
    with the taps, cut to the first T outputs (y[t] = sum_j w[j] x[t-j])."""
    r = rng(seed)
    x = r.standard_normal((B, T, H, D))
    w = r.standard_normal((H, D, W))
    y = conv(x, w, None)
    worst = 0.0
    for b in range(B):
        for h in range(H):
            for c in range(D):
                ref = np.convolve(x[b, :, h, c], w[h, c])[:T]
                worst = max(worst, np.max(np.abs(y[b, :, h, c] - ref)))
    return worst


def conv_impulse_response(conv, T=12, W=4, t0=5, seed=42):
    """A unit impulse at token t0 returns the taps at t0 .. t0 + W - 1 and
    zero elsewhere (nothing before t0: causal)."""
    r = rng(seed)
    w = r.standard_normal((1, 2, W))
    x = np.zeros((1, T, 1, 2))
    x[0, t0, 0, 1] = 1.0
    y = conv(x, w, None)
    want = np.zeros((T,))
    want[t0:t0 + W] = w[0, 1, :min(W, T - t0)]
    return max(np.max(np.abs(y[0, :, 0, 1] - want)), np.max(np.abs(y[0, :, 0, 0])))


def conv_isolates_sequences(conv, seed=43, W=4):
    """Packed sequences never see each other: the packed result equals the
    sequences run alone (each with zero history)."""
    r = rng(seed)
    lens = [5, 0, 1, 9, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = r.standard_normal((1, int(cu[-1]), 2, 3))
    w = r.standard_normal((2, 3, W))
    y = conv(x, w, cu)
    worst = 0.0
    for n in range(len(lens)):
        a, e = int(cu[n]), int(cu[n + 1])
        if e > a:
            worst = max(worst, np.max(np.abs(y[:, a:e] - conv(x[:, a:e], w, None))))
    return worst


def silu_identities(silu):
    """silu(0) = 0; silu(x) - silu(-x) = x; silu(1) = 1 / (1 + e^-1);
    silu(40) = 40 and silu(-40) = 0 to within 1e-15 of 40."""
    x = np.linspace(-6, 6, 25)
    one = silu(np.array([0.0, 1.0, 40.0, -40.0]))
    return max(abs(one[0]),
               np.max(np.abs(silu(x) - silu(-x) - x)),
               abs(one[1] - 1.0 / (1.0 + np.exp(-1.0))),
               abs(one[2] - 40.0) / 40.0,
               abs(one[3]))


# ------------------------------------- adjoint of the prologue path ---
# Checked against central finite differences of the forward path (a
# callable with the signature of oracle.conv_prologue) and a closed form.

def prologue_bwd_fd(bwd, fwd, normalize, varlen, seed=46, W=3, eps=1e-6):
    """Largest error of the adjoint's dx and dtaps against central finite
    differences of L = sum dy * fwd(x, taps), relative to the gradient's
    largest entry.  varlen: two packed sequences (5 and 4 tokens)."""
    r = rng(seed)
    T, H, D = 9, 2, 3
    cu = np.array([0, 5, 9]) if varlen else None
    x = r.standard_normal((1, T, H, D))
    w = r.standard_normal((H, D, W))
    dy = r.standard_normal((1, T, H, D))
    dx, dw = bwd(x, w, normalize, dy, cu)
    L = lambda xx, ww: float(np.sum(dy * fwd(xx, ww, normalize, cu)))

    def fd(arr, which):
        g = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            p, m = arr.copy(), arr.copy()
            p[i] += eps
            m[i] -= eps
            g[i] = (L(p, w) - L(m, w)) / (2 * eps) if which == "x" else \
                   (L(x, p) - L(x, m)) / (2 * eps)
        return g

    gx, gw = fd(x, "x"), fd(w, "w")
    return max(np.max(np.abs(dx - gx)) / np.max(np.abs(gx)),
               np.max(np.abs(dw - gw)) / np.max(np.abs(gw)))


def prologue_bwd_width_one(bwd, seed=47):
    """Width 1 with unit taps and no normalisation: y = silu(x), so
    dx = dy silu'(x) and dtaps = sum_t dy silu'(x) x, with
    silu'(x) = s (1 + x (1 - s)), s = 1 / (1 + e^-x)."""
    r = rng(seed)
    x = r.standard_normal((2, 6, 2, 4))
    dy = r.standard_normal((2, 6, 2, 4))
    s = 1.0 / (1.0 + np.exp(-x))
    d = dy * s * (1.0 + x * (1.0 - s))
    dx, dw = bwd(x, np.ones((2, 4, 1)), False, dy, None)
    return max(np.max(np.abs(dx - d)),
               np.max(np.abs(dw[:, :, 0] - np.sum(d * x, axis=(0, 1)))))
