"""Plain fp64 numpy oracle of the gated delta rule (TEST INFRASTRUCTURE).

Only tests, the smoke check and the CPU-baseline leg of the benchmark may use
this module; the HIP library never does.  Every function works on fp64 numpy
arrays that are exact upcasts of the values handed to the GPU.

Definition followed ("Gated Delta Networks: Improving Mamba2 with Delta Rule",
paper review, section "Method"): the state update is

    S_t = S_{t-1} alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T

with S_t of shape dv x dk (the write v k^T fixes the orientation).  The state
is stored transposed, M = S^T (dk x dv), and the per-token step reads

    Mt  = a_t * M_{t-1}                      (a_t = exp(log alpha_t))
    e_t = beta_t (v_t - Mt^T k_t)
    M_t = Mt + k_t e_t^T
    o_t = M_t^T q_t                          (output of the updated state)

Readings where the pages are silent (each is listed in the design notes):
  * the output o_t = S_t q_t is read with the updated state, no 1/sqrt(dk)
    scale (the pages never write the output);
  * the gate arrives as log alpha; alpha_t decays the old state before the
    rank-1 correction and the fresh write beta v k^T is not decayed ("Method":
    decay is applied before the correction; "Key idea": alpha -> 0 erases);
  * the per-channel (Kimi-Delta-style) gate puts Diag(alpha_t) in place of the
    scalar: it scales the dk rows of M.  Parity with any external definition
    of that gate is UNPINNED (the pages only name it); the pins fix that the
    all-equal-channels case equals the scalar gate.
  * the backward is the gradient of <dO, o> + <dS_final, S_final> with respect
    to q, k, v, beta, log alpha and S_0 (the pages give no backward).
  * Householder-product transitions (only named by the pages): nh delta
    steps per token after a single decay, output after the last step (see
    deltaproduct_fwd).  Parity with an external definition is UNPINNED; the
    pins fix its reductions and reflection properties.

  * short convolution + SiLU in front of q, k, v (the block design of
    "Method"; the pages give neither the width nor the tap layout): a
    causal depthwise convolution of caller-given width and taps, no bias,
    zero history at every sequence start (short_conv, conv_prologue,
    gdn_fwd_conv).  Pinned by numpy's own convolution, causality, sequence
    isolation and SiLU identities.

  * draft trees (TreeWY, only summarised by the pages): a node continues
    its parent's state with one step on its own token; the verification
    returns every node's output, the commit rebuilds the accepted node's
    state from its root path (tree_fwd, tree_commit).  Pinned by reductions
    to the chain (a path tree is a sequence, a star tree is independent
    single steps, every root path is a sequence) and by the tree WY form.

  * Gated DeltaNet-2 (only named by the pages, as decoupling erase and
    write): the strength of the erase factor and of the write get separate
    values (gdn2_fwd).  Parity with an external definition is UNPINNED; the
    pins fix its reductions (to the gated delta rule, to gated linear
    attention, to pure erasure) and its overwrite property.

Parity pins (tests/test_oracle_pins.py): chunked brute-force form, orthonormal
retrieval, beta = 0 gate product, DeltaNet limit, norm bound, alpha -> 0
erasure, gated-linear-attention limit, SGD reading, T = 1 closed form,
equal-channel reduction, boundary semantics, finite differences for the
adjoint and for the prologue path's adjoint, plus a hand-worked golden
example.  Nothing here is "parity
unpinned" except the matches of the per-channel gate, the Householder
products, the draft trees and Gated DeltaNet-2 to external definitions.
"""

from __future__ import annotations

import numpy as np

GATES = ("none", "scalar", "channel")


# --------------------------------------------------------------------------
# helpers (no method arithmetic)
# --------------------------------------------------------------------------

def _segments(B: int, T: int, cu_seqlens):
    """Yield (b, start, end, seq_index) for dense [B,T] or varlen packing."""
    if cu_seqlens is None:
        for b in range(B):
            yield b, 0, T, b
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        assert B == 1 and cu[0] == 0 and cu[-1] == T
        for n in range(len(cu) - 1):
            yield 0, int(cu[n]), int(cu[n + 1]), n


def _gate_rows(log_alpha_t, gate: str, dk: int):
    """Per-row multiplier of the state for one token (vector of length dk)."""
    if gate == "none":
        return np.ones(dk)
    if gate == "scalar":
        return np.full(dk, np.exp(float(log_alpha_t)))
    if gate == "channel":
        return np.exp(np.asarray(log_alpha_t, dtype=np.float64))
    raise ValueError(gate)


def normwise_rel_err(x, y, floor_frac: float = 1e-30):
    """max over leading slices of max|x-y| / max|y| (see README of tests).

    ``x`` and ``y`` have the same shape; the error is evaluated per slice of the
    last two axes when they exist.  A slice whose reference is below 1e-30 is
    judged by absolute error relative to the global max |y|.
    """
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    assert x.shape == y.shape, (x.shape, y.shape)
    if x.size == 0:
        return 0.0
    gmax = float(np.max(np.abs(y)))
    if x.ndim <= 2:
        x2, y2 = x.reshape(1, -1), y.reshape(1, -1)
    else:
        x2 = x.reshape(-1, x.shape[-2] * x.shape[-1])
        y2 = y.reshape(-1, y.shape[-2] * y.shape[-1])
    worst = 0.0
    for xs, ys in zip(x2, y2):
        ref = float(np.max(np.abs(ys)))
        diff = float(np.max(np.abs(xs - ys)))
        if not np.isfinite(diff):
            return float("inf")
        if ref < floor_frac:
            err = diff / gmax if gmax > 0 else diff
        else:
            err = diff / ref
        worst = max(worst, err)
    return worst


# --------------------------------------------------------------------------
# forward: the token-by-token recurrence ("Method")
# --------------------------------------------------------------------------

def gdn_fwd_chain(q, k, v, beta, log_alpha, m0, gate: str):
    """One (sequence, head): q,k [T,dk], v [T,dv], beta [T], log_alpha [T] /
    [T,dk] / None, m0 [dk,dv].  Returns (o [T,dv], M_T [dk,dv])."""
    T, dk = k.shape
    dv = v.shape[1]
    M = np.array(m0, dtype=np.float64, copy=True)
    o = np.zeros((T, dv))
    for t in range(T):
        a = _gate_rows(None if log_alpha is None else log_alpha[t], gate, dk)
        Mt = a[:, None] * M                      # decay the old state first
        e = beta[t] * (v[t] - Mt.T @ k[t])       # error of the decayed state
        M = Mt + np.outer(k[t], e)               # rank-1 delta correction
        o[t] = M.T @ q[t]                        # read the updated state
    return o, M


def gdn_fwd(q, k, v, beta, log_alpha, s0=None, gate: str = "scalar",
            cu_seqlens=None):
    """Whole batch.  q,k [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H];
    log_alpha [B,T,H] (scalar), [B,T,H,dk] (channel) or None (gate none);
    s0 [B|N,H,dk,dv] or None (zeros).  cu_seqlens [N+1] packs N sequences
    into B = 1.  Returns o [B,T,H,dv] and s_final [B|N,H,dk,dv]."""
    assert gate in GATES
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    nseq = B if cu_seqlens is None else len(cu_seqlens) - 1
    o = np.zeros((B, T, H, dv))
    sf = np.zeros((nseq, H, dk, dv))
    for b, t0, t1, n in _segments(B, T, cu_seqlens):
        for h in range(H):
            m0 = np.zeros((dk, dv)) if s0 is None else s0[n, h]
            la = None if gate == "none" else log_alpha[b, t0:t1, h]
            o[b, t0:t1, h], sf[n, h] = gdn_fwd_chain(
                q[b, t0:t1, h], k[b, t0:t1, h], v[b, t0:t1, h],
                beta[b, t0:t1, h], la, m0, gate)
    return o, sf


# --------------------------------------------------------------------------
# L2-normalised q and k ("Method": the block normalises q and k)
# --------------------------------------------------------------------------

def l2_normalize(x):
    """x / ||x|| over the last axis, each (token, head) row separately; an
    all-zero row stays zero."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.divide(x, n, out=np.zeros_like(x), where=n > 0)


def gdn_fwd_qknorm(q, k, v, beta, log_alpha, s0=None, gate: str = "scalar",
                   cu_seqlens=None):
    """The forward with q and k L2-normalised per (token, head) first ("Gated
    Delta Networks: Improving Mamba2 with Delta Rule", "Method": in the block
    design q and k go through an L2 normalisation for training stability,
    v does not).  Same shapes and returns as :func:`gdn_fwd`."""
    return gdn_fwd(l2_normalize(q), l2_normalize(k), v, beta, log_alpha, s0,
                   gate, cu_seqlens=cu_seqlens)


# --------------------------------------------------------------------------
# short causal convolution and SiLU in front of the recurrence ("Method":
# in the block design q and k pass through a projection, a short convolution
# and SiLU before the L2 normalisation; v takes the same path without it)
# --------------------------------------------------------------------------

def short_conv(x, taps, cu_seqlens=None):
    """Causal depthwise convolution over time, channel by channel:

        y[b, t, h, c] = sum_{j=0}^{W-1} taps[h, c, j] * x[b, t - j, h, c]

    tap j weighs the input j tokens back; inputs before the start of the
    sequence (dense row or packed varlen sequence) read as zero, so packed
    sequences never see each other.  x [B,T,H,D], taps [H,D,W]."""
    x = np.asarray(x, dtype=np.float64)
    taps = np.asarray(taps, dtype=np.float64)
    B, T, H, D = x.shape
    W = taps.shape[-1]
    y = np.zeros_like(x)
    for b, t0, t1, _ in _segments(B, T, cu_seqlens):
        for t in range(t0, t1):
            for j in range(W):
                if t - j >= t0:
                    y[b, t] += taps[:, :, j] * x[b, t - j]
    return y


def silu(x):
    """x * sigmoid(x)."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def conv_prologue(x, taps, normalize, cu_seqlens=None):
    """The path of one projection: short convolution, SiLU, and for q and k
    the L2 normalisation per (token, head)."""
    y = silu(short_conv(x, taps, cu_seqlens))
    return l2_normalize(y) if normalize else y


def conv_prologue_bwd(x, taps, normalize, dy, cu_seqlens=None):
    """Adjoint of :func:`conv_prologue`: the gradients of
    L = sum dy * conv_prologue(x, taps, normalize) with respect to x [B,T,H,D]
    and taps [H,D,W], taking the path's three steps back in reverse order:

      y = a / |a|        da = (dy - y (y . dy)) / |a|   (an all-zero row: 0)
      a = z sigmoid(z)   dz = da (s + a (1 - s)),  s = sigmoid(z)
      z[t] = sum_j taps[:, :, j] x[t - j]  (inside each sequence)
                         dx[t - j] += taps[:, :, j] dz[t]
                         dtaps[:, :, j] += dz[t] x[t - j]

    The pages define the forward path only; this is its chain rule.
    Returns (dx, dtaps)."""
    x = np.asarray(x, dtype=np.float64)
    taps = np.asarray(taps, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    B, T, H, D = x.shape
    W = taps.shape[-1]
    z = short_conv(x, taps, cu_seqlens)
    sg = 1.0 / (1.0 + np.exp(-z))
    a = z * sg
    if normalize:
        n = np.sqrt(np.sum(a * a, axis=-1, keepdims=True))
        y = np.divide(a, n, out=np.zeros_like(a), where=n > 0)
        proj = dy - y * np.sum(y * dy, axis=-1, keepdims=True)
        da = np.divide(proj, n, out=np.zeros_like(a), where=n > 0)
    else:
        da = dy
    dz = da * (sg + a * (1.0 - sg))
    dx = np.zeros_like(x)
    dtaps = np.zeros_like(taps)
    for b, t0, t1, _ in _segments(B, T, cu_seqlens):
        for t in range(t0, t1):
            for j in range(W):
                if t - j >= t0:
                    dx[b, t - j] += taps[:, :, j] * dz[b, t]
                    dtaps[:, :, j] += dz[b, t] * x[b, t - j]
    return dx, dtaps


def gdn_fwd_conv(xq, xk, xv, wq, wk, wv, beta, log_alpha, s0=None,
                 gate: str = "scalar", cu_seqlens=None):
    """The forward on the block's q, k, v paths: q = l2(silu(conv(xq))),
    k = l2(silu(conv(xk))), v = silu(conv(xv)), then :func:`gdn_fwd`.
    xq, xk [B,T,H,dk], xv [B,T,H,dv]; wq, wk [H,dk,W], wv [H,dv,W]."""
    return gdn_fwd(conv_prologue(xq, wq, True, cu_seqlens),
                   conv_prologue(xk, wk, True, cu_seqlens),
                   conv_prologue(xv, wv, False, cu_seqlens),
                   beta, log_alpha, s0, gate, cu_seqlens=cu_seqlens)


# --------------------------------------------------------------------------
# Householder-product transitions (several delta steps per token)
# --------------------------------------------------------------------------

def deltaproduct_fwd(q, k, v, beta, log_alpha, s0=None, gate: str = "scalar",
                     cu_seqlens=None):
    """Products of generalised Householder transitions per token ("Gated Delta
    Networks: Improving Mamba2 with Delta Rule", paper review, "Future work"
    and the closing section: Householder-product transitions can be grafted
    onto the gated delta rule).  The pages give no formula; the reading taken
    is the plainest one: token t carries nh (key, value, beta) triples, the
    state is decayed once by alpha_t and then takes the nh delta-rule steps
    in order,

        M <- a_t M;   for j = 1..nh:  e = beta_tj (v_tj - M^T k_tj),
                                      M <- M + k_tj e^T
        o_t = M^T q_t  (after the last step),

    so that S_t = S_{t-1} alpha_t H_t1 ... H_tnh + writes with
    H_tj = I - beta_tj k_tj k_tj^T.  nh = 1 is :func:`gdn_fwd`.

    Shapes: q [B,T,H,dk]; k [B,T,nh,H,dk]; v [B,T,nh,H,dv]; beta [B,T,nh,H];
    log_alpha [B,T,H] (scalar gate) or None (gate none); s0 as in gdn_fwd;
    cu_seqlens counts tokens.  Returns o [B,T,H,dv], s_final."""
    assert gate in ("none", "scalar")
    B, T, H, dk = q.shape
    nh = k.shape[2]
    dv = v.shape[-1]
    nseq = B if cu_seqlens is None else len(cu_seqlens) - 1
    o = np.zeros((B, T, H, dv))
    sf = np.zeros((nseq, H, dk, dv))
    for b, t0, t1, n in _segments(B, T, cu_seqlens):
        for h in range(H):
            M = np.zeros((dk, dv)) if s0 is None else np.array(s0[n, h], dtype=np.float64)
            for t in range(t0, t1):
                a = 1.0 if gate == "none" else float(np.exp(log_alpha[b, t, h]))
                M = a * M                                   # one decay per token
                for j in range(nh):
                    kj = k[b, t, j, h]
                    e = beta[b, t, j, h] * (v[b, t, j, h] - M.T @ kj)
                    M = M + np.outer(kj, e)                 # delta step j
                o[b, t, h] = M.T @ q[b, t, h]
            sf[n, h] = M
    return o, sf


def gdn_decode(q, k, v, beta, log_alpha, state, gate: str = "scalar"):
    """One token per (sequence, head): q,k [N,H,dk], v [N,H,dv], beta [N,H],
    log_alpha [N,H] / [N,H,dk] / None, state [N,H,dk,dv].  Returns
    (o [N,H,dv], new state); the input state is not modified."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((N, H, dv))
    new = np.array(state, dtype=np.float64, copy=True)
    for n in range(N):
        for h in range(H):
            la = None if gate == "none" else log_alpha[n, h][None]
            oo, mm = gdn_fwd_chain(q[n, h][None], k[n, h][None], v[n, h][None],
                                   beta[n, h][None], la, state[n, h], gate)
            o[n, h] = oo[0]
            new[n, h] = mm
    return o, new


# --------------------------------------------------------------------------
# draft trees: verification and commit ("TreeWY: Speculative Verification for
# Gated DeltaNet Hybrids")
# --------------------------------------------------------------------------

def _tree_parent(parent):
    """Parent array of one tree: node i's parent is an earlier node or -1
    (the committed state)."""
    p = np.asarray(parent, dtype=np.int64)
    assert p.ndim == 1 and np.all((p >= -1) & (p < np.arange(len(p)))), \
        "every parent precedes its child"
    return p


def _trees(B: int, n: int, parent, cu_seqlens):
    """Yield (b, start, end, tree index, parent array) for B dense trees of n
    nodes (parent [B, n]) or trees packed by cu_seqlens (parent [total])."""
    for b, t0, t1, m in _segments(B, n, cu_seqlens):
        par = parent[b] if cu_seqlens is None else parent[t0:t1]
        yield b, t0, t1, m, _tree_parent(par)


def tree_fwd(q, k, v, beta, log_alpha, parent, s0=None, gate: str = "scalar",
             cu_seqlens=None):
    """Every node of draft trees hanging off a committed state.  Node i takes
    one step of the recurrence on its own token from the state of its parent
    (the committed state when parent[i] = -1) and reads its output from the
    result, so each node sees exactly the tokens on its root path.
    q,k [B,n,H,dk]; v [B,n,H,dv]; beta [B,n,H]; log_alpha as in gdn_fwd;
    parent [B,n] int (indices inside the tree), or with cu_seqlens (trees
    packed into B = 1) parent [total] with each tree counting from 0;
    s0 [N,H,dk,dv] committed states (zeros if None).
    Returns (o [B,n,H,dv], states [B,n,H,dk,dv]: the state after each node)."""
    assert gate in GATES
    B, n, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, n, H, dv))
    st = np.zeros((B, n, H, dk, dv))
    for b, t0, t1, m, par in _trees(B, n, parent, cu_seqlens):
        for h in range(H):
            m0 = np.zeros((dk, dv)) if s0 is None else s0[m, h]
            for i in range(t1 - t0):
                t = t0 + i
                prev = m0 if par[i] < 0 else st[b, t0 + par[i], h]
                la = None if gate == "none" else log_alpha[b, t:t + 1, h]
                oo, mm = gdn_fwd_chain(q[b, t:t + 1, h], k[b, t:t + 1, h],
                                       v[b, t:t + 1, h], beta[b, t:t + 1, h],
                                       la, prev, gate)
                o[b, t, h], st[b, t, h] = oo[0], mm
    return o, st


def tree_path(parent, node):
    """Nodes from the root down to ``node`` (empty for node = -1)."""
    par = _tree_parent(parent)
    path = []
    while node >= 0:
        path.append(int(node))
        node = par[node]
    return path[::-1]


def tree_commit(k, v, beta, log_alpha, parent, accepted, s0=None,
                gate: str = "scalar", cu_seqlens=None):
    """New committed state of every tree after accepting node accepted[m]:
    the tokens on that node's root path, in order, run through the plain
    recurrence from the committed state; accepted = -1 keeps it.  Shapes as
    in tree_fwd; accepted [N].  Returns the states [N,H,dk,dv]."""
    assert gate in GATES
    B, n, H, dk = k.shape
    dv = v.shape[-1]
    N = B if cu_seqlens is None else len(cu_seqlens) - 1
    out = np.zeros((N, H, dk, dv))
    for b, t0, t1, m, par in _trees(B, n, parent, cu_seqlens):
        idx = [t0 + i for i in tree_path(par, int(accepted[m]))]
        for h in range(H):
            m0 = np.zeros((dk, dv)) if s0 is None else s0[m, h]
            if not idx:
                out[m, h] = m0
                continue
            la = None if gate == "none" else log_alpha[b, idx, h]
            _, out[m, h] = gdn_fwd_chain(np.zeros((len(idx), dk)), k[b, idx, h],
                                         v[b, idx, h], beta[b, idx, h], la, m0, gate)
    return out


def tree_wy_bruteforce(q, k, v, beta, log_alpha, parent, m0, gate: str):
    """The tree-structured WY form of one (tree, head), with an explicit
    dense inverse: the chunk equations of gdn_chunked_bruteforce with "i
    before r" replaced by "i is an ancestor of r" and the cumulative log gate
    summed along root paths,
        g_r = log alpha_r + g_parent(r),   gamma = exp(g),
        A_ri = beta_r exp(g_r - g_i) k_r.k_i   (i a strict ancestor of r),
        T = (I + A)^-1,  U = T diag(beta) V,  W = T diag(beta*gamma) K,
        E = U - W M0,    O = diag(gamma) Q M0 + (Q K^T o Gamma) E
    with Gamma_ri = exp(g_r - g_i) for i an ancestor of r or r itself and 0
    elsewhere: one triangular system verifies every node.  Returns O."""
    par = _tree_parent(parent)
    n, dk = k.shape
    anc = np.zeros((n, n), dtype=bool)
    for r in range(n):
        a = par[r]
        while a >= 0:
            anc[r, a] = True
            a = par[a]
    g = np.zeros((n, dk))
    for r in range(n):
        if gate == "scalar":
            own = np.full(dk, float(log_alpha[r]))
        elif gate == "channel":
            own = np.asarray(log_alpha[r], dtype=np.float64)
        else:
            own = np.zeros(dk)
        g[r] = own + (g[par[r]] if par[r] >= 0 else 0.0)
    A = np.zeros((n, n))
    P = np.zeros((n, n))
    for r in range(n):
        for i in range(n):
            if anc[r, i] or i == r:
                d = np.exp(g[r] - g[i])
                P[r, i] = np.sum(q[r] * k[i] * d)
                if i != r:
                    A[r, i] = beta[r] * np.sum(k[r] * k[i] * d)
    Tm = np.linalg.inv(np.eye(n) + A)
    U = Tm @ (beta[:, None] * v)
    W = Tm @ (beta[:, None] * k * np.exp(g))
    E = U - W @ m0
    return (q * np.exp(g)) @ m0 + P @ E


# --------------------------------------------------------------------------
# independent forms used only to pin the recurrence
# --------------------------------------------------------------------------

def delta_rule_ungated(q, k, v, beta, m0):
    """Plain delta rule with no gate at all ("Key idea": alpha -> 1 recovers
    the pure delta rule).  Written as an associative-memory update: read the
    current value stored under key k, move it toward v by beta."""
    M = np.array(m0, dtype=np.float64, copy=True)
    o = np.zeros((k.shape[0], v.shape[1]))
    for t in range(k.shape[0]):
        stored = M.T @ k[t]
        M = M + beta[t] * np.outer(k[t], v[t] - stored)
        o[t] = M.T @ q[t]
    return o, M


def gdn_sgd_form(q, k, v, beta, log_alpha, m0, gate: str):
    """Test-time-SGD reading ("Method"): the state is a fast weight decayed
    by alpha_t (adaptive weight decay), then one gradient step of learning
    rate beta_t on the loss 0.5 * ||Mt^T k_t - v_t||^2."""
    T, dk = k.shape
    M = np.array(m0, dtype=np.float64, copy=True)
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        a = _gate_rows(None if log_alpha is None else log_alpha[t], gate, dk)
        W = M * a[:, None]
        residual = W.T @ k[t] - v[t]             # prediction error
        grad = np.outer(k[t], residual)          # d/dW of 0.5*||W^T k - v||^2
        M = W - beta[t] * grad
        o[t] = M.T @ q[t]
    return o, M


def gdn_chunked_bruteforce(q, k, v, beta, log_alpha, m0, gate: str, C: int):
    """Chunkwise form of one chain with an explicit dense inverse.

    Within a chunk of c tokens, g is the inclusive chunk-local cumulative
    log-gate, gamma = exp(g), and (scalar gate)
        A_ri = beta_r exp(g_r - g_i) k_r.k_i   (i < r),  T = (I + A)^-1
        U = T diag(beta) V,   W = T diag(beta*gamma) K,   E = U - W M0
        O = diag(gamma) Q M0 + (Q K^T o Gamma) E,  Gamma_ri = exp(g_r-g_i), i<=r
        M_c = gamma_c M0 + (K o exp(g_c - g))^T E
    For the per-channel gate every exp(g_r - g_i) x.y becomes
    sum_c x_c y_c exp(g_rc - g_ic) and gamma multiplies channels.
    These equations are the unrolled recurrence (WY representation + UT
    transform named in "Method"); this routine checks them, not the GPU.
    """
    T, dk = k.shape
    dv = v.shape[1]
    M = np.array(m0, dtype=np.float64, copy=True)
    o = np.zeros((T, dv))
    for s in range(0, T, C):
        e_ = min(T, s + C)
        c = e_ - s
        K, Q, V, bt = k[s:e_], q[s:e_], v[s:e_], beta[s:e_]
        if gate == "none":
            g = np.zeros((c, dk))
        elif gate == "scalar":
            g = np.repeat(np.cumsum(log_alpha[s:e_])[:, None], dk, axis=1)
        else:
            g = np.cumsum(log_alpha[s:e_], axis=0)
        # pairwise decays D[r,i,c] = exp(g_rc - g_ic) for i <= r, 0 otherwise
        A = np.zeros((c, c))
        P = np.zeros((c, c))
        for r in range(c):
            for i in range(r + 1):
                d = np.exp(g[r] - g[i])
                P[r, i] = np.sum(Q[r] * K[i] * d)
                if i < r:
                    A[r, i] = bt[r] * np.sum(K[r] * K[i] * d)
        Tm = np.linalg.inv(np.eye(c) + A)
        U = Tm @ (bt[:, None] * V)
        W = Tm @ (bt[:, None] * K * np.exp(g))
        E = U - W @ M
        o[s:e_] = (Q * np.exp(g)) @ M + P @ E
        M = np.exp(g[-1])[:, None] * M + (K * np.exp(g[-1][None, :] - g)).T @ E
    return o, M


# --------------------------------------------------------------------------
# Gated DeltaNet-2: decoupled erase and write strengths ("Linear Attention
# Architectures: Mechanisms, Trade-offs, and Cross-Layer Routing", abstract,
# and the related-paper entry "Gated DeltaNet-2: Decoupling Erase and Write
# in Linear Attention"; the pages name the method and say it generalises
# Gated DeltaNet and Kimi Delta Attention, but print no formula)
# --------------------------------------------------------------------------

def gdn2_fwd_chain(q, k, v, erase, write, log_alpha, m0, gate: str):
    """One (sequence, head) of the reading taken here: the gated delta rule's
    single strength beta_t does two jobs, erasing the old value stored under
    k_t (the factor I - beta k k^T) and writing the new one (beta v k^T); the
    decoupled rule gives each job its own strength,

        S_t = S_{t-1} D_t (I - erase_t k_t k_t^T) + write_t v_t k_t^T,

    D_t = alpha_t (scalar gate) or Diag(alpha_t) (per-channel gate), so that
    erase = write is Gated DeltaNet (scalar gate) or the per-channel
    (Kimi-Delta-style) reading, and erase = 0 is gated linear attention.
    Stored orientation M = S^T: Mt = D M, e = write v - erase Mt^T k,
    M = Mt + k e^T, o = M^T q.  Shapes as gdn_fwd_chain; erase, write [T].
    Parity with any external definition of Gated DeltaNet-2 is UNPINNED."""
    T, dk = k.shape
    dv = v.shape[1]
    M = np.array(m0, dtype=np.float64, copy=True)
    o = np.zeros((T, dv))
    for t in range(T):
        a = _gate_rows(None if log_alpha is None else log_alpha[t], gate, dk)
        Mt = a[:, None] * M                              # decay first
        e = write[t] * v[t] - erase[t] * (Mt.T @ k[t])   # write minus erased value
        M = Mt + np.outer(k[t], e)
        o[t] = M.T @ q[t]
    return o, M


def gdn2_fwd(q, k, v, erase, write, log_alpha, s0=None, gate: str = "scalar",
             cu_seqlens=None):
    """Whole batch of :func:`gdn2_fwd_chain`; shapes and returns as
    :func:`gdn_fwd` with erase and write [B,T,H] in place of beta."""
    assert gate in GATES
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    nseq = B if cu_seqlens is None else len(cu_seqlens) - 1
    o = np.zeros((B, T, H, dv))
    sf = np.zeros((nseq, H, dk, dv))
    for b, t0, t1, n in _segments(B, T, cu_seqlens):
        for h in range(H):
            m0 = np.zeros((dk, dv)) if s0 is None else s0[n, h]
            la = None if gate == "none" else log_alpha[b, t0:t1, h]
            o[b, t0:t1, h], sf[n, h] = gdn2_fwd_chain(
                q[b, t0:t1, h], k[b, t0:t1, h], v[b, t0:t1, h], erase[b, t0:t1, h],
                write[b, t0:t1, h], la, m0, gate)
    return o, sf


def gdn2_decode(q, k, v, erase, write, log_alpha, state, gate: str = "scalar"):
    """One token per (sequence, head) of the decoupled rule: q,k [N,H,dk],
    v [N,H,dv], erase, write [N,H], log_alpha [N,H] / [N,H,dk] / None,
    state [N,H,dk,dv].  Returns (o [N,H,dv], new state)."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((N, H, dv))
    new = np.array(state, dtype=np.float64, copy=True)
    for n in range(N):
        for h in range(H):
            la = None if gate == "none" else log_alpha[n, h][None]
            oo, mm = gdn2_fwd_chain(q[n, h][None], k[n, h][None], v[n, h][None],
                                    erase[n, h][None], write[n, h][None], la,
                                    state[n, h], gate)
            o[n, h] = oo[0]
            new[n, h] = mm
    return o, new


def gdn2_chunked_bruteforce(q, k, v, erase, write, log_alpha, m0, gate: str, C: int):
    """Chunkwise form of one chain of the decoupled rule with an explicit
    dense inverse.  Unrolling e_r = write_r v_r - erase_r Mt_r^T k_r over a
    chunk gives (I + A) E = diag(write) V - diag(erase * gamma) K M0 with
    A_ri = erase_r exp(g_r - g_i) k_r.k_i (i < r): the erase strength enters
    A and W, the write strength only U:
        T = (I + A)^-1,  U = T diag(write) V,  W = T diag(erase*gamma) K,
        E = U - W M0,    O = diag(gamma) Q M0 + (Q K^T o Gamma) E,
        M_c = gamma_c M0 + (K o exp(g_c - g))^T E
    (per-channel gate: the decays move inside the key sums as in
    gdn_chunked_bruteforce).  Checks the equations, not the GPU."""
    T, dk = k.shape
    dv = v.shape[1]
    M = np.array(m0, dtype=np.float64, copy=True)
    o = np.zeros((T, dv))
    for s in range(0, T, C):
        e_ = min(T, s + C)
        c = e_ - s
        K, Q, V = k[s:e_], q[s:e_], v[s:e_]
        er, wr = erase[s:e_], write[s:e_]
        if gate == "none":
            g = np.zeros((c, dk))
        elif gate == "scalar":
            g = np.repeat(np.cumsum(log_alpha[s:e_])[:, None], dk, axis=1)
        else:
            g = np.cumsum(log_alpha[s:e_], axis=0)
        A = np.zeros((c, c))
        P = np.zeros((c, c))
        for r in range(c):
            for i in range(r + 1):
                d = np.exp(g[r] - g[i])
                P[r, i] = np.sum(Q[r] * K[i] * d)
                if i < r:
                    A[r, i] = er[r] * np.sum(K[r] * K[i] * d)
        Tm = np.linalg.inv(np.eye(c) + A)
        U = Tm @ (wr[:, None] * V)
        W = Tm @ (er[:, None] * K * np.exp(g))
        E = U - W @ M
        o[s:e_] = (Q * np.exp(g)) @ M + P @ E
        M = np.exp(g[-1])[:, None] * M + (K * np.exp(g[-1][None, :] - g)).T @ E
    return o, M


# --------------------------------------------------------------------------
# backward: adjoint of the token recurrence (derived by hand from "Method")
# --------------------------------------------------------------------------

def gdn_bwd_chain(q, k, v, beta, log_alpha, m0, do, dmT, gate: str,
                  ckpt: int = 64):
    """Adjoint of one chain.  Loss L = sum_t <dO_t, o_t> + <dmT, M_T>.

    With D = Diag(a_t), P = I - beta_t k_t k_t^T, Mt = D M_{t-1} and
    G = dL/dM_t (accumulated from the future):
        G   += q_t dO_t^T
        dq_t = M_t dO_t
        dv_t = beta_t G^T k_t
        dbeta_t = (G^T k_t) . (v_t - Mt^T k_t)
        dk_t = -beta_t (G Mt^T + Mt G^T) k_t + beta_t G v_t
        dla_t[i] = a_i sum_j (P G)_ij (M_{t-1})_ij   (scalar: summed over i)
        G    = D P G
    and dM_0 = G at the end.  States are checkpointed every ``ckpt`` tokens
    and recomputed segment by segment in reverse.
    Returns dq, dk, dv, dbeta, dla (None for gate none), dm0."""
    T, dk = k.shape
    dv = v.shape[1]
    # forward pass storing checkpoints M_{s} at segment starts
    starts = list(range(0, T, ckpt)) if T > 0 else []
    ck = {}
    M = np.array(m0, dtype=np.float64, copy=True)
    for t in range(T):
        if t % ckpt == 0:
            ck[t] = M.copy()
        a = _gate_rows(None if log_alpha is None else log_alpha[t], gate, dk)
        Mt = a[:, None] * M
        e = beta[t] * (v[t] - Mt.T @ k[t])
        M = Mt + np.outer(k[t], e)
    dq = np.zeros((T, dk))
    dkk = np.zeros((T, dk))
    dvv = np.zeros((T, dv))
    db = np.zeros(T)
    dla = None if gate == "none" else np.zeros(np.shape(log_alpha))
    G = np.zeros((dk, dv)) if dmT is None else np.array(dmT, dtype=np.float64)
    for s in reversed(starts):
        e_ = min(T, s + ckpt)
        # recompute the states of this segment: prev[t-s] = M_{t-1}
        prev = []
        M = ck[s].copy()
        for t in range(s, e_):
            prev.append(M.copy())
            a = _gate_rows(None if log_alpha is None else log_alpha[t], gate, dk)
            Mt = a[:, None] * M
            e = beta[t] * (v[t] - Mt.T @ k[t])
            M = Mt + np.outer(k[t], e)
        post = prev[1:] + [M]                    # post[t-s] = M_t
        for t in reversed(range(s, e_)):
            Mprev = prev[t - s]
            Mcur = post[t - s]
            a = _gate_rows(None if log_alpha is None else log_alpha[t], gate, dk)
            Mt = a[:, None] * Mprev
            kt, vt, bt = k[t], v[t], beta[t]
            G = G + np.outer(q[t], do[t])
            dq[t] = Mcur @ do[t]
            Gk = G.T @ kt
            dvv[t] = bt * Gk
            db[t] = Gk @ (vt - Mt.T @ kt)
            dkk[t] = -bt * (G @ (Mt.T @ kt) + Mt @ (G.T @ kt)) + bt * (G @ vt)
            PG = G - bt * np.outer(kt, kt @ G)
            if gate == "scalar":
                dla[t] = a[0] * np.sum(PG * Mprev)
            elif gate == "channel":
                dla[t] = a * np.sum(PG * Mprev, axis=1)
            G = a[:, None] * PG
    return dq, dkk, dvv, db, dla, G


def gdn_bwd(q, k, v, beta, log_alpha, s0, do, ds_final=None,
            gate: str = "scalar", cu_seqlens=None):
    """Batch adjoint.  Shapes as in :func:`gdn_fwd`; do [B,T,H,dv];
    ds_final [B|N,H,dk,dv] or None.  Returns dq, dk, dv, dbeta, dlog_alpha
    (None for gate none) and ds0 (gradient w.r.t. the initial state, also
    when s0 is None, i.e. zeros)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    nseq = B if cu_seqlens is None else len(cu_seqlens) - 1
    dq = np.zeros_like(q, dtype=np.float64)
    dk_ = np.zeros_like(k, dtype=np.float64)
    dv_ = np.zeros_like(v, dtype=np.float64)
    db = np.zeros_like(beta, dtype=np.float64)
    dla = None if gate == "none" else np.zeros_like(log_alpha, dtype=np.float64)
    ds0 = np.zeros((nseq, H, dk, dv))
    for b, t0, t1, n in _segments(B, T, cu_seqlens):
        for h in range(H):
            m0 = np.zeros((dk, dv)) if s0 is None else s0[n, h]
            la = None if gate == "none" else log_alpha[b, t0:t1, h]
            dmT = None if ds_final is None else ds_final[n, h]
            r = gdn_bwd_chain(q[b, t0:t1, h], k[b, t0:t1, h], v[b, t0:t1, h],
                              beta[b, t0:t1, h], la, m0, do[b, t0:t1, h],
                              dmT, gate)
            dq[b, t0:t1, h], dk_[b, t0:t1, h], dv_[b, t0:t1, h] = r[0], r[1], r[2]
            db[b, t0:t1, h] = r[3]
            if dla is not None:
                dla[b, t0:t1, h] = r[4]
            ds0[n, h] = r[5]
    return dq, dk_, dv_, db, dla, ds0
