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
