"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that the pins catch every one of them.  The copy is made by editing the
oracle's source text in memory; the oracle module itself is untouched."""

import inspect
import os
import types

import numpy as np
import pytest

import oracle.gdn_oracle as ref_mod
import pins
from test_oracle_pins import _read_golden

SRC = inspect.getsource(ref_mod)


def _mutant(old, new):
    assert SRC.count(old) >= 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "<oracle_mutant>", "exec"), mod.__dict__)
    return mod


def _golden_err(mod):
    g = _read_golden("hand_worked_t2.txt")
    T = len(g["beta"])
    o, M = mod.gdn_fwd_chain(g["q"].reshape(T, 2), g["k"].reshape(T, 2),
                             g["v"].reshape(T, 2), g["beta"], g["log_alpha"],
                             np.zeros((2, 2)), "scalar")
    return max(np.max(np.abs(o.reshape(-1) - g["o"])),
               np.max(np.abs(M.reshape(-1) - g["M_final"])))


def _forward_pins_pass(mod):
    c = mod.gdn_fwd_chain
    ok = _golden_err(mod) < 1e-12
    for gate in ("scalar", "channel"):
        ok &= pins.p2_orthonormal_retrieval(c, gate=gate) < 1e-12
        ok &= pins.p3_gate_product(c, gate=gate) < 1e-12
        ok &= pins.p6_erasure(c, gate=gate) < 1e-12
        ok &= pins.p7_gla_limit(c, gate=gate) < 1e-12
        ok &= pins.p9_single_token(c, gate=gate) < 1e-12
        ok &= pins.p5_norm_bound(c, gate=gate) <= 1 + 1e-12
    return bool(ok)


FWD_MUTANTS = {
    "write decayed with the state": (
        "        M = Mt + np.outer(k[t], e)               # rank-1 delta correction\n",
        "        M = a[:, None] * (M + np.outer(k[t], e))\n"),
    "output read before the update": (
        "        M = Mt + np.outer(k[t], e)               # rank-1 delta correction\n"
        "        o[t] = M.T @ q[t]                        # read the updated state\n",
        "        o[t] = Mt.T @ q[t]\n"
        "        M = Mt + np.outer(k[t], e)\n"),
    "transposed read": (
        "        o[t] = M.T @ q[t]                        # read the updated state\n",
        "        o[t] = (M @ q[t]) if M.shape[0] == M.shape[1] else M.T @ q[t]\n"),
    "error of the undecayed state": (
        "        e = beta[t] * (v[t] - Mt.T @ k[t])       # error of the decayed state\n",
        "        e = beta[t] * (v[t] - M.T @ k[t])\n"),
    "beta dropped from the error": (
        "        e = beta[t] * (v[t] - Mt.T @ k[t])       # error of the decayed state\n",
        "        e = (v[t] - Mt.T @ k[t])\n"),
    "wrong sign of the correction": (
        "        M = Mt + np.outer(k[t], e)               # rank-1 delta correction\n",
        "        M = Mt - np.outer(k[t], e)\n"),
    "gate exponent sign": (
        "        return np.full(dk, np.exp(float(log_alpha_t)))\n",
        "        return np.full(dk, np.exp(-float(log_alpha_t)))\n"),
}


def test_reference_oracle_passes_forward_pins():
    assert _forward_pins_pass(ref_mod)


@pytest.mark.parametrize("name", sorted(FWD_MUTANTS))
def test_forward_mutant_is_caught(name):
    mod = _mutant(*FWD_MUTANTS[name])
    assert not _forward_pins_pass(mod), name


def _adjoint_err(mod, gate):
    r = pins.rng(31)
    T, dk, dv = 6, 4, 3
    q = pins.unit(r.standard_normal((1, T, 1, dk)))
    k = pins.unit(r.standard_normal((1, T, 1, dk)))
    v = r.standard_normal((1, T, 1, dv))
    beta = 1.5 * r.random((1, T, 1))
    la = -0.7 * r.random((1, T, 1)) if gate == "scalar" else -0.7 * r.random((1, T, 1, dk))
    m0 = r.standard_normal((1, 1, dk, dv))
    do = r.standard_normal((1, T, 1, dv))
    dS = r.standard_normal((1, 1, dk, dv))
    g = mod.gdn_bwd(q, k, v, beta, la, m0, do, dS, gate)
    vals = [q, k, v, beta, la, m0]
    worst = 0.0
    h = 1e-6
    for j, x in enumerate(vals):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = [y.copy() for y in vals]; xp[j][idx] += h
            xm = [y.copy() for y in vals]; xm[j][idx] -= h
            lp = ref_mod.gdn_fwd(*xp, gate=gate)
            lm = ref_mod.gdn_fwd(*xm, gate=gate)
            fd[idx] = (np.sum(do * (lp[0] - lm[0])) + np.sum(dS * (lp[1] - lm[1]))) / (2 * h)
        worst = max(worst, np.max(np.abs(fd - g[j])) / np.max(np.abs(fd)))
    return worst


BWD_MUTANTS = {
    "dk misses the state-transpose term": (
        "            dkk[t] = -bt * (G @ (Mt.T @ kt) + Mt @ (G.T @ kt)) + bt * (G @ vt)\n",
        "            dkk[t] = -bt * (G @ (Mt.T @ kt)) + bt * (G @ vt)\n"),
    "dbeta uses the undecayed state": (
        "            db[t] = Gk @ (vt - Mt.T @ kt)\n",
        "            db[t] = Gk @ (vt - Mprev.T @ kt)\n"),
    "state adjoint skips the projection": (
        "            G = a[:, None] * PG\n",
        "            G = a[:, None] * G\n"),
    "dq reads the previous state": (
        "            dq[t] = Mcur @ do[t]\n",
        "            dq[t] = Mprev @ do[t]\n"),
    "dlog-alpha misses the gate factor": (
        "                dla[t] = a * np.sum(PG * Mprev, axis=1)\n",
        "                dla[t] = np.sum(PG * Mprev, axis=1)\n"),
}


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_reference_adjoint_passes(gate):
    assert _adjoint_err(ref_mod, gate) < 1e-7


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_adjoint_mutant_is_caught(name):
    mod = _mutant(*BWD_MUTANTS[name])
    gate = "channel" if "gate factor" in name else "scalar"
    assert _adjoint_err(mod, gate) > 1e-4, name


# ------------------------------------------- Householder-product transitions ---

def _dp_pins_pass(mod):
    f = mod.deltaproduct_fwd
    return bool(pins.dp_single_step_is_gdn(f, mod.gdn_fwd) < 1e-14
                and pins.dp_reflections(f) < 1e-12
                and pins.dp_two_step_closed_form(f) < 1e-13
                and pins.dp_gate_once_per_token(f, mod.gdn_fwd) < 1e-13)


DP_MUTANTS = {
    "decay at every step": (
        "                M = a * M                                   # one decay per token\n"
        "                for j in range(nh):\n",
        "                for j in range(nh):\n"
        "                    M = a * M\n"),
    "steps in reverse order": (
        "                    kj = k[b, t, j, h]\n"
        "                    e = beta[b, t, j, h] * (v[b, t, j, h] - M.T @ kj)\n",
        "                    kj = k[b, t, nh - 1 - j, h]\n"
        "                    e = beta[b, t, nh - 1 - j, h] * (v[b, t, nh - 1 - j, h] - M.T @ kj)\n"),
    "output after the first step": (
        "                    M = M + np.outer(kj, e)                 # delta step j\n"
        "                o[b, t, h] = M.T @ q[b, t, h]\n",
        "                    M = M + np.outer(kj, e)                 # delta step j\n"
        "                    if j == 0:\n"
        "                        o[b, t, h] = M.T @ q[b, t, h]\n"),
    "error of the state before the decay": (
        "                    e = beta[b, t, j, h] * (v[b, t, j, h] - M.T @ kj)\n",
        "                    e = beta[b, t, j, h] * (v[b, t, j, h] - (M / (a if j == 0 else 1.0)).T @ kj)\n"),
}


def test_reference_oracle_passes_dp_pins():
    assert _dp_pins_pass(ref_mod)


@pytest.mark.parametrize("name", sorted(DP_MUTANTS))
def test_dp_mutant_is_caught(name):
    mod = _mutant(*DP_MUTANTS[name])
    assert not _dp_pins_pass(mod), name


# ------------------------------------------------------------- draft trees ---

def _tree_pins_pass(mod):
    worst = 0.0
    for gate in ("scalar", "channel"):
        worst = max(worst,
                    pins.tree_chain_is_sequence(mod.tree_fwd, mod.gdn_fwd, gate),
                    pins.tree_star_is_single_steps(mod.tree_fwd, mod.gdn_decode, gate),
                    pins.tree_paths_are_sequences(mod.tree_fwd, mod.gdn_fwd, gate),
                    pins.tree_commit_is_node_state(mod.tree_commit, mod.tree_fwd, gate),
                    pins.tree_wy_matches_recurrence(mod.tree_wy_bruteforce, mod.tree_fwd,
                                                    gate))
    return worst < 1e-12


TREE_MUTANTS = {
    "node continues the previous node": (
        "                prev = m0 if par[i] < 0 else st[b, t0 + par[i], h]\n",
        "                prev = m0 if i == 0 else st[b, t - 1, h]\n"),
    "commit walks the path leaf first": (
        "    return path[::-1]\n",
        "    return path\n"),
    "WY mask over every earlier node": (
        "            if anc[r, i] or i == r:\n",
        "            if i <= r:\n"),
    "path gate summed over earlier nodes": (
        "        g[r] = own + (g[par[r]] if par[r] >= 0 else 0.0)\n",
        "        g[r] = own + (g[r - 1] if r > 0 else 0.0)\n"),
}


def test_reference_oracle_passes_tree_pins():
    assert _tree_pins_pass(ref_mod)


@pytest.mark.parametrize("name", sorted(TREE_MUTANTS))
def test_tree_mutant_is_caught(name):
    mod = _mutant(*TREE_MUTANTS[name])
    assert not _tree_pins_pass(mod), name


# ------------------------------------------------ Gated DeltaNet-2 ---

def _g2_pins_pass(mod):
    ok = True
    for gate in ("none", "scalar", "channel"):
        ok &= pins.g2_equal_strengths_is_gdn(mod.gdn2_fwd_chain, ref_mod.gdn_fwd_chain,
                                             gate) < 1e-13
        ok &= pins.g2_no_erase_is_linear_attention(mod.gdn2_fwd_chain, gate) < 1e-12
        ok &= pins.g2_no_write_is_erasure(mod.gdn2_fwd_chain, gate) < 1e-12
        ok &= pins.g2_full_erase_stores_write(mod.gdn2_fwd_chain, gate) < 1e-12
    return bool(ok)


G2_LINE = ("        e = write[t] * v[t] - erase[t] * (Mt.T @ k[t])"
           "   # write minus erased value\n")
G2_MUTANTS = {
    "erase and write swapped": (G2_LINE, "        e = erase[t] * v[t] - write[t] * (Mt.T @ k[t])\n"),
    "write strength used for both": (G2_LINE, "        e = write[t] * (v[t] - Mt.T @ k[t])\n"),
    "erase strength used for both": (G2_LINE, "        e = erase[t] * (v[t] - Mt.T @ k[t])\n"),
    "erase of the undecayed state": (G2_LINE,
                                     "        e = write[t] * v[t] - erase[t] * (M.T @ k[t])\n"),
    "write decayed with the state": (
        "        e = write[t] * v[t] - erase[t] * (Mt.T @ k[t])   # write minus erased value\n"
        "        M = Mt + np.outer(k[t], e)\n",
        "        e = write[t] * v[t] - erase[t] * (Mt.T @ k[t])\n"
        "        M = Mt + np.outer(k[t], e - write[t] * v[t] + write[t] * a[0] * v[t])\n"),
}


def test_reference_oracle_passes_g2_pins():
    assert _g2_pins_pass(ref_mod)


@pytest.mark.parametrize("name", sorted(G2_MUTANTS))
def test_g2_mutant_is_caught(name):
    assert not _g2_pins_pass(_mutant(*G2_MUTANTS[name]))


# ------------------------------------ short convolution + SiLU prologue ---

def _conv_pins_pass(mod):
    ok = pins.conv_equals_numpy_convolve(mod.short_conv) < 1e-13
    for W, t0 in ((1, 0), (3, 4), (4, 10)):
        ok &= pins.conv_impulse_response(mod.short_conv, W=W, t0=t0) < 1e-15
    ok &= pins.conv_isolates_sequences(mod.short_conv) < 1e-15
    ok &= pins.silu_identities(mod.silu) < 1e-12
    return bool(ok)


CONV_MUTANTS = {
    "taps applied forward in time": (
        "                    y[b, t] += taps[:, :, j] * x[b, t - j]\n",
        "                    y[b, t] += taps[:, :, W - 1 - j] * x[b, t - j]\n"),
    "history leaks across sequences": (
        "                if t - j >= t0:\n",
        "                if t - j >= 0:\n"),
    "current token skipped": (
        "                    y[b, t] += taps[:, :, j] * x[b, t - j]\n",
        "                    y[b, t] += taps[:, :, j] * x[b, t - j - 1] if t - j - 1 >= t0 else 0.0\n"),
    "sigmoid instead of SiLU": (
        "    return x / (1.0 + np.exp(-x))\n",
        "    return 1.0 / (1.0 + np.exp(-x))\n"),
}


def test_reference_oracle_passes_conv_pins():
    assert _conv_pins_pass(ref_mod)


@pytest.mark.parametrize("name", sorted(CONV_MUTANTS))
def test_conv_mutant_is_caught(name):
    assert not _conv_pins_pass(_mutant(*CONV_MUTANTS[name]))


# ------------------------------------- adjoint of the prologue path ---

def _prologue_bwd_pins_pass(mod):
    ok = True
    for normalize in (True, False):
        for varlen in (False, True):
            ok &= pins.prologue_bwd_fd(mod.conv_prologue_bwd, ref_mod.conv_prologue,
                                       normalize, varlen) < 1e-7
    ok &= pins.prologue_bwd_width_one(mod.conv_prologue_bwd) < 1e-14
    return bool(ok)


PROLOGUE_BWD_MUTANTS = {
    "norm projection sign flipped": (
        "        proj = dy - y * np.sum(y * dy, axis=-1, keepdims=True)\n",
        "        proj = dy + y * np.sum(y * dy, axis=-1, keepdims=True)\n"),
    "SiLU derivative without its second term": (
        "    dz = da * (sg + a * (1.0 - sg))\n",
        "    dz = da * sg\n"),
    "convolution adjoint reversed in time": (
        "                    dx[b, t - j] += taps[:, :, j] * dz[b, t]\n",
        "                    dx[b, t - j] += taps[:, :, W - 1 - j] * dz[b, t]\n"),
    "tap gradient against the current token": (
        "                    dtaps[:, :, j] += dz[b, t] * x[b, t - j]\n",
        "                    dtaps[:, :, j] += dz[b, t] * x[b, t]\n"),
}


def test_reference_oracle_passes_prologue_bwd_pins():
    assert _prologue_bwd_pins_pass(ref_mod)


@pytest.mark.parametrize("name", sorted(PROLOGUE_BWD_MUTANTS))
def test_prologue_bwd_mutant_is_caught(name):
    assert not _prologue_bwd_pins_pass(_mutant(*PROLOGUE_BWD_MUTANTS[name]))
