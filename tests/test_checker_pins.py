"""Pins of the two error measures every parity verdict goes through.

``oracle.normwise_rel_err`` (states, any [..., a, b] array) and
``gpu_util.slice_err`` (token outputs [B, T, H, D], dense or varlen) both
compute, per (sequence, head) slice, max|x - y| / max|y| over the slice and
report the worst slice; a slice whose reference is below 1e-30 is judged by
its absolute error relative to the whole tensor's max |y|.  These tests
plant errors of known size at known places so that a checker that
normalises by the wrong maximum, pairs the wrong slices, swallows a real
error in its small-reference branch, or lets a NaN through fails here."""

import numpy as np
import pytest

import oracle
from gpu_util import slice_err

TOL = 2e-2


def _tokens(seed=0, B=2, T=40, H=3, D=8):
    rng = np.random.default_rng(seed)
    y = rng.standard_normal((B, T, H, D))
    # slices of very different size: a per-slice normalisation matters
    y[1, :, 2] *= 1e-3
    y[0, :, 1] *= 50.0
    return y


def _states(seed=1, N=3, H=4, dk=6, dv=5):
    rng = np.random.default_rng(seed)
    y = rng.standard_normal((N, H, dk, dv))
    y[2, 3] *= 1e-4
    y[0, 0] *= 30.0
    return y


def _plant_token(y, b, t, h, d, frac):
    """x equal to y except one element, moved by frac * (its slice's max)."""
    x = y.copy()
    ref = np.max(np.abs(y[b, :, h]))
    x[b, t, h, d] += frac * ref
    return x


@pytest.mark.parametrize("where", [(1, 7, 2, 3), (0, 39, 1, 0), (1, 0, 0, 7)])
def test_slice_err_threshold_in_single_slice(where):
    y = _tokens()
    b, t, h, d = where
    assert slice_err(_plant_token(y, b, t, h, d, 1.01 * TOL), y) > TOL
    assert slice_err(_plant_token(y, b, t, h, d, 0.99 * TOL), y) < TOL
    # the value is the planted relative error itself
    e = slice_err(_plant_token(y, b, t, h, d, 0.5 * TOL), y)
    assert abs(e - 0.5 * TOL) < 1e-12


def test_slice_err_is_per_slice_not_global():
    # an error of 1.01 tol relative to the small slice is ~1e-5 of the global
    # max: a checker normalising by the global max would pass it
    y = _tokens()
    x = _plant_token(y, 1, 5, 2, 1, 1.01 * TOL)
    assert np.max(np.abs(x - y)) / np.max(np.abs(y)) < 1e-4
    assert slice_err(x, y) > TOL


def test_slice_err_varlen_slices():
    rng = np.random.default_rng(2)
    cu = np.array([0, 5, 5, 30, 31, 40])
    y = rng.standard_normal((1, 40, 2, 4))
    y[0, 5:30, 1] *= 1e-3            # sequence 2, head 1 is small
    x = y.copy()
    ref = np.max(np.abs(y[0, 5:30, 1]))
    x[0, 29, 1, 2] += 1.01 * TOL * ref
    assert slice_err(x, y, cu) > TOL
    x = y.copy()
    x[0, 29, 1, 2] += 0.99 * TOL * ref
    assert slice_err(x, y, cu) < TOL
    # an error on a token of a one-token sequence is judged against that token
    x = y.copy()
    x[0, 30, 0, 0] += 1.01 * TOL * np.max(np.abs(y[0, 30, 0]))
    assert slice_err(x, y, cu) > TOL


def test_slice_err_nan_and_inf():
    y = _tokens()
    x = y.copy()
    x[1, 3, 2, 4] = np.nan
    assert slice_err(x, y) == float("inf")
    x = y.copy()
    x[0, 0, 0, 0] = np.inf
    assert slice_err(x, y) == float("inf")


def test_slice_err_empty():
    y = np.zeros((2, 0, 3, 8))
    assert slice_err(y, y) == 0.0
    # empty sequences inside a varlen batch are skipped, others still count
    cu = np.array([0, 0, 4, 4])
    rng = np.random.default_rng(3)
    y = rng.standard_normal((1, 4, 1, 2))
    x = y.copy()
    x[0, 2, 0, 1] += 1.01 * TOL * np.max(np.abs(y[0, 0:4, 0]))
    assert slice_err(x, y, cu) > TOL


def test_slice_err_decayed_slice_uses_global_max():
    # a fully decayed reference slice (all below 1e-30): its error is judged
    # against the tensor's global max, so a real error there is still caught
    y = _tokens()
    y[0, :, 2] = 0.0
    gmax = np.max(np.abs(y))
    x = y.copy()
    x[0, 9, 2, 1] = 1.01 * TOL * gmax
    assert slice_err(x, y) > TOL
    x[0, 9, 2, 1] = 0.99 * TOL * gmax
    assert slice_err(x, y) < TOL
    x[0, 9, 2, 1] = 1e-12 * gmax           # rounding noise on a zero slice
    assert slice_err(x, y) < 1e-10


def test_normwise_threshold_in_single_slice():
    y = _states()
    for (n, h, i, j) in [(2, 3, 5, 4), (0, 0, 0, 0), (1, 2, 3, 1)]:
        ref = np.max(np.abs(y[n, h]))
        x = y.copy()
        x[n, h, i, j] += 1.01 * TOL * ref
        assert oracle.normwise_rel_err(x, y) > TOL
        x = y.copy()
        x[n, h, i, j] -= 0.99 * TOL * ref
        assert oracle.normwise_rel_err(x, y) < TOL


def test_normwise_is_per_slice_not_global():
    y = _states()
    x = y.copy()
    x[2, 3, 1, 1] += 1.01 * TOL * np.max(np.abs(y[2, 3]))
    assert np.max(np.abs(x - y)) / np.max(np.abs(y)) < 1e-4
    assert oracle.normwise_rel_err(x, y) > TOL


def test_normwise_slices_are_the_last_two_axes():
    # a [T, H, D]-shaped tensor would be sliced per T row by a wrong reshape;
    # states [N, H, dk, dv] must be sliced per (n, h) matrix
    y = _states()
    x = y.copy()
    # error relative to one row of the slice, but well under the slice max
    x[1, 1, 2, :] += 0.5 * TOL * np.max(np.abs(y[1, 1]))
    e = oracle.normwise_rel_err(x, y)
    assert abs(e - 0.5 * TOL) < 1e-12


def test_normwise_nan_empty_and_decayed():
    y = _states()
    x = y.copy()
    x[1, 0, 0, 0] = np.nan
    assert oracle.normwise_rel_err(x, y) == float("inf")
    z = np.zeros((0, 2, 4, 4))
    assert oracle.normwise_rel_err(z, z) == 0.0
    y[1, 2] = 0.0
    gmax = np.max(np.abs(y))
    x = y.copy()
    x[1, 2, 3, 3] = 1.01 * TOL * gmax
    assert oracle.normwise_rel_err(x, y) > TOL
    x[1, 2, 3, 3] = 0.99 * TOL * gmax
    assert oracle.normwise_rel_err(x, y) < TOL


def test_normwise_all_zero_reference():
    # nothing to normalise by: the absolute error is the measure
    y = np.zeros((2, 2, 3, 3))
    x = y.copy()
    x[0, 1, 2, 2] = 3e-5
    assert abs(oracle.normwise_rel_err(x, y) - 3e-5) < 1e-15


def test_checkers_are_symmetric_in_sign():
    y = _tokens()
    up = _plant_token(y, 0, 3, 0, 2, 1.01 * TOL)
    down = _plant_token(y, 0, 3, 0, 2, -1.01 * TOL)
    assert slice_err(up, y) > TOL and slice_err(down, y) > TOL


# ------------------------------------------------------------ teeth ---
# Planted mistakes in copies of slice_err: each must fail one of the pins
# above (run here against the copy instead of the real checker).

def _slices_mut(x, cu, shift=0):
    B, T, H = x.shape[:3]
    out = []
    if cu is None:
        for b in range(B):
            for h in range(H):
                out.append(x[b, :, h])
    else:
        for n in range(len(cu) - 1):
            for h in range(H):
                out.append(x[0, cu[n]:cu[n + 1], h])
    return out[shift:] + out[:shift]


def _mutant(kind):
    def err(x, y, cu=None):
        x = np.asarray(x, dtype=np.float64)
        y = np.asarray(y, dtype=np.float64)
        if x.size == 0:
            return 0.0
        if kind != "nan_ignored" and not np.all(np.isfinite(x)):
            return float("inf")
        gmax = float(np.max(np.abs(y)))
        worst = 0.0
        xs_all = _slices_mut(x, cu, 1 if kind == "mis_zipped" else 0)
        for xs, ys in zip(xs_all, _slices_mut(y, cu)):
            if xs.size == 0 or ys.size != xs.size:
                continue
            ref = float(np.max(np.abs(ys)))
            diff = float(np.nanmax(np.abs(xs - ys)))
            if kind == "global_max":
                ref = gmax
            if ref < 1e-30:
                if kind == "small_branch_zero":
                    continue
                worst = max(worst, diff / max(gmax, 1e-30))
            else:
                worst = max(worst, diff / ref)
        return worst
    return err


@pytest.mark.parametrize("kind", ["global_max", "mis_zipped", "small_branch_zero",
                                  "nan_ignored"])
def test_slice_err_mutant_is_caught(kind, monkeypatch):
    import sys
    mod = sys.modules[__name__]
    monkeypatch.setattr(mod, "slice_err", _mutant(kind))
    pins = [test_slice_err_is_per_slice_not_global, test_slice_err_varlen_slices,
            test_slice_err_nan_and_inf, test_slice_err_decayed_slice_uses_global_max,
            lambda: test_slice_err_threshold_in_single_slice((1, 7, 2, 3))]
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, kind
