"""Pins of the comparison functions that decide every parity verdict (CPU).

``oracle/compare.py`` turns a device output and the fp64 oracle into the
numbers the GPU tests assert on: the relative error against the unrounded
oracle (the letter's FP64 gold, "SwiftQK ...", Section IV-C), its max-abs /
mean-abs / RMSE context, the decoding of device bit patterns, and the
operand-scaled error of the LayerNorm extension (reading notes, Section 5e).
Each is pinned here by hand-computed values, and a set of planted mistakes,
each a plausible slip in one of these functions, must fail at least one pin
(``test_every_mutant_fails_a_pin``). Finally the GPU tests' own assertion
helper is driven on the CPU with a finite "device" value against NaN and
infinite oracle values, which it must reject.
"""
import math
import os
import types

import numpy as np
import pytest

from oracle import compare

INF, NAN = math.inf, math.nan


def _module_copy(name="compare_copy"):
    """A fresh copy of oracle/compare.py whose functions a mutant may replace
    (``report`` and ``layernorm_scaled_error`` look their helpers up in it)."""
    path = compare.__file__
    mod = types.ModuleType(name)
    mod.__file__ = path
    exec(compile(open(path).read(), path, "exec"), mod.__dict__)
    return mod


# ---------------------------------------------------------------- pins

def pin_rel_err_finite(c):
    e = c.rel_err(np.array([1.0, 2.0, -3.0, 2.0, -1.0]), np.array([1.0, 2.5, -2.0, 1.0, 1.0]))
    # |1-1|/1, |2-2.5|/2.5, |-3+2|/2, |2-1|/1 (relative to the oracle, not the result), |-1-1|/1
    np.testing.assert_array_equal(e, [0.0, 0.2, 0.5, 1.0, 2.0])


def pin_rel_err_zero_oracle(c):
    e = c.rel_err(np.array([0.0, -0.0, 1e-300, -5e-324]), np.array([0.0, 0.0, 0.0, -0.0]))
    np.testing.assert_array_equal(e, [0.0, 0.0, INF, INF])


def pin_rel_err_nan(c):
    got = np.array([NAN, 1.0, NAN, NAN, INF])
    ref = np.array([NAN, NAN, 1.0, 0.0, NAN])
    np.testing.assert_array_equal(c.rel_err(got, ref), [0.0, INF, INF, INF, INF])


def pin_rel_err_inf(c):
    got = np.array([INF, -INF, 1.0, INF, -INF, NAN])
    ref = np.array([INF, INF, -INF, 5.0, -INF, -INF])
    np.testing.assert_array_equal(c.rel_err(got, ref), [0.0, INF, INF, INF, 0.0, INF])


def pin_rel_err_never_nan(c):
    vals = np.array([0.0, -0.0, 1.0, -2.5, 1e-300, 3e300, INF, -INF, NAN])
    g, r = np.meshgrid(vals, vals)
    e = c.rel_err(g.ravel(), r.ravel())
    assert not np.isnan(e).any()
    # zero exactly where the two agree as values (NaN with NaN, zeros of either sign)
    agree = (g.ravel() == r.ravel()) | (np.isnan(g.ravel()) & np.isnan(r.ravel()))
    np.testing.assert_array_equal(e == 0.0, agree)


def pin_report_values(c):
    r = c.report(np.array([1.0, 2.0, 4.0]), np.array([1.0, 2.5, 2.0]))
    assert r["max_rel"] == 1.0
    assert r["max_abs"] == 2.0
    assert r["mean_abs"] == pytest.approx(2.5 / 3, rel=1e-15)
    assert r["rmse"] == pytest.approx(math.sqrt(4.25 / 3), rel=1e-15)
    assert r["n"] == 3


def pin_report_nonfinite(c):
    r = c.report(np.array([1.0, 2.0]), np.array([NAN, 2.0]))
    assert r["max_rel"] == INF and r["max_abs"] == INF
    r = c.report(np.array([NAN, 2.0, -INF]), np.array([NAN, 2.0, -INF]))
    assert r["max_rel"] == 0.0 and r["max_abs"] == 0.0 and r["rmse"] == 0.0
    r = c.report(np.array([], np.float64), np.array([], np.float64))
    assert r["max_rel"] == 0.0 and r["n"] == 0


def pin_fold_max(c):
    assert c.fold_max(0.0, 1.5) == 1.5 and c.fold_max(2.0, 1.5) == 2.0
    assert c.fold_max(0.0, NAN) == INF and c.fold_max(NAN, 0.0) == INF
    assert c.fold_max(1.0, INF) == INF


def pin_decode_bf16(c):
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F7F, 0x7F80, 0xFF80, 0x8000, 0x7FC0],
                    np.uint16)
    v = c.decode_out(bits)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127, INF, -INF, -0.0]
    np.testing.assert_array_equal(v[:8], want)
    assert np.signbit(v[7]) and np.isnan(v[8])


def pin_decode_f32_and_e4m3(c):
    f = np.array([0.1, -3.0, 2.0 ** -149], np.float32)
    np.testing.assert_array_equal(c.decode_out(f), [float(np.float32(0.1)), -3.0, 2.0 ** -149])
    codes = np.array([0x38, 0xB8, 0x7E, 0x01, 0x08, 0x7F], np.uint8)
    v = c.decode_out(codes)
    np.testing.assert_array_equal(v[:5], [1.0, -1.0, 448.0, 2.0 ** -9, 2.0 ** -6])
    assert np.isnan(v[5])


def _ln_case():
    """One row x = [1, 3]: mean 2, variance 1. eps = 0.5 (exact in fp32), so
    rstd = 1/sqrt(1.5) and the standard deviation recovered from rstd and eps is
    sqrt(1.5 - 0.5) = 1. gamma = [2, -1], beta = [0.5, 0]:
    y = (x - 2) rstd gamma + beta = [-2 rstd + 0.5, -rstd];
    scale = rstd |gamma| (|x| + 2 + 1) + |beta| = [8 rstd + 0.5, 6 rstd]."""
    rstd = 1.0 / math.sqrt(1.5)
    x = np.array([[1.0, 3.0]])
    y = np.array([[-2 * rstd + 0.5, -rstd]])
    scale = np.array([8 * rstd + 0.5, 6 * rstd])
    return x, y, np.array([2.0]), np.array([rstd]), np.array([2.0, -1.0]), np.array([0.5, 0.0]), scale


def pin_layernorm_scaled_values(c):
    x, y, mu, rs, g, b, scale = _ln_case()
    got = y + np.array([[0.07, -0.03]])
    err = c.layernorm_scaled_error(got, y, x, mu, rs, g, b, 0.5)
    np.testing.assert_allclose(err[0], [0.07 / scale[0], 0.03 / scale[1]], rtol=1e-12)
    # without beta the first scale loses its |beta| term
    err = c.layernorm_scaled_error(got, y, x, mu, rs, g, None, 0.5)
    np.testing.assert_allclose(err[0, 0], 0.07 / (8 * rs[0]), rtol=1e-12)


def pin_layernorm_scaled_special(c):
    x, y, mu, rs, g, b, _ = _ln_case()
    got = np.array([[NAN, y[0, 1]]])
    err = c.layernorm_scaled_error(got, y, x, mu, rs, g, b, 0.5)
    assert err[0, 0] == INF and err[0, 1] == 0.0
    # oracle NaN against a finite result is an infinite error; both NaN is exact
    yn = np.array([[NAN, NAN]])
    err = c.layernorm_scaled_error(np.array([[0.0, NAN]]), yn, x, mu, rs, g, b, 0.5)
    assert err[0, 0] == INF and err[0, 1] == 0.0
    # a zero operand scale (gamma = beta = 0: y = 0) accepts only the exact value
    z = np.zeros(2)
    err = c.layernorm_scaled_error(np.array([[0.0, 1e-3]]), np.zeros((1, 2)), x, mu, rs, z, z, 0.5)
    assert err[0, 0] == 0.0 and err[0, 1] == INF


PINS = [pin_rel_err_finite, pin_rel_err_zero_oracle, pin_rel_err_nan, pin_rel_err_inf,
        pin_rel_err_never_nan, pin_report_values, pin_report_nonfinite, pin_fold_max,
        pin_decode_bf16, pin_decode_f32_and_e4m3, pin_layernorm_scaled_values,
        pin_layernorm_scaled_special]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_compare_pin(pin):
    pin(compare)


# ---------------------------------------------------------------- mutants

def _mutant(kind):
    c = _module_copy()
    orig_rel, orig_ln = c.rel_err, c.layernorm_scaled_error
    if kind == "zero_oracle_accepts_anything":
        def rel_err(got, ref):
            e = orig_rel(got, ref)
            e[np.asarray(ref) == 0] = 0.0
            return e
        c.rel_err = rel_err
    elif kind == "relative_to_device_value":
        def rel_err(got, ref):
            got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
            with np.errstate(divide="ignore", invalid="ignore"):
                e = np.abs(got - ref) / np.abs(got)
            e[(ref == 0) & (got == 0)] = 0.0
            return e
        c.rel_err = rel_err
    elif kind == "absolute_error":
        c.rel_err = lambda got, ref: c.abs_diff(got, ref)
    elif kind == "nan_left_as_nan":
        # the plain quotient: a NaN or infinite oracle value gives NaN, not inf
        def rel_err(got, ref):
            got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
            with np.errstate(divide="ignore", invalid="ignore"):
                e = np.abs(got - ref) / np.abs(ref)
            z = ref == 0
            e[z] = np.where(got[z] == 0, 0.0, INF)
            e[np.isnan(got) & np.isnan(ref)] = 0.0
            return e
        c.rel_err = rel_err
    elif kind == "nan_result_accepted":
        def rel_err(got, ref):
            e = orig_rel(got, ref)
            e[np.isnan(np.asarray(got, np.float64))] = 0.0
            return e
        c.rel_err = rel_err
    elif kind == "opposite_infinities_agree":
        def rel_err(got, ref):
            e = orig_rel(got, ref)
            e[np.isinf(got) & np.isinf(ref)] = 0.0
            return e
        c.rel_err = rel_err
    elif kind == "fold_drops_nan":
        c.fold_max = lambda a, b: max(a, b)
    elif kind == "report_mean_not_max":
        orig_report = c.report

        def report(got, ref):
            r = orig_report(got, ref)
            r["max_rel"] = float(np.mean(c.rel_err(got, ref))) if np.size(got) else 0.0
            return r
        c.report = report
    elif kind == "bf16_low_half":
        orig_dec = c.decode_out

        def decode_out(a):
            if a.dtype == np.uint16:
                return a.astype(np.uint32).view(np.float32).astype(np.float64)
            return orig_dec(a)
        c.decode_out = decode_out
    elif kind == "bf16_as_fp16":
        orig_dec = c.decode_out

        def decode_out(a):
            if a.dtype == np.uint16:
                return a.view(np.float16).astype(np.float64)
            return orig_dec(a)
        c.decode_out = decode_out
    elif kind == "ln_scale_x10":
        c.layernorm_scaled_error = lambda *a: orig_ln(*a) / 10.0
    elif kind == "ln_sigma_without_eps":
        def ln(got, y, x, mean, rstd, gamma, beta, eps):
            # sigma taken as 1/rstd, i.e. sqrt(var + eps) instead of sqrt(var)
            g = np.abs(np.asarray(gamma, np.float64))[None, :]
            b = np.zeros_like(g) if beta is None else np.abs(np.asarray(beta, np.float64))[None, :]
            sigma = 1.0 / np.asarray(rstd, np.float64)
            scale = rstd[:, None] * g * (np.abs(x) + np.abs(mean)[:, None] + sigma[:, None]) + b
            d = c.abs_diff(got, y)
            with np.errstate(divide="ignore", invalid="ignore"):
                err = np.where(scale > 0, d / scale, INF)
            err[d == 0] = 0.0
            return err
        c.layernorm_scaled_error = ln
    elif kind == "ln_no_beta_term":
        c.layernorm_scaled_error = lambda got, y, x, m, r, g, b, e: orig_ln(got, y, x, m, r, g, None, e)
    elif kind == "ln_nan_mismatch_dropped":
        def ln(*a):
            err = orig_ln(*a)
            err[np.isinf(err)] = 0.0
            return err
        c.layernorm_scaled_error = ln
    else:
        raise KeyError(kind)
    return c


MUTANTS = ["zero_oracle_accepts_anything", "relative_to_device_value", "absolute_error",
           "nan_left_as_nan", "nan_result_accepted", "opposite_infinities_agree",
           "fold_drops_nan", "report_mean_not_max", "bf16_low_half", "bf16_as_fp16",
           "ln_scale_x10", "ln_sigma_without_eps", "ln_no_beta_term",
           "ln_nan_mismatch_dropped"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_every_mutant_fails_a_pin(kind):
    c = _mutant(kind)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(c)
        except (AssertionError, ValueError, TypeError):
            failed.append(pin.__name__)
    assert failed, f"mutant {kind} passed every pin"


# ---------------------------------------------------------------- the GPU tests' assertion

def test_assert_parity_rejects_finite_against_nonfinite_oracle():
    """tests/_gpu.py folds chunk maxima and asserts on them; run it on host arrays.
    A zero row with eps = 0 has the oracle value 0 * inf = NaN, and a row holding
    an infinity has NaN (inf * 0) or infinite outputs: a finite result there must
    fail, in every chunk position, and the oracle's own values must pass."""
    import _gpu
    from oracle import oracle
    H = 8
    x = np.random.default_rng(0).standard_normal((6, H)).astype(np.float32)
    x[2] = 0.0
    x[4, 3] = np.inf
    g = np.linspace(0.5, 1.5, H).astype(np.float32)
    y, _, _ = oracle.rmsnorm(x, g, 0.0)
    assert np.isnan(y[2]).all() and not np.isfinite(y[4]).all()
    good = y.astype(np.float32)
    _gpu.assert_parity(x, g, good, 0.0, "oracle values")
    for row in (2, 4):
        for chunk in (1, 4, 4096):
            bad = good.copy()
            bad[row] = 0.0
            with pytest.raises(AssertionError):
                r = _gpu.oracle_report(x, g, bad, 0.0, chunk=chunk)
                assert r["max_rel"] <= compare.TOL["f32"], r
            with pytest.raises(AssertionError):
                _gpu.assert_parity(x, g, bad, 0.0, "finite against non-finite")
