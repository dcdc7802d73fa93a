"""Error metrics of a device result against the fp64 oracle.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark's CPU leg).

The pass criterion is the elementwise relative error against the unrounded
fp64 oracle, with the convention that an exact zero in the oracle must be a
(signed) zero in the result. The letter reports max-abs, mean-abs and RMSE
against an FP64 RMSNorm of the gathered vector ("SwiftQK ...", Section IV-C);
``report`` returns those three as well, as context.
"""
from __future__ import annotations

import numpy as np

# Tolerances on the final outputs, by output dtype (relative error against the
# unrounded oracle). E4M3 outputs are checked by code instead: see e4m3_accepts.
TOL = {"bf16": 8e-3, "f32": 1e-5}
# Relative perturbation of the exact value within which either E4M3 neighbour is
# accepted: fp32 arithmetic may move a value lying that close to a rounding
# boundary across it.
E4M3_REL = 1e-5
E4M3_MAX = 448.0
# Tolerance on intermediate fp32 statistics (partials, reciprocal RMS).
TOL_STAT = 1e-5


def decode_out(a: np.ndarray) -> np.ndarray:
    """float64 values of a device output: bf16 bit patterns, float32 or E4M3 codes."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype == np.uint8:
        from oracle.oracle import decode_e4m3_np
        return decode_e4m3_np(a)
    return np.asarray(a, dtype=np.float64)


def layernorm_scaled_error(got, y, x, mean, rstd, gamma, beta, eps):
    """Elementwise |got - y| / s for LayerNorm outputs, with the operand scale
    s_j = rstd * |gamma_j| * (|x_j| + |mean| + sigma) + |beta_j| (sigma the row's
    standard deviation from the oracle's rstd and eps).

    An output near zero comes from x_j close to the mean, where the relative
    error of the result says nothing about the arithmetic; fp32 rounding of
    x - mean, of the statistics and of the final fma is bounded by a few ulp of
    this scale, and one bf16 rounding of the output by 2^-9 of it (|y_j| <= s_j).
    """
    got = np.asarray(got, np.float64)
    y = np.asarray(y, np.float64)
    xv = np.asarray(x, np.float64)
    g = np.abs(np.asarray(gamma, np.float64))[None, :]
    b = np.zeros_like(g) if beta is None else np.abs(np.asarray(beta, np.float64))[None, :]
    e = float(np.float32(eps))
    rstd = np.asarray(rstd, np.float64)
    mean = np.asarray(mean, np.float64)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        sigma = np.sqrt(np.maximum(1.0 / (rstd * rstd) - e, 0.0))
        scale = rstd[:, None] * g * (np.abs(xv) + np.abs(mean)[:, None] + sigma[:, None]) + b
    d = abs_diff(got, y)
    # identical values (non-finite ones included) are exact whatever the scale;
    # any other difference over a zero or non-finite scale is an infinite error
    ok = np.isfinite(scale) & (scale > 0)
    with np.errstate(divide="ignore", invalid="ignore"):
        err = np.where(ok, d / np.where(ok, scale, 1.0), np.inf)
    err[d == 0] = 0.0
    return err


def e4m3_rne(y: np.ndarray) -> np.ndarray:
    """E4M3 code (OCP OFP8 layout) nearest to each float64 value, ties to the even
    code; magnitudes of 448 and above (infinities included) saturate to the
    largest finite code, and NaN maps to the NaN code of its sign."""
    y = np.asarray(y, np.float64)
    neg = np.signbit(y).astype(np.int64)
    a = np.abs(y)
    with np.errstate(invalid="ignore", over="ignore"):
        # subnormal range [0, 2^-6): spacing 2^-9, code = rounded multiple (8 = 2^-6)
        m_sub = np.rint(np.ldexp(np.where(np.isfinite(a), a, 0.0), 9)).astype(np.int64)
        # normal range: a = 1.f * 2^e, 3 fraction bits kept
        _, E = np.frexp(np.where((a > 0) & np.isfinite(a), a, 1.0))
        e = E.astype(np.int64) - 1
        q = np.rint(np.ldexp(np.where(np.isfinite(a), a, 0.0), -(e - 3))).astype(np.int64)
    carry = q >= 16
    e = e + carry
    q = np.where(carry, 8, q)
    code = np.where(a < 2.0 ** -6, m_sub, ((e + 7) << 3) | (q - 8))
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = np.where(np.isnan(a), 0x7F, code)
    return (code | (neg << 7)).astype(np.uint8)


def e4m3_accepts(codes: np.ndarray, y: np.ndarray, rel: float = E4M3_REL) -> np.ndarray:
    """True where a device E4M3 code is the rounding of the exact value y, or, when
    y lies within ``rel`` of a rounding boundary, the code on the other side."""
    from oracle.oracle import decode_e4m3_np
    y = np.asarray(y, np.float64)
    got = decode_e4m3_np(np.asarray(codes, np.uint8))
    ok = np.zeros(y.shape, bool)
    for f in (1.0 - rel, 1.0, 1.0 + rel):
        want = decode_e4m3_np(e4m3_rne(y * f))
        ok |= (got == want) | (np.isnan(got) & np.isnan(want))
    return ok


def abs_diff(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """|got - ref| elementwise, where two identical non-finite values (both NaN, or
    the same infinity) differ by 0 and any other pair with a non-finite member
    differs by infinity."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    got, ref = np.broadcast_arrays(got, ref)
    with np.errstate(invalid="ignore", over="ignore"):
        d = np.abs(got - ref)
    d = np.where(np.isfinite(got) & np.isfinite(ref), d, np.inf)
    d[np.isnan(got) & np.isnan(ref)] = 0.0
    d[np.isinf(ref) & (got == ref)] = 0.0
    return d


def rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Elementwise |got - ref| / |ref| against the exact value ref.

    An exact zero in ref accepts only a (signed) zero. A non-finite ref accepts
    only the same value: NaN for NaN, the same infinity for an infinity. Every
    other disagreement (a NaN or an infinity against a finite ref, a finite value
    against a non-finite ref) is an infinite error, so no mismatch is ever NaN."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    got, ref = np.broadcast_arrays(got, ref)
    d = abs_diff(got, ref)
    e = np.full(ref.shape, np.inf)
    fin = np.isfinite(ref) & (ref != 0)
    with np.errstate(over="ignore"):
        e[fin] = d[fin] / np.abs(ref[fin])
    e[(ref == 0) & (got == 0)] = 0.0
    e[~np.isfinite(ref) & (d == 0)] = 0.0
    return e


def fold_max(a: float, b: float) -> float:
    """max(a, b) for folding error maxima over chunks: NaN in either counts as an
    infinite error (Python's max(0.0, nan) is 0.0, which would drop it)."""
    if a != a or b != b:
        return float("inf")
    return a if a >= b else b


def report(got: np.ndarray, ref: np.ndarray) -> dict:
    """Largest relative error (``rel_err``) and, as context, the max-abs,
    mean-abs and RMSE of the differences (``abs_diff``) the letter reports."""
    e = rel_err(got, ref)
    d = abs_diff(got, ref)
    return {
        "max_rel": float(e.max()) if e.size else 0.0,
        "max_abs": float(d.max()) if d.size else 0.0,
        "mean_abs": float(d.mean()) if d.size else 0.0,
        "rmse": float(np.sqrt(np.mean(d * d))) if d.size else 0.0,
        "n": int(e.size),
    }
