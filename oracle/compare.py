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

# Tolerances on the final outputs, by output dtype.
TOL = {"bf16": 8e-3, "f32": 1e-5}
# Tolerance on intermediate fp32 statistics (partials, reciprocal RMS).
TOL_STAT = 1e-5


def decode_out(a: np.ndarray) -> np.ndarray:
    """float64 values of a device output: bf16 bit patterns or float32."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.abs(got - ref) / np.abs(ref)
    zero = ref == 0
    e[zero] = np.where(got[zero] == 0, 0.0, np.inf)
    e[np.isnan(got) & ~np.isnan(ref)] = np.inf
    both_nan = np.isnan(got) & np.isnan(ref)
    e[both_nan] = 0.0
    return e


def report(got: np.ndarray, ref: np.ndarray) -> dict:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    e = rel_err(got, ref)
    d = np.abs(got - ref)
    return {
        "max_rel": float(e.max()) if e.size else 0.0,
        "max_abs": float(d.max()) if d.size else 0.0,
        "mean_abs": float(d.mean()) if d.size else 0.0,
        "rmse": float(np.sqrt(np.mean(d * d))) if d.size else 0.0,
        "n": int(e.size),
    }
