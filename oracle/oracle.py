"""Layerwise QK-Norm oracle (fp64, CPU).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the product. It shares no code
with the HIP library or its binding and imports nothing from them.

Three independent renderings of the same definitions (RMSNorm, and LayerNorm with
its two additive shard statistics):

* ``rmsnorm`` / ``shard_sumsq`` -- the plain C loops in ``qknorm_oracle.c``
  (fast enough for full-size sampled rows and for the CPU baseline);
* ``rmsnorm_np`` / ``shard_sumsq_np`` -- a NumPy mirror in float64;
* ``rmsnorm_exact`` -- exact rational sums of squares (``fractions``) and a
  50-digit ``decimal`` square root, for brute force on tiny inputs.

Definition followed (one factor per full Q or K vector of width H):
``y = x / sqrt(sum(x^2)/H + eps) * gamma`` -- "SwiftQK: Fast and
Communication-Efficient Tensor Parallelism for Query-Key Normalization",
Section II-A, Eq. (1); printed cleanly as Eq. (1) of the reading notes
"SwiftQK：当归一化层成为张量并行的瓶颈", Section 2. Shard partials follow
Algorithm 1, Phase A of the letter and Eqs. (3)-(4) of the notes' worked
example (Section 4b). LayerNorm (``layernorm``, ``shard_stats``) follows the notes'
Section 5e: mean and variance over the full vector, which shards reduce to two
additive statistics (sum x, sum x^2); the oracle itself uses the two-pass
definition of the variance. Headwise RMSNorm (``headwise``) normalises each
head of ``head_dim`` columns on its own (letter, Section II-A).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qknorm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPE_CODE = {"bf16": 0, "f32": 1, "e4m3": 2}
# the format of gamma for each input format: bf16 weights with E4M3 activations
GAMMA_FORMAT = {"bf16": "bf16", "f32": "f32", "e4m3": "bf16"}


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (plain -O2, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-shared",
             "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        lib.oracle_rmsnorm.restype = ctypes.c_int
        lib.oracle_rmsnorm.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_layernorm.restype = ctypes.c_int
        lib.oracle_layernorm.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p]
        lib.oracle_shard_stats.restype = ctypes.c_int
        lib.oracle_shard_stats.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_void_p]
        lib.oracle_headwise.restype = ctypes.c_int
        lib.oracle_headwise.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_decode_e4m3.restype = ctypes.c_int
        lib.oracle_decode_e4m3.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_shard_sumsq.restype = ctypes.c_int
        lib.oracle_shard_sumsq.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
        _lib = lib
    return _lib


def _dtype_of(a: np.ndarray) -> str:
    if a.dtype == np.uint16:
        return "bf16"
    if a.dtype == np.float32:
        return "f32"
    if a.dtype == np.uint8:
        return "e4m3"
    raise TypeError("oracle inputs are bf16 bit patterns (uint16), float32 or E4M3 codes "
                    f"(uint8), got {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float, want_y: bool = True,
            threads: int = 1):
    """fp64 RMSNorm of each row of ``x`` ([T][H]) via the C loops.

    ``eps`` is rounded to binary32 first: that is the value the GPU library
    receives. Returns ``(y, S, rinv)``; ``y`` is None when ``want_y`` is False.
    ``threads`` > 1 splits rows over a thread pool (the C call releases the GIL);
    the arithmetic per row is unchanged.
    """
    lib = _load()
    x = np.ascontiguousarray(x)
    gamma = np.ascontiguousarray(gamma)
    dt = _dtype_of(x)
    if _dtype_of(gamma) != GAMMA_FORMAT[dt]:
        raise TypeError(f"gamma must be {GAMMA_FORMAT[dt]} for {dt} inputs")
    T, H = x.shape
    if gamma.shape != (H,):
        raise ValueError("gamma must be [H]")
    y = np.empty((T, H), np.float64) if want_y else None
    S = np.empty(T, np.float64)
    r = np.empty(T, np.float64)

    def run(lo, hi):
        if hi <= lo:
            return
        rc = lib.oracle_rmsnorm(
            x.ctypes.data + lo * H * x.itemsize, gamma.ctypes.data, DTYPE_CODE[dt],
            hi - lo, H, ctypes.c_float(eps),
            None if y is None else y.ctypes.data + lo * H * 8,
            S.ctypes.data + lo * 8, r.ctypes.data + lo * 8)
        if rc != 0:
            raise ValueError("oracle_rmsnorm rejected its arguments")

    if threads <= 1 or T < 2 * threads:
        run(0, T)
    else:
        edges = np.linspace(0, T, threads + 1).astype(np.int64)
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda i: run(int(edges[i]), int(edges[i + 1])), range(threads)))
    return y, S, r


def layernorm(x: np.ndarray, gamma: np.ndarray, beta, eps: float, want_y: bool = True,
              threads: int = 1):
    """fp64 LayerNorm of each row of ``x`` via the C loops (two-pass definition).

    ``beta`` may be None (no shift). Returns ``(y, mean, rstd)``; ``y`` is None when
    ``want_y`` is False. Rows may be split over ``threads`` (arithmetic unchanged).
    """
    lib = _load()
    x = np.ascontiguousarray(x)
    gamma = np.ascontiguousarray(gamma)
    dt = _dtype_of(x)
    if _dtype_of(gamma) != GAMMA_FORMAT[dt]:
        raise TypeError(f"gamma must be {GAMMA_FORMAT[dt]} for {dt} inputs")
    if beta is not None:
        beta = np.ascontiguousarray(beta)
        if _dtype_of(beta) != GAMMA_FORMAT[dt] or beta.shape != gamma.shape:
            raise TypeError("beta must have the format and shape of gamma")
    T, H = x.shape
    if gamma.shape != (H,):
        raise ValueError("gamma must be [H]")
    y = np.empty((T, H), np.float64) if want_y else None
    mu = np.empty(T, np.float64)
    rs = np.empty(T, np.float64)

    def run(lo, hi):
        if hi <= lo:
            return
        rc = lib.oracle_layernorm(
            x.ctypes.data + lo * H * x.itemsize, gamma.ctypes.data,
            None if beta is None else beta.ctypes.data, DTYPE_CODE[dt], hi - lo, H,
            ctypes.c_float(eps), None if y is None else y.ctypes.data + lo * H * 8,
            mu.ctypes.data + lo * 8, rs.ctypes.data + lo * 8)
        if rc != 0:
            raise ValueError("oracle_layernorm rejected its arguments")

    if threads <= 1 or T < 2 * threads:
        run(0, T)
    else:
        edges = np.linspace(0, T, threads + 1).astype(np.int64)
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda i: run(int(edges[i]), int(edges[i + 1])), range(threads)))
    return y, mu, rs


def headwise(x: np.ndarray, gamma: np.ndarray, head_dim: int, eps: float, want_y: bool = True,
             threads: int = 1):
    """fp64 headwise RMSNorm via the C loops: one factor per (token, head) over the
    head's ``head_dim`` columns; ``gamma`` is [head_dim], shared by the heads.
    Returns ``(y, rinv)`` with ``rinv`` [T][n_heads]; ``y`` is None unless wanted."""
    lib = _load()
    x = np.ascontiguousarray(x)
    gamma = np.ascontiguousarray(gamma)
    dt = _dtype_of(x)
    if _dtype_of(gamma) != GAMMA_FORMAT[dt]:
        raise TypeError(f"gamma must be {GAMMA_FORMAT[dt]} for {dt} inputs")
    T, H = x.shape
    if head_dim < 1 or H % head_dim or gamma.shape != (head_dim,):
        raise ValueError("rows must be whole heads and gamma [head_dim]")
    nh = H // head_dim
    y = np.empty((T, H), np.float64) if want_y else None
    r = np.empty((T, nh), np.float64)

    def run(lo, hi):
        if hi <= lo:
            return
        rc = lib.oracle_headwise(x.ctypes.data + lo * H * x.itemsize, gamma.ctypes.data,
                                 DTYPE_CODE[dt], hi - lo, nh, head_dim, ctypes.c_float(eps),
                                 None if y is None else y.ctypes.data + lo * H * 8,
                                 r.ctypes.data + lo * nh * 8)
        if rc != 0:
            raise ValueError("oracle_headwise rejected its arguments")

    if threads <= 1 or T < 2 * threads:
        run(0, T)
    else:
        edges = np.linspace(0, T, threads + 1).astype(np.int64)
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda i: run(int(edges[i]), int(edges[i + 1])), range(threads)))
    return y, r


def shard_stats(x: np.ndarray, n_shards: int):
    """Per-shard sums and sums of squares, each ``[n_shards][T]`` (fp64), via the C loops."""
    lib = _load()
    x = np.ascontiguousarray(x)
    T, H = x.shape
    a = np.empty((n_shards, T), np.float64)
    b = np.empty((n_shards, T), np.float64)
    rc = lib.oracle_shard_stats(x.ctypes.data, DTYPE_CODE[_dtype_of(x)], T, H, n_shards,
                                a.ctypes.data, b.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_shard_stats rejected its arguments (H % N must be 0)")
    return a, b


def shard_sumsq(x: np.ndarray, n_shards: int) -> np.ndarray:
    """Shard-major partial sums of squares ``p[k][t]`` (fp64) via the C loops."""
    lib = _load()
    x = np.ascontiguousarray(x)
    T, H = x.shape
    p = np.empty((n_shards, T), np.float64)
    rc = lib.oracle_shard_sumsq(x.ctypes.data, DTYPE_CODE[_dtype_of(x)], T, H, n_shards,
                                p.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_shard_sumsq rejected its arguments (H % N must be 0)")
    return p


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """Exact values of E4M3 codes via the C decoder (OCP OFP8 E4M3 layout)."""
    lib = _load()
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    if lib.oracle_decode_e4m3(c.ctypes.data, c.size, out.ctypes.data) != 0:
        raise ValueError("oracle_decode_e4m3 rejected its arguments")
    return out


# ---------------------------------------------------------------- NumPy mirror

def decode_e4m3_np(codes: np.ndarray) -> np.ndarray:
    """NumPy rendering of the OCP E4M3 decoding: sign, 4-bit exponent with bias 7,
    3-bit mantissa; exponent 0 is zero or subnormal (m * 2^-9); S.1111.111 is NaN."""
    c = codes.astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    normal = np.ldexp(1.0 + m / 8.0, e - 7)
    sub = np.ldexp(m.astype(np.float64), -9)
    mag = np.where(e == 0, sub, normal)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def decode(a: np.ndarray) -> np.ndarray:
    """Exact float64 values of stored bf16 bit patterns, float32 values or E4M3 codes."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    if a.dtype == np.uint8:
        return decode_e4m3_np(a)
    raise TypeError(a.dtype)


def rmsnorm_np(x: np.ndarray, gamma: np.ndarray, eps: float):
    """NumPy float64 mirror of ``rmsnorm`` (same definition, numpy's sums)."""
    xv = decode(x)
    g = decode(gamma)
    H = xv.shape[1]
    S = np.sum(xv * xv, axis=1)
    denom = np.sqrt(S / H + float(np.float32(eps)))
    y = xv / denom[:, None] * g[None, :]
    return y, S, 1.0 / denom


def layernorm_np(x: np.ndarray, gamma: np.ndarray, beta, eps: float):
    """NumPy float64 mirror of ``layernorm`` (numpy's mean and centred variance)."""
    xv = decode(x)
    g = decode(gamma)
    b = np.zeros_like(g) if beta is None else decode(beta)
    mu = np.mean(xv, axis=1)
    var = np.mean((xv - mu[:, None]) ** 2, axis=1)
    denom = np.sqrt(var + float(np.float32(eps)))
    y = (xv - mu[:, None]) / denom[:, None] * g[None, :] + b[None, :]
    return y, mu, 1.0 / denom


def headwise_np(x: np.ndarray, gamma: np.ndarray, head_dim: int, eps: float):
    """NumPy float64 mirror of ``headwise`` (rows reshaped to [T, heads, head_dim])."""
    xv = decode(x)
    g = decode(gamma)
    T, H = xv.shape
    xh = xv.reshape(T, H // head_dim, head_dim)
    denom = np.sqrt(np.mean(xh * xh, axis=2) + float(np.float32(eps)))
    y = xh / denom[:, :, None] * g[None, None, :]
    return y.reshape(T, H), 1.0 / denom


def shard_stats_np(x: np.ndarray, n_shards: int):
    xv = decode(x)
    T, H = xv.shape
    if H % n_shards:
        raise ValueError("H % N must be 0")
    W = H // n_shards
    a = np.stack([np.sum(xv[:, k * W:(k + 1) * W], axis=1) for k in range(n_shards)])
    b = np.stack([np.sum(xv[:, k * W:(k + 1) * W] ** 2, axis=1) for k in range(n_shards)])
    return a, b


def shard_sumsq_np(x: np.ndarray, n_shards: int) -> np.ndarray:
    xv = decode(x)
    T, H = xv.shape
    if H % n_shards:
        raise ValueError("H % N must be 0")
    W = H // n_shards
    return np.stack([np.sum(xv[:, k * W:(k + 1) * W] ** 2, axis=1) for k in range(n_shards)])


# ---------------------------------------------------------------- exact brute force

def rmsnorm_exact(x: np.ndarray, gamma: np.ndarray, eps: float, digits: int = 50):
    """Exact S (rational) and a ``digits``-digit decimal y, row by row.

    Pure-Python loops: only for tiny inputs.
    """
    getcontext().prec = digits
    xv = decode(x)
    g = decode(gamma)
    T, H = xv.shape
    e = Fraction(float(np.float32(eps)))
    S_out, y_out, r_out = [], [], []
    for t in range(T):
        S = sum((Fraction(float(v)) ** 2 for v in xv[t]), Fraction(0))
        ms = S / H + e
        denom = (Decimal(ms.numerator) / Decimal(ms.denominator)).sqrt()
        S_out.append(S)
        r_out.append(1 / denom)
        y_out.append([Decimal(float(xv[t, j])) / denom * Decimal(float(g[j])) for j in range(H)])
    return y_out, S_out, r_out


def layernorm_exact(x: np.ndarray, gamma: np.ndarray, beta, eps: float, digits: int = 50):
    """Exact mean and variance (rationals) and a ``digits``-digit decimal y, row by row.

    Pure-Python loops: only for tiny inputs.
    """
    getcontext().prec = digits
    xv = decode(x)
    g = decode(gamma)
    b = np.zeros_like(g) if beta is None else decode(beta)
    T, H = xv.shape
    e = Fraction(float(np.float32(eps)))
    mu_out, var_out, y_out = [], [], []
    for t in range(T):
        vals = [Fraction(float(v)) for v in xv[t]]
        mu = sum(vals, Fraction(0)) / H
        var = sum(((v - mu) ** 2 for v in vals), Fraction(0)) / H
        ms = var + e
        denom = (Decimal(ms.numerator) / Decimal(ms.denominator)).sqrt()
        mud = Decimal(mu.numerator) / Decimal(mu.denominator)
        mu_out.append(mu)
        var_out.append(var)
        y_out.append([(Decimal(float(xv[t, j])) - mud) / denom * Decimal(float(g[j])) +
                      Decimal(float(b[j])) for j in range(H)])
    return y_out, mu_out, var_out
