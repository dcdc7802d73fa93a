"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each pin is a function of an oracle implementation ``impl`` with
``impl.rmsnorm(x, gamma, eps) -> (y, S, rinv)`` and
``impl.shard_sumsq(x, N) -> p[N][T]``. The same pins run on the C oracle, on
the NumPy mirror, and on deliberately broken copies of the NumPy mirror
(``test_every_mutant_fails_a_pin``), which shows that a plausible mistake
(a dropped term, a misplaced epsilon, a wrong divisor, index or sign) fails
at least one pin.
"""
import json
import math
import os
import types
from fractions import Fraction

import numpy as np
import pytest

from layerwise_qk_norm_amd import inputs
from oracle import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "p2_worked_example.json")

C_IMPL = types.SimpleNamespace(
    name="c",
    rmsnorm=lambda x, g, eps: oracle.rmsnorm(x, g, eps),
    shard_sumsq=oracle.shard_sumsq)
NP_IMPL = types.SimpleNamespace(
    name="numpy", rmsnorm=oracle.rmsnorm_np, shard_sumsq=oracle.shard_sumsq_np)
IMPLS = [C_IMPL, NP_IMPL]


def f32(a):
    return np.asarray(a, np.float32)


# ------------------------------------------------------------------ pins

def pin_worked_example(impl):
    """Reading notes, Section 4b, Eqs. (2)-(8)."""
    g = json.load(open(GOLDEN))
    x = f32([g["x"]])
    H = g["H_total"]
    gamma = f32([g["gamma"]] * H)
    for x_in, g_in in ((x, gamma), (inputs.f32_to_bf16_bits(x), inputs.f32_to_bf16_bits(gamma))):
        p = impl.shard_sumsq(x_in, g["n_shards"])
        assert list(p[:, 0]) == g["partials"]  # dyadic: exact
        y, S, r = impl.rmsnorm(x_in, g_in, g["eps"])
        assert S[0] == g["S_global"]
        assert S[0] / H == g["mean_square"]
        assert abs(1.0 / r[0] - g["rms_printed"]) < 5e-5
        assert abs(r[0] - g["rms_inv_printed"]) < g["rms_inv_tol"]
        assert np.max(np.abs(y[0] - np.array(g["y_printed"]))) < g["y_tol_abs"]


def pin_constant_row(impl):
    """Closed form: x_j = c for all j gives y_j = gamma_j * c / sqrt(c^2 + eps).

    eps is chosen large (2^-8) so that any misplacement of eps changes the
    result by far more than the tolerance.
    """
    H, c, eps = 64, 0.0625, 2.0 ** -8
    x = f32(np.full((1, H), c))
    gamma = f32(np.linspace(0.5, 1.5, H))
    y, S, r = impl.rmsnorm(x, gamma, eps)
    expect_r = 1.0 / math.sqrt(c * c + eps)
    assert abs(r[0] - expect_r) <= 1e-14 * expect_r
    np.testing.assert_allclose(y[0], gamma.astype(np.float64) * c * expect_r, rtol=1e-14)


def pin_one_hot_row(impl):
    """Closed form: one nonzero a at column j0: y_j0 = a*gamma_j0/sqrt(a^2/H + eps), else 0.

    The divisor must be the full width H (not a shard width); gamma must be
    indexed by column (gamma entries are all distinct).
    """
    H, a, j0, eps = 96, -3.0, 37, 1e-6
    x = np.zeros((1, H), np.float32)
    x[0, j0] = a
    gamma = f32(1.0 + np.arange(H) / 128.0)
    y, S, r = impl.rmsnorm(x, gamma, eps)
    e = float(np.float32(eps))
    expect = a * float(gamma[j0]) / math.sqrt(a * a / H + e)
    assert abs(y[0, j0] - expect) <= 1e-14 * abs(expect)
    y2 = y[0].copy()
    y2[j0] = 0
    assert np.all(y2 == 0)


def pin_zero_row(impl):
    """A zero row with eps > 0: reciprocal RMS 1/sqrt(eps), outputs exactly 0."""
    H, eps = 32, 1e-6
    x = np.zeros((2, H), np.float32)
    gamma = f32(np.linspace(0.5, 1.5, H))
    y, S, r = impl.rmsnorm(x, gamma, eps)
    assert np.all(S == 0)
    e = float(np.float32(eps))
    np.testing.assert_allclose(r, 1.0 / math.sqrt(e), rtol=1e-15)
    assert np.all(y == 0)


def pin_unit_rms(impl):
    """With gamma = 1 and eps = 0 the output has mean square exactly 1 (in exact math)."""
    rng = np.random.default_rng(7)
    x = f32(rng.standard_normal((5, 300)) * 3.0)
    y, S, r = impl.rmsnorm(x, f32(np.ones(300)), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-12)


def pin_partials_sum_to_total(impl):
    """sum_k p[k][t] = S[t]; bitwise on a dyadic grid (every term and sum exact)."""
    rng = np.random.default_rng(3)
    H = 256
    x = f32(rng.integers(-16, 17, (6, H)) / 8.0)  # m/8, exact in bf16 and fp32
    for N in (1, 2, 4, 8):
        p = impl.shard_sumsq(x, N)
        _, S, _ = impl.rmsnorm(x, f32(np.ones(H)), 1e-6)
        assert np.array_equal(p.sum(axis=0), S)
    # shards are contiguous column blocks: a row that is nonzero only in
    # block k has a single nonzero partial, at k
    for N in (2, 4, 8):
        W = H // N
        xs = np.zeros((N, H), np.float32)
        for k in range(N):
            xs[k, k * W:(k + 1) * W] = 0.5
        p = impl.shard_sumsq(xs, N)
        assert np.array_equal(p, np.diag(np.full(N, 0.25 * W)))


def pin_brute_force_tiny(impl):
    """The tiny workload (T=8, H=256, fp32) against exact rational sums."""
    w = inputs.TINY
    d = inputs.make_host(w)
    for name in ("q", "k"):
        x, g = d[name], d["gamma_" + name]
        y, S, r = impl.rmsnorm(x, g, w.eps)
        ye, Se, re_ = oracle.rmsnorm_exact(x, g, w.eps)
        for t in range(w.T):
            assert abs(Fraction(float(S[t])) - Se[t]) <= Fraction(1, 10 ** 12) * Se[t]
            assert abs(float(r[t]) - float(re_[t])) <= 1e-14 * float(re_[t])
            ref = np.array([float(v) for v in ye[t]])
            np.testing.assert_allclose(y[t], ref, rtol=1e-13, atol=0)


def pin_torch_rms_norm(impl):
    """N=1 special case: torch.nn.functional.rms_norm in float64 on the CPU."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    x = f32(rng.standard_normal((9, 640)) * 2.0)
    gamma = f32(rng.uniform(0.5, 1.5, 640))
    eps = 1e-6
    y, _, _ = impl.rmsnorm(x, gamma, eps)
    ref = torch.nn.functional.rms_norm(
        torch.from_numpy(x.astype(np.float64)), (640,),
        torch.from_numpy(gamma.astype(np.float64)), float(np.float32(eps))).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=0)


def pin_column_permutation(impl):
    """Permuting columns of x and gamma together permutes y the same way."""
    rng = np.random.default_rng(5)
    x = f32(rng.standard_normal((4, 128)))
    gamma = f32(rng.uniform(0.5, 1.5, 128))
    perm = rng.permutation(128)
    y, _, _ = impl.rmsnorm(x, gamma, 1e-6)
    yp, _, _ = impl.rmsnorm(np.ascontiguousarray(x[:, perm]), np.ascontiguousarray(gamma[perm]),
                            1e-6)
    np.testing.assert_allclose(yp, y[:, perm], rtol=1e-14)


PINS = [pin_worked_example, pin_constant_row, pin_one_hot_row, pin_zero_row, pin_unit_rms,
        pin_partials_sum_to_total, pin_brute_force_tiny, pin_torch_rms_norm,
        pin_column_permutation]


@pytest.mark.parametrize("impl", IMPLS, ids=lambda i: i.name)
@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(impl, pin):
    pin(impl)


def test_c_and_numpy_agree_on_workload_prefixes():
    for w in (inputs.DECODE.with_T(16), inputs.GQA.with_T(8), inputs.PREFILL.with_T(4)):
        d = inputs.make_host(w)
        for name in ("q", "k"):
            yc, Sc, rc = oracle.rmsnorm(d[name], d["gamma_" + name], w.eps)
            yn, Sn, rn = oracle.rmsnorm_np(d[name], d["gamma_" + name], w.eps)
            np.testing.assert_allclose(yc, yn, rtol=1e-13)
            np.testing.assert_allclose(rc, rn, rtol=1e-13)
            np.testing.assert_allclose(oracle.shard_sumsq(d[name], w.n_shards),
                                       oracle.shard_sumsq_np(d[name], w.n_shards), rtol=1e-13)


def test_threaded_rows_match_serial():
    w = inputs.DECODE.with_T(40)
    d = inputs.make_host(w)
    a = oracle.rmsnorm(d["q"], d["gamma_q"], w.eps, threads=1)
    b = oracle.rmsnorm(d["q"], d["gamma_q"], w.eps, threads=4)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_oracle_rejects_bad_arguments():
    x = np.zeros((2, 10), np.float32)
    with pytest.raises(ValueError):
        oracle.shard_sumsq(x, 3)  # 10 % 3 != 0
    with pytest.raises(TypeError):
        oracle.rmsnorm(np.zeros((2, 4), np.float64), np.zeros(4), 1e-6)


# ------------------------------------------------------------------ planted mistakes

def _mutant(kind):
    def rmsnorm(x, gamma, eps):
        xv = oracle.decode(x)
        g = oracle.decode(gamma)
        H = xv.shape[1]
        e = float(np.float32(eps))
        S = np.sum(xv * xv, axis=1)
        if kind == "abs_not_square":
            S = np.sum(np.abs(xv), axis=1)
        denom = np.sqrt(S / H + e)
        if kind == "eps_outside_sqrt":
            denom = np.sqrt(S / H) + e
        elif kind == "no_eps":
            denom = np.sqrt(S / H)
        elif kind == "shard_divisor":
            denom = np.sqrt(S / (H // 2) + e)
        elif kind == "sum_not_mean":
            denom = np.sqrt(S + e)
        elif kind == "no_sqrt":
            denom = S / H + e
        elif kind == "eps_squared":
            denom = np.sqrt(S / H + e * e)
        if kind == "gamma_reversed":
            g = g[::-1]
        if kind == "no_gamma":
            g = np.ones_like(g)
        if kind == "gamma_shifted":
            g = np.roll(g, 1)
        y = xv / denom[:, None] * g[None, :]
        if kind == "multiply_by_rms":
            y = xv * denom[:, None] * g[None, :]
        if kind == "sign":
            y = -y
        return y, S, 1.0 / denom

    def shard_sumsq(x, N):
        xv = oracle.decode(x)
        T, H = xv.shape
        W = H // N
        if kind == "strided_shards":
            return np.stack([np.sum(xv[:, k::N] ** 2, axis=1) for k in range(N)])
        if kind == "shard_off_by_one":
            return np.stack([np.sum(xv[:, k * W:(k + 1) * W - 1] ** 2, axis=1)
                             for k in range(N)])
        if kind == "shard_token_major":
            return np.stack([np.sum(xv[:, k * W:(k + 1) * W] ** 2, axis=1)
                             for k in range(N)]).T.reshape(N, T)
        return oracle.shard_sumsq_np(x, N)

    return types.SimpleNamespace(name=kind, rmsnorm=rmsnorm, shard_sumsq=shard_sumsq)


MUTANTS = ["abs_not_square", "eps_outside_sqrt", "no_eps", "shard_divisor", "sum_not_mean",
           "no_sqrt", "eps_squared", "gamma_reversed", "no_gamma", "multiply_by_rms", "sign",
           "gamma_shifted", "strided_shards", "shard_off_by_one", "shard_token_major"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_every_mutant_fails_a_pin(kind):
    impl = _mutant(kind)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(divide="ignore", invalid="ignore"):
                pin(impl)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"mutant {kind} passed every pin"
