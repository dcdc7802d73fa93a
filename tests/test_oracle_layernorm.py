"""Pins of the oracle's LayerNorm (CPU only).

The reading notes (Section 5e) extend the method to LayerNorm: the mean and
the variance of the whole vector follow from two additive shard statistics,
sum x and sum x^2. The oracle computes LayerNorm by its two-pass definition
(mean, then centred variance) in binary64, and the per-shard statistics by
plain sums. Every pin runs on the C oracle and on the NumPy mirror; planted
mistakes in a copy of the mirror must each fail a pin.
"""
import math
import types
from fractions import Fraction

import numpy as np
import pytest

from layerwise_qk_norm_amd import inputs
from oracle import oracle

C_IMPL = types.SimpleNamespace(
    name="c", layernorm=lambda x, g, b, eps: oracle.layernorm(x, g, b, eps),
    shard_stats=oracle.shard_stats)
NP_IMPL = types.SimpleNamespace(
    name="numpy", layernorm=oracle.layernorm_np, shard_stats=oracle.shard_stats_np)


def f32(a):
    return np.asarray(a, np.float32)


def pin_constant_row(impl):
    """x_j = c: mean c, variance 0, so y = beta exactly and rstd = 1/sqrt(eps)."""
    H, c, eps = 64, 0.375, 2.0 ** -8
    g = f32(np.linspace(0.5, 1.5, H))
    b = f32(np.linspace(-0.5, 0.5, H))
    y, mu, r = impl.layernorm(f32(np.full((1, H), c)), g, b, eps)
    assert mu[0] == c
    assert abs(r[0] - 1.0 / math.sqrt(eps)) <= 1e-15 * r[0]
    assert np.array_equal(y[0], b.astype(np.float64))


def pin_two_valued_row(impl):
    """Alternating +a, -a: mean 0, variance a^2; y_j = +-a/sqrt(a^2 + eps) gamma_j + beta_j.
    eps = 2^-8 is large enough for any misplacement of it to show."""
    H, a, eps = 128, 0.75, 2.0 ** -8
    x = f32([[a if j % 2 == 0 else -a for j in range(H)]])
    g = f32(1.0 + np.arange(H) / 256.0)
    b = f32(np.linspace(-0.5, 0.5, H))
    y, mu, r = impl.layernorm(x, g, b, eps)
    assert mu[0] == 0.0
    s = np.where(np.arange(H) % 2 == 0, 1.0, -1.0)
    want = s * a / math.sqrt(a * a + eps) * g.astype(np.float64) + b.astype(np.float64)
    np.testing.assert_allclose(y[0], want, rtol=1e-14, atol=1e-15)


def pin_shift_invariance(impl):
    """LN(x + c) = LN(x): the mean is subtracted from every element and from the variance."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 96))
    g = f32(rng.uniform(0.5, 1.5, 96))
    b = f32(rng.uniform(-0.5, 0.5, 96))
    y0, _, r0 = impl.layernorm(f32(x), g, b, 1e-6)
    y1, _, r1 = impl.layernorm(f32(x + 3.0), g, b, 1e-6)
    # x + 3 is rounded to fp32 again, so compare at fp32-input precision
    np.testing.assert_allclose(y1, y0, rtol=0, atol=2e-6)
    np.testing.assert_allclose(r1, r0, rtol=2e-6)


def pin_scale_invariance(impl):
    """With eps = 0, LN(4x) = LN(x) (scaling by a power of two is exact)."""
    rng = np.random.default_rng(4)
    x = f32(rng.standard_normal((3, 80)))
    g = f32(rng.uniform(0.5, 1.5, 80))
    y0, _, _ = impl.layernorm(x, g, None, 0.0)
    y1, _, _ = impl.layernorm(x * 4, g, None, 0.0)
    np.testing.assert_allclose(y1, y0, rtol=1e-13, atol=1e-14)


def pin_zero_mean_is_rmsnorm(impl):
    """Rows with an exactly zero mean (x next to -x): LayerNorm without beta is the
    RMSNorm pinned in test_oracle.py."""
    rng = np.random.default_rng(6)
    h = f32(rng.standard_normal((5, 64)))
    x = np.ascontiguousarray(np.concatenate([h, -h], axis=1))
    g = f32(rng.uniform(0.5, 1.5, 128))
    y, mu, r = impl.layernorm(x, g, None, 1e-6)
    assert np.all(mu == 0)
    yr, _, rr = oracle.rmsnorm(x, g, 1e-6)
    np.testing.assert_allclose(y, yr, rtol=1e-14)
    np.testing.assert_allclose(r, rr, rtol=1e-14)


def pin_torch_layer_norm(impl):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    x = f32(rng.standard_normal((9, 640)) * 2.0 + 0.5)
    g = f32(rng.uniform(0.5, 1.5, 640))
    b = f32(rng.uniform(-0.5, 0.5, 640))
    y, _, _ = impl.layernorm(x, g, b, 1e-6)
    ref = torch.nn.functional.layer_norm(
        torch.from_numpy(x.astype(np.float64)), (640,), torch.from_numpy(g.astype(np.float64)),
        torch.from_numpy(b.astype(np.float64)), float(np.float32(1e-6))).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


def pin_unit_variance(impl):
    """gamma = 1, beta = 0, eps = 0: every row has mean 0 and mean square 1."""
    rng = np.random.default_rng(8)
    x = f32(rng.standard_normal((6, 300)) * 3.0 + 1.0)
    y, _, _ = impl.layernorm(x, f32(np.ones(300)), f32(np.zeros(300)), 0.0)
    np.testing.assert_allclose(np.mean(y, axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-12)


def pin_stats_additive(impl):
    """Shard statistics add up to the row's sum and sum of squares, bitwise on a
    dyadic grid; a row nonzero only in block k has nonzero statistics only at k."""
    rng = np.random.default_rng(3)
    H = 256
    x = f32(rng.integers(-16, 17, (6, H)) / 8.0)
    xv = x.astype(np.float64)
    for N in (1, 2, 4, 8):
        a, b = impl.shard_stats(x, N)
        assert np.array_equal(a.sum(axis=0), xv.sum(axis=1))
        assert np.array_equal(b.sum(axis=0), (xv * xv).sum(axis=1))
    for N in (2, 4):
        W = H // N
        xs = np.zeros((N, H), np.float32)
        for k in range(N):
            xs[k, k * W:(k + 1) * W] = -0.5
        a, b = impl.shard_stats(xs, N)
        assert np.array_equal(a, np.diag(np.full(N, -0.5 * W)))
        assert np.array_equal(b, np.diag(np.full(N, 0.25 * W)))


def pin_stats_give_mean_and_variance(impl):
    """mean = sum/H and var = sumsq/H - mean^2 from the combined shard statistics."""
    w = inputs.LN_SHIFTED.with_T(6)
    d = inputs.make_host(w)
    x, g, b = d["q"], d["gamma_q"], d["beta_q"]
    _, mu, r = impl.layernorm(x, g, b, w.eps)
    a, s2 = impl.shard_stats(x, w.n_shards)
    H = x.shape[1]
    m = a.sum(axis=0) / H
    var = s2.sum(axis=0) / H - m * m
    np.testing.assert_allclose(m, mu, rtol=1e-13)
    np.testing.assert_allclose(1.0 / np.sqrt(var + float(np.float32(w.eps))), r, rtol=1e-11)


def pin_brute_force_tiny(impl):
    w = inputs.LN_TINY
    d = inputs.make_host(w)
    for t_ in ("q", "k"):
        x, g, b = d[t_], d["gamma_" + t_], d["beta_" + t_]
        y, mu, r = impl.layernorm(x, g, b, w.eps)
        ye, me, ve = oracle.layernorm_exact(x, g, b, w.eps)
        for t in range(w.T):
            assert abs(Fraction(float(mu[t])) - me[t]) <= Fraction(1, 10 ** 14) * (abs(me[t]) + 1)
            e = float(np.float32(w.eps))
            assert abs(float(r[t]) - 1.0 / math.sqrt(float(ve[t]) + e)) <= 1e-13 * float(r[t])
            np.testing.assert_allclose(y[t], [float(v) for v in ye[t]], rtol=1e-12, atol=1e-14)


PINS = [pin_constant_row, pin_two_valued_row, pin_shift_invariance, pin_scale_invariance,
        pin_zero_mean_is_rmsnorm, pin_torch_layer_norm, pin_unit_variance, pin_stats_additive,
        pin_stats_give_mean_and_variance, pin_brute_force_tiny]


@pytest.mark.parametrize("impl", [C_IMPL, NP_IMPL], ids=lambda i: i.name)
@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_layernorm_pin(impl, pin):
    pin(impl)


def test_c_and_numpy_agree_on_workload_prefixes():
    for w in (inputs.LN_DECODE.with_T(16), inputs.LN_GQA.with_T(8), inputs.LN_SHIFTED.with_T(8)):
        d = inputs.make_host(w)
        for t in ("q", "k"):
            a = oracle.layernorm(d[t], d["gamma_" + t], d["beta_" + t], w.eps)
            b = oracle.layernorm_np(d[t], d["gamma_" + t], d["beta_" + t], w.eps)
            for u, v in zip(a, b):
                np.testing.assert_allclose(u, v, rtol=1e-12, atol=1e-13)


def _mutant(kind):
    def layernorm(x, gamma, beta, eps):
        xv = oracle.decode(x)
        g = oracle.decode(gamma)
        b = np.zeros_like(g) if beta is None else oracle.decode(beta)
        H = xv.shape[1]
        e = float(np.float32(eps))
        mu = np.mean(xv, axis=1)
        if kind == "mean_over_shard":
            mu = np.sum(xv, axis=1) / (H // 2)
        c = xv - mu[:, None]
        var = np.mean(c * c, axis=1)
        if kind == "uncentred_variance":
            var = np.mean(xv * xv, axis=1)
        elif kind == "unbiased_variance":
            var = np.sum(c * c, axis=1) / (H - 1)
        denom = np.sqrt(var + e)
        if kind == "eps_outside_sqrt":
            denom = np.sqrt(var) + e
        num = xv if kind == "mean_not_subtracted" else c
        if kind == "mean_added":
            num = xv + mu[:, None]
        y = num / denom[:, None] * g[None, :] + b[None, :]
        if kind == "no_beta":
            y = num / denom[:, None] * g[None, :]
        elif kind == "beta_scaled":
            y = (num / denom[:, None] + b[None, :]) * g[None, :]
        elif kind == "gamma_reversed":
            y = num / denom[:, None] * g[None, ::-1] + b[None, :]
        return y, mu, 1.0 / denom

    def shard_stats(x, N):
        xv = oracle.decode(x)
        T, H = xv.shape
        W = H // N
        if kind == "abs_sums":
            return (np.stack([np.abs(xv[:, k * W:(k + 1) * W]).sum(axis=1) for k in range(N)]),
                    np.stack([(xv[:, k * W:(k + 1) * W] ** 2).sum(axis=1) for k in range(N)]))
        if kind == "strided_stats":
            return (np.stack([xv[:, k::N].sum(axis=1) for k in range(N)]),
                    np.stack([(xv[:, k::N] ** 2).sum(axis=1) for k in range(N)]))
        return oracle.shard_stats_np(x, N)

    return types.SimpleNamespace(name=kind, layernorm=layernorm, shard_stats=shard_stats)


MUTANTS = ["mean_over_shard", "uncentred_variance", "unbiased_variance", "eps_outside_sqrt",
           "mean_not_subtracted", "mean_added", "no_beta", "beta_scaled", "gamma_reversed",
           "abs_sums", "strided_stats"]


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
