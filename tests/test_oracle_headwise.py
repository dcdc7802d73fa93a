"""Pins of the oracle's headwise RMSNorm (CPU only).

Headwise QK-Norm computes one factor per attention head instead of one per
full Q or K vector ("SwiftQK ...", Section II-A). Every pin runs on the C
oracle and on the NumPy mirror; planted mistakes in a copy of the mirror must
each fail a pin.
"""
import math
import types
from fractions import Fraction

import numpy as np
import pytest

from layerwise_qk_norm_amd import inputs
from oracle import oracle

C = types.SimpleNamespace(name="c", headwise=lambda x, g, D, eps: oracle.headwise(x, g, D, eps))
NP = types.SimpleNamespace(name="numpy", headwise=oracle.headwise_np)


def f32(a):
    return np.asarray(a, np.float32)


def pin_one_head_is_layerwise(impl):
    """A single head spanning the row is the layerwise RMSNorm pinned in test_oracle.py."""
    rng = np.random.default_rng(1)
    x = f32(rng.standard_normal((5, 256)))
    g = f32(rng.uniform(0.5, 1.5, 256))
    y, r = impl.headwise(x, g, 256, 1e-6)
    yl, _, rl = oracle.rmsnorm(x, g, 1e-6)
    np.testing.assert_allclose(y, yl, rtol=1e-14)
    np.testing.assert_allclose(r[:, 0], rl, rtol=1e-14)


def pin_heads_are_independent(impl):
    """Changing one head leaves every other head's output bit for bit unchanged."""
    rng = np.random.default_rng(2)
    D, nh = 64, 6
    x = f32(rng.standard_normal((4, D * nh)))
    g = f32(rng.uniform(0.5, 1.5, D))
    y0, _ = impl.headwise(x, g, D, 1e-6)
    x2 = x.copy()
    x2[:, 2 * D:3 * D] = f32(rng.standard_normal((4, D)))  # new values, not a rescaling
    y1, _ = impl.headwise(x2, g, D, 1e-6)
    keep = np.r_[0:2 * D, 3 * D:nh * D]
    assert np.array_equal(y0[:, keep], y1[:, keep])
    assert not np.allclose(y0[:, 2 * D:3 * D], y1[:, 2 * D:3 * D])


def pin_each_head_is_an_rmsnorm_row(impl):
    """Head h of token t equals the pinned layerwise RMSNorm of that head's D values."""
    rng = np.random.default_rng(3)
    D, nh = 128, 5
    x = f32(rng.standard_normal((3, D * nh)) * 2.0)
    g = f32(rng.uniform(0.5, 1.5, D))
    y, r = impl.headwise(x, g, D, 1e-6)
    yl, _, rl = oracle.rmsnorm(np.ascontiguousarray(x.reshape(3 * nh, D)), g, 1e-6)
    np.testing.assert_allclose(y, yl.reshape(3, nh * D), rtol=1e-14)
    np.testing.assert_allclose(r.reshape(-1), rl, rtol=1e-14)


def pin_torch_rms_norm_last_dim(impl):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    D, nh = 128, 8
    x = f32(rng.standard_normal((7, D * nh)))
    g = f32(rng.uniform(0.5, 1.5, D))
    y, _ = impl.headwise(x, g, D, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x.astype(np.float64)).reshape(7, nh, D),
                                       (D,), torch.from_numpy(g.astype(np.float64)),
                                       float(np.float32(1e-6))).reshape(7, nh * D).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-13)


def pin_closed_forms(impl):
    """Head 0 constant c: y = gamma*c/sqrt(c^2 + eps); head 1 one-hot a at j0:
    y_j0 = a*gamma_j0/sqrt(a^2/D + eps); the divisor is D, not the row width."""
    D, c, a, j0, eps = 32, 0.25, -3.0, 5, 2.0 ** -8
    x = np.zeros((1, 2 * D), np.float32)
    x[0, :D] = c
    x[0, D + j0] = a
    g = f32(1.0 + np.arange(D) / 64.0)
    y, r = impl.headwise(x, g, D, eps)
    g64 = g.astype(np.float64)
    np.testing.assert_allclose(y[0, :D], g64 * c / math.sqrt(c * c + eps), rtol=1e-14)
    assert abs(y[0, D + j0] - a * g64[j0] / math.sqrt(a * a / D + eps)) <= 1e-14 * abs(y[0, D + j0])
    assert np.count_nonzero(y[0, D:]) == 1


def pin_brute_force_tiny(impl):
    w = inputs.HW_TINY
    d = inputs.make_host(w)
    D = w.head_dim
    for t_ in ("q", "k"):
        x, g = d[t_], d["gamma_" + t_]
        y, r = impl.headwise(x, g, D, w.eps)
        nh = x.shape[1] // D
        rows = np.ascontiguousarray(x.reshape(w.T * nh, D))
        ye, Se, re_ = oracle.rmsnorm_exact(rows, g, w.eps)
        for i in range(w.T * nh):
            assert abs(float(r.reshape(-1)[i]) - float(re_[i])) <= 1e-14 * float(re_[i])
            np.testing.assert_allclose(y.reshape(-1, D)[i], [float(v) for v in ye[i]], rtol=1e-13)


PINS = [pin_one_head_is_layerwise, pin_heads_are_independent, pin_each_head_is_an_rmsnorm_row,
        pin_torch_rms_norm_last_dim, pin_closed_forms, pin_brute_force_tiny]


@pytest.mark.parametrize("impl", [C, NP], ids=lambda i: i.name)
@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_headwise_pin(impl, pin):
    pin(impl)


def test_c_and_numpy_agree_on_workloads():
    for w in (inputs.HW_DECODE.with_T(8), inputs.HW_GQA.with_T(4)):
        d = inputs.make_host(w)
        for t in ("q", "k"):
            a = oracle.headwise(d[t], d["gamma_" + t], w.head_dim, w.eps)
            b = oracle.headwise_np(d[t], d["gamma_" + t], w.head_dim, w.eps)
            np.testing.assert_allclose(a[0], b[0], rtol=1e-13)


def _mutant(kind):
    def headwise(x, gamma, D, eps):
        xv = oracle.decode(x)
        g = oracle.decode(gamma)
        T, H = xv.shape
        e = float(np.float32(eps))
        xh = xv.reshape(T, H // D, D)
        S = np.sum(xh * xh, axis=2)
        if kind == "one_factor_per_row":
            S = np.repeat(np.sum(xv * xv, axis=1, keepdims=True) * D / H, H // D, axis=1)
        div = H if kind == "row_divisor" else D
        denom = np.sqrt(S / div + e)
        if kind == "eps_outside_sqrt":
            denom = np.sqrt(S / div) + e
        if kind == "gamma_reversed":
            g = g[::-1]
        y = xh / denom[:, :, None] * g[None, None, :]
        if kind == "heads_shifted":
            y = np.roll(y, 1, axis=1)
        return y.reshape(T, H), 1.0 / denom

    return types.SimpleNamespace(name=kind, headwise=headwise)


MUTANTS = ["one_factor_per_row", "row_divisor", "eps_outside_sqrt", "gamma_reversed",
           "heads_shifted"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_every_mutant_fails_a_pin(kind):
    impl = _mutant(kind)
    failed = []
    for pin in PINS:
        try:
            pin(impl)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {kind} passed every pin"
