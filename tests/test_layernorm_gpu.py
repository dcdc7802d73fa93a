"""LayerNorm with two additive shard statistics on the HIP path (GPU).

The reading notes (Section 5e) extend the method to LayerNorm: each shard
reduces sum x and sum x^2; the exchanged sums give the mean and the variance
of the whole vector. Outputs are compared with the fp64 oracle by the
operand-scaled error of ``compare.layernorm_scaled_error`` (bf16 8e-3, fp32
1e-5): outputs near zero come from x close to the mean, where a relative
error would not measure the arithmetic.
"""
import zlib

import numpy as np
import pytest
import torch

from layerwise_qk_norm_amd import inputs, ops
from oracle import compare, oracle

from _gpu import (assert_layernorm_parity, device_layernorm_check, group_tile_rows, needs_gpu, to_dev,
                  to_host)

pytestmark = [pytest.mark.gpu, needs_gpu]

REDUCED = {"ln_tiny": 8, "ln_decode": 64, "ln_prefill": 389, "ln_gqa": 1001, "ln_shifted": 257}


def run_ln(d, N, eps, with_beta=True):
    q, k = to_dev(d["q"]), to_dev(d["k"])
    gq, gk = to_dev(d["gamma_q"]), to_dev(d["gamma_k"])
    bq = to_dev(d["beta_q"]) if with_beta else None
    bk = to_dev(d["beta_k"]) if with_beta else None
    oq, ok = ops.layernorm_fwd(q, k, gq, gk, N, eps, beta_q=bq, beta_k=bk)
    torch.cuda.synchronize()
    assert ops.check_fault() == ops.QKN_OK
    return to_host(oq), to_host(ok)


def run_ln_split(x, g, b, N, eps):
    xd, gd = to_dev(x), to_dev(g)
    bd = None if b is None else to_dev(b)
    s1, s2 = ops.shard_stats(xd, N)
    mu, rs = ops.combine_stats(s1, s2, x.shape[1], eps)
    y = ops.apply_norm(xd, gd, bd, mu, rs)
    torch.cuda.synchronize()
    return to_host(s1), to_host(s2), to_host(mu), to_host(rs), to_host(y)


@pytest.mark.parametrize("with_beta", [True, False])
@pytest.mark.parametrize("name", list(REDUCED))
def test_fused_reduced(name, with_beta):
    w = inputs.LN_CONFIGS[name].with_T(REDUCED[name])
    d = inputs.make_host(w)
    oq, ok = run_ln(d, w.n_shards, w.eps, with_beta)
    for t, o in (("q", oq), ("k", ok)):
        b = d["beta_" + t] if with_beta else None
        r = assert_layernorm_parity(d[t], d["gamma_" + t], b, o, w.eps, f"{name} {t}")
        print(name, t, with_beta, r)


@pytest.mark.parametrize("name", ["ln_decode", "ln_prefill", "ln_gqa"])
def test_fused_full_size_all_rows(name):
    w = inputs.LN_CONFIGS[name]
    d = inputs.make_host(w)
    oq, ok = run_ln(d, w.n_shards, w.eps)
    for t, o in (("q", oq), ("k", ok)):
        r = assert_layernorm_parity(d[t], d["gamma_" + t], d["beta_" + t], o, w.eps, f"{name} {t}")
        print(name, t, r)


@pytest.mark.parametrize("name", list(REDUCED))
def test_split_reduced(name):
    w = inputs.LN_CONFIGS[name].with_T(REDUCED[name])
    d = inputs.make_host(w)
    for t in ("q", "k"):
        x, g, b = d[t], d["gamma_" + t], d["beta_" + t]
        s1, s2, mu, rs, y = run_ln_split(x, g, b, w.n_shards, w.eps)
        e1, e2 = oracle.shard_stats(x, w.n_shards)
        xa = np.abs(compare.decode_out(x))
        W = x.shape[1] // w.n_shards
        absum = np.stack([xa[:, k * W:(k + 1) * W].sum(axis=1) for k in range(w.n_shards)])
        # a sum of mixed signs is judged against the sum of magnitudes
        assert np.all(np.abs(s1 - e1) <= compare.TOL_STAT * absum)
        assert compare.report(s2, e2)["max_rel"] <= compare.TOL_STAT
        _, me, re_ = oracle.layernorm(x, g, b, w.eps, want_y=False)
        sig2 = 1.0 / (re_ * re_)
        m2 = (compare.decode_out(x) ** 2).mean(axis=1)
        assert np.all(np.abs(mu - me) <= compare.TOL_STAT * np.sqrt(m2))
        # the variance comes from S2/H - mean^2: its error grows with mean^2 / variance
        assert np.all(np.abs(rs - re_) <= compare.TOL_STAT * re_ * m2 / sig2 * 4)
        assert_layernorm_parity(x, g, b, y, w.eps, f"{name} {t} split")


@pytest.mark.parametrize("N", [1, 2, 4, 8, 16])
def test_dyadic_stats_bitwise_and_fused_equals_split(N):
    """Values k/8 (|k| <= 16) make every fp32 sum and sum of squares exact: the
    device statistics equal the oracle's bit for bit, and the fused outputs
    equal the split path's (same statistics, same expressions)."""
    rng = np.random.default_rng(N)
    T, H = 37, 2048
    q = inputs.f32_to_bf16_bits((rng.integers(-16, 17, (T, H)) / 8.0).astype(np.float32))
    k = inputs.f32_to_bf16_bits((rng.integers(-16, 17, (T, H)) / 8.0 + 0.5).astype(np.float32))
    g = inputs.f32_to_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
    b = inputs.f32_to_bf16_bits(rng.uniform(-0.5, 0.5, H).astype(np.float32))
    for x in (q, k):
        s1, s2, _, _, ys = run_ln_split(x, g, b, N, 1e-6)
        e1, e2 = oracle.shard_stats(x, N)
        assert np.array_equal(s1.astype(np.float64), e1) and np.array_equal(s2.astype(np.float64), e2)
    oq, ok = run_ln({"q": q, "k": k, "gamma_q": g, "gamma_k": g, "beta_q": b, "beta_k": b}, N, 1e-6)
    assert np.array_equal(oq, run_ln_split(q, g, b, N, 1e-6)[4])
    assert np.array_equal(ok, run_ln_split(k, g, b, N, 1e-6)[4])


def test_null_beta_equals_zero_beta():
    w = inputs.LN_DECODE.with_T(40)
    d = inputs.make_host(w)
    z = dict(d, beta_q=np.zeros_like(d["beta_q"]), beta_k=np.zeros_like(d["beta_k"]))
    a = run_ln(d, w.n_shards, w.eps, with_beta=False)
    b = run_ln(z, w.n_shards, w.eps, with_beta=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_constant_rows_give_beta():
    """A constant row has zero variance: y = beta up to fp32 rounding of the two
    products u*rstd and mean*rstd*gamma (rstd = 1/sqrt(eps) = 1000 here)."""
    T, H = 6, 1024
    x = inputs.f32_to_bf16_bits(np.repeat(np.array([0.5, -2.0, 0.0, 1.0, 3.0, -0.25],
                                                   np.float32)[:, None], H, axis=1))
    rng = np.random.default_rng(0)
    g = inputs.f32_to_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
    b = inputs.f32_to_bf16_bits(rng.uniform(-0.5, 0.5, H).astype(np.float32))
    oq, _ = run_ln({"q": x, "k": x, "gamma_q": g, "gamma_k": g, "beta_q": b, "beta_k": b}, 4, 1e-6)
    assert_layernorm_parity(x, g, b, oq, 1e-6, "constant rows")
    np.testing.assert_allclose(compare.decode_out(oq), np.tile(compare.decode_out(b), (T, 1)),
                               atol=4e-3)


@pytest.mark.parametrize("N,H,dt", [(16, 4096, "bf16"), (32, 4096, "bf16"), (3, 3072, "f32"),
                                    (4, 4100, "bf16"), (2, 16384, "f32")])
def test_shard_counts_and_split_fallback(N, H, dt):
    """N = 16 still fits one comm wave; N = 32 (4 x 32 statistics), shard widths that
    are not whole vectors and rows too wide for any variant run the split kernels."""
    w = inputs.Workload("ln_shards", 70, H, H, N, dt, norm="layer")
    d = inputs.make_host(w)
    oq, ok = run_ln(d, N, w.eps)
    assert_layernorm_parity(d["q"], d["gamma_q"], d["beta_q"], oq, w.eps, f"N={N} H={H}")
    assert_layernorm_parity(d["k"], d["gamma_k"], d["beta_k"], ok, w.eps, f"N={N} H={H}")


def test_in_place():
    w = inputs.LN_DECODE.with_T(33)
    d = inputs.make_host(w)
    q, k = to_dev(d["q"]), to_dev(d["k"])
    g = [to_dev(d[n]) for n in ("gamma_q", "gamma_k", "beta_q", "beta_k")]
    ops.layernorm_fwd(q, k, g[0], g[1], w.n_shards, w.eps, beta_q=g[2], beta_k=g[3],
                      out_q=q, out_k=k)
    torch.cuda.synchronize()
    assert_layernorm_parity(d["q"], d["gamma_q"], d["beta_q"], to_host(q), w.eps, "in place q")
    assert_layernorm_parity(d["k"], d["gamma_k"], d["beta_k"], to_host(k), w.eps, "in place k")


SWEEP = list(inputs.sweep_layernorm())


@pytest.mark.parametrize("w", SWEEP, ids=[w.name for w in SWEEP])
def test_sweep_full_size(w):
    torch.cuda.empty_cache()
    q = inputs.make_device_activations(w, "q", "cuda:0", torch)
    k = inputs.make_device_activations(w, "k", "cuda:0", torch)
    hd = inputs.make_host(w.with_T(1))
    gq, gk = to_dev(hd["gamma_q"]), to_dev(hd["gamma_k"])
    bq, bk = to_dev(hd["beta_q"]), to_dev(hd["beta_k"])
    oq, ok = ops.layernorm_fwd(q, k, gq, gk, w.n_shards, w.eps, beta_q=bq, beta_k=bk)
    assert ops.check_fault() == ops.QKN_OK
    rows = np.unique(np.concatenate([[0, 1, w.T // 2, w.T - 1],
                                     np.random.default_rng(zlib.crc32(w.name.encode()))
                                     .integers(0, w.T, 40)]))
    # plus every row of the first and last tile of every group of the launch made
    plan_q, plan_k = group_tile_rows(w.fmt, w.T, w.Hq, w.Hk, w.n_shards)
    for x, g, b, y, gh, bh, pr in ((q, gq, bq, oq, hd["gamma_q"], hd["beta_q"], plan_q),
                                   (k, gk, bk, ok, hd["gamma_k"], hd["beta_k"], plan_k)):
        idx = torch.as_tensor(np.union1d(rows, pr), device="cuda:0")
        assert_layernorm_parity(to_host(x.index_select(0, idx)), gh, bh,
                                to_host(y.index_select(0, idx)), w.eps, w.name)
        # every element of every row against a plain fp64 reference on the device
        device_layernorm_check(x, g, b, y, w.eps, compare.TOL[w.dtype], w.name)
    del q, k, oq, ok
