"""Parity of the HIP path with the fp64 oracle on every workload (GPU).

* the four named workloads element by element, at reduced token counts
  (several tiles and a ragged tail) and at their full sizes (all rows);
* the split entry points (partials, reciprocal RMS, outputs);
* all 320 sweep points at full size, in the launch configuration the
  benchmark uses: sampled rows against the oracle, every row against the
  unit-RMS property.
Tolerances: max relative error 8e-3 for bf16 outputs, 1e-5 for fp32 outputs,
1e-5 for fp32 statistics.
"""
import zlib

import numpy as np
import pytest
import torch

from layerwise_qk_norm_amd import inputs, ops
from oracle import compare, oracle

from _gpu import assert_parity, needs_gpu, run_fused, run_split, to_dev, to_host

pytestmark = [pytest.mark.gpu, needs_gpu]

REDUCED = {"tiny": 8, "decode": 64, "prefill": 389, "gqa": 1001}


@pytest.mark.parametrize("name", list(REDUCED))
def test_fused_reduced(name):
    w = inputs.CONFIGS[name].with_T(REDUCED[name])
    d = inputs.make_host(w)
    oq, ok = run_fused(d, w.n_shards, w.eps)
    rq = assert_parity(d["q"], d["gamma_q"], oq, w.eps, f"{name} q")
    rk = assert_parity(d["k"], d["gamma_k"], ok, w.eps, f"{name} k")
    print(name, "q", rq, "k", rk)


@pytest.mark.parametrize("name", ["decode", "prefill", "gqa"])
def test_fused_full_size_all_rows(name):
    w = inputs.CONFIGS[name]
    d = inputs.make_host(w)
    oq, ok = run_fused(d, w.n_shards, w.eps)
    rq = assert_parity(d["q"], d["gamma_q"], oq, w.eps, f"{name} q")
    rk = assert_parity(d["k"], d["gamma_k"], ok, w.eps, f"{name} k")
    print(name, "q", rq, "k", rk)


@pytest.mark.parametrize("name", list(REDUCED))
def test_split_reduced(name):
    w = inputs.CONFIGS[name].with_T(REDUCED[name])
    d = inputs.make_host(w)
    for t in ("q", "k"):
        x, g = d[t], d["gamma_" + t]
        p, r, y = run_split(x, g, w.n_shards, w.eps)
        pe = oracle.shard_sumsq(x, w.n_shards)
        _, _, re_ = oracle.rmsnorm(x, g, w.eps, want_y=False)
        assert compare.report(p, pe)["max_rel"] <= compare.TOL_STAT
        assert compare.report(r, re_)["max_rel"] <= compare.TOL_STAT
        assert_parity(x, g, y, w.eps, f"{name} {t} split")


def _sample_rows(T: int, rng) -> np.ndarray:
    fixed = [0, 1, T // 2, T - 2, T - 1]
    return np.unique(np.concatenate([fixed, rng.integers(0, T, 40)]).clip(0, T - 1))


def _unit_rms_property(x: torch.Tensor, g: torch.Tensor, y: torch.Tensor, eps: float, tol: float):
    """Every row: mean((y/gamma)^2) = m/(m+eps) with m = mean(x^2), checked in fp64."""
    gd = g.double()
    for lo in range(0, x.shape[0], 4096):
        xs, ys = x[lo:lo + 4096].double(), y[lo:lo + 4096].double()
        m = (xs * xs).mean(dim=1)
        want = m / (m + float(np.float32(eps)))
        got = ((ys / gd) ** 2).mean(dim=1)
        err = ((got - want).abs() / want).max().item()
        assert err <= tol, f"unit-RMS property off by {err:.3e}"


SWEEP = list(inputs.sweep())


@pytest.mark.parametrize("w", SWEEP, ids=[w.name for w in SWEEP])
def test_sweep_full_size(w):
    torch.cuda.empty_cache()
    q = inputs.make_device_activations(w, "q", "cuda:0", torch)
    k = inputs.make_device_activations(w, "k", "cuda:0", torch)
    hd = inputs.make_host(w.with_T(1))
    gq, gk = to_dev(hd["gamma_q"]), to_dev(hd["gamma_k"])
    oq, ok = ops.layerwise_fwd(q, k, gq, gk, w.n_shards, w.eps)
    assert ops.check_fault() == ops.QKN_OK
    rows = _sample_rows(w.T, np.random.default_rng(zlib.crc32(w.name.encode())))
    idx = torch.as_tensor(rows, device="cuda:0")
    for x, g, y, gh in ((q, gq, oq, hd["gamma_q"]), (k, gk, ok, hd["gamma_k"])):
        assert_parity(to_host(x.index_select(0, idx)), gh, to_host(y.index_select(0, idx)),
                      w.eps, w.name)
        _unit_rms_property(x, g, y, w.eps, 1e-2 if w.dtype == "bf16" else 1e-5)
    del q, k, oq, ok
