"""Parity of the HIP path with the fp64 oracle on every workload (GPU).

* the four named workloads element by element, at reduced token counts
  (several tiles and a ragged tail) and at their full sizes (all rows);
* the split entry points (partials, reciprocal RMS, outputs);
* all 320 sweep points at full size, in the launch configuration the
  benchmark uses: against the oracle on sampled rows and on every row of the
  first and last tile of every workgroup group of the launch made; every row
  against a plain fp64 reference computed on the device.
Tolerances: max relative error 8e-3 for bf16 outputs, 1e-5 for fp32 outputs,
1e-5 for fp32 statistics.
"""
import zlib

import numpy as np
import pytest
import torch

from layerwise_qk_norm_amd import inputs, ops
from oracle import compare, oracle

from _gpu import (assert_parity, device_rms_check, group_tile_rows, needs_gpu, run_fused, run_split,
                  to_dev, to_host)

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


SWEEP = list(inputs.sweep())


@pytest.mark.parametrize("w", SWEEP, ids=[w.name for w in SWEEP])
def test_sweep_full_size(w):
    """Oracle on 45 sampled rows plus every row of the first and last tile of every
    workgroup group of the launch actually made; every row of both tensors against a
    plain fp64 reference on the device."""
    torch.cuda.empty_cache()
    q = inputs.make_device_activations(w, "q", "cuda:0", torch)
    k = inputs.make_device_activations(w, "k", "cuda:0", torch)
    hd = inputs.make_host(w.with_T(1))
    gq, gk = to_dev(hd["gamma_q"]), to_dev(hd["gamma_k"])
    oq, ok = ops.layerwise_fwd(q, k, gq, gk, w.n_shards, w.eps)
    assert ops.check_fault() == ops.QKN_OK
    sample = _sample_rows(w.T, np.random.default_rng(zlib.crc32(w.name.encode())))
    plan_q, plan_k = group_tile_rows(w.fmt, w.T, w.Hq, w.Hk, w.n_shards)
    for x, g, y, gh, pr in ((q, gq, oq, hd["gamma_q"], plan_q), (k, gk, ok, hd["gamma_k"], plan_k)):
        idx = torch.as_tensor(np.union1d(sample, pr), device="cuda:0")
        assert_parity(to_host(x.index_select(0, idx)), gh, to_host(y.index_select(0, idx)),
                      w.eps, w.name)
        device_rms_check(x, g, y, w.eps, compare.TOL[w.dtype], w.name)
    del q, k, oq, ok
