"""Shared helpers of the GPU tests: host<->device transfer and oracle checks."""
import numpy as np
import pytest
import torch

from layerwise_qk_norm_amd import inputs
from oracle import compare, oracle

DEV = "cuda:0"

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def to_dev(a: np.ndarray) -> torch.Tensor:
    return inputs.to_device(a, DEV, torch)


def to_host(t: torch.Tensor) -> np.ndarray:
    return inputs.from_device(t)


def dtype_name(a) -> str:
    if isinstance(a, torch.Tensor):
        return "bf16" if a.dtype == torch.bfloat16 else "f32"
    return "bf16" if a.dtype == np.uint16 else "f32"


def oracle_report(x: np.ndarray, gamma: np.ndarray, out: np.ndarray, eps: float,
                  chunk: int = 4096, threads: int = 8) -> dict:
    """Elementwise comparison of a device output with the fp64 oracle, by row chunks."""
    worst = {"max_rel": 0.0, "max_abs": 0.0, "sum_abs": 0.0, "sum_sq": 0.0, "n": 0}
    for lo in range(0, x.shape[0], chunk):
        hi = min(x.shape[0], lo + chunk)
        y, _, _ = oracle.rmsnorm(x[lo:hi], gamma, eps, threads=threads)
        got = compare.decode_out(out[lo:hi])
        r = compare.report(got, y)
        worst["max_rel"] = max(worst["max_rel"], r["max_rel"])
        worst["max_abs"] = max(worst["max_abs"], r["max_abs"])
        d = np.abs(got - y)
        worst["sum_abs"] += float(d.sum())
        worst["sum_sq"] += float((d * d).sum())
        worst["n"] += r["n"]
    n = max(1, worst["n"])
    return {"max_rel": worst["max_rel"], "max_abs": worst["max_abs"],
            "mean_abs": worst["sum_abs"] / n, "rmse": (worst["sum_sq"] / n) ** 0.5, "n": worst["n"]}


def assert_parity(x, gamma, out, eps, what=""):
    dt = dtype_name(x)
    r = oracle_report(x, gamma, out, eps)
    tol = compare.TOL[dt]
    assert r["max_rel"] <= tol, f"{what}: max rel err {r['max_rel']:.3e} > {tol} ({r})"
    return r


def run_fused(d: dict, n_shards: int, eps: float):
    q, k = to_dev(d["q"]), to_dev(d["k"])
    gq, gk = to_dev(d["gamma_q"]), to_dev(d["gamma_k"])
    from layerwise_qk_norm_amd import ops
    oq, ok = ops.layerwise_fwd(q, k, gq, gk, n_shards, eps)
    torch.cuda.synchronize()
    return to_host(oq), to_host(ok)


def run_split(x: np.ndarray, gamma: np.ndarray, n_shards: int, eps: float):
    from layerwise_qk_norm_amd import ops
    xd, gd = to_dev(x), to_dev(gamma)
    p = ops.shard_sumsq(xd, n_shards)
    r = ops.combine_scale(p, x.shape[1], eps)
    y = ops.apply_scale(xd, gd, r)
    torch.cuda.synchronize()
    return to_host(p), to_host(r), to_host(y)
