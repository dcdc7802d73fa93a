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
    """"bf16", "f32" or "e4m3" of a torch tensor or of its host array."""
    if isinstance(a, torch.Tensor):
        return {torch.bfloat16: "bf16", torch.float32: "f32", torch.float8_e4m3fn: "e4m3"}[a.dtype]
    return {np.dtype(np.uint16): "bf16", np.dtype(np.float32): "f32",
            np.dtype(np.uint8): "e4m3"}[a.dtype]


def rows_of(t: torch.Tensor, idx: torch.Tensor) -> torch.Tensor:
    """t[idx] for any dtype (E4M3 rows are gathered as bytes)."""
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).index_select(0, idx).view(torch.float8_e4m3fn)
    return t.index_select(0, idx)


def oracle_report(x: np.ndarray, gamma: np.ndarray, out: np.ndarray, eps: float,
                  chunk: int = 4096, threads: int = 8) -> dict:
    """Elementwise comparison of a device output with the fp64 oracle, by row chunks.
    For E4M3 outputs ``rejected`` counts codes that are not the rounding of the
    exact value (nor, within 1e-5 of a tie, its other neighbour)."""
    worst = {"max_rel": 0.0, "max_abs": 0.0, "sum_abs": 0.0, "sum_sq": 0.0, "n": 0,
             "rejected": 0}
    for lo in range(0, x.shape[0], chunk):
        hi = min(x.shape[0], lo + chunk)
        y, _, _ = oracle.rmsnorm(x[lo:hi], gamma, eps, threads=threads)
        got = compare.decode_out(out[lo:hi])
        if out.dtype == np.uint8:
            worst["rejected"] += int(np.count_nonzero(~compare.e4m3_accepts(out[lo:hi], y)))
        r = compare.report(got, y)
        worst["max_rel"] = compare.fold_max(worst["max_rel"], r["max_rel"])
        worst["max_abs"] = compare.fold_max(worst["max_abs"], r["max_abs"])
        d = compare.abs_diff(got, y)
        worst["sum_abs"] += float(d.sum())
        worst["sum_sq"] += float((d * d).sum())
        worst["n"] += r["n"]
    n = max(1, worst["n"])
    return {"max_rel": worst["max_rel"], "max_abs": worst["max_abs"],
            "mean_abs": worst["sum_abs"] / n, "rmse": (worst["sum_sq"] / n) ** 0.5, "n": worst["n"],
            "rejected": worst["rejected"]}


def assert_parity(x, gamma, out, eps, what=""):
    """The bar of the output's format: relative error for bf16 and fp32, the
    rounding of the exact value for E4M3."""
    r = oracle_report(x, gamma, out, eps)
    kind = dtype_name(out)
    if kind == "e4m3":
        assert r["rejected"] == 0, f"{what}: {r['rejected']} E4M3 codes are not the rounding ({r})"
    else:
        tol = compare.TOL[kind]
        assert r["max_rel"] <= tol, f"{what}: max rel err {r['max_rel']:.3e} > {tol} ({r})"
    return r


TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32, "e4m3": torch.float8_e4m3fn}


def run_fused(d: dict, n_shards: int, eps: float, out: str = ""):
    """Fused call on host arrays; ``out`` names the output dtype of E4M3 inputs."""
    q, k = to_dev(d["q"]), to_dev(d["k"])
    gq, gk = to_dev(d["gamma_q"]), to_dev(d["gamma_k"])
    from layerwise_qk_norm_amd import ops
    oq, ok = ops.layerwise_fwd(q, k, gq, gk, n_shards, eps,
                               out_dtype=TORCH_DTYPE[out] if out else None)
    torch.cuda.synchronize()
    return to_host(oq), to_host(ok)


def run_split(x: np.ndarray, gamma: np.ndarray, n_shards: int, eps: float, out: str = ""):
    from layerwise_qk_norm_amd import ops
    xd, gd = to_dev(x), to_dev(gamma)
    p = ops.shard_sumsq(xd, n_shards)
    r = ops.combine_scale(p, x.shape[1], eps)
    y = ops.apply_scale(xd, gd, r, out_dtype=TORCH_DTYPE[out] if out else None)
    torch.cuda.synchronize()
    return to_host(p), to_host(r), to_host(y)


def layernorm_report(x, gamma, beta, out, eps, chunk: int = 4096, threads: int = 8) -> dict:
    """LayerNorm output against the fp64 oracle: the largest operand-scaled error
    (``compare.layernorm_scaled_error``) and, as context, max-abs and RMSE."""
    worst, sum_sq, n, max_abs = 0.0, 0.0, 0, 0.0
    for lo in range(0, x.shape[0], chunk):
        hi = min(x.shape[0], lo + chunk)
        y, mu, rs = oracle.layernorm(x[lo:hi], gamma, beta, eps, threads=threads)
        got = compare.decode_out(out[lo:hi])
        err = compare.layernorm_scaled_error(got, y, compare.decode_out(x[lo:hi]), mu, rs,
                                             compare.decode_out(gamma),
                                             None if beta is None else compare.decode_out(beta), eps)
        worst = compare.fold_max(worst, float(err.max()) if err.size else 0.0)
        d = compare.abs_diff(got, y)
        max_abs = compare.fold_max(max_abs, float(d.max()) if d.size else 0.0)
        sum_sq += float((d * d).sum())
        n += d.size
    return {"max_scaled": worst, "max_abs": max_abs, "rmse": (sum_sq / max(n, 1)) ** 0.5, "n": n}


def assert_layernorm_parity(x, gamma, beta, out, eps, what=""):
    r = layernorm_report(x, gamma, beta, out, eps)
    tol = compare.TOL[dtype_name(out)]
    assert r["max_scaled"] <= tol, f"{what}: max scaled err {r['max_scaled']:.3e} > {tol} ({r})"
    return r
