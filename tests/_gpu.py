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


# ---------------------------------------------------------------- launch coverage

_FMT_BYTES = {"bf16": (2, 2), "f32": (4, 4), "e4m3_bf16": (1, 2), "e4m3_e4m3": (1, 1),
              "ln_bf16": (2, 2), "ln_f32": (4, 4)}


def launched_plans(fmt: str, T: int, Hq: int, Hk: int, n_shards: int):
    """[(first token, plan)] of the fused launches one call makes: the host runs
    tensors that reach 2^31 - 2^16 bytes as consecutive launches over token
    ranges (the buffer descriptors take 32-bit offsets), each planned on its own."""
    from layerwise_qk_norm_amd import ops
    e_in, e_out = _FMT_BYTES[fmt]
    tmax = ((1 << 31) - (1 << 16)) // (max(Hq, Hk) * max(e_in, e_out))
    out = []
    for t0 in range(0, T, tmax):
        tc = min(tmax, T - t0)
        out.append((t0, ops.current_plan(fmt, tc, Hq, Hk, n_shards)))
    return out


def group_tile_rows(fmt: str, T: int, Hq: int, Hk: int, n_shards: int):
    """Token rows of Q and of K (two sorted arrays) held by the first and the last
    tile of every workgroup group of the launches a call makes, plus, with
    single-tensor tiles, the last Q tile and the first K tile. Group g walks
    tiles g, g + n_groups, ... (the stride loop), so checking these rows element
    by element compares every group's work with the oracle."""
    rq, rk = [], []
    for t0, pl in launched_plans(fmt, T, Hq, Hk, n_shards):
        if pl["variant"] < 0:
            continue
        tc = min(T - t0, ((1 << 31) - (1 << 16)) // (max(Hq, Hk) * max(_FMT_BYTES[fmt])))
        G, n, r, st = pl["n_groups"], pl["n_tiles"], pl["rows"], pl["st"]
        g = np.arange(min(G, n))
        tiles = np.concatenate([g, g + ((n - 1 - g) // G) * G])
        nq = (tc + r - 1) // r if st else n
        if st:
            tiles = np.concatenate([tiles, [nq - 1, nq]])
        tiles = np.unique(tiles[(tiles >= 0) & (tiles < n)])
        for t in tiles:
            if st and t >= nq:
                lo = (t - nq) * r
                rk.append(np.arange(t0 + lo, t0 + min(tc, lo + r)))
            else:
                lo = t * r
                rows = np.arange(t0 + lo, t0 + min(tc, lo + r))
                rq.append(rows)
                if not st:
                    rk.append(rows)
    cat = lambda a: np.unique(np.concatenate(a)) if a else np.zeros(0, np.int64)
    return cat(rq), cat(rk)


# ---------------------------------------------------------------- every row, fp64 on the device

def _rel_err_dev(got, ref):
    """Elementwise relative error on the device with the oracle checker's rules: an
    exact zero must be a zero, and NaN anywhere it is not matched is infinite."""
    err = (got - ref).abs() / ref.abs()
    err = torch.where(ref == 0, torch.where(got == 0, 0.0, float("inf")), err)
    same_nan = torch.isnan(got) & torch.isnan(ref)
    err = torch.where(same_nan, 0.0, torch.nan_to_num(err, nan=float("inf")))
    return err


def device_rms_check(x, g, y, eps: float, tol: float, what: str = ""):
    """Every element of every row against x * gamma / sqrt(mean(x^2) + eps) computed in
    fp64 by PyTorch on the device (a plain reference beside the oracle, which checks
    the sampled rows): max relative error <= tol."""
    e = float(np.float32(eps))
    gd = g.double()
    rows = max(1, (1 << 24) // x.shape[1])
    worst = 0.0
    for lo in range(0, x.shape[0], rows):
        xs = x[lo:lo + rows].double()
        ref = xs * gd * torch.rsqrt((xs * xs).mean(dim=1, keepdim=True) + e)
        worst = compare.fold_max(worst, _rel_err_dev(y[lo:lo + rows].double(), ref).max().item())
    assert worst <= tol, f"{what}: every-row fp64 check, max rel err {worst:.3e} > {tol}"
    return worst


def device_headwise_check(x, g, y, D: int, eps: float, tol: float, what: str = ""):
    """device_rms_check per head of D columns (gamma [D] shared by the heads)."""
    e = float(np.float32(eps))
    gd = g.double()
    rows = max(1, (1 << 24) // x.shape[1])
    worst = 0.0
    for lo in range(0, x.shape[0], rows):
        xs = x[lo:lo + rows].double().reshape(-1, D)
        ref = xs * gd * torch.rsqrt((xs * xs).mean(dim=1, keepdim=True) + e)
        got = y[lo:lo + rows].double().reshape(-1, D)
        worst = compare.fold_max(worst, _rel_err_dev(got, ref).max().item())
    assert worst <= tol, f"{what}: every-row fp64 check, max rel err {worst:.3e} > {tol}"
    return worst


def device_layernorm_check(x, g, b, y, eps: float, tol: float, what: str = ""):
    """Every element against (x - mean) / sqrt(var + eps) * gamma + beta in fp64 on the
    device (two-pass variance), the error taken against the operand scale
    rstd * |gamma| * (|x| + |mean| + sigma) + |beta| as the oracle's LayerNorm check."""
    e = float(np.float32(eps))
    gd, bd = g.double(), (torch.zeros_like(g, dtype=torch.float64) if b is None else b.double())
    rows = max(1, (1 << 24) // x.shape[1])
    worst = 0.0
    for lo in range(0, x.shape[0], rows):
        xs = x[lo:lo + rows].double()
        mu = xs.mean(dim=1, keepdim=True)
        var = ((xs - mu) ** 2).mean(dim=1, keepdim=True)
        rstd = torch.rsqrt(var + e)
        ref = (xs - mu) * rstd * gd + bd
        scale = rstd * gd.abs() * (xs.abs() + mu.abs() + var.sqrt()) + bd.abs()
        d = (y[lo:lo + rows].double() - ref).abs()
        err = torch.nan_to_num(torch.where(d == 0, 0.0, d / scale), nan=float("inf"))
        worst = compare.fold_max(worst, err.max().item())
    assert worst <= tol, f"{what}: every-row fp64 check, max scaled err {worst:.3e} > {tol}"
    return worst
