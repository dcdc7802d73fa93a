"""Seeded synthetic inputs for layerwise QK-Norm workloads.

This module only draws numbers: it holds none of the normalisation
arithmetic, imports neither the HIP binding nor the oracle, and serves both.

Recipe (stated once, used everywhere):

* Per-tensor streams come from ``numpy.random.SeedSequence(seed).spawn(8)`` in
  the order [q, k, gamma_q, gamma_k, outlier_q, outlier_k, beta_q, beta_k]
  (a child's stream does not depend on how many children are spawned).
* Activations: ``N(0, sigma^2)`` (``standard_normal * sigma``) or Student-t
  with 3 degrees of freedom; drawn in float64 row-major, in row chunks (the
  stream is consumed in C order, so the first T' rows of a T-row draw equal a
  T'-row draw).
* Outlier channels: a fixed set of ``max(1, round(p * H))`` columns per tensor,
  the first entries of a seeded permutation, shared by every token; those
  columns are multiplied by the outlier scale before rounding.
* gamma: ``U(0.5, 1.5)`` or ``N(1, 0.1^2)``, drawn in float64.
* LayerNorm workloads add beta ``U(-0.5, 0.5)`` in gamma's format, and may shift
  the activations by a constant ``mu`` (mean offset) before rounding.
* Headwise workloads draw gamma of length ``head_dim`` (one vector shared by
  every head).
* Storage: float64 -> float32 (round to nearest even), then for bf16
  float32 -> bf16 round to nearest even on the bit pattern. bf16 tensors are
  numpy ``uint16`` bit patterns. For E4M3 activations float32 -> E4M3 (OCP
  OFP8 E4M3: round to nearest even, magnitudes clipped to 448 first), stored
  as numpy ``uint8`` codes; gamma is then bf16. No input scale factor is
  applied: RMSNorm divides any common scale out (up to its effect on eps).

The shapes and distributions are the stand-in for the Q/K activations of the
models the letter evaluates ("SwiftQK ...", Section IV-A and the Q/K sizes of
Fig. 2(a)); no dataset values are used.
"""
from __future__ import annotations

import dataclasses
import itertools
from typing import Iterator

import numpy as np

EPS = 1e-6


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    Hq: int
    Hk: int
    n_shards: int
    dtype: str  # input format: "bf16", "f32" (gamma and outputs share it) or "e4m3"
    dist: str = "normal"  # "normal" or "t3"
    sigma: float = 1.0
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    gamma_dist: str = "uniform"  # "uniform" (0.5, 1.5) or "normal" (1, 0.1)
    eps: float = EPS
    seed: int = 0
    out_dtype: str = ""  # output format; "" = the input format (E4M3: "bf16" or "e4m3")
    norm: str = "rms"    # "rms" (RMSNorm), "layer" (LayerNorm with beta) or "head" (headwise)
    mu: float = 0.0      # constant added to every activation draw
    head_dim: int = 0    # headwise: columns per head (gamma is [head_dim], shared by heads)

    def with_T(self, T: int) -> "Workload":
        return dataclasses.replace(self, T=T)

    @property
    def out(self) -> str:
        return self.out_dtype or self.dtype

    @property
    def gamma_dtype(self) -> str:
        return "bf16" if self.dtype == "e4m3" else self.dtype

    @property
    def fmt(self) -> str:
        """Kernel format name: "bf16", "f32", "e4m3_bf16", "e4m3_e4m3", "ln_bf16" or "ln_f32"."""
        if self.norm == "layer":
            return f"ln_{self.dtype}"
        return f"e4m3_{self.out}" if self.dtype == "e4m3" else self.dtype

    @property
    def elem_bytes(self) -> int:
        """Bytes per input element."""
        return _BYTES[self.dtype]

    @property
    def out_bytes(self) -> int:
        return _BYTES[self.out]

    def algorithmic_bytes(self) -> int:
        """One read and one write of Q and K, plus gamma (and beta) of Q and K once."""
        per_col = self.elem_bytes + self.out_bytes
        params = 2 if self.norm == "layer" else 1
        cols = 2 * self.head_dim if self.norm == "head" else self.Hq + self.Hk
        return (self.T * (self.Hq + self.Hk) * per_col +
                params * cols * _BYTES[self.gamma_dtype])

    def outlier_count(self, H: int) -> int:
        if self.outlier_frac <= 0:
            return 0
        return max(1, int(round(self.outlier_frac * H)))


_BYTES = {"bf16": 2, "f32": 4, "e4m3": 1}

TINY = Workload("tiny", 8, 256, 256, 2, "f32", gamma_dist="normal")
DECODE = Workload("decode", 64, 4096, 4096, 4, "bf16", outlier_frac=0.01, outlier_scale=20.0)
PREFILL = Workload("prefill", 16384, 5120, 5120, 2, "bf16", sigma=2.0)
GQA = Workload("gqa", 8192, 5120, 1024, 4, "bf16", outlier_frac=0.005, outlier_scale=50.0)
CONFIGS = {w.name: w for w in (TINY, DECODE, PREFILL, GQA)}

# FP8-E4M3 activations (the letter's second precision, Section IV-C) at the same
# shapes: E4M3 in, bf16 gamma, bf16 or E4M3 out
TINY_E4M3 = Workload("tiny_e4m3", 8, 256, 256, 2, "e4m3", gamma_dist="normal", out_dtype="e4m3")
DECODE_E4M3 = Workload("decode_e4m3", 64, 4096, 4096, 4, "e4m3", outlier_frac=0.01,
                       outlier_scale=20.0, out_dtype="e4m3")
PREFILL_E4M3 = Workload("prefill_e4m3", 16384, 5120, 5120, 2, "e4m3", sigma=2.0, out_dtype="bf16")
GQA_E4M3 = Workload("gqa_e4m3", 8192, 5120, 1024, 4, "e4m3", outlier_frac=0.005,
                    outlier_scale=50.0, out_dtype="bf16")
E4M3_CONFIGS = {w.name: w for w in (TINY_E4M3, DECODE_E4M3, PREFILL_E4M3, GQA_E4M3)}

# LayerNorm with two additive shard statistics (reading notes, Section 5e) at the
# same shapes, plus rows with a non-zero mean
LN_TINY = Workload("ln_tiny", 8, 256, 256, 2, "f32", gamma_dist="normal", norm="layer")
LN_DECODE = Workload("ln_decode", 64, 4096, 4096, 4, "bf16", outlier_frac=0.01,
                     outlier_scale=20.0, norm="layer")
LN_PREFILL = Workload("ln_prefill", 16384, 5120, 5120, 2, "bf16", sigma=2.0, norm="layer")
LN_GQA = Workload("ln_gqa", 8192, 5120, 1024, 4, "bf16", outlier_frac=0.005, outlier_scale=50.0,
                  norm="layer")
LN_SHIFTED = Workload("ln_shifted", 1024, 4096, 4096, 4, "f32", mu=1.0, norm="layer")
LN_CONFIGS = {w.name: w for w in (LN_TINY, LN_DECODE, LN_PREFILL, LN_GQA, LN_SHIFTED)}

# headwise QK-Norm (one factor per head of 128 columns; letter, Section II-A) at the
# same Q/K widths: 40 heads (5120), 32 heads (4096), 8 KV heads (1024)
HW_TINY = Workload("hw_tiny", 8, 256, 256, 1, "f32", gamma_dist="normal", norm="head", head_dim=128)
HW_DECODE = Workload("hw_decode", 64, 4096, 4096, 1, "bf16", outlier_frac=0.01, outlier_scale=20.0,
                     norm="head", head_dim=128)
HW_PREFILL = Workload("hw_prefill", 16384, 5120, 5120, 1, "bf16", sigma=2.0, norm="head",
                      head_dim=128)
HW_GQA = Workload("hw_gqa", 8192, 5120, 1024, 1, "bf16", outlier_frac=0.005, outlier_scale=50.0,
                  norm="head", head_dim=128)
HW_CONFIGS = {w.name: w for w in (HW_TINY, HW_DECODE, HW_PREFILL, HW_GQA)}

SWEEP_T = (4096, 4097, 16384, 65536)
SWEEP_H = (1024, 3072, 5120, 8192, 16384)
SWEEP_N = (1, 2, 4, 8)
SWEEP_DTYPE = ("bf16", "f32")
SWEEP_DIST = ("normal", "t3")


def sweep() -> Iterator[Workload]:
    for T, H, N, dt, dist in itertools.product(SWEEP_T, SWEEP_H, SWEEP_N, SWEEP_DTYPE,
                                               SWEEP_DIST):
        yield Workload(f"sweep_T{T}_H{H}_N{N}_{dt}_{dist}", T, H, H, N, dt, dist=dist)


def sweep_layernorm() -> Iterator[Workload]:
    """LayerNorm over a reduced sweep grid: T in {4096, 16384}, H in {1024, 5120, 16384},
    N in {1, 2, 4, 8}, bf16 and fp32, normal draws (48 points)."""
    for T, H, N, dt in itertools.product((4096, 16384), (1024, 5120, 16384), SWEEP_N, SWEEP_DTYPE):
        yield Workload(f"ln_sweep_T{T}_H{H}_N{N}_{dt}", T, H, H, N, dt, norm="layer")


def sweep_headwise() -> Iterator[Workload]:
    """Headwise RMSNorm: T in {4097, 16384}, H in {2048, 5120, 16384}, head_dim in
    {64, 128, 256}, bf16 and fp32, normal draws (36 points)."""
    for T, H, D, dt in itertools.product((4097, 16384), (2048, 5120, 16384), (64, 128, 256),
                                         SWEEP_DTYPE):
        yield Workload(f"hw_sweep_T{T}_H{H}_D{D}_{dt}", T, H, H, 1, dt, norm="head", head_dim=D)


def sweep_e4m3() -> Iterator[Workload]:
    """The sweep grid with E4M3 activations: bf16 outputs for the normal draws,
    E4M3 outputs for the Student-t draws (160 points)."""
    for T, H, N, dist in itertools.product(SWEEP_T, SWEEP_H, SWEEP_N, SWEEP_DIST):
        out = "bf16" if dist == "normal" else "e4m3"
        yield Workload(f"sweep_T{T}_H{H}_N{N}_e4m3_{out}_{dist}", T, H, H, N, "e4m3", dist=dist,
                       out_dtype=out)


# ---------------------------------------------------------------- rounding

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even; NaN -> 0x7FC0."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0) | (((u[nan] >> 16) & np.uint32(0x8000)).astype(np.uint16))
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


E4M3_MAX = 448.0


def f32_to_e4m3_codes(a: np.ndarray) -> np.ndarray:
    """float32 -> E4M3 codes (uint8): clip to +-448, then PyTorch's float8_e4m3fn
    conversion (round to nearest even)."""
    import torch
    a = np.clip(np.ascontiguousarray(a, dtype=np.float32), -E4M3_MAX, E4M3_MAX)
    return torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def store(a64: np.ndarray, dtype: str) -> np.ndarray:
    f32 = a64.astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(f32)
    if dtype == "e4m3":
        return f32_to_e4m3_codes(f32)
    return f32


# ---------------------------------------------------------------- host draws

def _streams(seed: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(8)]


_NP = {"bf16": np.uint16, "f32": np.float32, "e4m3": np.uint8}


def _activations(rng, T, H, w: Workload, outlier_cols, chunk_rows: int) -> np.ndarray:
    out = np.empty((T, H), _NP[w.dtype])
    for lo in range(0, T, chunk_rows):
        hi = min(T, lo + chunk_rows)
        if w.dist == "normal":
            a = rng.standard_normal((hi - lo, H)) * w.sigma
        elif w.dist == "t3":
            a = rng.standard_t(3, (hi - lo, H)) * w.sigma
        else:
            raise ValueError(w.dist)
        if outlier_cols is not None:
            a[:, outlier_cols] *= w.outlier_scale
        if w.mu:
            a += w.mu
        out[lo:hi] = store(a, w.dtype)
    return out


def _beta(rng, H, w: Workload) -> np.ndarray:
    return store(rng.uniform(-0.5, 0.5, H), w.gamma_dtype)


def _gamma(rng, H, w: Workload) -> np.ndarray:
    if w.gamma_dist == "uniform":
        g = rng.uniform(0.5, 1.5, H)
    elif w.gamma_dist == "normal":
        g = rng.normal(1.0, 0.1, H)
    else:
        raise ValueError(w.gamma_dist)
    return store(g, w.gamma_dtype)


def outlier_columns(w: Workload, which: str):
    """The outlier column indices of tensor ``which`` ("q" or "k"), or None."""
    H = w.Hq if which == "q" else w.Hk
    n = w.outlier_count(H)
    if n == 0:
        return None
    rng = _streams(w.seed)[4 if which == "q" else 5]
    return np.sort(rng.permutation(H)[:n])


def make_host(w: Workload, chunk_rows: int = 2048) -> dict:
    """Host arrays ``q, k, gamma_q, gamma_k`` (and ``beta_q, beta_k`` for LayerNorm)."""
    rq, rk, rgq, rgk, _, _, rbq, rbk = _streams(w.seed)
    gq_len = w.head_dim if w.norm == "head" else w.Hq
    gk_len = w.head_dim if w.norm == "head" else w.Hk
    d = {
        "q": _activations(rq, w.T, w.Hq, w, outlier_columns(w, "q"), chunk_rows),
        "k": _activations(rk, w.T, w.Hk, w, outlier_columns(w, "k"), chunk_rows),
        "gamma_q": _gamma(rgq, gq_len, w),
        "gamma_k": _gamma(rgk, gk_len, w),
    }
    if w.norm == "layer":
        d["beta_q"] = _beta(rbq, w.Hq, w)
        d["beta_k"] = _beta(rbk, w.Hk, w)
    return d


# ---------------------------------------------------------------- device draws

def make_device_activations(w: Workload, which: str, device, torch):
    """Device-side draw of one activation tensor with torch's seeded generator.

    Used only where a host draw would dominate a test's run time (the
    largest sweep points). Same distribution as the host draw, different
    values; the oracle then reads back exactly the rows it checks.
    Returns a torch tensor of dtype bfloat16, float32 or float8_e4m3fn on ``device``.
    """
    H = w.Hq if which == "q" else w.Hk
    seed = int(np.random.SeedSequence(w.seed).spawn(6)[0 if which == "q" else 1]
               .generate_state(1)[0])
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out_dtype = {"bf16": torch.bfloat16, "f32": torch.float32,
                 "e4m3": torch.float8_e4m3fn}[w.dtype]
    out = torch.empty((w.T, H), dtype=out_dtype, device=device)
    rows = max(1, (1 << 26) // H)
    for lo in range(0, w.T, rows):
        hi = min(w.T, lo + rows)
        a = torch.randn((hi - lo, H), generator=g, device=device, dtype=torch.float32)
        if w.dist == "t3":
            chi = sum(torch.randn((hi - lo, H), generator=g, device=device,
                                  dtype=torch.float32) ** 2 for _ in range(3))
            a = a / torch.sqrt(chi / 3.0)
        a = a * w.sigma
        cols = outlier_columns(w, which)
        if cols is not None:
            a[:, torch.as_tensor(cols, device=device)] *= w.outlier_scale
        if w.mu:
            a = a + w.mu
        if w.dtype == "e4m3":
            a = a.clamp(-E4M3_MAX, E4M3_MAX)
        out[lo:hi] = a.to(out_dtype)
    return out


# ---------------------------------------------------------------- transfers

def to_device(a: np.ndarray, device, torch):
    """numpy bf16 bit patterns (uint16), float32 or E4M3 codes (uint8) -> torch
    tensor (bfloat16, float32, float8_e4m3fn) on ``device``."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to(device)
    if a.dtype == np.uint8:
        return torch.from_numpy(a).to(device).view(torch.float8_e4m3fn)
    raise TypeError(a.dtype)


def from_device(t) -> np.ndarray:
    """torch tensor -> numpy bf16 bit patterns (uint16), float32 or E4M3 codes (uint8)."""
    import torch
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()
