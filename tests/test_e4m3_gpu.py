"""FP8-E4M3 activations on the HIP path against the fp64 oracle (GPU).

The letter evaluates FP8-E4M3 activations next to BF16, accumulating in FP32
("SwiftQK ...", Section IV-C). Here q and k are OCP E4M3 codes, gamma is bf16,
and outputs are bf16 (8e-3 relative bar) or E4M3 (each code must be the
rounding of the exact value; within 1e-5 of a tie either neighbour).

* the converters: every one of the 256 codes decoded, and every rounding case
  (all codes, every tie, saturation, infinities, NaN) encoded, through both
  the 128-bit and the scalar paths of the split kernel;
* the fused path on the E4M3 workloads (reduced and full size, both output
  formats), the split path, exact partials on a dyadic grid, the E4M3 sweep
  (160 points at full size) and edge cases.
"""
import zlib

import numpy as np
import pytest
import torch

from layerwise_qk_norm_amd import inputs, ops
from oracle import compare, oracle

from _gpu import (assert_parity, device_rms_check, group_tile_rows, needs_gpu, rows_of, run_fused,
                  run_split, to_dev, to_host)

pytestmark = [pytest.mark.gpu, needs_gpu]

E4 = torch.float8_e4m3fn
ALL = np.arange(256, dtype=np.uint8)


def bf16(a):
    return inputs.f32_to_bf16_bits(np.asarray(a, np.float32))


@pytest.mark.parametrize("H", [256, 255])  # 128-bit path, scalar path
def test_every_code_decodes_exactly(H):
    """gamma = 1 and rms_inv = 1: the bf16 output is the code's value (exact in bf16)."""
    T = 3
    codes = np.resize(ALL, (T, H)).copy()
    x = to_dev(codes)
    g = to_dev(bf16(np.ones(H)))
    r = torch.ones(T, dtype=torch.float32, device="cuda:0")
    y = to_host(ops.apply_scale(x, g, r, out_dtype=torch.bfloat16))
    got = compare.decode_out(y)
    want = oracle.decode_e4m3(codes)
    assert np.array_equal(got, want, equal_nan=True)
    assert np.array_equal(np.signbit(got[~np.isnan(want)]), np.signbit(want[~np.isnan(want)]))


def _rounding_cases():
    v = oracle.decode_e4m3(ALL)
    vals = np.sort(v[~np.isnan(v) & (v >= 0)])
    mids = (vals[1:] + vals[:-1]) / 2  # every tie: 5 significant bits, exact in bf16
    near = np.concatenate([mids * (1 + 2.0 ** -7), mids * (1 - 2.0 ** -7)])
    special = [449.0, 464.0, 480.0, 500.0, 1e4, np.inf, np.nan, 2.0 ** -11, 0.0]
    a = np.concatenate([vals, mids, near, special])
    a = np.concatenate([a, -a])
    g = bf16(a)  # every case is exact in bf16 except `near`, whose bf16 value is tested
    return g


@pytest.mark.parametrize("H", [None, "scalar"])
def test_every_rounding_case_encodes_to_nearest_even(H):
    """x = 1 (code 0x38), rms_inv = 1: y = gamma exactly in fp32, so the E4M3 output
    must be exactly the round-to-nearest-even code, saturated at +-448."""
    g = _rounding_cases()
    n = g.size if H is None else g.size - (g.size % 16) - 1  # odd width: scalar path
    g = g[:n]
    x = to_dev(np.full((2, n), 0x38, np.uint8))
    r = torch.ones(2, dtype=torch.float32, device="cuda:0")
    y = to_host(ops.apply_scale(x, to_dev(g), r, out_dtype=E4))
    want = oracle.decode_e4m3(compare.e4m3_rne(compare.decode_out(g)))
    for row in y:
        got = oracle.decode_e4m3(row)  # values: -0 and +0 compare equal
        bad = np.nonzero(~((got == want) | (np.isnan(got) & np.isnan(want))))[0]
        assert bad.size == 0, (bad[:8], compare.decode_out(g)[bad[:8]], got[bad[:8]], want[bad[:8]])


REDUCED = {"tiny_e4m3": 8, "decode_e4m3": 64, "prefill_e4m3": 389, "gqa_e4m3": 1001}


@pytest.mark.parametrize("out", ["bf16", "e4m3"])
@pytest.mark.parametrize("name", list(REDUCED))
def test_fused_reduced(name, out):
    w = inputs.E4M3_CONFIGS[name].with_T(REDUCED[name])
    d = inputs.make_host(w)
    oq, ok = run_fused(d, w.n_shards, w.eps, out)
    rq = assert_parity(d["q"], d["gamma_q"], oq, w.eps, f"{name} q -> {out}")
    rk = assert_parity(d["k"], d["gamma_k"], ok, w.eps, f"{name} k -> {out}")
    print(name, out, "q", rq, "k", rk)


@pytest.mark.parametrize("name", ["decode_e4m3", "prefill_e4m3", "gqa_e4m3"])
def test_fused_full_size_all_rows(name):
    w = inputs.E4M3_CONFIGS[name]
    d = inputs.make_host(w)
    oq, ok = run_fused(d, w.n_shards, w.eps, w.out)
    rq = assert_parity(d["q"], d["gamma_q"], oq, w.eps, f"{name} q")
    rk = assert_parity(d["k"], d["gamma_k"], ok, w.eps, f"{name} k")
    print(name, "q", rq, "k", rk)


def test_gqa_e4m3_outputs_full_size():
    """The GQA workload at full size (8192 tokens, the measured launch for its
    shards) with E4M3 outputs, every row against the oracle."""
    w = inputs.E4M3_CONFIGS["gqa_e4m3"]
    d = inputs.make_host(w)
    oq, ok = run_fused(d, w.n_shards, w.eps, "e4m3")
    assert_parity(d["q"], d["gamma_q"], oq, w.eps, "gqa q -> e4m3")
    assert_parity(d["k"], d["gamma_k"], ok, w.eps, "gqa k -> e4m3")
    assert ops.check_fault() == ops.QKN_OK


@pytest.mark.parametrize("out", ["bf16", "e4m3"])
@pytest.mark.parametrize("name", list(REDUCED))
def test_split_reduced(name, out):
    w = inputs.E4M3_CONFIGS[name].with_T(REDUCED[name])
    d = inputs.make_host(w)
    for t in ("q", "k"):
        x, g = d[t], d["gamma_" + t]
        p, r, y = run_split(x, g, w.n_shards, w.eps, out)
        pe = oracle.shard_sumsq(x, w.n_shards)
        _, _, re_ = oracle.rmsnorm(x, g, w.eps, want_y=False)
        assert compare.report(p, pe)["max_rel"] <= compare.TOL_STAT
        assert compare.report(r, re_)["max_rel"] <= compare.TOL_STAT
        assert_parity(x, g, y, w.eps, f"{name} {t} split -> {out}")


@pytest.mark.parametrize("N", [1, 2, 4, 8])
def test_dyadic_partials_bitwise_and_fused_equals_split(N):
    """Values k/8 with |k| <= 16 are E4M3 codes whose squares and sums are exact in
    fp32: the device partials equal the oracle's bit for bit, and the fused
    outputs equal the split path's (same fp32 factor, same rounding)."""
    rng = np.random.default_rng(N)
    T, H = 37, 1024
    vals = rng.integers(-16, 17, (2, T, H)) / 8.0
    q8, k8 = compare.e4m3_rne(vals[0]), compare.e4m3_rne(vals[1])
    assert np.array_equal(oracle.decode_e4m3(q8), vals[0])
    g = bf16(rng.uniform(0.5, 1.5, H))
    p = to_host(ops.shard_sumsq(to_dev(q8), N))
    assert np.array_equal(p.astype(np.float64), oracle.shard_sumsq(q8, N))
    for out in ("bf16", "e4m3"):
        fq, fk = run_fused({"q": q8, "k": k8, "gamma_q": g, "gamma_k": g}, N, 1e-6, out)
        _, _, sq = run_split(q8, g, N, 1e-6, out)
        _, _, sk = run_split(k8, g, N, 1e-6, out)
        assert np.array_equal(fq, sq) and np.array_equal(fk, sk), out


SWEEP = list(inputs.sweep_e4m3())


def _unit_rms(x, g, y, eps, tol):
    gd = g.double()
    for lo in range(0, x.shape[0], 4096):
        xs, ys = x[lo:lo + 4096].double(), y[lo:lo + 4096].double()
        m = (xs * xs).mean(dim=1)
        want = m / (m + float(np.float32(eps)))
        got = ((ys / gd) ** 2).mean(dim=1)
        err = ((got - want).abs() / want).max().item()
        assert err <= tol, f"unit-RMS property off by {err:.3e}"


@pytest.mark.parametrize("w", SWEEP, ids=[w.name for w in SWEEP])
def test_sweep_full_size(w):
    torch.cuda.empty_cache()
    q = inputs.make_device_activations(w, "q", "cuda:0", torch)
    k = inputs.make_device_activations(w, "k", "cuda:0", torch)
    hd = inputs.make_host(w.with_T(1))
    gq, gk = to_dev(hd["gamma_q"]), to_dev(hd["gamma_k"])
    odt = torch.bfloat16 if w.out == "bf16" else E4
    oq, ok = ops.layerwise_fwd(q, k, gq, gk, w.n_shards, w.eps, out_dtype=odt)
    assert ops.check_fault() == ops.QKN_OK
    rows = np.unique(np.concatenate([[0, 1, w.T // 2, w.T - 1],
                                     np.random.default_rng(zlib.crc32(w.name.encode()))
                                     .integers(0, w.T, 40)]))
    # plus every row of the first and last tile of every group of the launch made
    plan_q, plan_k = group_tile_rows(w.fmt, w.T, w.Hq, w.Hk, w.n_shards)
    for x, g, y, gh, pr in ((q, gq, oq, hd["gamma_q"], plan_q), (k, gk, ok, hd["gamma_k"], plan_k)):
        idx = torch.as_tensor(np.union1d(rows, pr), device="cuda:0")
        assert_parity(to_host(rows_of(x, idx)), gh, to_host(rows_of(y, idx)), w.eps, w.name)
        if w.out == "bf16":
            # every element of every row against a plain fp64 reference on the device
            device_rms_check(x, g, y, w.eps, compare.TOL["bf16"], w.name)
        else:
            # E4M3 outputs are checked by code, on the rows above. An E4M3 output lies
            # within a factor (1 +- 2^-4) of the exact value (normal range), so a mean
            # of squares moves by at most (1 + 2^-4)^2 - 1 = 0.129 (reached by
            # heavy-tailed rows that a few large values dominate); subnormal outputs
            # add at most 2^-12 each against a mean square near 1.
            _unit_rms(x, g, y, w.eps, 0.13)
    del q, k, oq, ok


@pytest.mark.parametrize("T", [1, 5, 63, 65, 4097])
def test_ragged_token_counts(T):
    w = inputs.PREFILL_E4M3.with_T(T)
    d = inputs.make_host(w)
    for out in ("bf16", "e4m3"):
        oq, ok = run_fused(d, w.n_shards, w.eps, out)
        assert_parity(d["q"], d["gamma_q"], oq, w.eps, f"T={T} {out}")
        assert_parity(d["k"], d["gamma_k"], ok, w.eps, f"T={T} {out}")


@pytest.mark.parametrize("N,H", [(1, 4096), (3, 3072), (5, 5120), (16, 4096), (32, 4096),
                                 (4, 4100), (8, 1032)])
def test_shard_counts_and_split_fallback(N, H):
    """Shard widths that are whole 16-column vectors take the fused kernel; the
    others (4100/4, 1032/8) run the split kernels from the same entry point."""
    w = inputs.Workload("e4m3_shards", 70, H, H, N, "e4m3", out_dtype="e4m3")
    d = inputs.make_host(w)
    fused = (H // N) % 16 == 0
    assert (ops.current_plan("e4m3_e4m3", 70, H, H, N)["variant"] >= 0) == fused
    for out in ("bf16", "e4m3"):
        oq, ok = run_fused(d, N, w.eps, out)
        assert_parity(d["q"], d["gamma_q"], oq, w.eps, f"N={N} H={H} {out}")
        assert_parity(d["k"], d["gamma_k"], ok, w.eps, f"N={N} H={H} {out}")


def test_in_place_e4m3_output():
    w = inputs.DECODE_E4M3.with_T(33)
    d = inputs.make_host(w)
    q, k = to_dev(d["q"]), to_dev(d["k"])
    gq, gk = to_dev(d["gamma_q"]), to_dev(d["gamma_k"])
    ops.layerwise_fwd(q, k, gq, gk, w.n_shards, w.eps, out_q=q, out_k=k)
    torch.cuda.synchronize()
    assert_parity(d["q"], d["gamma_q"], to_host(q), w.eps, "in place q")
    assert_parity(d["k"], d["gamma_k"], to_host(k), w.eps, "in place k")


def test_nan_codes_and_saturation():
    """A NaN code makes its row NaN; a large gamma saturates E4M3 outputs at 448."""
    T, H = 4, 256
    x = np.full((T, H), 0x38, np.uint8)  # 1.0
    x[1, 7] = 0x7F  # NaN
    g = bf16(np.full(H, 1.0))
    g16 = g.copy()
    g16[3] = bf16([1000.0])[0]
    for out in ("bf16", "e4m3"):
        oq, ok = run_fused({"q": x, "k": x, "gamma_q": g, "gamma_k": g16}, 2, 1e-6, out)
        vq = compare.decode_out(oq)
        assert np.all(np.isnan(vq[1])) and not np.any(np.isnan(vq[[0, 2, 3]]))
        vk = compare.decode_out(ok)
        if out == "e4m3":
            assert vk[0, 3] == 448.0  # 1000 * 1/sqrt(1 + eps) saturates
        assert_parity(x[[0]], g16, ok[[0]], 1e-6, f"saturation {out}")


@pytest.mark.parametrize("layout", [1, 2])
@pytest.mark.parametrize("T,H,N", [(64, 1024, 2), (37, 5120, 4), (300, 4096, 1), (129, 2560, 2),
                                   (1, 4096, 8), (4097, 2048, 8)])
def test_unsaturated_conversion_matches_saturating_split_path(T, H, N, layout):
    """The fused E4M3 -> E4M3 path converts without saturation in waves whose gammas
    keep sqrt(H)|gamma| under 448 (|x_j| * rms_inv <= sqrt(H) in every row). On a
    dyadic grid (exact sums) its codes must equal the split path's, which always
    saturates: rows that reach the bound (a single nonzero element, |y_j| close to
    sqrt(H)|gamma_j|) against gammas under the skip limit, just over it, far over
    448/sqrt(H) (those outputs saturate), NaN and infinite."""
    rng = np.random.default_rng(H + T + N)
    lim = 440.0 / (np.sqrt(H) * (1.0 + H * 1.2e-7))
    xs, gs = [], []
    for t_ in range(2):
        v = rng.integers(-16, 17, (T, H)) / 8.0
        for t in range(t_, T, 3):  # one row in three: one nonzero element
            v[t] = 0.0
            v[t, (t * 37 + 11 * t_) % H] = 2.0 if t % 2 else -2.0
        xs.append(compare.e4m3_rne(v))
        gv = rng.uniform(0.5, 0.98, H) * lim
        blk = np.array_split(rng.permutation(H) if t_ else np.arange(H), 5)
        gv[blk[1]] = 1.02 * lim
        gv[blk[2]] = -1.2 * 448 / np.sqrt(H)
        gv[blk[3][0]] = np.nan
        gv[blk[4][0]] = np.inf
        gs.append(bf16(gv))
    old = ops.get_option("tile_layout")
    try:
        ops.set_option("tile_layout", layout)
        oq, ok = run_fused({"q": xs[0], "k": xs[1], "gamma_q": gs[0], "gamma_k": gs[1]}, N, 1e-6, "e4m3")
    finally:
        ops.set_option("tile_layout", old)
    for x, g, o in ((xs[0], gs[0], oq), (xs[1], gs[1], ok)):
        _, _, ys = run_split(x, g, N, 1e-6, "e4m3")
        assert np.array_equal(o, ys), np.argwhere(o != ys)[:8]
    # the far-over block saturated where a row reached the bound
    big = np.array_split(np.arange(H), 5)[2]
    one_hot = [t for t in range(0, T, 3) if (t * 37) % H in big]
    for t in one_hot:
        assert oracle.decode_e4m3(oq[t, (t * 37) % H]) in (448.0, -448.0), t
    assert ops.check_fault() == ops.QKN_OK


def test_wrong_dtypes_are_rejected():
    q = torch.zeros((4, 64), dtype=E4, device="cuda:0")
    g = torch.ones(64, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(TypeError):
        ops.layerwise_fwd(q, q, g.float(), g.float(), 2)  # gamma must be bf16
    with pytest.raises(TypeError):
        ops.layerwise_fwd(q, q, g, g, 2, out_dtype=torch.float32)
    L = ops.lib()
    s = torch.cuda.current_stream().cuda_stream
    o = torch.empty((4, 64), dtype=torch.bfloat16, device="cuda:0")
    assert L.qknorm_layerwise_fwd_e4m3(q.data_ptr(), q.data_ptr(), g.data_ptr(), g.data_ptr(), 4,
                                       64, 64, 2, 1e-6, o.data_ptr(), o.data_ptr() + 128 * 2,
                                       ops.QKN_F32, s) == ops.QKN_EINVAL
