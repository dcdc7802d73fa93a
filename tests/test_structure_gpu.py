"""Bit-exact partition checks and structural invariants of the HIP path (GPU).

* Dyadic inputs (values m/8, |m| <= 16) make every square and every partial
  sum exact in fp32, so the split path's partials must equal the oracle's
  bitwise, and the fused path (same exact partials, same ascending combine,
  same scaling) must equal the split path bitwise.
* Column-coded inputs: token t is nonzero only in shard t % N. Exactly one
  partial per token is nonzero, at shard t % N; the fused output is nonzero
  exactly where the input is.
* Determinism, independence of Q from K, token-permutation equivariance and
  power-of-two scale invariance at eps = 0.
"""
import numpy as np
import pytest
import torch

from layerwise_qk_norm_amd import inputs, ops
from oracle import oracle

from _gpu import assert_layernorm_parity, assert_parity, needs_gpu, run_fused, run_split, to_dev, to_host

pytestmark = [pytest.mark.gpu, needs_gpu]

SHAPES = [(64, 4096, 4096), (300, 5120, 5120), (129, 5120, 1024), (77, 1024, 1024)]


def dyadic(T, H, dtype, seed):
    rng = np.random.default_rng(seed)
    a = (rng.integers(-16, 17, (T, H)) / 8.0).astype(np.float32)
    return inputs.f32_to_bf16_bits(a) if dtype == "bf16" else a


def gamma_of(H, dtype, seed=1):
    g = np.random.default_rng(seed).uniform(0.5, 1.5, H)
    return inputs.store(g, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N", [1, 2, 4, 8])
def test_split_partials_bitwise_on_dyadic_grid(dtype, N):
    for T, Hq, _ in SHAPES:
        x = dyadic(T, Hq, dtype, T)
        p, _, _ = run_split(x, gamma_of(Hq, dtype), N, 1e-6)
        pe = oracle.shard_sumsq(x, N)
        assert np.array_equal(p.astype(np.float64), pe), (T, Hq, N)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N", [1, 2, 4, 8])
def test_fused_equals_split_bitwise_on_dyadic_grid(dtype, N):
    for T, Hq, Hk in SHAPES:
        q, k = dyadic(T, Hq, dtype, 2 * T), dyadic(T, Hk, dtype, 2 * T + 1)
        gq, gk = gamma_of(Hq, dtype, 3), gamma_of(Hk, dtype, 4)
        oq, ok = ops.layerwise_fwd(to_dev(q), to_dev(k), to_dev(gq), to_dev(gk), N, 1e-6)
        _, _, yq = run_split(q, gq, N, 1e-6)
        _, _, yk = run_split(k, gk, N, 1e-6)
        assert np.array_equal(to_host(oq), yq), (T, Hq, N)
        assert np.array_equal(to_host(ok), yk), (T, Hk, N)
        assert_parity(q, gq, to_host(oq), 1e-6)


@pytest.mark.parametrize("N", [2, 4, 8])
def test_column_coded_partition(N):
    T, Hq, Hk = 96, 4096, 1024
    rng = np.random.default_rng(N)
    q = np.zeros((T, Hq), np.float32)
    k = np.zeros((T, Hk), np.float32)
    for t in range(T):
        s = t % N
        Wq, Wk = Hq // N, Hk // N
        q[t, s * Wq:(s + 1) * Wq] = (1 + (np.arange(Wq) % 7)) / 8.0 * (1 + t % 3)
        k[t, s * Wk:(s + 1) * Wk] = (1 + (np.arange(Wk) % 5)) / 4.0
    for dtype in ("bf16", "f32"):
        qd, kd = inputs.store(q.astype(np.float64), dtype), inputs.store(k.astype(np.float64), dtype)
        p, _, _ = run_split(qd, gamma_of(Hq, dtype), N, 1e-6)
        nz = p != 0
        assert np.array_equal(nz, np.arange(N)[:, None] == (np.arange(T) % N)[None, :])
        assert np.array_equal(p.astype(np.float64), oracle.shard_sumsq(qd, N))
        gq, gk = gamma_of(Hq, dtype, 5), gamma_of(Hk, dtype, 6)
        oq, ok = ops.layerwise_fwd(to_dev(qd), to_dev(kd), to_dev(gq), to_dev(gk), N, 1e-6)
        oq, ok = to_host(oq), to_host(ok)
        assert np.array_equal(oq != 0, q != 0)
        assert np.array_equal(ok != 0, k != 0)
        assert_parity(qd, gq, oq, 1e-6)
        assert_parity(kd, gk, ok, 1e-6)


def _dev(w):
    d = inputs.make_host(w)
    return [to_dev(d[n]) for n in ("q", "k", "gamma_q", "gamma_k")]


@pytest.mark.parametrize("name", ["decode", "gqa"])
def test_deterministic_and_q_independent_of_k(name):
    w = inputs.CONFIGS[name].with_T(257)
    q, k, gq, gk = _dev(w)
    a = [to_host(t) for t in ops.layerwise_fwd(q, k, gq, gk, w.n_shards)]
    b = [to_host(t) for t in ops.layerwise_fwd(q, k, gq, gk, w.n_shards)]
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    k2 = k * 3 + 1
    c = [to_host(t) for t in ops.layerwise_fwd(q, k2, gq, gk, w.n_shards)]
    assert np.array_equal(a[0], c[0])
    assert not np.array_equal(a[1], c[1])


def test_token_permutation_equivariance():
    """Bitwise when every token is alone in its tile (its arithmetic is then
    independent of its position); within tolerance for the default plan."""
    w = inputs.PREFILL.with_T(500)
    q, k, gq, gk = _dev(w)
    perm = torch.randperm(500, generator=torch.Generator().manual_seed(0)).to("cuda:0")
    qp, kp = q[perm].contiguous(), k[perm].contiguous()
    old = ops.get_option("rows")
    try:
        ops.set_option("rows", 1)
        assert ops.current_plan("bf16", 500, 5120, 5120, 2)["rows"] == 1
        oq, ok = ops.layerwise_fwd(q, k, gq, gk, w.n_shards)
        pq, pk = ops.layerwise_fwd(qp, kp, gq, gk, w.n_shards)
        assert torch.equal(oq[perm], pq) and torch.equal(ok[perm], pk)
    finally:
        ops.set_option("rows", old)
    oq, ok = ops.layerwise_fwd(q, k, gq, gk, w.n_shards)
    pq, pk = ops.layerwise_fwd(qp, kp, gq, gk, w.n_shards)
    for a, b in ((oq[perm], pq), (ok[perm], pk)):
        rel = ((a.float() - b.float()).abs() / a.float().abs().clamp_min(1e-30)).max().item()
        assert rel <= 2 * 2 ** -8  # two valid roundings differ by at most one bf16 ulp each


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_power_of_two_scale_invariance_at_eps_zero(dtype):
    w = inputs.Workload("s", 200, 2048, 1024, 4, dtype)
    q, k, gq, gk = _dev(w)
    a = [to_host(t) for t in ops.layerwise_fwd(q, k, gq, gk, 4, 0.0)]
    for m in (-3, 5):
        b = [to_host(t) for t in ops.layerwise_fwd(q * 2.0 ** m, k * 2.0 ** m, gq, gk, 4, 0.0)]
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.fixture
def _layout_option():
    old = ops.get_option("tile_layout")
    yield
    ops.set_option("tile_layout", old)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,H,N", [(37, 5120, 2), (1001, 4096, 1), (999, 5120, 4), (513, 5120, 8),
                                   (4097, 1024, 2), (3, 256, 2), (16384, 5120, 2)])
def test_single_tensor_tiles(dtype, T, H, N, _layout_option):
    # Tiles that hold rows of one tensor (Q's tiles, then K's) compute every row
    # exactly as mixed Q+K tiles do: on dyadic inputs (exact sums) the outputs are
    # bitwise equal to the mixed layout's and to the split path's; on Gaussian
    # inputs they meet the oracle's bar. Both layouts are forced explicitly.
    q, k = dyadic(T, H, dtype, 5 * T), dyadic(T, H, dtype, 5 * T + 1)
    gq, gk = gamma_of(H, dtype, 6), gamma_of(H, dtype, 7)
    dq, dk, dgq, dgk = to_dev(q), to_dev(k), to_dev(gq), to_dev(gk)
    outs = {}
    for layout in (1, 2):
        ops.set_option("tile_layout", layout)
        assert ops.current_plan(dtype, T, H, H, N)["st"] == (layout == 2)
        outs[layout] = [to_host(t) for t in ops.layerwise_fwd(dq, dk, dgq, dgk, N, 1e-6)]
    assert np.array_equal(outs[1][0], outs[2][0]) and np.array_equal(outs[1][1], outs[2][1])
    if T <= 1001:
        _, _, yq = run_split(q, gq, N, 1e-6)
        assert np.array_equal(outs[2][0], yq)
    w = inputs.Workload("st", T, H, H, N, dtype)
    d = inputs.make_host(w)
    ops.set_option("tile_layout", 2)
    oq, ok = ops.layerwise_fwd(to_dev(d["q"]), to_dev(d["k"]), to_dev(d["gamma_q"]),
                               to_dev(d["gamma_k"]), N, w.eps)
    rows = slice(None) if T <= 4097 else np.r_[0:64, T // 2 - 32:T // 2 + 32, T - 64:T]
    assert_parity(d["q"][rows], d["gamma_q"], to_host(oq)[rows], w.eps, "single-tensor tiles, q")
    assert_parity(d["k"][rows], d["gamma_k"], to_host(ok)[rows], w.eps, "single-tensor tiles, k")
    assert ops.check_fault() == ops.QKN_OK


@pytest.mark.parametrize("dtype,T,H,N", [("bf16", 4096, 3072, 8), ("f32", 4097, 2048, 4),
                                         ("bf16", 8192, 4096, 4)])
def test_wide_split_default_plan_uses_single_tensor_tiles(dtype, T, H, N, _layout_option):
    # Streaming RMSNorm shards split 4-8 ways run on single-tensor tiles when
    # nothing is forced: the scored mixed launch with twice the rows per tile.
    # Same outputs as mixed tiles (bitwise on dyadic inputs) and the oracle's bar
    # on Gaussian inputs, at sampled rows.
    ops.set_option("tile_layout", 0)
    p = ops.current_plan(dtype, T, H, H, N)
    ops.set_option("tile_layout", 1)
    m = ops.current_plan(dtype, T, H, H, N)
    assert p["st"] == 1 and m["st"] == 0, (p, m)
    assert (p["variant"], p["data_waves"], p["rows"]) == (m["variant"], m["data_waves"], 2 * m["rows"])
    q, k = dyadic(T, H, dtype, 11 * T), dyadic(T, H, dtype, 11 * T + 1)
    gq, gk = gamma_of(H, dtype, 12), gamma_of(H, dtype, 13)
    dq, dk, dgq, dgk = to_dev(q), to_dev(k), to_dev(gq), to_dev(gk)
    outs = {}
    for layout in (0, 1):
        ops.set_option("tile_layout", layout)
        outs[layout] = [to_host(t) for t in ops.layerwise_fwd(dq, dk, dgq, dgk, N, 1e-6)]
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    ops.set_option("tile_layout", 0)
    w = inputs.Workload("st_default", T, H, H, N, dtype)
    d = inputs.make_host(w)
    oq, ok = ops.layerwise_fwd(to_dev(d["q"]), to_dev(d["k"]), to_dev(d["gamma_q"]),
                               to_dev(d["gamma_k"]), N, w.eps)
    rows = np.r_[0:64, T // 2 - 32:T // 2 + 32, T - 64:T]
    assert_parity(d["q"][rows], d["gamma_q"], to_host(oq)[rows], w.eps, "default plan, q")
    assert_parity(d["k"][rows], d["gamma_k"], to_host(ok)[rows], w.eps, "default plan, k")
    assert ops.check_fault() == ops.QKN_OK


@pytest.mark.parametrize("fmt", ["ln_bf16", "ln_f32", "e4m3_bf16", "e4m3_e4m3"])
@pytest.mark.parametrize("T,H,N", [(37, 5120, 2), (999, 5120, 4), (513, 4096, 8), (1001, 2048, 1)])
def test_single_tensor_tiles_other_formats(fmt, T, H, N, _layout_option):
    # LayerNorm (four LDS images: gamma and beta of each tensor) and E4M3 (two-word
    # bf16 stores) on single-tensor tiles: bitwise equal to mixed tiles on dyadic
    # inputs (exact statistics), and held to the oracle on Gaussian inputs.
    ln = fmt.startswith("ln")
    rng = np.random.default_rng(T + N)
    vq = torch.from_numpy((rng.integers(-16, 17, (T, H)) / 8.0).astype(np.float32)).cuda()
    vk = torch.from_numpy((rng.integers(-16, 17, (T, H)) / 8.0).astype(np.float32)).cuda()
    g = torch.from_numpy(rng.uniform(0.5, 1.5, (2, H)).astype(np.float32)).cuda()
    if ln:
        dt = torch.bfloat16 if fmt == "ln_bf16" else torch.float32
        q, k, gq, gk = vq.to(dt), vk.to(dt), g[0].to(dt), g[1].to(dt)
        bq, bk = (g[0] - 1).to(dt), (1 - g[1]).to(dt)
        call = lambda: ops.layernorm_fwd(q, k, gq, gk, N, 1e-5, beta_q=bq, beta_k=bk)
    else:
        odt = torch.bfloat16 if fmt == "e4m3_bf16" else torch.float8_e4m3fn
        q, k = vq.to(torch.float8_e4m3fn), vk.to(torch.float8_e4m3fn)
        gq, gk = g[0].to(torch.bfloat16), g[1].to(torch.bfloat16)
        call = lambda: ops.layerwise_fwd(q, k, gq, gk, N, 1e-6, out_dtype=odt)
    outs = {}
    for layout in (1, 2):
        ops.set_option("tile_layout", layout)
        assert ops.current_plan(fmt, T, H, H, N)["st"] == (layout == 2)
        outs[layout] = [to_host(t) for t in call()]
    assert np.array_equal(outs[1][0], outs[2][0]) and np.array_equal(outs[1][1], outs[2][1])
    ops.set_option("tile_layout", 2)
    if ln:
        w = inputs.Workload("st", T, H, H, N, "bf16" if fmt == "ln_bf16" else "f32", norm="layer")
        d = inputs.make_host(w)
        t = {n: to_dev(d[n]) for n in ("q", "k", "gamma_q", "gamma_k", "beta_q", "beta_k")}
        oq, ok = ops.layernorm_fwd(t["q"], t["k"], t["gamma_q"], t["gamma_k"], N, w.eps,
                                   beta_q=t["beta_q"], beta_k=t["beta_k"])
        assert_layernorm_parity(d["q"], d["gamma_q"], d["beta_q"], to_host(oq), w.eps, "st q")
        assert_layernorm_parity(d["k"], d["gamma_k"], d["beta_k"], to_host(ok), w.eps, "st k")
    else:
        w = inputs.Workload("st", T, H, H, N, "e4m3", out_dtype=fmt.split("_")[1])
        d = inputs.make_host(w)
        oq, ok = run_fused(d, N, w.eps, w.out_dtype)
        assert_parity(d["q"], d["gamma_q"], oq, w.eps, "st q")
        assert_parity(d["k"], d["gamma_k"], ok, w.eps, "st k")
    assert ops.check_fault() == ops.QKN_OK
