"""Edge cases, launch options and error paths of the HIP path (GPU)."""
import numpy as np
import pytest
import torch

from layerwise_qk_norm_amd import inputs, ops
from oracle import compare, oracle

from _gpu import DEV, assert_layernorm_parity, assert_parity, needs_gpu, run_fused, run_split, to_dev, to_host

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.fixture(autouse=True)
def _restore_options():
    saved = {n: ops.get_option(n) for n in ops.OPT}
    yield
    for n, v in saved.items():
        ops.set_option(n, v)


def test_empty_batch_is_a_noop():
    for dt in (torch.bfloat16, torch.float32):
        q = torch.empty((0, 256), dtype=dt, device="cuda:0")
        g = torch.ones(256, dtype=dt, device="cuda:0")
        oq, ok = ops.layerwise_fwd(q, q.clone(), g, g, 2)
        assert oq.shape == (0, 256)


@pytest.mark.parametrize("T", [1, 2, 3, 5, 63, 65, 4097])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_token_counts(T, dtype):
    w = inputs.Workload("r", T, 1024, 512, 2, dtype)
    d = inputs.make_host(w)
    oq, ok = run_fused(d, 2, w.eps)
    assert_parity(d["q"], d["gamma_q"], oq, w.eps)
    assert_parity(d["k"], d["gamma_k"], ok, w.eps)


@pytest.mark.parametrize("N", [1, 3, 5, 16, 32, 48, 64])
def test_shard_counts(N):
    H = 256 * N  # 256-wide bf16 shards: every N divides H
    w = inputs.Workload("n", 130, H, H, N, "bf16")
    d = inputs.make_host(w)
    oq, ok = run_fused(d, N, w.eps)
    assert_parity(d["q"], d["gamma_q"], oq, w.eps)
    assert_parity(d["k"], d["gamma_k"], ok, w.eps)


@pytest.mark.parametrize("N", [33, 64])
def test_wide_splits_on_single_tensor_tiles(N):
    """More than 32 shards fit the exchange wave only with single-tensor tiles of
    one row (one segment per tile): forced here, the fused kernel runs 64-member
    groups; the planner's default for such splits is the split kernels."""
    H = 64 * N
    w = inputs.Workload("wide", 77, H, H, N, "bf16")
    d = inputs.make_host(w)
    try:
        ops.set_option("tile_layout", 2)
        plan = ops.current_plan("bf16", w.T, H, H, N)
        assert plan["variant"] >= 0 and plan["st"] == 1 and plan["rows"] == 1, plan
        assert plan["grid"] % N == 0
        oq, ok = run_fused(d, N, w.eps)
    finally:
        ops.set_option("tile_layout", 0)
    assert ops.check_fault() == ops.QKN_OK
    assert_parity(d["q"], d["gamma_q"], oq, w.eps)
    assert_parity(d["k"], d["gamma_k"], ok, w.eps)
    # by default the planner runs such splits on the split kernels
    assert ops.current_plan("bf16", w.T, H, H, N)["variant"] == -1
    p, r, y = run_split(d["q"], d["gamma_q"], N, w.eps)
    assert_parity(d["q"], d["gamma_q"], y, w.eps)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_unaligned_shapes_and_pointers(dtype):
    # 25-wide shards cannot use 16-byte accesses: the library runs the split kernels
    w = inputs.Workload("u", 70, 100, 60, 4, dtype)
    d = inputs.make_host(w)
    oq, ok = run_fused(d, 4, w.eps)
    assert_parity(d["q"], d["gamma_q"], oq, w.eps)
    assert_parity(d["k"], d["gamma_k"], ok, w.eps)
    # 16-byte-aligned shapes at an odd element offset
    w = inputs.Workload("o", 33, 1024, 1024, 2, dtype)
    d = inputs.make_host(w)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    bufs = []
    for name in ("q", "k"):
        flat = torch.empty(d[name].size + 1, dtype=dt, device="cuda:0")
        flat[1:] = to_dev(d[name]).reshape(-1)
        bufs.append(flat[1:].view(33, 1024))
    oq, ok = ops.layerwise_fwd(bufs[0], bufs[1], to_dev(d["gamma_q"]), to_dev(d["gamma_k"]), 2)
    assert_parity(d["q"], d["gamma_q"], to_host(oq), w.eps)
    assert_parity(d["k"], d["gamma_k"], to_host(ok), w.eps)


def test_in_place():
    w = inputs.DECODE
    d = inputs.make_host(w)
    q, k = to_dev(d["q"]), to_dev(d["k"])
    ops.layerwise_fwd(q, k, to_dev(d["gamma_q"]), to_dev(d["gamma_k"]), 4, out_q=q, out_k=k)
    assert_parity(d["q"], d["gamma_q"], to_host(q), w.eps)
    assert_parity(d["k"], d["gamma_k"], to_host(k), w.eps)


def test_overlap_is_rejected():
    q = torch.zeros((8, 256), dtype=torch.bfloat16, device="cuda:0")
    k = torch.zeros((8, 256), dtype=torch.bfloat16, device="cuda:0")
    g = torch.ones(256, dtype=torch.bfloat16, device="cuda:0")
    buf = torch.empty(8 * 256 + 8, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ops.QKNormError) as e:
        ops.layerwise_fwd(q, k, g, g, 2, out_q=k, out_k=q)
    assert e.value.status == ops.QKN_EOVERLAP
    with pytest.raises(ops.QKNormError) as e:
        ops.layerwise_fwd(q, k, g, g, 2, out_q=buf[:2048].view(8, 256), out_k=buf[8:].view(8, 256))
    assert e.value.status == ops.QKN_EOVERLAP


def test_degenerate_rows():
    H = 512
    x = np.zeros((4, H), np.float32)
    x[1, 3] = np.inf
    x[2, 7] = np.nan
    x[3, :] = 1e-3
    g = np.linspace(0.5, 1.5, H).astype(np.float32)
    for dtype in ("bf16", "f32"):
        xd = inputs.store(x.astype(np.float64), dtype)
        gd = inputs.store(g.astype(np.float64), dtype)
        d = {"q": xd, "k": xd, "gamma_q": gd, "gamma_k": gd}
        oq, _ = run_fused(d, 2, 1e-6)
        y = compare.decode_out(oq)
        ye, _, _ = oracle.rmsnorm(xd, gd, 1e-6)
        assert np.all(y[0] == 0)  # zero row, eps > 0
        assert np.isnan(y[1, 3]) and np.all(y[1, np.arange(H) != 3] == 0)
        assert np.all(np.isnan(y[2]))
        assert compare.report(y[3], ye[3])["max_rel"] <= compare.TOL[dtype]
        oq0, _ = run_fused(d, 2, 0.0)  # zero row with eps = 0: 0 * inf
        assert np.all(np.isnan(compare.decode_out(oq0)[0]))


def test_launch_options_preserve_results():
    w = inputs.PREFILL.with_T(1000)
    d = inputs.make_host(w)
    base = run_fused(d, 2, w.eps)
    for name, val in (("xcd_map", 0), ("xcd_map", 1), ("cooperative", 1), ("max_groups", 8)):
        ops.set_option(name, val)
        got = run_fused(d, 2, w.eps)
        assert np.array_equal(got[0], base[0]) and np.array_equal(got[1], base[1]), name
        ops.set_option(name, {"xcd_map": -1, "cooperative": 0, "max_groups": 0}[name])
    for v in range(ops.NUM_VARIANTS):
        ops.set_option("force_variant", v)
        got = run_fused(d, 2, w.eps)
        assert_parity(d["q"], d["gamma_q"], got[0], w.eps, f"variant {v}")
    ops.set_option("force_variant", -1)
    ops.set_option("force_split", 1)
    got = run_fused(d, 2, w.eps)
    assert_parity(d["q"], d["gamma_q"], got[0], w.eps, "split")
    assert_parity(d["k"], d["gamma_k"], got[1], w.eps, "split")


def test_bf16_output_rounds_to_nearest_even():
    # y = x * gamma * r with gamma = 1 and a chosen r: 1 * (1 + 2^-8 + 2^-10)
    # lies 0.625 ulp above 1.0 in bf16, so RNE gives 1 + 2^-7 (truncation: 1.0);
    # 1 * (1 + 2^-8) is an exact tie between 1.0 (even) and 1 + 2^-7.
    H = 64
    x = to_dev(inputs.f32_to_bf16_bits(np.ones((2, H), np.float32)))
    g = to_dev(inputs.f32_to_bf16_bits(np.ones(H, np.float32)))
    r = torch.tensor([1 + 2 ** -8 + 2 ** -10, 1 + 2 ** -8], dtype=torch.float32, device="cuda:0")
    y = to_host(ops.apply_scale(x, g, r))
    assert np.all(y[0] == 0x3F81) and np.all(y[1] == 0x3F80)


def _fused_calls():
    """Fused calls of several kinds on fixed tensors, each returning its outputs:
    the decode and a ragged prefill-shaped batch (fused kernel), an unaligned
    shape (the split fallback of the fused entry point), E4M3 and LayerNorm, and
    the no-allocation entry point through the C ABI."""
    calls = []
    for w in (inputs.DECODE, inputs.PREFILL.with_T(389), inputs.Workload("u", 70, 100, 60, 4, "bf16")):
        d = inputs.make_host(w)
        t = [to_dev(d[n]) for n in ("q", "k", "gamma_q", "gamma_k")]
        o = [torch.empty_like(t[0]), torch.empty_like(t[1])]
        calls.append((lambda t=t, o=o, w=w: ops.layerwise_fwd(*t, w.n_shards, w.eps, out_q=o[0], out_k=o[1]), o))
    d8 = inputs.make_host(inputs.DECODE_E4M3.with_T(77))
    t8 = [to_dev(d8[n]) for n in ("q", "k", "gamma_q", "gamma_k")]
    o8 = [torch.empty(t8[0].shape, dtype=torch.bfloat16, device=DEV),
          torch.empty(t8[1].shape, dtype=torch.bfloat16, device=DEV)]
    calls.append((lambda: ops.layerwise_fwd(*t8, 4, 1e-6, out_q=o8[0], out_k=o8[1]), o8))
    wl = inputs.LN_DECODE
    dl = inputs.make_host(wl)
    tl = {n: to_dev(dl[n]) for n in dl}
    ol = [torch.empty_like(tl["q"]), torch.empty_like(tl["k"])]
    calls.append((lambda: ops.layernorm_fwd(tl["q"], tl["k"], tl["gamma_q"], tl["gamma_k"], wl.n_shards,
                                            wl.eps, beta_q=tl["beta_q"], beta_k=tl["beta_k"],
                                            out_q=ol[0], out_k=ol[1]), ol))
    dn = inputs.make_host(inputs.GQA.with_T(300))
    tn = [to_dev(dn[n]) for n in ("q", "k", "gamma_q", "gamma_k")]
    on = [torch.empty_like(tn[0]), torch.empty_like(tn[1])]

    def noalloc():
        rc = ops.lib().qknorm_layerwise_fwd_bf16_noalloc(
            tn[0].data_ptr(), tn[1].data_ptr(), tn[2].data_ptr(), tn[3].data_ptr(), 300, 5120, 1024, 4,
            1e-6, on[0].data_ptr(), on[1].data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert rc == ops.QKN_OK
    calls.append((noalloc, on))
    return calls


def test_graph_capture():
    """Fused calls are recordable: each records a clearing kernel and the fused
    kernel on the scratch reserved for recorded launches. Replays, with eager work
    and synchronisation between them, give the eager outputs bit for bit."""
    calls = _fused_calls()
    for fn, _ in calls:
        fn()
    torch.cuda.synchronize()
    eager = [[t.clone() for t in outs] for _, outs in calls]
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for fn, _ in calls:
                fn()
    torch.cuda.current_stream().wait_stream(s)
    w = inputs.DECODE
    d = inputs.make_host(w)
    q, gq = to_dev(d["q"]), to_dev(d["gamma_q"])
    k, gk = to_dev(d["k"]), to_dev(d["gamma_k"])
    for rep in range(3):
        for _, outs in calls:
            for t in outs:
                t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (_, outs), ref in zip(calls, eager):
            for t, r in zip(outs, ref):
                assert torch.equal(t, r), f"replay {rep}"
        ops.layerwise_fwd(q, k, gq, gk, 4)  # eager work between replays
        ops.check_fault()
        torch.cuda.synchronize()
    assert ops.check_fault() == ops.QKN_OK
    # the split path is capturable too; replays match eager
    p = torch.empty((4, w.T), dtype=torch.float32, device="cuda:0")
    r = torch.empty((w.T,), dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(q)
    ops.shard_sumsq(q, 4, p)
    ops.combine_scale(p, w.Hq, w.eps, r)
    ops.apply_scale(q, gq, r, y)
    eager_y = y.clone()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        ops.shard_sumsq(q, 4, p)
        ops.combine_scale(p, w.Hq, w.eps, r)
        ops.apply_scale(q, gq, r, y)
    for _ in range(3):
        y.zero_()
        p.zero_()
        g2.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager_y)
        ops.layerwise_fwd(q, k, gq, gk, 4)  # eager work between replays
        torch.cuda.synchronize()


def test_graph_replay_reports_a_timeout():
    """A recorded launch whose exchange times out (forced by the never-publish test
    hook, recorded with a 1 ms spin limit) sets the fault word that check_fault reports;
    the options are restored for later tests."""
    w = inputs.DECODE
    d = inputs.make_host(w)
    q, k = to_dev(d["q"]), to_dev(d["k"])
    gq, gk = to_dev(d["gamma_q"]), to_dev(d["gamma_k"])
    oq, ok = torch.empty_like(q), torch.empty_like(k)
    assert ops.check_fault() == ops.QKN_OK
    g = torch.cuda.CUDAGraph()
    try:
        ops.set_option("spin_limit_ns", 1_000_000)
        ops.set_option("test_skip_publish", 1)
        with torch.cuda.graph(g):
            ops.layerwise_fwd(q, k, gq, gk, 4, w.eps, out_q=oq, out_k=ok)
    finally:
        ops.set_option("test_skip_publish", 0)
        ops.set_option("spin_limit_ns", 1_000_000_000)
    g.replay()
    torch.cuda.synchronize()
    assert ops.check_fault() == ops.QKN_ETIMEOUT
    assert ops.check_fault() == ops.QKN_OK


def test_timeout_is_reported_and_recovers():
    w = inputs.DECODE
    d = inputs.make_host(w)
    assert ops.check_fault() == ops.QKN_OK
    try:
        ops.set_option("spin_limit_ns", 1_000_000)  # 1 ms
        ops.set_option("test_skip_publish", 1)     # no partial is ever published
        run_fused(d, 4, w.eps)
        assert ops.check_fault() == ops.QKN_ETIMEOUT
        assert ops.check_fault() == ops.QKN_OK  # cleared
    finally:
        # restore the defaults even when an assertion failed, so later tests do
        # not inherit a 1 ms spin limit and a kernel that never publishes
        ops.set_option("test_skip_publish", 0)
        ops.set_option("spin_limit_ns", 1_000_000_000)
        ops.check_fault()
    oq, ok = run_fused(d, 4, w.eps)
    assert ops.check_fault() == ops.QKN_OK
    assert_parity(d["q"], d["gamma_q"], oq, w.eps)


def test_timeout_is_loud_at_the_next_python_call():
    """A timed-out launch issued through the C ABI (no check) sets the device's
    pinned timeout flag: fault_pending() sees it without synchronising once the
    launch has ended, the next call through the binding raises QKN_ETIMEOUT
    without issuing, and check_fault() clears everything."""
    w = inputs.DECODE
    d = inputs.make_host(w)
    q, k = to_dev(d["q"]), to_dev(d["k"])
    gq, gk = to_dev(d["gamma_q"]), to_dev(d["gamma_k"])
    oq, ok = torch.empty_like(q), torch.empty_like(k)
    assert ops.check_fault() == ops.QKN_OK
    ops.layerwise_fwd(q, k, gq, gk, 4, w.eps, out_q=oq, out_k=ok)  # the flag exists from here
    torch.cuda.synchronize()
    assert not ops.fault_pending()
    try:
        ops.set_option("spin_limit_ns", 1_000_000)
        ops.set_option("test_skip_publish", 1)
        rc = ops.lib().qknorm_layerwise_fwd_bf16(q.data_ptr(), k.data_ptr(), gq.data_ptr(), gk.data_ptr(),
                                                 w.T, w.Hq, w.Hk, 4, w.eps, oq.data_ptr(), ok.data_ptr(),
                                                 torch.cuda.current_stream().cuda_stream)
        assert rc == ops.QKN_OK
        torch.cuda.synchronize()
    finally:
        ops.set_option("test_skip_publish", 0)
        ops.set_option("spin_limit_ns", 1_000_000_000)
    try:
        assert ops.fault_pending()
        oq.fill_(7.0)
        with pytest.raises(ops.QKNormError) as e:
            ops.layerwise_fwd(q, k, gq, gk, 4, w.eps, out_q=oq, out_k=ok)
        assert e.value.status == ops.QKN_ETIMEOUT
        torch.cuda.synchronize()
        assert bool((oq == 7.0).all())  # nothing was issued
    finally:
        assert ops.check_fault() == ops.QKN_ETIMEOUT
    assert not ops.fault_pending()
    assert ops.check_fault() == ops.QKN_OK
    ops.layerwise_fwd(q, k, gq, gk, 4, w.eps, out_q=oq, out_k=ok)
    torch.cuda.synchronize()
    assert_parity(d["q"], d["gamma_q"], to_host(oq), w.eps)


def test_coresidency_query():
    """The co-resident capacity the library reports for the prefill shape holds the
    grid it plans, is a whole number of workgroups per CU, and fits the CU's wave
    slots (4 SIMDs x 8 waves on gfx950) for that launch's workgroup size."""
    plan = ops.current_plan("bf16", 16384, 5120, 5120, 2)
    n = ops.max_coresident_workgroups("bf16", 5120, 5120, 2)
    bpc, cu = ops.device_occupancy("bf16")
    assert cu == torch.cuda.get_device_properties(0).multi_processor_count
    assert n % cu == 0 and n // cu >= 1
    assert plan["grid"] <= n, (plan, n)
    assert n // cu <= 32 // (plan["data_waves"] + 1), (plan, n, cu)
    if not plan["st"]:
        assert n == bpc[plan["variant"]][plan["data_waves"]] * cu


def test_bench_helpers_compute_the_same():
    w = inputs.DECODE
    d = inputs.make_host(w)
    q, k = to_dev(d["q"]), to_dev(d["k"])
    gq, gk = to_dev(d["gamma_q"]), to_dev(d["gamma_k"])
    ref = [to_host(t) for t in ops.layerwise_fwd(q, k, gq, gk, 4)]
    oq, ok = torch.empty_like(q), torch.empty_like(k)
    ops.bench_fused(q, k, gq, gk, 4, w.eps, oq, ok, 3)
    assert np.array_equal(to_host(oq), ref[0]) and np.array_equal(to_host(ok), ref[1])
    ops.bench_copy(q, k, oq, ok)
    assert torch.equal(oq, q) and torch.equal(ok, k)
    # sizes that end mid-workgroup and mid-vector
    a = torch.randn(3, 1001, device="cuda:0").to(torch.bfloat16)
    b = torch.randn(5, 777, device="cuda:0")
    oa, ob = torch.zeros_like(a), torch.zeros_like(b)
    ops.bench_copy(a, b, oa, ob)
    assert torch.equal(oa, a) and torch.equal(ob, b)
    # the widening ceiling: each byte becomes a zero-extended 16-bit word (byte
    # counts with and without whole 8-byte chunks, and a tensor of tail bytes only)
    g = torch.Generator(device="cuda:0").manual_seed(7)
    for na, nb in ((3 * 1003, 7), (4096, 2048 * 8 + 5), (8, 0)):
        e = torch.randint(0, 256, (na,), dtype=torch.uint8, device="cuda:0", generator=g)
        f = torch.randint(0, 256, (max(nb, 1),), dtype=torch.uint8, device="cuda:0", generator=g)[:nb]
        oe = torch.full((na,), -1, dtype=torch.int16, device="cuda:0")
        of = torch.full((max(nb, 1),), -1, dtype=torch.int16, device="cuda:0")[:nb]
        ops.bench_widen(e, f, oe, of)
        assert torch.equal(oe, e.to(torch.int16)) and torch.equal(of, f.to(torch.int16))



@pytest.mark.parametrize("case", [("bf16", 37, 1000, 1), ("bf16", 19, 5120, 2), ("f32", 23, 1000, 4), ("f32", 23, 1160, 2),
                                  ("e4m3", 29, 2080, 2)])
def test_split_vector_widths(case):
    # The split kernels' 16-byte paths at every vector count per thread. Rows of
    # 125 / 640 / 250 / 290 / 130 vectors do not divide a workgroup's span of vectors,
    # so workgroups straddle rows and the last one is partial. Every width adds
    # each lane's vectors in the same order and scales elementwise alike, so the
    # results are bitwise equal; the library's default is also held to the oracle.
    dtype, T, H, N = case
    w = inputs.Workload("sv", T, H, H, N, dtype, out_dtype="bf16" if dtype == "e4m3" else "")
    d = inputs.make_host(w)
    base = run_split(d["q"], d["gamma_q"], N, w.eps, w.out_dtype)
    assert_parity(d["q"], d["gamma_q"], base[2], w.eps, "split")
    pe = oracle.shard_sumsq(d["q"], N)
    assert np.max(np.abs(base[0] - pe) / pe) <= compare.TOL_STAT
    for v in (1, 2, 4, 8):
        ops.set_option("split_vectors", v)
        got = run_split(d["q"], d["gamma_q"], N, w.eps, w.out_dtype)
        for a, b in zip(base, got):
            assert np.array_equal(a, b), (case, v)
    ops.set_option("split_vectors", 0)
    if dtype == "e4m3":
        return
    x, g = to_dev(d["q"]), to_dev(d["gamma_q"])
    beta = to_dev(d["gamma_k"])  # any vector of the format serves as beta here
    ref = None
    for v in (0, 1, 2, 4, 8):
        ops.set_option("split_vectors", v)
        s1, s2 = ops.shard_stats(x, N)
        mean, rstd = ops.combine_stats(s1, s2, H, w.eps)
        y = ops.apply_norm(x, g, beta, mean, rstd)
        torch.cuda.synchronize()
        got = [to_host(t) for t in (s1, s2, mean, rstd, y)]
        if ref is None:
            ref = got
            assert_layernorm_parity(d["q"], d["gamma_q"], d["gamma_k"], got[4], w.eps, "split LN")
        for a, b in zip(ref, got):
            assert np.array_equal(a, b), (case, v)


def _eq(a, b):
    return all(np.array_equal(to_host(x), to_host(y)) for x, y in zip(a, b))


def test_prepared_calls_match_direct_calls():
    # A prepared call validates once and then issues the same C call; its outputs
    # must equal the direct call's bit for bit, on every call, and follow changes
    # of the inputs' contents between calls.
    w = inputs.DECODE
    d = inputs.make_host(w)
    q, k, gq, gk = (to_dev(d[n]) for n in ("q", "k", "gamma_q", "gamma_k"))
    ref = ops.layerwise_fwd(q, k, gq, gk, w.n_shards, w.eps)
    call = ops.prepare_layerwise_fwd(q, k, gq, gk, w.n_shards, w.eps)
    for _ in range(3):
        assert _eq(call(), ref)
    q.copy_(k)
    got = call()
    assert _eq(got, ops.layerwise_fwd(q, k, gq, gk, w.n_shards, w.eps))
    assert_parity(d["k"], d["gamma_q"], to_host(got[0]), w.eps, "prepared, new contents")
    # given outputs are written in place and returned
    oq, ok = torch.empty_like(q), torch.empty_like(k)
    c2 = ops.prepare_layerwise_fwd(q, k, gq, gk, w.n_shards, w.eps, out_q=oq, out_k=ok)
    outs = c2()
    assert outs[0] is oq and outs[1] is ok and _eq(outs, got)
    # E4M3 inputs with E4M3 outputs
    w8 = inputs.E4M3_CONFIGS["decode_e4m3"]
    d8 = inputs.make_host(w8)
    q8, k8, g8q, g8k = (to_dev(d8[n]) for n in ("q", "k", "gamma_q", "gamma_k"))
    e4 = torch.float8_e4m3fn
    c8 = ops.prepare_layerwise_fwd(q8, k8, g8q, g8k, w8.n_shards, w8.eps, out_dtype=e4)
    assert _eq(c8(), ops.layerwise_fwd(q8, k8, g8q, g8k, w8.n_shards, w8.eps, out_dtype=e4))
    # LayerNorm with beta, and headwise
    wl = inputs.LN_DECODE
    dl = inputs.make_host(wl)
    tl = {n: to_dev(dl[n]) for n in ("q", "k", "gamma_q", "gamma_k", "beta_q", "beta_k")}
    cl = ops.prepare_layernorm_fwd(tl["q"], tl["k"], tl["gamma_q"], tl["gamma_k"], wl.n_shards,
                                   wl.eps, beta_q=tl["beta_q"], beta_k=tl["beta_k"])
    assert _eq(cl(), ops.layernorm_fwd(tl["q"], tl["k"], tl["gamma_q"], tl["gamma_k"], wl.n_shards,
                                       wl.eps, beta_q=tl["beta_q"], beta_k=tl["beta_k"]))
    wh = inputs.HW_DECODE
    dh = inputs.make_host(wh)
    th = {n: to_dev(dh[n]) for n in ("q", "k", "gamma_q", "gamma_k")}
    ch = ops.prepare_headwise_fwd(th["q"], th["k"], th["gamma_q"], th["gamma_k"], wh.head_dim, wh.eps)
    assert _eq(ch(), ops.headwise_fwd(th["q"], th["k"], th["gamma_q"], th["gamma_k"], wh.head_dim,
                                      wh.eps))


def test_prepared_call_validates_once_and_reports_errors():
    w = inputs.DECODE
    d = inputs.make_host(w)
    q, k, gq, gk = (to_dev(d[n]) for n in ("q", "k", "gamma_q", "gamma_k"))
    with pytest.raises(ValueError):
        ops.prepare_layerwise_fwd(q, k[:3], gq, gk, w.n_shards)
    with pytest.raises(TypeError):
        ops.prepare_layerwise_fwd(q, k.float(), gq, gk, w.n_shards)
    # the library's own checks still run on every call
    bad = ops.prepare_layerwise_fwd(q, k, gq, gk, 3)  # 4096 is not a multiple of 3
    with pytest.raises(ops.QKNormError) as e:
        bad()
    assert e.value.status == ops.QKN_EINVAL


def _random_bytes(shape, dtype, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    n = int(np.prod(shape)) * torch.empty(0, dtype=dtype).element_size()
    return torch.randint(0, 256, (n,), generator=g, dtype=torch.uint8, device=DEV).view(dtype).view(shape)


@pytest.mark.parametrize("fmt,T,Hq,Hk,N,layout", [
    ("bf16", 389, 5120, 5120, 2, 0), ("bf16", 389, 5120, 5120, 2, 1), ("bf16", 389, 5120, 5120, 2, 2),
    ("bf16", 1001, 5120, 1024, 4, 0), ("bf16", 16384, 5120, 5120, 2, 0), ("bf16", 8192, 5120, 1024, 4, 0),
    ("f32", 200, 2048, 1024, 2, 0), ("ln_bf16", 300, 4096, 4096, 4, 0),
    ("e4m3_e4m3", 777, 5120, 5120, 2, 0), ("e4m3_bf16", 500, 5120, 5120, 2, 0),
    ("e4m3_bf16", 16384, 5120, 5120, 2, 0),
])
def test_bench_skeleton_moves_every_byte(fmt, T, Hq, Hk, N, layout):
    """The copy skeleton of a fused launch (the fused call's own plan, without the
    arithmetic) stores every byte of q and k, unchanged or zero-extended."""
    ops.set_option("tile_layout", layout)
    tin = {"bf16": torch.bfloat16, "f32": torch.float32, "ln_bf16": torch.bfloat16,
           "e4m3_e4m3": torch.float8_e4m3fn, "e4m3_bf16": torch.float8_e4m3fn}[fmt]
    tout = torch.bfloat16 if fmt == "e4m3_bf16" else tin
    q, k = _random_bytes((T, Hq), tin, 1), _random_bytes((T, Hk), tin, 2)
    oq = torch.full((T, Hq), 0, dtype=torch.uint8 if tout == torch.float8_e4m3fn else torch.int16, device=DEV)
    ok = torch.full((T, Hk), 0, dtype=oq.dtype, device=DEV)
    if tout == torch.float32:
        oq, ok = oq.to(torch.int32), ok.to(torch.int32)
    oq.fill_(-1 if oq.dtype != torch.uint8 else 0xAB)
    ok.fill_(-1 if ok.dtype != torch.uint8 else 0xAB)
    oq, ok = oq.view(tout), ok.view(tout)
    ops.bench_skeleton(q, k, oq, ok, N, fmt)
    torch.cuda.synchronize()
    for x, y in ((q, oq), (k, ok)):
        xb = x.view(torch.uint8)
        if fmt == "e4m3_bf16":
            assert torch.equal(y.view(torch.int16).to(torch.int32) & 0xffff, xb.to(torch.int32)), fmt
        else:
            assert torch.equal(y.contiguous().view(torch.uint8), xb), (fmt, T, Hq, Hk, N, layout)


@pytest.mark.parametrize("fmt,T,Hq,Hk,N,rate", [
    ("bf16", 8192, 5120, 1024, 4, -1),      # the tuned GQA launch, paced by default
    ("bf16", 16384, 5120, 5120, 2, -1),     # the tuned prefill launch, staggered by default
    ("bf16", 4099, 5120, 5120, 2, 4000),    # staggered, groups of 17 and 16 tiles, barriers held
    ("bf16", 4096, 5120, 5120, 1, -1),      # the tuned one-shard launch, staggered by default
    ("bf16", 4099, 5120, 5120, 1, 6000),    # the same, ragged, at a set rate
    ("ln_bf16", 16384, 5120, 5120, 2, -1),  # the tuned LayerNorm launch, staggered by default
    ("ln_bf16", 4099, 5120, 5120, 2, 4000), # staggered LayerNorm (lean), ragged, barriers held
    ("bf16", 4096, 5120, 1024, 4, 4000),    # a rate below the launch's own: barriers held
    ("e4m3_bf16", 16384, 5120, 5120, 2, -1),  # the tuned E4M3 -> bf16 launch, staggered
    ("e4m3_bf16", 4099, 5120, 5120, 2, 4000), # the same, ragged, barriers held
    ("e4m3_bf16", 4096, 5120, 5120, 4, -1),
    ("e4m3_bf16", 4099, 5120, 5120, 1, 4000),
    ("e4m3_bf16", 8192, 5120, 5120, 8, -1),
    ("e4m3_e4m3", 4096, 5120, 5120, 2, -1),
])
def test_pacing_changes_no_output(fmt, T, Hq, Hk, N, rate):
    """Pacing only holds barriers: a paced launch's outputs are bitwise those of the
    unpaced one, no exchange times out, and the paced launch skeleton still stores
    every byte."""
    g = torch.Generator(device=DEV).manual_seed(T + Hq + N)
    e4 = fmt.startswith("e4m3")
    tin = torch.float8_e4m3fn if e4 else (torch.float32 if fmt == "f32" else torch.bfloat16)
    tout = torch.float8_e4m3fn if fmt == "e4m3_e4m3" else (torch.bfloat16 if e4 else tin)
    tg = torch.bfloat16 if e4 else tin
    q = (torch.randn(T, Hq, generator=g, device=DEV) * 2).to(tin)
    k = (torch.randn(T, Hk, generator=g, device=DEV) * 2).to(tin)
    gq = (torch.rand(Hq, generator=g, device=DEV) + 0.5).to(tg)
    gk = (torch.rand(Hk, generator=g, device=DEV) + 0.5).to(tg)

    def run():
        oq = torch.empty(T, Hq, dtype=tout, device=DEV)
        ok = torch.empty(T, Hk, dtype=tout, device=DEV)
        if fmt.startswith("ln"):
            ops.layernorm_fwd(q, k, gq, gk, N, 1e-6, beta_q=gq, beta_k=gk, out_q=oq, out_k=ok)
        else:
            ops.layerwise_fwd(q, k, gq, gk, N, 1e-6, out_q=oq, out_k=ok)
        torch.cuda.synchronize()
        assert ops.check_fault() == ops.QKN_OK
        return oq.view(torch.uint8), ok.view(torch.uint8)

    ops.set_option("pace", 0)
    assert ops.current_plan(fmt, T, Hq, Hk, N)["pace_gbs"] == 0
    ref = run()
    ops.set_option("pace", rate)
    p = ops.current_plan(fmt, T, Hq, Hk, N)
    assert p["pace_gbs"] > 0 and p["iters"] > 2, p
    for _ in range(3):
        got = run()
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), (fmt, T, Hq, Hk, N)
    # the skeleton of the paced launch moves every byte
    sq, sk = torch.empty_like(q), torch.empty_like(k)
    if fmt == "e4m3_bf16":
        sq, sk = torch.empty(T, Hq, dtype=torch.bfloat16, device=DEV), torch.empty(T, Hk, dtype=torch.bfloat16, device=DEV)
    ops.bench_skeleton(q, k, sq, sk, N, fmt)
    torch.cuda.synchronize()
    for x, y in ((q, sq), (k, sk)):
        if fmt == "e4m3_bf16":
            assert torch.equal(y.view(torch.int16).to(torch.int32) & 0xffff, x.view(torch.uint8).to(torch.int32))
        else:
            assert torch.equal(y.view(torch.uint8), x.view(torch.uint8))


def test_bench_skeleton_refuses_split_shapes():
    # shard widths that are not whole vectors run the split kernels: no fused plan to mirror
    q = torch.zeros((8, 100), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ops.QKNormError):
        ops.bench_skeleton(q, q.clone(), torch.empty_like(q), torch.empty_like(q), 4)
