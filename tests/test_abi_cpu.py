"""The C-ABI library on the CPU: exports, host-only validation, launch planning.

Nothing here launches a kernel: every call either is pure host logic or is
rejected by argument validation before any HIP call.
"""
import ctypes
import os
import re

import pytest

from layerwise_qk_norm_amd import inputs, ops

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "qknorm.h")
CU = 256


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qknorm_\w+)\s*\(", text)))


def test_every_declared_function_is_exported_and_bound():
    names = declared_functions()
    assert "qknorm_layerwise_fwd_bf16" in names and len(names) >= 15
    L = ops.lib()
    for n in names:
        assert hasattr(L, n), n
        assert n in ops._SIGS, n


def test_strerror_and_options():
    for code in range(0, -9, -1):
        assert ops.strerror(code) and ops.strerror(code) != "unknown status"
    assert ops.strerror(-99) == "unknown status"
    old = ops.get_option("rows")
    ops.set_option("rows", 2)
    assert ops.get_option("rows") == 2
    ops.set_option("rows", old)
    with pytest.raises(ops.QKNormError):
        ops.set_option("force_variant", 99)
    assert ops.lib().qknorm_set_option(12345, 1) == ops.QKN_EINVAL


def test_option_ids_match_header():
    hdr = open(HEADER).read()
    ids = {m.group(1).lower(): int(m.group(2))
           for m in re.finditer(r"QKN_OPT_([A-Z_]+)\s*=\s*(\d+)", hdr)}
    assert ids == ops.OPT
    for n in ops.OPT:  # every option reads back what it was set to
        v = ops.get_option(n)
        ops.set_option(n, v)
        assert ops.get_option(n) == v


FAKE = [0x10000 * (i + 1) for i in range(6)]  # never dereferenced: rejected first


def fwd(T=4, Hq=64, Hk=64, N=2, eps=1e-6, ptrs=None, fn="qknorm_layerwise_fwd_bf16"):
    q, k, gq, gk, oq, ok = ptrs or FAKE
    return getattr(ops.lib(), fn)(q, k, gq, gk, T, Hq, Hk, N, eps, oq, ok, None)


@pytest.mark.parametrize("kw", [dict(N=0), dict(N=65), dict(N=3), dict(Hq=0), dict(Hk=-2),
                                dict(T=-1), dict(eps=-1e-6), dict(eps=float("nan")),
                                dict(eps=float("inf")), dict(Hq=100, Hk=64, N=8)])
def test_fused_rejects_bad_arguments(kw):
    assert fwd(**kw) == ops.QKN_EINVAL
    assert fwd(fn="qknorm_layerwise_fwd_f32", **kw) == ops.QKN_EINVAL


def test_fused_null_and_empty():
    assert fwd(T=0, ptrs=[0] * 6) == ops.QKN_OK  # T == 0 is a no-op
    for i in range(6):
        p = list(FAKE)
        p[i] = 0
        assert fwd(ptrs=p) == ops.QKN_EINVAL


def test_fused_rejects_partial_overlap():
    T, H = 4, 64  # 512 bytes per bf16 tensor
    q, k, gq, gk, oq, ok = FAKE
    assert fwd(ptrs=[q, k, gq, gk, q + 16, ok]) == ops.QKN_EOVERLAP  # out_q straddles q
    assert fwd(ptrs=[q, k, gq, gk, oq, oq + 256]) == ops.QKN_EOVERLAP  # outputs overlap
    assert fwd(ptrs=[q, k, gq, gk, k, ok]) == ops.QKN_EOVERLAP  # out_q aliases k
    assert fwd(ptrs=[q, k, gq, gk, oq, gk]) == ops.QKN_EOVERLAP  # out_k over gamma_k


def fwd8(T=4, Hq=64, Hk=64, N=2, eps=1e-6, ptrs=None, out=ops.QKN_BF16):
    q, k, gq, gk, oq, ok = ptrs or FAKE
    return ops.lib().qknorm_layerwise_fwd_e4m3(q, k, gq, gk, T, Hq, Hk, N, eps, oq, ok, out, None)


def test_e4m3_entry_points_reject_bad_arguments():
    L = ops.lib()
    for bad in (ops.QKN_F32, 7, -1):  # outputs are bf16 or e4m3 only
        assert fwd8(out=bad) == ops.QKN_EINVAL
        assert L.qknorm_apply_scale_e4m3(*FAKE[:3], 4, 64, FAKE[3], bad, None) == ops.QKN_EINVAL
    for kw in (dict(N=3), dict(T=-1), dict(eps=-1.0), dict(Hq=0)):
        assert fwd8(**kw) == ops.QKN_EINVAL
    assert fwd8(T=0, ptrs=[0] * 6) == ops.QKN_OK
    q, k, gq, gk, oq, ok = FAKE
    # a bf16 output at q's address covers 512 bytes, q only 256: not an exact alias
    assert fwd8(ptrs=[q, k, gq, gk, q, ok], out=ops.QKN_BF16) == ops.QKN_EOVERLAP
    # out_k (4 x 64 bf16 = 512 B) reaching into gamma_k
    assert fwd8(ptrs=[q, k, gq, gk, oq, gk - 256]) == ops.QKN_EOVERLAP
    # e4m3 x of 256 B just below the partials: no overlap; 8 bytes in: overlap
    assert L.qknorm_shard_sumsq_e4m3(FAKE[0], 4, 64, 2, FAKE[0] + 8, None) == ops.QKN_EOVERLAP
    assert L.qknorm_shard_sumsq_e4m3(FAKE[0], 4, 64, 3, FAKE[1], None) == ops.QKN_EINVAL
    assert L.qknorm_apply_scale_e4m3(FAKE[0], FAKE[1], FAKE[2], 4, 64, FAKE[0] + 2,
                                     ops.QKN_E4M3, None) == ops.QKN_EOVERLAP


def test_layernorm_entry_points_reject_bad_arguments():
    L = ops.lib()
    q, k, gq, gk, oq, ok = FAKE
    bq, bk = 0x90000, 0xA0000

    def ln(T=4, Hq=64, Hk=64, N=2, eps=1e-6, ptrs=None, betas=(bq, bk), fn="bf16"):
        a = ptrs or FAKE
        return getattr(L, f"qknorm_layernorm_fwd_{fn}")(a[0], a[1], a[2], a[3], betas[0], betas[1],
                                                        T, Hq, Hk, N, eps, a[4], a[5], None)
    for kw in (dict(N=3), dict(T=-1), dict(eps=-1.0), dict(Hq=0), dict(N=65)):
        assert ln(**kw) == ops.QKN_EINVAL
        assert ln(fn="f32", **kw) == ops.QKN_EINVAL
    assert ln(T=0, ptrs=[0] * 6, betas=(0, 0)) == ops.QKN_OK
    assert ln(ptrs=[q, k, gq, gk, oq, bk - 16]) == ops.QKN_EOVERLAP  # out_k runs into beta_k
    assert ln(ptrs=[q, k, gq, gk, bq, ok]) == ops.QKN_EOVERLAP       # out_q over beta_q
    assert L.qknorm_shard_stats_bf16(q, 4, 64, 3, gq, gk, None) == ops.QKN_EINVAL
    assert L.qknorm_shard_stats_f32(q, 4, 64, 2, gq, gq + 8, None) == ops.QKN_EOVERLAP
    assert L.qknorm_shard_stats_f32(q, 4, 64, 2, q + 8, gk, None) == ops.QKN_EOVERLAP
    assert L.qknorm_combine_stats(q, k, 4, 64, 2, -1.0, gq, gk, None) == ops.QKN_EINVAL
    assert L.qknorm_combine_stats(q, k, 4, 64, 2, 1e-6, gq, gq + 4, None) == ops.QKN_EOVERLAP
    assert L.qknorm_combine_stats(q, k, 4, 64, 2, 1e-6, q + 4, gk, None) == ops.QKN_EOVERLAP
    assert L.qknorm_apply_norm_bf16(q, 0, bq, gq, gk, 4, 64, oq, None) == ops.QKN_EINVAL
    assert L.qknorm_apply_norm_bf16(q, k, bq, gq, gk, 4, 64, bq - 2, None) == ops.QKN_EOVERLAP
    assert L.qknorm_apply_norm_f32(q, k, 0, gq, gk, 0, 64, oq, None) == ops.QKN_OK


def test_split_entry_points_reject_bad_arguments():
    L = ops.lib()
    assert L.qknorm_shard_sumsq_bf16(FAKE[0], 4, 64, 3, FAKE[1], None) == ops.QKN_EINVAL
    assert L.qknorm_shard_sumsq_f32(0, 4, 64, 2, FAKE[1], None) == ops.QKN_EINVAL
    assert L.qknorm_shard_sumsq_f32(FAKE[0], 0, 64, 2, 0, None) == ops.QKN_OK
    assert L.qknorm_shard_sumsq_f32(FAKE[0], 4, 64, 2, FAKE[0] + 8, None) == ops.QKN_EOVERLAP
    assert L.qknorm_combine_scale(FAKE[0], 4, 64, 2, -1.0, FAKE[1], None) == ops.QKN_EINVAL
    assert L.qknorm_combine_scale(FAKE[0], 4, 64, 2, 1e-6, FAKE[0] + 4, None) == ops.QKN_EOVERLAP
    assert L.qknorm_apply_scale_bf16(FAKE[0], FAKE[1], FAKE[2], 4, 64, FAKE[0] + 2, None) == \
        ops.QKN_EOVERLAP
    assert L.qknorm_apply_scale_f32(FAKE[0], 0, FAKE[2], 4, 64, FAKE[3], None) == ops.QKN_EINVAL
    assert L.qknorm_bench_copy(FAKE[0] + 4, FAKE[1], FAKE[2], FAKE[3], 64, 64, None) == \
        ops.QKN_EINVAL
    assert L.qknorm_bench_widen(FAKE[0] + 4, FAKE[1], FAKE[2], FAKE[3], 64, 64, None) == \
        ops.QKN_EINVAL
    # out_q (128 bytes from FAKE[2]) reaching into k
    assert L.qknorm_bench_widen(FAKE[0], FAKE[2] + 64, FAKE[2], FAKE[3], 64, 64, None) == \
        ops.QKN_EOVERLAP
    assert L.qknorm_bench_widen(FAKE[0], FAKE[1], FAKE[2], FAKE[3], 0, 0, None) == ops.QKN_OK
    assert L.qknorm_bench_widen(FAKE[0], 0, FAKE[2], 0, 64, 8, None) == ops.QKN_EINVAL
    assert L.qknorm_bench_copy(0, FAKE[1], FAKE[2], FAKE[3], 16, 16, None) == ops.QKN_EINVAL
    # out_k (64 bytes from FAKE[2] + 48) reaching over out_q's last 16 bytes
    assert L.qknorm_bench_copy(FAKE[0], FAKE[1], FAKE[2], FAKE[2] + 48, 64, 64, None) == \
        ops.QKN_EOVERLAP
    assert L.qknorm_bench_copy(FAKE[0], FAKE[1], FAKE[0], FAKE[3], 64, 64, None) == ops.QKN_EOVERLAP
    # one launch each: tensors (widening: outputs) up to 2^31 - 2^16 bytes
    far = [i << 40 for i in range(1, 5)]
    big = (1 << 31) - (1 << 16)
    assert L.qknorm_bench_copy(far[0], far[1], far[2], far[3], big + 16, 16, None) == ops.QKN_EINVAL
    assert L.qknorm_bench_copy(far[0], far[1], far[2], far[3], 16, big + 16, None) == ops.QKN_EINVAL
    assert L.qknorm_bench_widen(far[0], far[1], far[2], far[3], big // 2 + 8, 8, None) == ops.QKN_EINVAL


def test_bench_skeleton_rejects_bad_arguments():
    """The copy skeleton of a fused launch validates like the fused call (no GPU
    is touched before the arguments pass)."""
    L = ops.lib()
    q, k, oq, ok = FAKE[:4]
    bf16 = ops.FORMATS["bf16"]
    assert L.qknorm_bench_skeleton(99, q, k, oq, ok, 4, 64, 64, 2, None) == ops.QKN_EINVAL
    assert L.qknorm_bench_skeleton(bf16, q + 4, k, oq, ok, 4, 64, 64, 2, None) == ops.QKN_EINVAL
    assert L.qknorm_bench_skeleton(bf16, q, 0, oq, ok, 4, 64, 64, 2, None) == ops.QKN_EINVAL
    assert L.qknorm_bench_skeleton(bf16, q, k, oq, ok, -1, 64, 64, 2, None) == ops.QKN_EINVAL
    assert L.qknorm_bench_skeleton(bf16, q, k, oq, ok, 4, 64, 64, 3, None) == ops.QKN_EINVAL
    assert L.qknorm_bench_skeleton(bf16, q, k, oq, ok, 0, 64, 64, 2, None) == ops.QKN_OK
    # out_q (512 bytes) reaching into k; out_k on top of out_q
    assert L.qknorm_bench_skeleton(bf16, q, k, k - 256, ok, 4, 64, 64, 2, None) == ops.QKN_EOVERLAP
    assert L.qknorm_bench_skeleton(bf16, q, k, oq, oq + 16, 4, 64, 64, 2, None) == ops.QKN_EOVERLAP
    # E4M3 inputs with bf16 outputs: out_q holds twice q's bytes (256 -> 512)
    e4b = ops.FORMATS["e4m3_bf16"]
    assert L.qknorm_bench_skeleton(e4b, q, k, k - 256, ok, 4, 64, 64, 2, None) == ops.QKN_EOVERLAP
    # one launch only: tensors below 2^31 - 2^16 bytes
    far = [(i + 1) << 40 for i in range(4)]  # 1 TiB apart: no overlap even at this size
    assert L.qknorm_bench_skeleton(bf16, *far, 1 << 20, 4096, 4096, 2, None) == ops.QKN_EINVAL


# ------------------------------------------------------------------ planner

CU = 256
VPT = [1, 2, 3, 4, 6, 9, 1, 2, 3, 4, 5]
# data waves per variant (launch bound / 64 - 1) and rough register use, per format;
# 0 = not instantiated for that format
MAXW = {"bf16": [15, 15, 15, 15, 11, 0, 15, 15, 11, 7, 4],
        "f32": [15, 15, 15, 15, 11, 15, 15, 15, 11, 7, 0],
        "e4m3": [15, 15, 11, 0, 0, 0, 15, 11, 0, 0, 0],
        "ln_bf16": [15, 15, 15, 15, 7, 0, 15, 15, 11, 7, 0],
        "ln_f32": [15, 15, 15, 15, 7, 0, 15, 15, 11, 7, 0]}
VGPR = {"bf16": [32, 56, 80, 104, 168, 120, 48, 80, 136, 184, 232],
        "f32": [32, 56, 80, 104, 168, 120, 48, 80, 104, 128, 1],
        "e4m3": [56, 104, 144, 1, 1, 1, 96, 168, 1, 1, 1],
        "ln_bf16": [48, 73, 96, 121, 168, 1, 59, 99, 143, 184, 1],
        "ln_f32": [32, 58, 71, 95, 124, 1, 40, 72, 98, 139, 1]}
EV = {"bf16": 8, "f32": 4, "e4m3_bf16": 16, "e4m3_e4m3": 16, "ln_bf16": 8, "ln_f32": 4}
KGAM = {"bf16": 1, "f32": 1, "e4m3_bf16": 2, "e4m3_e4m3": 2, "ln_bf16": 2, "ln_f32": 2}  # x params
STATS = {"bf16": 1, "f32": 1, "e4m3_bf16": 1, "e4m3_e4m3": 1, "ln_bf16": 2, "ln_f32": 2}
FORMATS = list(EV)
assert set(FORMATS) == set(ops.FORMATS)


def _fam(fmt):
    return "e4m3" if fmt.startswith("e4m3") else fmt


def occupancy_model(dtype="bf16", lds_kb=160, waves_per_simd=8):
    """Synthetic blocks_per_cu[v][w] of a format: register file, wave slots and LDS limits."""
    fam = _fam(dtype)
    table = []
    for v in range(ops.NUM_VARIANTS):
        row = [0] * (ops.MAX_DATA_WAVES + 1)
        for w in range(1, MAXW[fam][v] + 1):
            waves = w + 1
            per_simd = -(-waves // 4)
            by_regs = min(waves_per_simd, 512 // VGPR[fam][v]) // per_simd
            by_lds = (lds_kb * 1024) // (VPT[v] * 64 * w * 16 * KGAM[dtype] + 1024)
            row[w] = max(0, min(by_regs, by_lds, 32 // waves))
        table.append(row)
    return table


BPC = {f: occupancy_model(f) for f in FORMATS}


def check_plan(p, dtype, T, Hq, Hk, N, cu=CU, bpc=None):
    bpc = bpc or BPC[dtype]
    if p["variant"] < 0:
        return
    v, w = p["variant"], p["data_waves"]
    assert MAXW[_fam(dtype)][v] > 0, "variant not instantiated for this format"
    assert p["threads"] == 64 * (w + 1) and 1 <= w <= MAXW[_fam(dtype)][v]
    assert p["slots"] == VPT[v]
    cap = bpc[v][w] * cu
    assert p["grid"] == p["n_groups"] * N
    assert p["grid"] <= cap, "grid must not exceed co-resident capacity"
    ev = EV[dtype]
    wvq, wvk = Hq // N // ev, Hk // N // ev
    if p["st"]:
        # single-tensor tiles: Hq == Hk, rows of one tensor, Q's tiles then K's,
        # one segment per row
        assert Hq == Hk and v not in (4, 5)
        assert 1 <= p["rows"] <= 8
        assert N * p["rows"] * STATS[dtype] <= 64
        assert p["n_tiles"] == 2 * -(-T // p["rows"])
        need = p["rows"] * wvq
    else:
        assert 1 <= p["rows"] <= 4
        assert N * 2 * p["rows"] * STATS[dtype] <= 64
        assert p["n_tiles"] == -(-T // p["rows"])
        # Q's part of a tile is padded to whole waves, then K's part follows
        need = -(-p["rows"] * wvq // 64) * 64 + p["rows"] * wvk
    assert 1 <= p["n_groups"] <= p["n_tiles"]
    assert p["iters"] * p["n_groups"] >= p["n_tiles"] > (p["iters"] - 1) * p["n_groups"]
    assert need <= w * 64 * p["slots"]  # data threads x slots
    if p["xcd_map"]:
        assert p["n_groups"] % 8 == 0


def plan(dtype, T, Hq, Hk, N, cu=CU, bpc=None, aligned=True):
    return ops.plan_fused(dtype, T, Hq, Hk, N, cu, bpc or BPC[dtype], aligned)


def test_plan_named_workloads():
    for w in (inputs.TINY, inputs.DECODE, inputs.PREFILL, inputs.GQA,
              *inputs.E4M3_CONFIGS.values(), *inputs.LN_CONFIGS.values()):
        p = plan(w.fmt, w.T, w.Hq, w.Hk, w.n_shards)
        assert p["variant"] >= 0, w.name
        check_plan(p, w.fmt, w.T, w.Hq, w.Hk, w.n_shards)
    d = plan("bf16", 64, 4096, 4096, 4)
    assert d["rows"] == 1 and d["grid"] == 256 and d["xcd_map"] == 1


def test_plan_every_sweep_point():
    for w in [*inputs.sweep(), *inputs.sweep_e4m3(), *inputs.sweep_layernorm()]:
        p = plan(w.fmt, w.T, w.Hq, w.Hk, w.n_shards)
        # every shape whose one-row tile fits some variant's slots runs fused
        ev = EV[w.fmt]
        wvq, wvk = w.Hq // w.n_shards // ev, w.Hk // w.n_shards // ev
        need = -(-wvq // 64) * 64 + wvk
        fam = _fam(w.fmt)
        room = max(64 * MAXW[fam][v] * VPT[v] for v in range(ops.NUM_VARIANTS)
                   if MAXW[fam][v] and (w.n_shards > 1 or v < 6))
        assert (p["variant"] >= 0) == (need <= room), w.name
        if w.norm == "rms":
            assert p["variant"] >= 0, w.name  # every RMSNorm sweep shape runs fused
        check_plan(p, w.fmt, w.T, w.Hq, w.Hk, w.n_shards)


def test_plan_latency_bound_batches_take_one_vector_per_thread():
    # Batches whose loads are below 32 KB per CU run one tile pass per call, so the
    # planner spreads a tile over as many waves as it needs at one 16-byte vector
    # per thread (measured on MI355X: 3.7 us per single-token call against 4.8 us
    # with four vectors per thread on one wave). Streaming batches keep wider slots.
    for dt in ("bf16", "e4m3_bf16", "ln_bf16"):
        for T, H, N in ((1, 4096, 4), (2, 5120, 2), (64, 4096, 4), (128, 4096, 2), (256, 2048, 2)):
            p = plan(dt, T, H, H, N)
            check_plan(p, dt, T, H, H, N)
            assert p["slots"] == 1 and p["rows"] == 1, (dt, T, H, N, p)
    assert plan("bf16", 16384, 5120, 5120, 2)["slots"] > 1


def test_plan_tile_layout_option():
    old = ops.get_option("tile_layout")
    try:
        ops.set_option("tile_layout", 2)  # single-tensor tiles wherever allowed
        for dt in FORMATS:
            for T, H, N in ((4097, 5120, 2), (16384, 4096, 1), (999, 5120, 4), (513, 5120, 8), (3, 1024, 2)):
                p = plan(dt, T, H, H, N)
                check_plan(p, dt, T, H, H, N)
                assert p["st"] == 1, (dt, T, H, N, p)
        # not allowed: Q and K of different widths
        for dt in FORMATS:
            p = plan(dt, 4096, 5120, 1024, 4)
            check_plan(p, dt, 4096, 5120, 1024, 4)
            assert p["st"] == 0
        ops.set_option("tile_layout", 1)  # mixed tiles only
        for T in (4096, 16384):
            p = plan("bf16", T, 5120, 5120, 2)
            check_plan(p, "bf16", T, 5120, 5120, 2)
            assert p["st"] == 0
        with pytest.raises(ops.QKNormError):
            ops.set_option("tile_layout", 3)
    finally:
        ops.set_option("tile_layout", old)


def test_plan_prefill_shards_use_single_tensor_tiles():
    # the measured launches of the bf16 prefill shards (width 5120 split 1-8 ways)
    for N in (1, 2, 4, 8):
        p = plan("bf16", 16384, 5120, 5120, N)
        check_plan(p, "bf16", 16384, 5120, 5120, N)
        assert p["st"] == 1, (N, p)
    assert plan("bf16", 8192, 5120, 1024, 4)["st"] == 0  # GQA: widths differ
    # the two-way prefill split: four data waves of five vectors (one wave per
    # SIMD), four-row tiles, members on one XCD, on the staggered schedule
    p = plan("bf16", 16384, 5120, 5120, 2)
    assert (p["variant"], p["data_waves"], p["rows"], p["st"], p["xcd_map"], p["pace_gbs"]) == (10, 4, 4, 1, 1, 7100), p
    p = plan("bf16", 16384, 5120, 5120, 1)  # unsplit: the same tile as 2-row tiles
    assert (p["variant"], p["data_waves"], p["rows"], p["st"], p["pace_gbs"]) == (10, 4, 2, 1, 7100), p
    # E4M3 entries, timed with rotating buffer sets (inputs beyond the Infinity Cache)
    p = plan("e4m3_e4m3", 16384, 5120, 5120, 2)
    assert (p["variant"], p["data_waves"], p["rows"], p["st"]) == (7, 10, 8, 1), p
    p = plan("e4m3_e4m3", 16384, 5120, 5120, 4)
    assert (p["variant"], p["data_waves"], p["rows"], p["st"], p["n_groups"]) == (7, 3, 2, 0, 3 * 256 // 4), p
    p = plan("e4m3_bf16", 16384, 5120, 5120, 4)
    assert (p["variant"], p["data_waves"], p["rows"], p["st"], p["n_groups"]) == (7, 3, 2, 0, 3 * 256 // 4), p
    assert p["xcd_map"] == 0, p
    # GQA entries (5120/1024 over 4 shards), retimed with exact workgroups per CU
    for fmt in ("e4m3_bf16", "e4m3_e4m3"):
        p = plan(fmt, 8192, 5120, 1024, 4)
        assert (p["variant"], p["data_waves"], p["rows"], p["n_groups"]) == (7, 3, 4, 3 * 256 // 4), (fmt, p)
    p = plan("ln_bf16", 8192, 5120, 1024, 4)
    assert (p["variant"], p["data_waves"], p["rows"], p["n_groups"]) == (6, 12, 4, 2 * 256 // 4), p


def test_plan_streaming_wide_splits_use_single_tensor_tiles():
    # untuned streaming RMSNorm shards split 4 to 8 ways: the scored mixed
    # launch, moved to single-tensor tiles of twice the rows
    old = ops.get_option("tile_layout")
    try:
        for dt in ("bf16", "f32"):
            for T, H, N in ((16384, 3072, 4), (16384, 8192, 8), (8192, 16384, 4), (16384, 1024, 8)):
                ops.set_option("tile_layout", 0)
                p = plan(dt, T, H, H, N)
                check_plan(p, dt, T, H, H, N)
                ops.set_option("tile_layout", 1)
                m = plan(dt, T, H, H, N)
                assert p["st"] == 1 and m["st"] == 0, (dt, T, H, N, p, m)
                assert (p["variant"], p["data_waves"], p["rows"]) == (m["variant"], m["data_waves"], 2 * m["rows"])
                assert p["n_groups"] == m["n_groups"]
        ops.set_option("tile_layout", 0)
        # N = 1, 2 or 16, other formats, latency-bound batches: mixed tiles
        for dt, T, H, N in (("bf16", 16384, 3072, 2), ("f32", 16384, 8192, 1), ("bf16", 16384, 8192, 16),
                            ("ln_bf16", 16384, 3072, 4),
                            ("e4m3_bf16", 16384, 3072, 8), ("bf16", 64, 4096, 4)):
            assert plan(dt, T, H, H, N)["st"] == 0, (dt, T, H, N)
        assert plan("bf16", 16384, 8192, 2048, 4)["st"] == 0  # widths differ
    finally:
        ops.set_option("tile_layout", old)


def test_plan_refuses_grid_beyond_residency():
    one = [[1] * (ops.MAX_DATA_WAVES + 1) for _ in range(ops.NUM_VARIANTS)]
    with pytest.raises(ops.QKNormError) as e:
        plan("bf16", 64, 4096, 4096, 8, cu=4, bpc=one)  # capacity 4 < 8
    assert e.value.status == ops.QKN_ERESIDENCY
    two = [[2] * (ops.MAX_DATA_WAVES + 1) for _ in range(ops.NUM_VARIANTS)]
    p = plan("bf16", 100000, 4096, 4096, 8, cu=4, bpc=two)  # capacity exactly 8
    assert p["grid"] == 8 and p["n_groups"] == 1


def test_plan_split_fallbacks():
    assert plan("bf16", 64, 4096, 4096, 4, aligned=False)["variant"] == -1
    assert plan("bf16", 64, 100, 100, 4)["variant"] == -1  # 25-wide shards
    # rows too wide for any bf16 variant's registers
    assert plan("bf16", 64, 65536, 65536, 1)["variant"] == -1
    # unlaunchable variants are skipped
    t = occupancy_model("bf16")
    for v in (0, 1, 6, 7):
        t[v] = [0] * (ops.MAX_DATA_WAVES + 1)
    p = plan("bf16", 64, 4096, 4096, 4, bpc=t)
    assert p["variant"] not in (0, 1, 6, 7)
    check_plan(p, "bf16", 64, 4096, 4096, 4, bpc=t)


def test_plan_forced_options_are_honoured():
    old = {n: ops.get_option(n) for n in ("force_variant", "data_waves", "rows")}
    try:
        ops.set_option("force_variant", 1)
        ops.set_option("data_waves", 6)
        ops.set_option("rows", 1)
        p = plan("bf16", 16384, 5120, 5120, 2)
        assert (p["variant"], p["data_waves"], p["rows"]) == (1, 6, 1)
        check_plan(p, "bf16", 16384, 5120, 5120, 2)
    finally:
        for n, v in old.items():
            ops.set_option(n, v)


def test_plan_forced_workgroups_per_cu():
    # QKN_OPT_WPC fixes the workgroups per CU of the planner's search (launch timing)
    old = {n: ops.get_option(n) for n in ("force_variant", "rows", "wpc")}
    try:
        ops.set_option("force_variant", 9)
        ops.set_option("rows", 4)
        for wpc in (1, 2):
            ops.set_option("wpc", wpc)
            p = plan("bf16", 8192, 5120, 1024, 4)
            check_plan(p, "bf16", 8192, 5120, 1024, 4)
            assert (p["variant"], p["rows"]) == (9, 4)
            assert p["n_groups"] == min(p["n_tiles"], wpc * CU // 4), p
        with pytest.raises(ops.QKNormError):
            ops.set_option("wpc", -1)
    finally:
        for n, v in old.items():
            ops.set_option(n, v)


def test_plan_narrow_e4m3_shards_use_several_workgroups_per_cu():
    # E4M3 -> E4M3 over shards of at most 160 vectors of Q and K per token: the
    # scored search starts at three workgroups per CU
    for T, H, N in ((16384, 2048, 2), (16384, 4096, 4), (16384, 2560, 2), (8192, 6144, 8)):
        p = plan("e4m3_e4m3", T, H, H, N)
        check_plan(p, "e4m3_e4m3", T, H, H, N)
        assert p["grid"] >= 3 * CU, (T, H, N, p)
    # latency-bound calls keep one token per tile
    p = plan("e4m3_e4m3", 64, 2048, 2048, 2)
    assert p["rows"] == 1 and p["slots"] == 1, p


def test_plan_many_shards_uses_narrow_tiles():
    for N in (16, 32):
        p = plan("bf16", 4096, 4096, 4096, N)
        assert p["variant"] >= 0 and N * (1 if p["st"] else 2) * p["rows"] <= 64
        check_plan(p, "bf16", 4096, 4096, 4096, N)
    # LayerNorm exchanges two statistics: 16 shards fit one comm wave, 32 do not
    p = plan("ln_bf16", 4096, 4096, 4096, 16)
    assert p["variant"] >= 0 and p["rows"] == 1
    check_plan(p, "ln_bf16", 4096, 4096, 4096, 16)
    assert plan("ln_bf16", 4096, 4096, 4096, 32)["variant"] == -1


def test_plan_randomised_invariants():
    import random
    rnd = random.Random(1)
    for _ in range(3000):
        N = rnd.choice([1, 2, 3, 4, 5, 8, 16, 32])
        dt = rnd.choice(FORMATS)
        ev = EV[dt]
        Hq = N * ev * rnd.randint(1, 600)
        Hk = N * ev * rnd.randint(1, 600)
        T = rnd.choice([1, 2, 3, 7, 63, 64, 65, 1000, 4097, rnd.randint(1, 200000)])
        cu = rnd.choice([1, 8, 80, 256])
        bpc = [[rnd.randint(0, 8) if w else 0 for w in range(ops.MAX_DATA_WAVES + 1)]
               for _ in range(ops.NUM_VARIANTS)]
        try:
            p = plan(dt, T, Hq, Hk, N, cu=cu, bpc=bpc)
        except ops.QKNormError as e:
            assert e.value.status == ops.QKN_ERESIDENCY if hasattr(e, "value") else True
            assert e.status == ops.QKN_ERESIDENCY
            continue
        check_plan(p, dt, T, Hq, Hk, N, cu, bpc)


def test_plan_xcd_mapping_follows_the_tuned_launch():
    """With the option at -1 a tuned launch keeps its measured XCD placement: a
    group's members on one XCD for the bf16 prefill split two ways, spread over
    XCDs for GQA and the eight-way splits; 0 and 1 force it either way. (A device
    roomy enough for every tuned launch.)"""
    roomy = [[0] + [8] * 15 for _ in range(ops.NUM_VARIANTS)]
    assert ops.get_option("xcd_map") == -1
    p = plan("bf16", 16384, 5120, 5120, 2, bpc=roomy)
    assert p["xcd_map"] == 1 and (p["variant"], p["rows"], p["st"]) == (10, 4, 1), p
    g = plan("bf16", 8192, 5120, 1024, 4, bpc=roomy)
    assert g["xcd_map"] == 0 and (g["variant"], g["data_waves"], g["rows"], g["n_groups"]) == (8, 2, 2, 256), g
    for dt in ("bf16", "e4m3_bf16", "e4m3_e4m3", "ln_bf16"):
        assert plan(dt, 16384, 5120, 5120, 8, bpc=roomy)["xcd_map"] == 0, dt
    assert plan("e4m3_e4m3", 8192, 5120, 1024, 4, bpc=roomy)["xcd_map"] == 1
    e = plan("e4m3_bf16", 16384, 5120, 5120, 2, bpc=roomy)
    assert e["xcd_map"] == 1 and (e["variant"], e["data_waves"], e["rows"], e["st"]) == (7, 10, 8, 1), e
    try:
        ops.set_option("xcd_map", 1)
        assert plan("bf16", 8192, 5120, 1024, 4, bpc=roomy)["xcd_map"] == 1
        ops.set_option("xcd_map", 0)
        assert plan("bf16", 16384, 5120, 5120, 2, bpc=roomy)["xcd_map"] == 0
    finally:
        ops.set_option("xcd_map", -1)


def test_plan_pace_follows_the_tuned_launch():
    """Tuned launches measured faster paced carry their pacing rate in the plan
    (bf16 split 1 and 2 ways on the staggered schedule 7100 GB/s, LayerNorm bf16 split 2
    ways staggered 6900 GB/s on single-tensor tiles, 6700 on mixed ones; bf16 GQA
    6700 GB/s; E4M3 -> bf16 split 2 ways staggered
    6800 GB/s; E4M3 -> bf16 split 1, 4 and 8 ways and E4M3 -> E4M3 split 2 ways 6600 GB/s);
    every other launch, forced launches included, has none unless the option
    sets a rate and its kernel has a paced build; 0 turns pacing off."""
    roomy = [[0] + [8] * 15 for _ in range(ops.NUM_VARIANTS)]
    pace = lambda *a: plan(*a, bpc=roomy)["pace_gbs"]
    assert ops.get_option("pace") == -1
    assert pace("bf16", 8192, 5120, 1024, 4) == 6700
    assert pace("bf16", 16384, 5120, 5120, 2) == 7100
    assert pace("bf16", 16384, 5120, 5120, 1) == 7100
    assert pace("ln_bf16", 16384, 5120, 5120, 2) == 6900
    ln = plan("ln_bf16", 16384, 5120, 5120, 2, bpc=roomy)
    assert (ln["variant"], ln["data_waves"], ln["rows"], ln["st"]) == (7, 10, 4, 1), ln
    try:
        # mixed tiles asked for: the mixed-tile staggered entry
        ops.set_option("tile_layout", 1)
        ln = plan("ln_bf16", 16384, 5120, 5120, 2, bpc=roomy)
        assert (ln["variant"], ln["rows"], ln["st"], ln["pace_gbs"]) == (7, 2, 0, 6700), ln
    finally:
        ops.set_option("tile_layout", 0)
    for N in (1, 4, 8):
        assert pace("e4m3_bf16", 16384, 5120, 5120, N) == 6600, N
    assert pace("e4m3_bf16", 16384, 5120, 5120, 2) == 6800
    assert pace("e4m3_e4m3", 16384, 5120, 5120, 2) == 6600
    for dt, N in (("bf16", 4), ("bf16", 8), ("e4m3_e4m3", 1),
                  ("e4m3_e4m3", 4), ("e4m3_e4m3", 8), ("ln_bf16", 4)):
        assert pace(dt, 16384, 5120, 5120, N) == 0, (dt, N)
    assert pace("bf16", 16384, 3072, 3072, 4) == 0 and pace("f32", 16384, 8192, 8192, 8) == 0
    assert pace("bf16", 64, 4096, 4096, 4) == 0
    try:
        # a forced launch is not the tuned one, even on the tuned launch's kernel
        for n, v in (("force_variant", 8), ("data_waves", 2), ("rows", 2), ("tile_layout", 1)):
            ops.set_option(n, v)
        assert plan("bf16", 8192, 5120, 1024, 4, bpc=roomy)["variant"] == 8
        assert pace("bf16", 8192, 5120, 1024, 4) == 0
        ops.set_option("pace", 7000)
        assert pace("bf16", 8192, 5120, 1024, 4) == 7000
    finally:
        for n, v in (("force_variant", -1), ("data_waves", 0), ("rows", 0), ("tile_layout", 0)):
            ops.set_option(n, v)
    try:
        ops.set_option("pace", 0)
        assert pace("bf16", 8192, 5120, 1024, 4) == 0
        ops.set_option("pace", 5000)
        assert pace("bf16", 8192, 5120, 1024, 4) == 5000
        assert pace("e4m3_e4m3", 16384, 5120, 5120, 2) == 5000
        # kernels without a paced build run unpaced whatever the option says
        assert pace("bf16", 16384, 3072, 3072, 2) == 0 and pace("bf16", 16384, 5120, 5120, 4) == 0
        assert pace("bf16", 16384, 5120, 5120, 2) == 5000
        for bad in (-2, 100001):
            assert ops.lib().qknorm_set_option(ops.OPT["pace"], bad) == ops.QKN_EINVAL
    finally:
        ops.set_option("pace", -1)


def test_plan_xcd_rule_for_untuned_shapes():
    """Untuned streaming shapes spread a group's members over XCDs for fp32 split
    4-8 ways and for bf16 split 4 ways with shard rows of at least 1 KiB; every
    other untuned shape, latency-bound batches, forced launches and LayerNorm or
    E4M3 keep them on one XCD; the option still forces either way."""
    roomy = [[0] + [8] * 15 for _ in range(ops.NUM_VARIANTS)]
    xm = lambda *a, **kw: plan(*a, bpc=roomy, **kw)["xcd_map"]
    for T in (4096, 16384, 65536):
        for H in (1024, 3072, 8192):
            assert xm("f32", T, H, H, 4) == 0 and xm("f32", T, H, H, 8) == 0, (T, H)
            assert xm("f32", T, H, H, 2) == 1, (T, H)
            assert xm("bf16", T, H, H, 2) == 1 and xm("bf16", T, H, H, 8) == 1, (T, H)
            # bf16 four ways: shard rows of H / 4 * 2 bytes
            assert xm("bf16", T, H, H, 4) == (0 if H // 4 * 2 >= 1024 else 1), (T, H)
            for dt in ("ln_bf16", "e4m3_bf16", "e4m3_e4m3"):
                assert xm(dt, T, H, H, 4) == 1 and xm(dt, T, H, H, 8) == 1, (dt, T, H)
    # a narrow K shard keeps bf16 on one XCD (K rows of 256 columns = 512 bytes)
    assert xm("bf16", 16384, 4096, 1024, 4) == 1
    assert xm("bf16", 16384, 4096, 4096, 4) == 0
    # latency-bound (decode-sized) batches: one XCD
    assert xm("f32", 64, 4096, 4096, 4) == 1 and xm("bf16", 64, 4096, 4096, 4) == 1
    try:
        ops.set_option("rows", 2)  # a forced launch follows the option alone
        assert xm("f32", 16384, 3072, 3072, 4) == 1
    finally:
        ops.set_option("rows", 0)
    try:
        ops.set_option("xcd_map", 1)
        assert xm("f32", 16384, 3072, 3072, 4) == 1
        ops.set_option("xcd_map", 0)
        assert xm("bf16", 16384, 3072, 3072, 2) == 0
    finally:
        ops.set_option("xcd_map", -1)


def test_plan_forced_single_tensor_only_variant():
    """Variant 10 exists for single-tensor tiles only: forcing it plans it on such
    tiles, and never on mixed tiles (the forced search then finds no launch)."""
    try:
        for n, v in (("force_variant", 10), ("data_waves", 4), ("rows", 4), ("tile_layout", 2)):
            ops.set_option(n, v)
        p = plan("bf16", 16384, 5120, 5120, 2)
        assert (p["variant"], p["data_waves"], p["rows"], p["st"]) == (10, 4, 4, 1), p
        ops.set_option("rows", 2)
        p = plan("bf16", 16384, 5120, 5120, 1)
        assert (p["variant"], p["rows"], p["st"]) == (10, 2, 1), p
        ops.set_option("tile_layout", 1)
        assert plan("bf16", 16384, 5120, 5120, 2)["variant"] != 10
    finally:
        for n, v in (("force_variant", -1), ("data_waves", 0), ("rows", 0), ("tile_layout", 0)):
            ops.set_option(n, v)
