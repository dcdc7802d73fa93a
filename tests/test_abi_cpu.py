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
# plausible blocks-per-CU for the five fused variants on a 256-CU device
BPC = [6, 3, 2, 1, 1]
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
    for code in range(0, -8, -1):
        assert ops.strerror(code) and ops.strerror(code) != "unknown status"
    assert ops.strerror(-99) == "unknown status"
    old = ops.get_option("rows")
    ops.set_option("rows", 2)
    assert ops.get_option("rows") == 2
    ops.set_option("rows", old)
    with pytest.raises(ops.QKNormError):
        ops.set_option("force_variant", 99)
    assert ops.lib().qknorm_set_option(12345, 1) == ops.QKN_EINVAL


FAKE = [0x10000 * (i + 1) for i in range(6)]  # never dereferenced: rejected first


def fwd(T=4, Hq=64, Hk=64, N=2, eps=1e-6, ptrs=None, fn="qknorm_layerwise_fwd_bf16"):
    q, k, gq, gk, oq, ok = ptrs or FAKE
    return getattr(ops.lib(), fn)(q, k, gq, gk, T, Hq, Hk, N, eps, oq, ok, None)


@pytest.mark.parametrize("kw", [dict(N=0), dict(N=33), dict(N=3), dict(Hq=0), dict(Hk=-2),
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


# ------------------------------------------------------------------ planner

def check_plan(p, dtype, T, Hq, Hk, N, cu=CU, bpc=BPC):
    if p["variant"] < 0:
        return
    v = p["variant"]
    cap = bpc[v] * cu
    assert p["grid"] == p["n_groups"] * N
    assert p["grid"] <= cap, "grid must not exceed co-resident capacity"
    assert 1 <= p["rows"]
    assert N * 2 * p["rows"] <= 64
    assert p["n_tiles"] == -(-T // p["rows"])
    assert 1 <= p["n_groups"] <= p["n_tiles"]
    assert p["iters"] * p["n_groups"] >= p["n_tiles"] > (p["iters"] - 1) * p["n_groups"]
    ev = 8 if dtype == "bf16" else 4
    vrow = (Hq // N + Hk // N) // ev
    assert p["rows"] * vrow <= (p["threads"] - 64) * p["slots"]  # data threads x slots
    if p["xcd_map"]:
        assert p["n_groups"] % 8 == 0


def test_plan_named_workloads():
    for w in (inputs.TINY, inputs.DECODE, inputs.PREFILL, inputs.GQA):
        p = ops.plan_fused(w.dtype, w.T, w.Hq, w.Hk, w.n_shards, CU, BPC)
        assert p["variant"] >= 0, w.name
        check_plan(p, w.dtype, w.T, w.Hq, w.Hk, w.n_shards)
    d = ops.plan_fused("bf16", 64, 4096, 4096, 4, CU, BPC)
    assert d["rows"] == 1 and d["grid"] == 256 and d["xcd_map"] == 1


def test_plan_every_sweep_point():
    for w in inputs.sweep():
        p = ops.plan_fused(w.dtype, w.T, w.Hq, w.Hk, w.n_shards, CU, BPC)
        assert p["variant"] >= 0, w.name  # every sweep shape fits a fused variant
        check_plan(p, w.dtype, w.T, w.Hq, w.Hk, w.n_shards)


def test_plan_refuses_grid_beyond_residency():
    with pytest.raises(ops.QKNormError) as e:
        ops.plan_fused("bf16", 64, 4096, 4096, 8, 4, [1, 1, 1, 1, 1])  # capacity 4 < 8
    assert e.value.status == ops.QKN_ERESIDENCY
    p = ops.plan_fused("bf16", 100000, 4096, 4096, 8, 4, [2, 2, 2, 2, 2])  # capacity exactly 8
    assert p["grid"] == 8 and p["n_groups"] == 1


def test_plan_split_fallbacks():
    assert ops.plan_fused("bf16", 64, 4096, 4096, 4, CU, BPC, aligned=False)["variant"] == -1
    assert ops.plan_fused("bf16", 64, 100, 100, 4, CU, BPC)["variant"] == -1  # 25-wide shards
    # rows too wide for any bf16 variant's registers
    assert ops.plan_fused("bf16", 64, 65536, 65536, 1, CU, BPC)["variant"] == -1
    # variant unusable on this device (zero occupancy): next one up is used
    p = ops.plan_fused("bf16", 64, 4096, 4096, 4, CU, [0, 3, 2, 1, 1])
    assert p["variant"] == 1


def test_plan_many_shards_uses_narrow_tiles():
    for N in (16, 32):
        p = ops.plan_fused("bf16", 4096, 4096, 4096, N, CU, BPC)
        assert p["variant"] >= 0 and N * 2 * p["rows"] <= 64
        check_plan(p, "bf16", 4096, 4096, 4096, N)


def test_plan_randomised_invariants():
    import random
    rnd = random.Random(1)
    for _ in range(3000):
        N = rnd.choice([1, 2, 3, 4, 5, 8, 16, 32])
        dt = rnd.choice(["bf16", "f32"])
        ev = 8 if dt == "bf16" else 4
        Hq = N * ev * rnd.randint(1, 600)
        Hk = N * ev * rnd.randint(1, 600)
        T = rnd.choice([1, 2, 3, 7, 63, 64, 65, 1000, 4097, rnd.randint(1, 200000)])
        cu = rnd.choice([1, 8, 80, 256])
        bpc = [rnd.randint(0, 8) for _ in range(5)]
        try:
            p = ops.plan_fused(dt, T, Hq, Hk, N, cu, bpc)
        except ops.QKNormError as e:
            assert e.status == ops.QKN_ERESIDENCY
            continue
        check_plan(p, dt, T, Hq, Hk, N, cu, bpc)
