"""Headwise QK-Norm on the HIP path against the fp64 oracle (GPU).

One factor per (token, head) over head_dim columns, gamma [head_dim] shared by
the heads ("SwiftQK ...", Section II-A). The 128-bit path reduces each head
inside its lanes; other shapes take the one-wave-per-head path. Tolerances as
for the layerwise path: 8e-3 relative for bf16, 1e-5 for fp32.
"""
import zlib

import numpy as np
import pytest
import torch

from layerwise_qk_norm_amd import inputs, ops
from oracle import compare, oracle

from _gpu import device_headwise_check, needs_gpu, to_dev, to_host

pytestmark = [pytest.mark.gpu, needs_gpu]


def run_hw(d, D, eps):
    q, k = to_dev(d["q"]), to_dev(d["k"])
    oq, ok = ops.headwise_fwd(q, k, to_dev(d["gamma_q"]), to_dev(d["gamma_k"]), D, eps)
    torch.cuda.synchronize()
    return to_host(oq), to_host(ok)


def assert_hw_parity(x, g, D, out, eps, what=""):
    worst = 0.0
    for lo in range(0, x.shape[0], 4096):
        y, _ = oracle.headwise(x[lo:lo + 4096], g, D, eps, threads=8)
        worst = compare.fold_max(worst, compare.report(compare.decode_out(out[lo:lo + 4096]), y)["max_rel"])
    tol = compare.TOL["bf16" if out.dtype == np.uint16 else "f32"]
    assert worst <= tol, f"{what}: max rel err {worst:.3e} > {tol}"
    return worst


REDUCED = {"hw_tiny": 8, "hw_decode": 64, "hw_prefill": 389, "hw_gqa": 1001}


@pytest.mark.parametrize("name", list(REDUCED))
def test_reduced(name):
    w = inputs.HW_CONFIGS[name].with_T(REDUCED[name])
    d = inputs.make_host(w)
    oq, ok = run_hw(d, w.head_dim, w.eps)
    assert_hw_parity(d["q"], d["gamma_q"], w.head_dim, oq, w.eps, f"{name} q")
    assert_hw_parity(d["k"], d["gamma_k"], w.head_dim, ok, w.eps, f"{name} k")


@pytest.mark.parametrize("name", ["hw_decode", "hw_prefill", "hw_gqa"])
def test_full_size_all_rows(name):
    w = inputs.HW_CONFIGS[name]
    d = inputs.make_host(w)
    oq, ok = run_hw(d, w.head_dim, w.eps)
    assert_hw_parity(d["q"], d["gamma_q"], w.head_dim, oq, w.eps, f"{name} q")
    assert_hw_parity(d["k"], d["gamma_k"], w.head_dim, ok, w.eps, f"{name} k")


@pytest.mark.parametrize("D,dt", [(96, "bf16"), (100, "bf16"), (48, "f32"), (1024, "bf16"),
                                  (8, "bf16"), (4, "f32"), (512, "bf16"), (256, "f32")])
def test_head_dims_and_scalar_path(D, dt):
    """Powers of two from 1 to 64 vectors per head take the 128-bit path (8, 4, 512, 256);
    the rest (96: 12 vectors, 100: not whole vectors, 48 fp32: 12, 1024: 128) the
    one-wave-per-head path."""
    w = inputs.Workload("hw_dims", 37, 8 * D, 2 * D, 1, dt, norm="head", head_dim=D)
    d = inputs.make_host(w)
    oq, ok = run_hw(d, D, w.eps)
    assert_hw_parity(d["q"], d["gamma_q"], D, oq, w.eps, f"D={D} q")
    assert_hw_parity(d["k"], d["gamma_k"], D, ok, w.eps, f"D={D} k")


def test_unaligned_pointers_take_the_scalar_path():
    w = inputs.HW_DECODE.with_T(20)
    d = inputs.make_host(w)
    k = to_dev(d["k"])
    buf = torch.empty(20 * w.Hq + 1, dtype=torch.bfloat16, device="cuda:0")
    qo = buf[1:].view(20, w.Hq)  # contiguous, at a 2-byte offset from 16-byte alignment
    qo.copy_(to_dev(d["q"]))
    assert qo.data_ptr() % 16 == 2
    oq, ok = ops.headwise_fwd(qo, k, to_dev(d["gamma_q"]), to_dev(d["gamma_k"]), w.head_dim, w.eps)
    torch.cuda.synchronize()
    assert_hw_parity(d["q"], d["gamma_q"], w.head_dim, to_host(oq), w.eps, "unaligned q")
    assert_hw_parity(d["k"], d["gamma_k"], w.head_dim, to_host(ok), w.eps, "unaligned k")


def test_heads_are_independent_and_paths_agree_on_dyadic_inputs():
    """On values k/8 every sum of squares is exact, so the 128-bit path and the
    one-wave-per-head path agree bit for bit; changing one head changes no other."""
    rng = np.random.default_rng(0)
    T, nh, D = 33, 16, 128
    x = inputs.f32_to_bf16_bits((rng.integers(-16, 17, (T, nh * D)) / 8.0).astype(np.float32))
    g = inputs.f32_to_bf16_bits(rng.uniform(0.5, 1.5, D).astype(np.float32))
    a, _ = run_hw({"q": x, "k": x[:, :4 * D].copy(), "gamma_q": g, "gamma_k": g}, D, 1e-6)
    # the same heads through the scalar path: shift the data by one element in a bigger buffer
    buf = torch.empty(T * nh * D + 1, dtype=torch.bfloat16, device="cuda:0")
    xo = buf[1:].view(T, nh * D)
    xo.copy_(to_dev(x))
    b, _ = ops.headwise_fwd(xo, to_dev(x[:, :4 * D].copy()), to_dev(g), to_dev(g), D, 1e-6)
    assert np.array_equal(a, to_host(b))
    x2 = x.copy()
    x2[:, 5 * D:6 * D] = inputs.f32_to_bf16_bits(rng.standard_normal((T, D)).astype(np.float32))
    c, _ = run_hw({"q": x2, "k": x[:, :4 * D].copy(), "gamma_q": g, "gamma_k": g}, D, 1e-6)
    keep = np.r_[0:5 * D, 6 * D:nh * D]
    assert np.array_equal(a[:, keep], c[:, keep])


def test_in_place_empty_and_errors():
    w = inputs.HW_DECODE.with_T(9)
    d = inputs.make_host(w)
    q, k = to_dev(d["q"]), to_dev(d["k"])
    ops.headwise_fwd(q, k, to_dev(d["gamma_q"]), to_dev(d["gamma_k"]), w.head_dim, w.eps,
                     out_q=q, out_k=k)
    torch.cuda.synchronize()
    assert_hw_parity(d["q"], d["gamma_q"], w.head_dim, to_host(q), w.eps, "in place")
    e = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda:0")
    g = torch.ones(128, dtype=torch.bfloat16, device="cuda:0")
    ops.headwise_fwd(e, e.clone(), g, g, 128)
    L = ops.lib()
    s = torch.cuda.current_stream().cuda_stream
    p = to_dev(d["q"])
    for bad in ((0, 32, 128), (32, 0, 128), (32, 32, 0)):
        assert L.qknorm_headwise_fwd_bf16(p.data_ptr(), p.data_ptr(), g.data_ptr(), g.data_ptr(),
                                          9, *bad, 1e-6, p.data_ptr(), p.data_ptr(), s) == ops.QKN_EINVAL
    # out_q overlapping k partially
    assert L.qknorm_headwise_fwd_bf16(p.data_ptr(), p.data_ptr() + 1024, g.data_ptr(), g.data_ptr(),
                                      2, 4, 4, 128, 1e-6, p.data_ptr() + 512, p.data_ptr() + 4096,
                                      s) == ops.QKN_EOVERLAP


SWEEP = list(inputs.sweep_headwise())


@pytest.mark.parametrize("w", SWEEP, ids=[w.name for w in SWEEP])
def test_sweep_full_size(w):
    torch.cuda.empty_cache()
    q = inputs.make_device_activations(w, "q", "cuda:0", torch)
    k = inputs.make_device_activations(w, "k", "cuda:0", torch)
    hd = inputs.make_host(w.with_T(1))
    gq, gk = to_dev(hd["gamma_q"]), to_dev(hd["gamma_k"])
    oq, ok = ops.headwise_fwd(q, k, gq, gk, w.head_dim, w.eps)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, w.T // 2, w.T - 1],
                                     np.random.default_rng(zlib.crc32(w.name.encode()))
                                     .integers(0, w.T, 40)]))
    idx = torch.as_tensor(rows, device="cuda:0")
    D = w.head_dim
    for x, g, y, gh in ((q, gq, oq, hd["gamma_q"]), (k, gk, ok, hd["gamma_k"])):
        assert_hw_parity(to_host(x.index_select(0, idx)), gh, D, to_host(y.index_select(0, idx)),
                         w.eps, w.name)
        # every element of every head against a plain fp64 reference on the device
        device_headwise_check(x, g, y, D, w.eps, compare.TOL[w.dtype], w.name)
    del q, k, oq, ok
