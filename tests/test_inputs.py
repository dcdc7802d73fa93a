"""The seeded input generator: reproducibility, rounding and structure (CPU)."""
import numpy as np
import pytest

from layerwise_qk_norm_amd import inputs


def test_same_seed_same_bits_other_seed_differs():
    w = inputs.DECODE.with_T(8)
    a, b = inputs.make_host(w), inputs.make_host(w)
    for key in a:
        assert np.array_equal(a[key], b[key])
    c = inputs.make_host(inputs.Workload("x", 8, 4096, 4096, 4, "bf16", seed=1))
    assert not np.array_equal(a["q"], c["q"])


def test_prefix_rows_equal_smaller_draw():
    for w in (inputs.PREFILL, inputs.GQA):
        small = inputs.make_host(w.with_T(5))
        big = inputs.make_host(w.with_T(37), chunk_rows=16)
        assert np.array_equal(big["q"][:5], small["q"])
        assert np.array_equal(big["k"][:5], small["k"])
        assert np.array_equal(big["gamma_q"], small["gamma_q"])


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(100000) * 10).astype(np.float32)
    # exact ties between two bf16 values, both parities, and specials
    base = inputs.bf16_bits_to_f32(np.arange(0x3F80, 0x3FA0, dtype=np.uint16))
    ties = (base.view(np.uint32) + np.uint32(0x8000)).view(np.float32)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, 1e-40, -1e-45], np.float32)
    a = np.concatenate([a, ties, specials])
    ours = inputs.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    nan = inputs.f32_to_bf16_bits(np.array([np.nan], np.float32))
    assert (int(nan[0]) & 0x7FC0) == 0x7FC0


def test_outlier_columns_count_and_scale():
    w = inputs.DECODE
    cols = inputs.outlier_columns(w, "q")
    assert len(cols) == 41 and len(np.unique(cols)) == 41
    g = inputs.GQA
    assert len(inputs.outlier_columns(g, "q")) == 26
    assert len(inputs.outlier_columns(g, "k")) == 5
    assert inputs.outlier_columns(inputs.PREFILL, "q") is None
    d = inputs.make_host(w.with_T(64))
    x = inputs.bf16_bits_to_f32(d["q"]).astype(np.float64)
    mask = np.zeros(w.Hq, bool)
    mask[cols] = True
    assert 15 < x[:, mask].std() < 25
    assert 0.9 < x[:, ~mask].std() < 1.1


def test_distributions():
    d = inputs.make_host(inputs.PREFILL.with_T(64))
    x = inputs.bf16_bits_to_f32(d["q"]).astype(np.float64)
    assert 1.9 < x.std() < 2.1
    g = inputs.bf16_bits_to_f32(d["gamma_q"])
    assert g.min() >= 0.5 and g.max() <= 1.5
    t = inputs.make_host(inputs.Workload("t", 256, 1024, 1024, 1, "f32", dist="t3"))["q"]
    # Student-t(3): median |x| = 0.7649, heavy tails
    assert abs(np.median(np.abs(t)) - 0.765) < 0.02
    assert np.abs(t).max() > 20
    tiny = inputs.make_host(inputs.TINY)
    assert tiny["q"].dtype == np.float32 and tiny["q"].shape == (8, 256)
    assert 0.6 < tiny["gamma_q"].mean() < 1.4 and tiny["gamma_q"].std() < 0.2


def test_sweep_grid_and_bytes():
    pts = list(inputs.sweep())
    assert len(pts) == 320
    assert inputs.PREFILL.algorithmic_bytes() == 671_109_120
    assert inputs.DECODE.algorithmic_bytes() == 2_113_536
    assert inputs.GQA.algorithmic_bytes() == 201_338_880
    assert inputs.TINY.algorithmic_bytes() == 34_816


def test_e4m3_workloads():
    assert len(list(inputs.sweep_e4m3())) == 160
    w = inputs.PREFILL_E4M3
    assert w.fmt == "e4m3_bf16" and w.gamma_dtype == "bf16" and w.out_bytes == 2
    # 1 byte read + 2 bytes written per element, gamma in bf16
    assert w.algorithmic_bytes() == 16384 * 10240 * 3 + 10240 * 2
    assert inputs.DECODE_E4M3.fmt == "e4m3_e4m3"
    assert inputs.DECODE_E4M3.algorithmic_bytes() == 64 * 8192 * 2 + 8192 * 2
    d = inputs.make_host(w.with_T(32))
    assert d["q"].dtype == np.uint8 and d["gamma_q"].dtype == np.uint16
    codes = d["q"]
    assert not np.any((codes & 0x7F) == 0x7F), "no NaN codes"
    # codes are the nearest E4M3 values of the float32 draws of the q stream
    torch = pytest.importorskip("torch")
    a = (np.random.default_rng(np.random.SeedSequence(w.seed).spawn(6)[0])
         .standard_normal((32, w.Hq)) * w.sigma).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def test_e4m3_clipping_and_transfer_round_trip():
    torch = pytest.importorskip("torch")
    big = np.array([1000.0, -1e6, 448.0, 449.0, 0.0], np.float32)
    c = inputs.f32_to_e4m3_codes(big)
    assert list(c) == [0x7E, 0xFE, 0x7E, 0x7E, 0x00]
    t = inputs.to_device(c, "cpu", torch)
    assert t.dtype == torch.float8_e4m3fn
    assert np.array_equal(inputs.from_device(t), c)
