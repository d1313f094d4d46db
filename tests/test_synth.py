"""The seeded input generators: determinism, shapes and the stated distributions (CPU only)."""
import numpy as np

import synth


def test_deterministic_and_shaped():
    cfg = synth.CONFIGS["tiny"]
    a = synth.make_layer_inputs(cfg)
    b = synth.make_layer_inputs(cfg)
    for k in ("x", "w", "bias", "outliers"):
        assert np.array_equal(a[k], b[k])
    assert a["x"].shape == (256, 256) and a["x"].dtype == np.uint16
    assert a["w"].shape == (256, 512) and a["bias"].shape == (512,)
    assert len(a["outliers"]) == 4 and len(set(a["outliers"].tolist())) == 4
    c = synth.make_layer_inputs(cfg, seed=1)
    assert not np.array_equal(a["x"], c["x"])


def test_outlier_channels_and_scales():
    cfg = synth.CONFIGS["tiny"]
    d = synth.make_layer_inputs(cfg)
    x = synth.f32_from_bf16_bits(d["x"]).astype(np.float64)
    std = x.std(axis=0)
    o = d["outliers"]
    rest = np.setdiff1d(np.arange(cfg.K), o)
    assert np.all(std[o] > 10) and abs(std[rest].mean() - 1) < 0.05
    w = synth.f32_from_bf16_bits(d["w"]).astype(np.float64)
    assert abs(w.std() - 0.02) < 0.001
    bias = synth.f32_from_bf16_bits(d["bias"]).astype(np.float64)
    assert abs(bias.std() - 0.01) < 0.002


def test_flux_configs_table():
    c = synth.CONFIGS
    assert (c["up"].M, c["up"].K, c["up"].N, c["up"].rank) == (4608, 3072, 12288, 32)
    assert (c["down"].K, c["down"].N, c["down"].gelu_input) == (12288, 3072, True)
    assert c["attn"].n_outliers == 31 and c["down"].n_outliers == 123
    assert [c[f"qkv_r{r}"].rank for r in (32, 128, 256)] == [32, 128, 256]
    assert c["awq"].kind == "w4a16" and not c["awq"].has_bias


def test_gelu_input_distribution():
    cfg = synth.CONFIGS["down"]
    d = synth.make_layer_inputs(cfg, M=64)
    x = synth.f32_from_bf16_bits(d["x"]).astype(np.float64)
    rest = np.setdiff1d(np.arange(cfg.K), d["outliers"])
    assert x[:, rest].min() > -0.2      # GELU(z) >= -0.17
    assert abs(x[:, rest].mean() - 0.282) < 0.02   # E[GELU(Z)] = 1/sqrt(2*pi)


def test_bf16_helpers_roundtrip():
    v = np.array([1.0, -2.5, 3.0e-5, 1.0 + 2 ** -8], np.float32)
    b = synth.bf16_bits_from_f32(v)
    f = synth.f32_from_bf16_bits(b)
    assert f[0] == 1.0 and f[1] == -2.5 and f[3] == 1.0
