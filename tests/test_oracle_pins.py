"""Pins of the CPU oracle against what the method and plain mathematics fix (CPU only).

Each test checks the oracle against something other than itself: hand-worked cases, closed
forms, invariants, brute force in pure Python, or an independent library routine.
"""
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------------------------
# pure-Python helpers (independent of numpy's float32 arithmetic)
# ---------------------------------------------------------------------------------------------
def f32(v: float) -> float:
    """Round a Python float (binary64) to the nearest binary32 value."""
    return struct.unpack("f", struct.pack("f", v))[0]


def f32_div(a: float, b: float) -> float:
    # binary64 quotient then rounding to binary32 equals the correctly rounded binary32 quotient,
    # because 53 >= 2*24 + 2 (double rounding is innocuous for division at these precisions).
    return f32(a / b)


def py_rule_group(vals):
    """The INT4 group rule evaluated element by element with Python scalars."""
    amax = max(abs(v) for v in vals)
    s = f32_div(amax, 7.0)
    if s == 0.0:
        return s, [0] * len(vals)
    codes = []
    for v in vals:
        q = f32_div(v, s)
        c = round(q)  # Python's round() is round-half-to-even
        codes.append(max(-8, min(7, int(c))))
    return s, codes


def bf16_candidates(x: float):
    """The two bf16 neighbours of a float32 value (truncate, truncate + 1 ulp)."""
    u = struct.unpack("I", struct.pack("f", x))[0]
    lo = u & 0xFFFF0000
    hi = lo + 0x10000
    flo = struct.unpack("f", struct.pack("I", lo))[0]
    fhi = struct.unpack("f", struct.pack("I", hi & 0xFFFFFFFF))[0]
    return (flo, lo >> 16), (fhi, (hi >> 16) & 0xFFFF)


def bf16_nearest_by_definition(x: float) -> float:
    (a, abits), (b, bbits) = bf16_candidates(x)
    da, db = abs(Fraction(x) - Fraction(a)), abs(Fraction(x) - Fraction(b))
    if da < db:
        return a
    if db < da:
        return b
    return a if abits % 2 == 0 else b


# ---------------------------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------------------------
def test_bf16_round_matches_definition():
    rng = np.random.default_rng(11)
    vals = np.concatenate([
        rng.standard_normal(3000).astype(np.float32),
        (rng.standard_normal(500) * 1e-30).astype(np.float32),
        np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0, 2 ** -130], np.float32),
    ])
    got = oracle.bf16_round(vals)
    for v, g in zip(vals.tolist(), got.tolist()):
        assert g == bf16_nearest_by_definition(v), v


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 lies exactly between 1 and 1 + 2^-7: the even neighbour is 1.
    assert oracle.bf16_round(np.float32(1.0 + 2 ** -8)) == 1.0
    # 1 + 3*2^-8 lies between 1 + 2^-7 (odd) and 1 + 2^-6 (even).
    assert oracle.bf16_round(np.float32(1.0 + 3 * 2 ** -8)) == np.float32(1.0 + 2 ** -6)


# ---------------------------------------------------------------------------------------------
# INT4 group rule
# ---------------------------------------------------------------------------------------------
def _parse_rle(s):
    out = []
    for item in s.split():
        v, n = item.split("*")
        out += [float(v)] * int(n)
    return out


def test_golden_hand_worked_groups():
    cases = []
    with open(os.path.join(GOLDEN, "int4_rule_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split("->")
            scale_s, codes_s = rhs.split("|")
            vals = _parse_rle(lhs)
            codes = [int(c) for c in _parse_rle(codes_s)]
            assert len(vals) == 64 and len(codes) == 64
            cases.append((vals, float(scale_s), codes))
    assert len(cases) == 4
    for vals, scale, codes in cases:
        c, s = oracle.int4_quantize_rows(np.array([vals], np.float32))
        assert s[0, 0] == np.float32(scale)
        assert c[0].tolist() == codes


def test_grid_values_are_fixed_points():
    """Quantize->dequantize is the identity on values already on the INT4 grid."""
    rng = np.random.default_rng(3)
    for e in range(-20, 21, 3):
        s = 2.0 ** e
        c = rng.integers(-7, 8, size=(5, 64))
        c[:, 5] = np.where(rng.random(5) < 0.5, 7, -7)    # every group attains |code| = 7
        v = (c * s).astype(np.float32)
        codes, scales = oracle.int4_quantize_rows(v)
        assert np.array_equal(codes, c)
        assert np.all(scales == np.float32(s))
        assert np.array_equal((codes.astype(np.float64) * scales.repeat(64, axis=1)), v.astype(np.float64))


def test_power_of_two_covariance_and_sign_symmetry():
    rng = np.random.default_rng(4)
    v = (rng.standard_normal((16, 256)) * rng.uniform(0.01, 10, size=(16, 1))).astype(np.float32)
    c0, s0 = oracle.int4_quantize_rows(v)
    for j in (-7, -1, 1, 5):
        c1, s1 = oracle.int4_quantize_rows((v * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(c0, c1)
        assert np.array_equal(s1, (s0 * np.float32(2.0 ** j)).astype(np.float32))
    cn, sn = oracle.int4_quantize_rows(-v)
    assert np.array_equal(cn, -c0)
    assert np.array_equal(sn, s0)


def test_normal_scale_groups_hit_seven_and_never_minus_eight():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((64, 1024)).astype(np.float32)
    c, s = oracle.int4_quantize_rows(v)
    cg = c.reshape(64, 16, 64)
    assert np.all(np.max(np.abs(cg), axis=2) == 7)
    assert c.min() >= -7


def test_rule_brute_force_per_element():
    rng = np.random.default_rng(6)
    v = (rng.standard_normal((6, 192)) * np.float32(3.0)).astype(np.float32)
    v[0, :64] *= np.float32(1e-3)
    v[1, 64:128] = 0.0
    c, s = oracle.int4_quantize_rows(v)
    for r in range(v.shape[0]):
        for g in range(3):
            vals = [float(x) for x in v[r, 64 * g:64 * g + 64]]
            ps, pc = py_rule_group(vals)
            assert float(s[r, g]) == ps
            assert c[r, 64 * g:64 * g + 64].tolist() == pc


def test_subnormal_scale_reaches_clamp():
    """With a subnormal scale the quotient can exceed 7.5 and the clamp (to -8 / 7) is live."""
    # absmax = 2^-147 * 9 -> amax/7 rounds to a subnormal whose relative error is large.
    tiny = np.float32(9 * 2.0 ** -149)
    vals = np.zeros(64, np.float32)
    vals[0] = -tiny
    vals[1] = tiny
    vals[2] = np.float32(5 * 2.0 ** -149)
    c, s = oracle.int4_quantize_rows(vals[None, :])
    ps, pc = py_rule_group([float(x) for x in vals])
    assert float(s[0, 0]) == ps and ps != 0.0
    assert c[0].tolist() == pc
    assert c[0, 0] == -8 and c[0, 1] == 7          # 9/1 -> clamp(9) on both sides of the range


def test_zero_group_rule():
    v = np.zeros((2, 128), np.float32)
    v[1, 64:] = np.float32(2.0 ** -149)            # amax/7 underflows to 0 -> zero group too
    c, s = oracle.int4_quantize_rows(v)
    assert np.all(c == 0) and np.all(s == 0)


def test_weight_quantization_is_along_k_per_column():
    rng = np.random.default_rng(7)
    r = rng.standard_normal((128, 24)).astype(np.float32)
    qw, sw = oracle.quantize_weights_w4a4(r)
    assert qw.shape == (128, 24) and sw.shape == (2, 24)
    for n in range(24):
        for g in range(2):
            ps, pc = py_rule_group([float(x) for x in r[64 * g:64 * g + 64, n]])
            assert float(sw[g, n]) == ps
            assert qw[64 * g:64 * g + 64, n].tolist() == pc


# ---------------------------------------------------------------------------------------------
# group sums and the dequantized product
# ---------------------------------------------------------------------------------------------
def test_group_sums_brute_force_and_closed_form():
    rng = np.random.default_rng(8)
    qa = rng.integers(-8, 8, size=(5, 128)).astype(np.int8)
    qw = rng.integers(-8, 8, size=(128, 7)).astype(np.int8)
    P = oracle.group_sums(qa, qw)
    assert P.shape == (2, 5, 7)
    for g in range(2):
        for m in range(5):
            for n in range(7):
                s = 0
                for k in range(64 * g, 64 * g + 64):
                    s += int(qa[m, k]) * int(qw[k, n])
                assert P[g, m, n] == s
    ones = oracle.group_sums(np.ones((3, 192), np.int8), np.ones((192, 4), np.int8))
    assert np.all(ones == 64)
    ext = oracle.group_sums(np.full((1, 64), -8, np.int8), np.full((64, 1), -8, np.int8))
    assert ext[0, 0, 0] == 4096


def test_dequant_product_triple_loop():
    rng = np.random.default_rng(9)
    M, K, N = 6, 128, 5
    qa = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(K, N)).astype(np.int8)
    sa = rng.uniform(0.01, 1, size=(K // 64, M)).astype(np.float32)
    sw = rng.uniform(0.001, 0.1, size=(K // 64, N)).astype(np.float32)
    y = oracle.dequant_product(qa, sa, qw, sw)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(qa[m, k]) * float(sa[k // 64, m]) * float(qw[k, n]) * float(sw[k // 64, n])
            assert abs(y[m, n] - acc) <= 1e-12 * max(1.0, abs(acc))
    # closed form: all codes 1, unit scales -> every output equals K
    y1 = oracle.dequant_product(np.ones((2, K), np.int8), np.ones((2, 2), np.float32),
                                np.ones((K, 3), np.int8), np.ones((2, 3), np.float32))
    assert np.all(y1 == K)


def _small_problem(seed=12, M=32, K=128, N=48, r=16):
    rng = np.random.default_rng(seed)
    x = oracle.bf16_round(rng.standard_normal((M, K)).astype(np.float32))
    x[:, 3] *= 20
    x = oracle.bf16_round(x)
    w = oracle.bf16_round((rng.standard_normal((K, N)) * 0.02).astype(np.float32))
    b = oracle.bf16_round((rng.standard_normal(N) * 0.01).astype(np.float32))
    return x, w, b, r


def test_zero_residual_leaves_lowrank_plus_bias():
    """R = 0 => the 4-bit branch contributes nothing: Y = T L2 + b (checked by explicit loops)."""
    x, w, b, r = _small_problem()
    d = oracle.svdq_decompose(x, w, r)
    out = oracle.svdq_layer(x, d["inv"], d["l1_bf16"], d["l2_bf16"], np.zeros_like(d["resid"]), b)
    assert np.all(out["qw"] == 0) and np.all(out["sw"] == 0)
    t, l2 = out["t"], d["l2_bf16"]
    M, N = out["y64"].shape
    for m in range(0, M, 7):
        for n in range(0, N, 5):
            ref = sum(float(t[m, j]) * float(l2[j, n]) for j in range(r)) + float(b[n])
            assert abs(out["y64"][m, n] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_rank_zero_is_pure_w4a4_plus_bias():
    x, w, b, _ = _small_problem()
    d = oracle.svdq_decompose(x, w, 0)
    assert np.array_equal(d["resid"], d["w_hat"].astype(np.float32))
    qa, sa, t = oracle.quantize_activations(x, d["inv"], None)
    qw, sw = oracle.quantize_weights_w4a4(d["resid"])
    y64, _ = oracle.svdq_linear(qa, sa, qw, sw, None, None, b)
    P = oracle.group_sums(qa, qw)
    ref = np.einsum("gmn,gm,gn->mn", P.astype(np.float64), sa.astype(np.float64), sw.astype(np.float64)) + b
    assert np.allclose(y64, ref, rtol=1e-12, atol=1e-15)


def test_lowrank_down_brute_force():
    rng = np.random.default_rng(13)
    xh = (rng.standard_normal((4, 64)) * 3).astype(np.float32)
    l1 = oracle.bf16_round(rng.standard_normal((64, 16)).astype(np.float32))
    t = oracle.lowrank_down(xh, l1)
    for m in range(4):
        for j in range(16):
            acc = 0.0
            for k in range(64):
                acc += bf16_nearest_by_definition(float(xh[m, k])) * float(l1[k, j])
            assert t[m, j] == bf16_nearest_by_definition(f32(acc))


def test_activation_step_fuses_independent_pieces():
    """Engine figure (b): the fused down-projection + quantize equals the two pieces run apart."""
    x, w, b, r = _small_problem()
    d = oracle.svdq_decompose(x, w, r)
    qa, sa, t = oracle.quantize_activations(x, d["inv"], d["l1_bf16"])
    xh = (x * d["inv"]).astype(np.float32)
    for m in range(0, x.shape[0], 5):
        for g in range(x.shape[1] // 64):
            ps, pc = py_rule_group([float(f32(float(x[m, k]) * float(d["inv"][k])))
                                    for k in range(64 * g, 64 * g + 64)])
            assert float(sa[g, m]) == ps
            assert qa[m, 64 * g:64 * g + 64].tolist() == pc
    assert np.array_equal(t, oracle.lowrank_down(xh, d["l1_bf16"]))


# ---------------------------------------------------------------------------------------------
# offline preparation: smoothing and truncated SVD
# ---------------------------------------------------------------------------------------------
def test_smoothing_identity_and_degenerate_channels():
    x, w, _, _ = _small_problem()
    x = x.copy()
    x[:, 7] = 0.0                                    # a dead channel -> lambda = 1
    inv, lam = oracle.smoothing_factors(x, w)
    assert inv[7] == np.float32(1.0) and lam[7] == 1.0
    xs = x.astype(np.float64) * inv.astype(np.float64)
    ws = lam[:, None] * w.astype(np.float64)
    assert np.allclose(xs @ ws, x.astype(np.float64) @ w.astype(np.float64), rtol=1e-12, atol=1e-13)
    # smoothing equalises channel ranges: max|x_k|/lambda_k == max|w_k|*lambda_k (up to rounding)
    k = 3
    a = np.max(np.abs(x[:, k])) / math.sqrt(np.max(np.abs(x[:, k])) / np.max(np.abs(w[k])))
    bb = np.max(np.abs(w[k])) * math.sqrt(np.max(np.abs(x[:, k])) / np.max(np.abs(w[k])))
    assert abs(a - bb) <= 1e-12 * a


def test_truncated_svd_eckart_young():
    x, w, _, r = _small_problem(K=128, N=96)
    d = oracle.svdq_decompose(x, w, r)
    res64 = d["w_hat"] - d["l1"] @ d["l2"]
    s = d["sigma"]
    assert abs(np.sum(res64 ** 2) - np.sum(s[r:] ** 2)) <= 1e-9 * np.sum(s[r:] ** 2)
    # the singular values agree with an independent routine (eigenvalues of W_hat^T W_hat)
    ev = np.sort(np.linalg.eigvalsh(d["w_hat"].T @ d["w_hat"]))[::-1][: len(s)]
    assert np.allclose(np.sqrt(np.maximum(ev, 0)), s, rtol=1e-8, atol=1e-10 * s[0])
    # best rank-r approximation: no worse than a perturbed rank-r factorisation
    rng = np.random.default_rng(1)
    alt = (d["l1"] + 1e-3 * rng.standard_normal(d["l1"].shape)) @ d["l2"]
    assert np.sum((d["w_hat"] - alt) ** 2) >= np.sum(res64 ** 2)
    # the stored residual is W_hat minus the bf16 factors the runtime uses
    rec = d["resid"].astype(np.float64) + d["l1_bf16"].astype(np.float64) @ d["l2_bf16"].astype(np.float64)
    assert np.allclose(rec, d["w_hat"], rtol=0, atol=1e-6 * np.abs(d["w_hat"]).max())
    assert np.sum(d["resid"].astype(np.float64) ** 2) >= np.sum(s[r:] ** 2) * (1 - 1e-6)


def test_method_reduces_error_on_outlier_data():
    """The overview figure's claim: smoothing + low-rank make the 4-bit product more accurate."""
    cfg = synth.CONFIGS["tiny"]
    inp = synth.make_layer_inputs(cfg)
    x = synth.f32_from_bf16_bits(inp["x"])
    w = synth.f32_from_bf16_bits(inp["w"])
    exact = x.astype(np.float64) @ w.astype(np.float64)

    def err(rank, smooth=True):
        d = oracle.svdq_decompose(x, w, rank)
        if not smooth:
            d = oracle.svdq_decompose(x, w, 0) if rank == 0 else d
            inv = np.ones(x.shape[1], np.float32)
            qa, sa, _ = oracle.quantize_activations(x, inv, None)
            qw, sw = oracle.quantize_weights_w4a4(w)
            y, _ = oracle.svdq_linear(qa, sa, qw, sw)
            return np.linalg.norm(y - exact) / np.linalg.norm(exact)
        out = oracle.svdq_layer(x, d["inv"], d["l1_bf16"], d["l2_bf16"], d["resid"], None)
        return np.linalg.norm(out["y64"] - exact) / np.linalg.norm(exact)

    e_plain = err(0, smooth=False)
    e_smooth = err(0)
    e_r16 = err(16)
    assert e_smooth < e_plain
    assert e_r16 < e_smooth


# ---------------------------------------------------------------------------------------------
# W4A16 projection
# ---------------------------------------------------------------------------------------------
def test_w4a16_rule_brute_force_and_grid():
    rng = np.random.default_rng(14)
    w = (rng.standard_normal((128, 12)) * 0.02).astype(np.float32)
    w[:64, 3] = 0.0
    codes, s = oracle.quantize_weights_w4a16(w)
    for n in range(12):
        for g in range(2):
            col = [float(v) for v in w[64 * g:64 * g + 64, n]]
            amax = max(abs(v) for v in col)
            sb = bf16_nearest_by_definition(f32_div(amax, 7.0))
            assert float(s[g, n]) == sb
            exp = [0] * 64 if sb == 0 else [max(-8, min(7, int(round(f32_div(v, sb))))) for v in col]
            assert codes[64 * g:64 * g + 64, n].tolist() == exp
    # grid identity with power-of-two scales
    c = rng.integers(-7, 8, size=(64, 4))
    c[0] = 7
    wg = (c * 2.0 ** -9).astype(np.float32)
    cc, ss = oracle.quantize_weights_w4a16(wg)
    assert np.array_equal(cc, c) and np.all(ss == np.float32(2.0 ** -9))


def test_awq_linear_triple_loop():
    rng = np.random.default_rng(15)
    x = oracle.bf16_round(rng.standard_normal((3, 128)).astype(np.float32))
    codes = rng.integers(-8, 8, size=(128, 5)).astype(np.int8)
    s = oracle.bf16_round(rng.uniform(1e-3, 1e-2, size=(2, 5)).astype(np.float32))
    b = oracle.bf16_round(rng.standard_normal(5).astype(np.float32))
    y64, y = oracle.awq_linear(x, codes, s, b)
    for m in range(3):
        for n in range(5):
            acc = float(b[n])
            for k in range(128):
                acc += float(x[m, k]) * float(codes[k, n]) * float(s[k // 64, n])
            assert abs(y64[m, n] - acc) <= 1e-12 * max(1.0, abs(acc))
            assert y[m, n] == bf16_nearest_by_definition(f32(y64[m, n]))


# ---------------------------------------------------------------------------------------------
# GELU (tanh form) of the MLP path
# ---------------------------------------------------------------------------------------------
def test_gelu_tanh_against_library_and_identities():
    """Pinned to torch's tanh-form GELU in float64 (CPU), to the identity gelu(x) - gelu(-x) = x
    of this form, to gelu'(0) = 1/2, to its limits, and to the tabulated gelu_tanh(1)."""
    import torch
    x = np.concatenate([np.linspace(-12.0, 12.0, 2401), [0.0, 1e-30, -1e-30, 1e6, -1e6]])
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    got = oracle.gelu_tanh(x)
    # absolute agreement: in the negative tail 1 + tanh(u) cancels in both implementations
    assert np.all(np.abs(got - ref) <= 1e-15 * np.maximum(1.0, np.abs(x)))
    assert np.allclose(oracle.gelu_tanh(x) - oracle.gelu_tanh(-x), x, rtol=1e-12, atol=1e-12)
    h = 1e-6
    assert abs((oracle.gelu_tanh(h) - oracle.gelu_tanh(-h)) / (2 * h) - 0.5) < 1e-9
    assert oracle.gelu_tanh(0.0) == 0.0
    assert oracle.gelu_tanh(40.0) == 40.0 and oracle.gelu_tanh(-40.0) == 0.0
    assert abs(float(oracle.gelu_tanh(1.0)) - 0.8411919906082768) < 1e-15


def test_svdq_linear_gelu_is_gelu_of_the_layer():
    """The MLP form applies the activation to the unrounded layer output, then rounds to bf16
    (checked through torch's GELU on the layer's float64 output)."""
    import torch
    cfg = synth.CONFIGS["tiny"]
    inp = synth.make_layer_inputs(cfg)
    x = synth.f32_from_bf16_bits(inp["x"])
    w = synth.f32_from_bf16_bits(inp["w"])
    b = synth.f32_from_bf16_bits(inp["bias"])
    d = oracle.svdq_decompose(x, w, cfg.rank)
    out = oracle.svdq_layer(x, d["inv"], d["l1_bf16"], d["l2_bf16"], d["resid"], b)
    g64, g = oracle.svdq_linear_gelu(out["qa"], out["sa"], out["qw"], out["sw"], out["t"], d["l2_bf16"], b)
    ref = torch.nn.functional.gelu(torch.from_numpy(out["y64"]), approximate="tanh").numpy()
    assert np.all(np.abs(g64 - ref) <= 1e-15 * np.maximum(1.0, np.abs(out["y64"])))
    gr = oracle.bf16_round(ref.astype(np.float32))
    assert np.mean(g == gr) > 0.999 and np.all(np.abs(g - gr) <= 2.0 ** -8 * np.abs(gr) + 1e-30)
    # negative pre-activations shrink towards 0, positive ones stay close to themselves
    assert np.all(np.abs(g64) <= np.abs(out["y64"]) + 1e-12)


# ---------------------------------------------------------------------------------------------
# fused QKV: per-head RMS normalisation and rotary embedding of Q and K
# ---------------------------------------------------------------------------------------------
def _qkv_case(M=5, heads=3, seed=81):
    D = 128
    rng = np.random.default_rng(seed)
    y = oracle.bf16_round(rng.standard_normal((M, 3 * heads * D)).astype(np.float32) * 3.0)
    q_w = rng.uniform(0.5, 1.5, D)
    k_w = rng.uniform(0.5, 1.5, D)
    ang = rng.uniform(-np.pi, np.pi, (M, D // 2))
    return y, heads, q_w, k_w, np.cos(ang), np.sin(ang), ang


def test_qkv_norm_against_torch_rms_norm_and_identity_rotation():
    """With zero angles the Q/K parts are torch's RMS norm (float64), rounded to bf16; V passes."""
    import torch
    y, H, q_w, k_w, _, _, _ = _qkv_case()
    M, D = y.shape[0], 128
    out = oracle.qkv_norm_rope(y, H, q_w, k_w, np.ones((M, D // 2)), np.zeros((M, D // 2)))
    for part, w in ((0, q_w), (1, k_w)):
        v = torch.from_numpy(y[:, part * H * D:(part + 1) * H * D].astype(np.float64).reshape(M, H, D))
        ref = torch.nn.functional.rms_norm(v, (D,), torch.from_numpy(w), eps=1e-6).numpy().reshape(M, H * D)
        assert np.array_equal(out[:, part * H * D:(part + 1) * H * D], oracle.bf16_round(ref.astype(np.float32)))
    assert np.array_equal(out[:, 2 * H * D:], y[:, 2 * H * D:])


def test_qkv_rotary_is_a_complex_rotation_of_pairs():
    """Rotating pair (a, b) by angle t equals (a + ib) e^{it}; pair norms are preserved; rotating
    by t then by -t restores the normalised values (checked before the bf16 rounding)."""
    y, H, q_w, k_w, c, s, ang = _qkv_case(seed=82)
    M, D = y.shape[0], 128
    ones, zeros = np.ones((M, D // 2)), np.zeros((M, D // 2))
    plain = oracle.qkv_norm_rope(y, H, q_w, k_w, ones, zeros)
    rot = oracle.qkv_norm_rope(y, H, q_w, k_w, c, s)
    # recompute unrounded normalised Q to compare in float64
    v = y[:, :H * D].astype(np.float64).reshape(M, H, D)
    u = v / np.sqrt(np.mean(v * v, axis=2, keepdims=True) + 1e-6) * q_w
    z = (u[:, :, 0::2] + 1j * u[:, :, 1::2]) * np.exp(1j * ang)[:, None, :]
    ref = np.empty_like(u)
    ref[:, :, 0::2], ref[:, :, 1::2] = z.real, z.imag
    assert np.array_equal(rot[:, :H * D], oracle.bf16_round(ref.reshape(M, H * D).astype(np.float32)))
    # norms of the pairs are preserved up to the bf16 rounding of both sides
    pn = lambda a: np.hypot(a[:, 0::2], a[:, 1::2])
    assert np.allclose(pn(rot[:, :2 * H * D]), pn(plain[:, :2 * H * D]), rtol=2 ** -6, atol=1e-6)
    assert np.array_equal(rot[:, 2 * H * D:], y[:, 2 * H * D:])



def test_naive_form_reduces_to_the_fused_layer():
    """The unfused (naive) form differs from the layer only by its two extra 16-bit roundings: with a
    zero L1 the output is the fused layer's bit for bit (T = 0, Y = bf16(bf16(Y0))), and with unit
    smoothing on bf16 inputs its down projection is the fused T bit for bit (diag(inv) L1 = L1 exactly,
    bf16(X_hat) = X)."""
    cfg = synth.LayerConfig("nv", 40, 128, 96, 16, seed=17, n_outliers=2, outlier_scale=20.0)
    inp = synth.make_layer_inputs(cfg)
    x = synth.f32_from_bf16_bits(inp["x"])
    w = synth.f32_from_bf16_bits(inp["w"])
    b = synth.f32_from_bf16_bits(inp["bias"])
    d = oracle.svdq_decompose(x, w, cfg.rank)
    zero_l1 = np.zeros_like(d["l1_bf16"])
    nv = oracle.svdq_layer_naive(x, d["inv"], zero_l1, d["l2_bf16"], d["resid"], b)
    fu = oracle.svdq_layer(x, d["inv"], zero_l1, d["l2_bf16"], d["resid"], b)
    assert np.array_equal(nv["t"], np.zeros_like(nv["t"]))
    assert np.array_equal(nv["y"], fu["y"])
    ones = np.ones_like(d["inv"])
    nv1 = oracle.svdq_layer_naive(x, ones, d["l1_bf16"], d["l2_bf16"], d["resid"], b)
    fu1 = oracle.svdq_layer(x, ones, d["l1_bf16"], d["l2_bf16"], d["resid"], b)
    assert np.array_equal(nv1["l1s"], d["l1_bf16"])
    assert np.array_equal(nv1["t"], fu1["t"])
    # and the naive output is the bf16 rounding of Y0 + T L2, Y0 being the 4-bit branch's bf16 output
    y0 = oracle.bf16_round((oracle.dequant_product(fu1["qa"], fu1["sa"], fu1["qw"], fu1["sw"]) +
                            b.astype(np.float64)).astype(np.float32))
    assert np.array_equal(nv1["y0"], y0)
