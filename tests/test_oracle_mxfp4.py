"""Pins of the oracle's 4-bit float (MXFP4) variant against what its definition fixes (CPU only).

The rule (a reading: the pages name a 4-bit float precision beside INT4 but do not define it; the
CDNA4 matrix cores take the OCP Microscaling formats, so the variant is MXFP4): E2M1 elements, one
E8M0 scale 2^e per block of 32 along K with e = floor(log2(absmax)) - 2, elements rounded to the
nearest E2M1 value with ties to the even mantissa and saturated at 6. Each test checks the oracle
against hand-worked cases, a pure-Python evaluation with exact rationals, or an invariant.
"""
import math
import os
from fractions import Fraction

import numpy as np

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
# E2M1 magnitudes as the OCP MX specification lists them (sign bit separate)
SPEC_MAGNITUDES = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
                   Fraction(6)]


def py_block_rule(vals):
    """The block rule element by element with Python scalars and exact rationals."""
    amax = max(abs(v) for v in vals)
    if amax == 0.0:
        e = -127
    else:
        m, ex = math.frexp(amax)       # amax = m 2^ex, m in [0.5, 1)
        e = max(-127, min(127, ex - 1 - 2))
    X = Fraction(2) ** e
    codes = []
    for v in vals:
        q = abs(Fraction(v) / X)
        if q > 6:
            mag = 7
        else:
            d = [abs(q - g) for g in SPEC_MAGNITUDES]
            best = min(d)
            cand = [c for c in range(8) if d[c] == best]
            mag = cand[0] if len(cand) == 1 else [c for c in cand if c % 2 == 0][0]
        sign = 1 if math.copysign(1.0, v) < 0 else 0
        codes.append((sign << 3) | mag)
    return e + 127, codes


def test_e2m1_decode_matches_the_specification_table():
    vals = oracle.e2m1_decode(np.arange(16))
    for c in range(16):
        mag = SPEC_MAGNITUDES[c & 7]
        assert Fraction(float(vals[c])) == (-mag if c >= 8 else mag), c


def _parse_runs(text):
    out = []
    for item in text.split():
        v, n = item.split("*")
        out += [float(v)] * int(n)
    return out


def test_golden_cases():
    n = 0
    for line in open(os.path.join(GOLDEN, "mxfp4_rule_cases.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        lhs, rhs = line.split("->")
        byte_s, elems_s = rhs.split("|")
        vals = _parse_runs(lhs)
        assert len(vals) == 32
        codes, scales = oracle.mxfp4_quantize_rows(np.array([vals], np.float32))
        assert int(scales[0, 0]) == int(byte_s), line
        expect = _parse_runs(elems_s)
        got = oracle.e2m1_decode(codes[0])
        assert np.array_equal(got, np.array(expect)), (line, got)
        n += 1
    assert n == 5


def test_rule_matches_pure_python_brute_force():
    rng = np.random.default_rng(3)
    rows = [rng.standard_normal(32) * 10.0 ** rng.integers(-6, 6) for _ in range(60)]
    # values on and around the E2M1 midpoints of a block with absmax 6 (X = 1)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for d in (0.0, 2 ** -20, -2 ** -20):
        r = np.concatenate([[6.0], mids + d, -(mids + d), rng.uniform(-6, 6, 32 - 15)])
        rows.append(r)
    rows.append(np.concatenate([[7.99], rng.uniform(6.0, 7.99, 31)]))           # saturation
    rows.append(np.full(32, 1e-40))                                                # subnormal absmax
    rows.append(np.concatenate([[-0.0], np.zeros(31)]))                            # signed zeros
    v = np.array(rows, dtype=np.float32)
    codes, scales = oracle.mxfp4_quantize_rows(v)
    for i, row in enumerate(v.tolist()):
        byte, c = py_block_rule(row)
        assert int(scales[i, 0]) == byte, i
        assert codes[i].tolist() == c, i


def test_grid_values_are_fixed_points():
    rng = np.random.default_rng(5)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    for _ in range(200):
        e = int(rng.integers(-100, 100))
        g = rng.choice(grid, 32) * rng.choice([-1.0, 1.0], 32)
        g[rng.integers(32)] = rng.choice([4.0, 6.0, -4.0, -6.0])                 # absmax in [4, 8)
        v = np.ldexp(g, e).astype(np.float32)
        codes, scales = oracle.mxfp4_quantize_rows(v[None, :])
        assert int(scales[0, 0]) == e + 127
        assert np.array_equal(oracle.mxfp4_dequant(codes, scales)[0], v.astype(np.float64))


def test_power_of_two_covariance_and_sign_symmetry():
    rng = np.random.default_rng(7)
    v = (rng.standard_normal((40, 96)) * 3).astype(np.float32)
    c0, s0 = oracle.mxfp4_quantize_rows(v)
    for j in (-20, -1, 1, 13):
        c, s = oracle.mxfp4_quantize_rows(np.ldexp(v, j).astype(np.float32))
        assert np.array_equal(c, c0) and np.array_equal(s.astype(int), s0.astype(int) + j)
    cn, sn = oracle.mxfp4_quantize_rows(-v)
    assert np.array_equal(cn, c0 ^ 8) and np.array_equal(sn, s0)


def test_error_bound_and_saturation():
    rng = np.random.default_rng(9)
    v = (rng.standard_normal((200, 64)) * rng.uniform(0.01, 100, (200, 1))).astype(np.float32)
    codes, scales = oracle.mxfp4_quantize_rows(v)
    X = np.repeat(np.ldexp(1.0, scales.astype(int) - 127), 32, axis=1)
    dq = oracle.mxfp4_dequant(codes, scales)
    q = np.abs(v.astype(np.float64)) / X
    err = np.abs(dq - v)
    # below 6 the nearest grid point is within half the widest gap (4 -> 6): X; saturated values
    # (6 <= q < 8) lose less than 2X
    assert np.all(err[q <= 6] <= X[q <= 6])
    assert np.all(q < 8)
    assert np.all(err[q > 6] < 2 * X[q > 6])
    assert np.all(np.abs(dq[q > 6]) == 6 * X[q > 6])
    # every block's absmax lands in [4, 8) X: its element is 4 or 6
    qb = q.reshape(200, 2, 32).max(axis=2)
    assert np.all((qb >= 4) & (qb < 8))


def test_product_matches_triple_loop():
    rng = np.random.default_rng(13)
    M, K, N = 5, 64, 7
    a = (rng.standard_normal((M, K)) * 2).astype(np.float32)
    w = (rng.standard_normal((K, N)) * 0.05).astype(np.float32)
    qa, sa = oracle.mxfp4_quantize_rows(a)
    qw, sw = oracle.quantize_weights_mxfp4(w)
    y, _ = oracle.svdq_linear_mxfp4(qa, sa, qw, sw)
    for m in range(M):
        for n in range(N):
            ref = Fraction(0)
            for k in range(K):
                va = SPEC_MAGNITUDES[int(qa[m, k]) & 7] * (-1 if qa[m, k] & 8 else 1) * Fraction(2) ** (int(sa[m, k // 32]) - 127)
                vw = SPEC_MAGNITUDES[int(qw[n, k]) & 7] * (-1 if qw[n, k] & 8 else 1) * Fraction(2) ** (int(sw[n, k // 32]) - 127)
                ref += va * vw
            assert abs(Fraction(y[m, n]) - ref) <= abs(ref) * Fraction(1, 2 ** 50), (m, n)


def test_zero_residual_and_rank_zero():
    cfg = synth.LayerConfig("mx", 48, 128, 64, 16, seed=21, n_outliers=2, outlier_scale=20.0)
    inp = synth.make_layer_inputs(cfg)
    x = synth.f32_from_bf16_bits(inp["x"])
    w = synth.f32_from_bf16_bits(inp["w"])
    b = synth.f32_from_bf16_bits(inp["bias"])
    d = oracle.svdq_decompose(x, w, cfg.rank)
    out = oracle.svdq_layer_mxfp4(x, d["inv"], d["l1_bf16"], d["l2_bf16"], np.zeros_like(d["resid"]), b)
    # R = 0: every weight block is all zeros (byte 0, codes 0) and Y is the low-rank part plus the bias
    assert np.all(out["sw"] == 0) and np.all(out["qw"] == 0)
    ref = out["t"].astype(np.float64) @ d["l2_bf16"].astype(np.float64) + b.astype(np.float64)[None, :]
    assert np.array_equal(out["y64"], ref)
    # r = 0: the layer is the dequantized MXFP4 product alone
    d0 = oracle.svdq_decompose(x, w, 0)
    out0 = oracle.svdq_layer_mxfp4(x, d0["inv"], d0["l1_bf16"], d0["l2_bf16"], d0["resid"], None)
    assert out0["t"] is None
    assert np.allclose(out0["y64"], oracle.mxfp4_dequant(out0["qa"], out0["sa"]) @
                       oracle.mxfp4_dequant(out0["qw"], out0["sw"]).T, rtol=0, atol=0)
