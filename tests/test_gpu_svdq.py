"""GPU parity of the HIP path against the CPU oracle, through the C ABI (needs an MI355X).

Bar: INT4 codes, scales and per-group integer sums bit-exact; T within one bf16 ulp;
Y (bf16) with max|err| <= 1e-2 * max|Y_ref| and sum|err| / sum|Y_ref| <= 2e-3.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from guard import Guarded
from problems import (decode_qact, random_w4a4_problem, tolerance_report, w4a16_problem, w4a4_problem,
                      within_one_bf16_ulp)

pytestmark = pytest.mark.gpu

MAX_REL = 1e-2
MEAN_REL = 2e-3


@pytest.fixture(scope="module")
def gpu():
    import torch
    import quantized_gemm_amd as q
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    q.load_library()
    q.svdq_check_device()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev_bf16(bits: np.ndarray, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def to_dev(a: np.ndarray, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bf16_to_np(t) -> np.ndarray:
    import torch
    return synth.f32_from_bf16_bits(t.view(torch.int16).cpu().numpy().view(np.uint16))


class Layer:
    """The packed layer on the device (weights packed by the library's host packer)."""

    def __init__(self, p, dev, resid=None):
        import quantized_gemm_amd as q
        cfg = p["cfg"]
        self.r = cfg.rank
        qw, sw = q.svdq_pack_weights(q.SVDQ_FMT_W4A4_F32SCALE, p["resid"] if resid is None else resid)
        self.qw, self.sw = to_dev(qw, dev), to_dev(sw, dev)
        self.inv = to_dev(p["inv"], dev)
        if self.r:
            l1t, l2t = q.svdq_pack_lowrank(p["l1"], p["l2"])
            self.l1t, self.l2t = to_dev_bf16(l1t, dev), to_dev_bf16(l2t, dev)
        else:
            self.l1t = self.l2t = None
        self.bias = None if p["bias_bits"] is None else to_dev_bf16(p["bias_bits"], dev)

    def run(self, x_bits, dev):
        """Both kernels into outputs fenced by canary bytes (checked after the launches)."""
        import torch
        import quantized_gemm_amd as q
        x = to_dev_bf16(x_bits, dev)
        M, K = x.shape
        N = self.sw.shape[1]
        gq = Guarded((K // 64, M, 32), torch.uint8, dev)
        gs = Guarded((K // 64, M), torch.float32, dev)
        gt = Guarded((M, self.r), torch.bfloat16, dev) if self.r else None
        gy = Guarded((M, N), torch.bfloat16, dev)
        qact, ascale, t = q.svdq_quantize_act(x, self.inv, self.l1t, gq.tensor, gs.tensor,
                                              gt.tensor if self.r else None)
        y = q.svdq_linear_w4a4(qact, ascale, self.qw, self.sw, t, self.l2t, self.bias, gy.tensor)
        for g, what in ((gq, "qact"), (gs, "ascale"), (gt, "lora_act"), (gy, "y")):
            if g is not None:
                g.check(what)
        return qact, ascale, t, y


def check_activation_outputs(p, qact, ascale, t, rows=None):
    M, K = p["x"].shape if rows is None else (rows, p["x"].shape[1])
    codes = decode_qact(qact.cpu().numpy(), M, K)
    assert np.array_equal(codes, p["qa"][:M]), "INT4 activation codes differ"
    sa = ascale.cpu().numpy()
    assert np.array_equal(sa.view(np.uint32), np.ascontiguousarray(p["sa"][:, :M]).view(np.uint32)), \
        "activation scales differ"
    if p["cfg"].rank:
        tg = bf16_to_np(t)
        tr = p["t"][:M]
        ok = within_one_bf16_ulp(tg, tr, abs_floor=2.0 ** -16 * float(np.abs(tr).max()))
        assert ok.all(), f"T beyond one bf16 ulp at {np.argwhere(~ok)[:5]}"
        say(f"  T exact fraction {np.mean(tg == tr):.6f}")


def check_y(p, y, rows=None):
    yr = p["y"] if rows is None else p["y"][:rows]
    yg = bf16_to_np(y)
    mx, mean = tolerance_report(yg, yr)
    say(f"  Y max|err|/max|Y| = {mx:.3e}, mean rel = {mean:.3e}")
    assert mx <= MAX_REL and mean <= MEAN_REL


# ---------------------------------------------------------------------------------------------
# whole-layer parity on every W4A4 configuration
# ---------------------------------------------------------------------------------------------
W4A4_CASES = [("tiny", None), ("attn", None), ("up", None), ("down", None),
              ("qkv_r32", 32), ("qkv_r32", 128), ("qkv_r32", 256)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,rank", W4A4_CASES, ids=[f"{n}-r{r or ''}" for n, r in W4A4_CASES])
def test_w4a4_layer_parity(gpu, name, rank):
    import quantized_gemm_amd as q
    say(f"[w4a4 parity] {name} rank={rank}: building oracle problem")
    p = w4a4_problem(name, rank=rank)
    cfg = p["cfg"]
    M, K = p["x"].shape
    N = p["resid"].shape[1]
    say(f"[w4a4 parity] {cfg.name} M={M} K={K} N={N} r={cfg.rank}: running GPU")
    layer = Layer(p, gpu)
    qact, ascale, t, y = layer.run(p["x_bits"], gpu)
    check_activation_outputs(p, qact, ascale, t)
    check_y(p, y)
    # exact per-group integer sums on windows: the corner, the ragged far corner, the middle
    # windows: the corner, a whole 128 x 128 tile away from the corner, the ragged far corner, a
    # window across tile boundaries
    wins = [(0, 0, min(M, 64), min(N, 64)), (M - 37, N - 53, 37, 53), (M // 2 - 20, N // 2 - 24, 40, 48)]
    if M >= 256 and N >= 256:
        wins.append((128, 128, 128, 128))
    for (m0, n0, tm, tn) in wins:
        got = q.svdq_debug_group_sums(qact, layer.qw, N, m0, n0, tm, tn).cpu().numpy()
        ref = oracle.group_sums(p["qa"][m0:m0 + tm], p["qw"][:, n0:n0 + tn])
        assert np.array_equal(got, ref), f"group sums differ in window {(m0, n0, tm, tn)}"
    # run-to-run determinism (no atomics, fixed reduction order)
    qact2, ascale2, t2, y2 = layer.run(p["x_bits"], gpu)
    import torch
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert np.array_equal(qact.cpu().numpy(), qact2.cpu().numpy())


# (M, K, N, rank): 1, 2, 7, 10, 16 and 50 groups (fewer groups than waves, every tail length of the
# GEMM's six-step loop, a quantizer chunk that is full then partial), ragged M and N, ranks 0 to 112;
# then token counts above 256 16-token tiles (on a 256-CU MI355X): at r = 32 .. 64 the quantizer runs
# 24-token blocks (second tile half full), with a last block holding 17, 8, 20 and 23 tokens (its
# half tile with one token, empty, four and seven tokens); at r >= 128 32-token blocks, with a last
# block holding 17 and 31 tokens (its second tile one token, 15 tokens)
SMALL_SHAPES = [(33, 64, 48, 16), (130, 128, 272, 48), (77, 448, 144, 0), (200, 640, 400, 112),
                (16, 1024, 1040, 64), (40, 3200, 160, 32),
                (4097, 256, 128, 32), (4112, 192, 144, 32), (4100, 128, 160, 64), (4127, 64, 128, 48),
                (4113, 128, 272, 128), (4127, 320, 272, 256)]


@pytest.mark.parametrize("M,K,N,rank", SMALL_SHAPES, ids=[f"M{m}K{k}N{n}r{r}" for m, k, n, r in SMALL_SHAPES])
def test_w4a4_small_shapes(gpu, M, K, N, rank):
    import quantized_gemm_amd as q
    say(f"[w4a4 shapes] M={M} K={K} N={N} r={rank}")
    p = random_w4a4_problem(M, K, N, rank, seed=M + K + N + rank)
    layer = Layer(p, gpu)
    qact, ascale, t, y = layer.run(p["x_bits"], gpu)
    check_activation_outputs(p, qact, ascale, t)
    check_y(p, y)
    got = q.svdq_debug_group_sums(qact, layer.qw, N, 0, 0, M, N).cpu().numpy()
    assert np.array_equal(got, oracle.group_sums(p["qa"], p["qw"]))


# (M, K, N, ka, kw, r): ragged token and column counts, 2 to 8 groups, and the FLUX token count and
# hidden size (all 48 groups of K = 3072, 24-token quantizer blocks); activation scale 2^-ka, weight
# scale 2^-kw; low-rank rank r (0: no branch and no bias)
EXACT_SHAPES = [(200, 512, 272, 3, 5, 32), (129, 128, 160, 0, 0, 0), (33, 320, 48, 7, 2, 256),
                (4100, 256, 144, 4, 6, 16), (4608, 3072, 384, 2, 3, 32)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("M,K,N,ka,kw,r", EXACT_SHAPES,
                         ids=[f"M{m}K{k}N{n}r{r}" for m, k, n, _, _, r in EXACT_SHAPES])
def test_product_kernel_exact_with_power_of_two_scales(gpu, M, K, N, ka, kw, r):
    """The product kernel itself (scale loads, rescale FMAs, epilogue and store), not its debug
    instantiation, checked bit for bit. With every group's activation scale 2^-ka and weight scale
    2^-kw, each rescaled group sum 256 P[g] 2^-(ka+kw) and their running float32 sum stay exact
    while |sum 256 P| < 2^24 units of 2^-(ka+kw): codes in [-7, 7] up to 8 groups, in [-3, 3] (and
    one +-7 per group) beyond. The epilogue's low-rank product T L2 (T integers in [-8, 8] times
    2^-ka, L2 integers in [-4, 4] times 2^-kw) and the bias (integers times 2^-(ka+kw)) add exactly
    in the same units. Y must then be exactly bf16(2^-(ka+kw) * (sum_g P[g] + T_int L2_int + b_int)):
    the integer result, scaled and rounded once."""
    import torch
    import quantized_gemm_amd as q
    say(f"[exact product] M={M} K={K} N={N} 2^-{ka} 2^-{kw}")
    G = K // 64
    c = 7 if G <= 8 else 3
    assert G * (63 * c * c + 49) * 256 < 2 ** 24, "partial sums would not be exact"
    rng = np.random.default_rng(M * 7 + K + N)
    qa = rng.integers(-c, c + 1, size=(M, G, 64))
    qw = rng.integers(-c, c + 1, size=(G, 64, N))
    # a +-7 in every group, so absmax / 7 is exactly the power of two
    qa[:, :, 5] = 7 * np.where(rng.random((M, G)) < 0.5, -1, 1)
    qw[:, 9, :] = 7 * np.where(rng.random((G, N)) < 0.5, -1, 1)
    qa = qa.reshape(M, K)
    qw = qw.reshape(K, N)
    x_bits = synth.bf16_bits_from_f32((qa * 2.0 ** -ka).astype(np.float32))
    w = (qw * 2.0 ** -kw).astype(np.float32)
    pw, psw = q.svdq_pack_weights(q.SVDQ_FMT_W4A4_F32SCALE, w)
    assert np.all(psw == np.float32(2.0 ** -kw))
    gq = Guarded((G, M, 32), torch.uint8, gpu)
    gs = Guarded((G, M), torch.float32, gpu)
    gy = Guarded((M, N), torch.bfloat16, gpu)
    qact, ascale, _ = q.svdq_quantize_act(to_dev_bf16(x_bits, gpu), None, None, gq.tensor, gs.tensor, None)
    ti = rng.integers(-8, 9, size=(M, r))
    li = rng.integers(-4, 5, size=(r, N))
    bi = rng.integers(-50, 51, size=N)
    t_dev = l2t_dev = b_dev = None
    if r:
        def grid(v, e):
            return np.ldexp(v.astype(np.float64), e).astype(np.float32)
        _, l2t = q.svdq_pack_lowrank(np.zeros((K, r), np.float32), grid(li, -kw))
        l2t_dev = to_dev_bf16(l2t, gpu)
        t_dev = to_dev_bf16(synth.bf16_bits_from_f32(grid(ti, -ka)), gpu)
        b_dev = to_dev_bf16(synth.bf16_bits_from_f32(grid(bi, -(ka + kw))), gpu)
    y = q.svdq_linear_w4a4(qact, ascale, to_dev(pw, gpu), to_dev(psw, gpu), t_dev, l2t_dev, b_dev, gy.tensor)
    for g, what in ((gq, "qact"), (gs, "ascale"), (gy, "y")):
        g.check(what)
    assert np.array_equal(decode_qact(qact.cpu().numpy(), M, K), qa), "activation codes differ"
    assert np.all(ascale.cpu().numpy() == np.float32(2.0 ** -ka)), "activation scales differ"
    if G <= 8:
        total = oracle.group_sums(qa, qw).sum(axis=0).astype(np.float64)
    else:  # the same integers through a float64 product (every partial sum below 2^53 is exact)
        total = qa.astype(np.float64) @ qw.astype(np.float64)
    if r:
        total = total + ti.astype(np.float64) @ li.astype(np.float64) + bi
    ref = oracle.bf16_round(total * 2.0 ** -(ka + kw))
    got = bf16_to_np(y)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} outputs differ, first at {bad[:3].tolist()}"


# (M, K, r): 16-token blocks (r = 16, and M 100), 24-token blocks (r = 32, 48, 64 at M 4608 and a
# ragged 4100), 32-token blocks (r = 128, 256)
T_EXACT = [(100, 3072, 16), (4608, 3072, 32), (4100, 1600, 48), (4608, 3072, 64), (4113, 3072, 128),
           (4608, 3072, 256)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("M,K,r", T_EXACT, ids=[f"M{m}K{k}r{r}" for m, k, r in T_EXACT])
def test_down_projection_exact_with_grid_inputs(gpu, M, K, r):
    """The fused down projection of kernel (a) checked bit for bit: with X integers in [-8, 8] times
    2^-3, no smoothing and L1 integers in [-4, 4] times 2^-5, the bf16 operands are exact, every
    float32 sum of the MFMAs and of the fixed-order reduction over the waves is an integer multiple of
    2^-8 below 32 K of them (< 2^24), so T must be exactly bf16(X L1). The codes and scales of the same
    launch are checked against the oracle."""
    import torch
    import quantized_gemm_amd as q
    say(f"[down projection exact] M={M} K={K} r={r}")
    assert 32 * K < 2 ** 24
    rng = np.random.default_rng(M + K + r)
    xi = rng.integers(-8, 9, size=(M, K))
    li = rng.integers(-4, 5, size=(K, r))
    x = np.ldexp(xi.astype(np.float64), -3).astype(np.float32)
    l1 = np.ldexp(li.astype(np.float64), -5).astype(np.float32)
    l2 = np.zeros((r, 16), np.float32)
    xb = synth.bf16_bits_from_f32(x)
    l1t, _ = q.svdq_pack_lowrank(l1, l2)
    gq, gs = Guarded((K // 64, M, 32), torch.uint8, gpu), Guarded((K // 64, M), torch.float32, gpu)
    gt = Guarded((M, r), torch.bfloat16, gpu)
    qact, ascale, t = q.svdq_quantize_act(to_dev_bf16(xb, gpu), None, to_dev_bf16(l1t, gpu), gq.tensor, gs.tensor,
                                          gt.tensor)
    for g, what in ((gq, "qact"), (gs, "ascale"), (gt, "lora_act")):
        g.check(what)
    qa_ref, sa_ref = oracle.quantize_activations(x, np.ones(K, np.float32))[:2]
    assert np.array_equal(decode_qact(qact.cpu().numpy(), M, K), qa_ref), "activation codes differ"
    assert np.array_equal(ascale.cpu().numpy().view(np.uint32), np.ascontiguousarray(sa_ref).view(np.uint32))
    ref = oracle.bf16_round(np.ldexp(xi.astype(np.float64) @ li.astype(np.float64), -8))
    got = bf16_to_np(t)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} T values differ, first at {bad[:3].tolist()}"


def test_tiny_full_group_sums(gpu):
    import quantized_gemm_amd as q
    p = w4a4_problem("tiny")
    layer = Layer(p, gpu)
    qact, _, _, _ = layer.run(p["x_bits"], gpu)
    M, K = p["x"].shape
    N = p["resid"].shape[1]
    got = q.svdq_debug_group_sums(qact, layer.qw, N, 0, 0, M, N).cpu().numpy()
    assert np.array_equal(got, oracle.group_sums(p["qa"], p["qw"]))


@pytest.mark.parametrize("rows", [1, 7, 16, 17, 100, 129, 255])
def test_ragged_token_counts(gpu, rows):
    """Rows are independent: a prefix of the tokens gives the prefix of every output."""
    p = w4a4_problem("tiny")
    layer = Layer(p, gpu)
    qact, ascale, t, y = layer.run(p["x_bits"][:rows], gpu)
    check_activation_outputs(p, qact, ascale, t, rows=rows)
    check_y(p, y, rows=rows)


def test_rank_zero(gpu):
    p = w4a4_problem("tiny", rank=0)
    assert p["t"] is None
    layer = Layer(p, gpu)
    qact, ascale, t, y = layer.run(p["x_bits"], gpu)
    assert t is None
    check_activation_outputs(p, qact, ascale, t)
    check_y(p, y)


def test_zero_residual_gives_lowrank_plus_bias(gpu):
    p = w4a4_problem("tiny")
    zero = np.zeros_like(p["resid"])
    ref = oracle.svdq_layer(p["x"], p["inv"], p["l1"], p["l2"], zero, p["bias"])
    layer = Layer(p, gpu, resid=zero)
    _, _, _, y = layer.run(p["x_bits"], gpu)
    mx, mean = tolerance_report(bf16_to_np(y), ref["y"])
    assert mx <= MAX_REL and mean <= MEAN_REL


def test_column_slice_invariance(gpu):
    """Output columns are independent (fused Q|K|V slices): an N-slice of the packed weights gives
    that slice of the full output, bit for bit."""
    import torch
    import quantized_gemm_amd as q
    p = w4a4_problem("tiny")
    layer = Layer(p, gpu)
    qact, ascale, t, y = layer.run(p["x_bits"], gpu)
    K = p["x"].shape[1]
    for n0, n1 in [(0, 16), (128, 384), (496, 512)]:
        qw = layer.qw.view(K // 64, -1, 32)[:, n0:n1].contiguous()
        sw = layer.sw[:, n0:n1].contiguous()
        l2t = layer.l2t[n0:n1].contiguous()
        b = layer.bias[n0:n1].contiguous()
        ys = q.svdq_linear_w4a4(qact, ascale, qw, sw, t, l2t, b)
        torch.cuda.synchronize()
        assert torch.equal(ys.view(torch.int16), y[:, n0:n1].contiguous().view(torch.int16))


def test_activation_edge_values(gpu):
    """Zero rows, subnormal scales (including one where the clamp to -8 / 7 is live), exact
    half-integer quotients with an inexact reciprocal, and huge outliers: codes and scales
    bit-exact."""
    import torch
    import quantized_gemm_amd as q
    rng = np.random.default_rng(31)
    M, K = 48, 256
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[3] = 0.0                                                   # zero token
    x[5, :64] = 0.0
    x[5, 0] = np.float32(9 * 2.0 ** -130)                        # scale subnormal after /7
    x[6, 64:128] = np.float32(2.0 ** -133) * rng.integers(-9, 10, 64).astype(np.float32)
    x[7, :64] = np.float32(2.0 ** -133) * rng.integers(-9, 10, 64).astype(np.float32)
    x[7, 0], x[7, 1] = np.float32(-9 * 2.0 ** -133), np.float32(9 * 2.0 ** -133)
    # scale 9/32 (absmax 63/32 = 14 * 9/64): values c * 9/64 give quotients c / 2
    half = np.array([14, 5, -5, 7, -7, 3, 1, -1, 9, 11, 13, -13], np.float32) * np.float32(9.0 / 64.0)
    x[8, :12] = half
    x[8, 12:64] = np.float32(2 * 9.0 / 64.0)
    x[9, :] *= 1e4
    xb = synth.bf16_bits_from_f32(x)
    xv = synth.f32_from_bf16_bits(xb)
    tiny_first_group = np.ones(K, np.float32)
    tiny_first_group[:64] = np.float32(2.0 ** -16)               # x_hat = c * 2^-149: scale 2^-149
    invs = [np.ones(K, np.float32), (1.0 / rng.uniform(0.5, 3, K)).astype(np.float32), tiny_first_group]
    for n, inv in enumerate(invs):
        qa, sa, _ = oracle.quantize_activations(xv, inv, None)
        qact, ascale, _ = q.svdq_quantize_act(to_dev_bf16(xb, gpu), to_dev(inv, gpu), None)
        torch.cuda.synchronize()
        assert np.array_equal(decode_qact(qact.cpu().numpy(), M, K), qa), f"codes differ (inv #{n})"
        assert np.array_equal(ascale.cpu().numpy().view(np.uint32), sa.view(np.uint32)), f"scales differ (inv #{n})"
        if n == 0:
            assert qa[8, :12].tolist() == [7, 2, -2, 4, -4, 2, 0, 0, 4, 6, 6, -6]
        if n == 2:
            assert qa[7, 0] == -8 and qa[7, 1] == 7          # clamp live on both ends


def test_no_smoothing_pointer(gpu):
    import torch
    import quantized_gemm_amd as q
    p = w4a4_problem("tiny")
    M, K = p["x"].shape
    qa, sa, _ = oracle.quantize_activations(p["x"], np.ones(K, np.float32), None)
    qact, ascale, _ = q.svdq_quantize_act(to_dev_bf16(p["x_bits"], gpu), None, None)
    torch.cuda.synchronize()
    assert np.array_equal(decode_qact(qact.cpu().numpy(), M, K), qa)
    assert np.array_equal(ascale.cpu().numpy(), sa)


# ---------------------------------------------------------------------------------------------
# MLP up projection with the GELU fused into the epilogue
# ---------------------------------------------------------------------------------------------
@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["tiny", "up"])
def test_w4a4_gelu_parity(gpu, name):
    import torch
    import quantized_gemm_amd as q
    say(f"[w4a4 gelu parity] {name}: building oracle problem")
    p = w4a4_problem(name)
    layer = Layer(p, gpu)
    x = to_dev_bf16(p["x_bits"], gpu)
    qact, ascale, t = q.svdq_quantize_act(x, layer.inv, layer.l1t)
    y = q.svdq_linear_w4a4(qact, ascale, layer.qw, layer.sw, t, layer.l2t, layer.bias, activation="gelu_tanh")
    y_plain = q.svdq_linear_w4a4(qact, ascale, layer.qw, layer.sw, t, layer.l2t, layer.bias)
    torch.cuda.synchronize()
    _, y_ref = oracle.svdq_linear_gelu(p["qa"], p["sa"], p["qw"], p["sw"], p["t"], p["l2"], p["bias"])
    mx, mean = tolerance_report(bf16_to_np(y), y_ref)
    say(f"  GELU(Y) max|err|/max|Y| = {mx:.3e}, mean rel = {mean:.3e}")
    assert mx <= MAX_REL and mean <= MEAN_REL
    # the plain entry point is unchanged by the flag
    check_y(p, y_plain)


@pytest.mark.parametrize("M,K,N,rank", [(33, 64, 48, 16), (77, 448, 144, 0), (130, 128, 272, 48)])
def test_w4a4_gelu_small_shapes(gpu, M, K, N, rank):
    """The GELU epilogue on ragged token counts, rank 0 and column counts that leave partial tiles."""
    import torch
    import quantized_gemm_amd as q
    say(f"[w4a4 gelu shapes] M={M} K={K} N={N} r={rank}")
    p = random_w4a4_problem(M, K, N, rank, seed=M + K + N + rank + 1)
    layer = Layer(p, gpu)
    qact, ascale, t = q.svdq_quantize_act(to_dev_bf16(p["x_bits"], gpu), layer.inv, layer.l1t)
    y = q.svdq_linear_w4a4(qact, ascale, layer.qw, layer.sw, t, layer.l2t, layer.bias, activation="gelu_tanh")
    torch.cuda.synchronize()
    _, y_ref = oracle.svdq_linear_gelu(p["qa"], p["sa"], p["qw"], p["sw"], p["t"], p["l2"], p["bias"])
    mx, mean = tolerance_report(bf16_to_np(y), y_ref)
    say(f"  GELU(Y) max|err|/max|Y| = {mx:.3e}, mean rel = {mean:.3e}")
    assert mx <= MAX_REL and mean <= MEAN_REL


def test_mlp_pair_chained_on_real_intermediates(gpu):
    """Up projection with the fused GELU, then the down projection quantizing that output: the
    intermediate against the oracle's, and the down layer bit-exact (codes, scales) and within
    tolerance (Y) against the oracle run on the intermediate the GPU produced."""
    import torch
    import quantized_gemm_amd as q
    M, D, F, r = 256, 256, 512, 16
    say(f"[mlp pair] M={M} D={D} F={F} r={r}")
    up = random_w4a4_problem(M, D, F, r, seed=71)
    h_ref64, h_ref = oracle.svdq_linear_gelu(up["qa"], up["sa"], up["qw"], up["sw"], up["t"], up["l2"], up["bias"])
    # the down layer, prepared from the oracle's intermediate (its smoothing needs activation maxima)
    w_dn = synth.random_f32((F, D), seed=72, scale=0.02)
    b_dn = oracle.bf16_round(synth.random_f32((D,), seed=73, scale=0.01))
    d_dn = oracle.svdq_decompose(h_ref, w_dn, r)
    upl = Layer(up, gpu)
    x = to_dev_bf16(up["x_bits"], gpu)
    qa1, sa1, t1 = q.svdq_quantize_act(x, upl.inv, upl.l1t)
    h = q.svdq_linear_w4a4(qa1, sa1, upl.qw, upl.sw, t1, upl.l2t, upl.bias, activation="gelu_tanh")
    qw2, sw2 = q.svdq_pack_weights(q.SVDQ_FMT_W4A4_F32SCALE, d_dn["resid"])
    l1t2, l2t2 = q.svdq_pack_lowrank(d_dn["l1_bf16"], d_dn["l2_bf16"])
    qa2, sa2, t2 = q.svdq_quantize_act(h, to_dev(d_dn["inv"], gpu), to_dev_bf16(l1t2, gpu))
    y = q.svdq_linear_w4a4(qa2, sa2, to_dev(qw2, gpu), to_dev(sw2, gpu), t2, to_dev_bf16(l2t2, gpu),
                           to_dev_bf16(synth.bf16_bits_from_f32(b_dn), gpu))
    torch.cuda.synchronize()
    h_gpu = bf16_to_np(h)
    mx, mean = tolerance_report(h_gpu, h_ref)
    say(f"  H = GELU(up) max|err|/max|H| = {mx:.3e}, mean rel = {mean:.3e}")
    assert mx <= MAX_REL and mean <= MEAN_REL
    dn = oracle.svdq_layer(h_gpu, d_dn["inv"], d_dn["l1_bf16"], d_dn["l2_bf16"], d_dn["resid"], b_dn)
    assert np.array_equal(decode_qact(qa2.cpu().numpy(), M, F), dn["qa"]), "down-layer codes differ"
    assert np.array_equal(sa2.cpu().numpy().view(np.uint32), np.ascontiguousarray(dn["sa"]).view(np.uint32))
    mx, mean = tolerance_report(bf16_to_np(y), dn["y"])
    say(f"  Y = down(H) max|err|/max|Y| = {mx:.3e}, mean rel = {mean:.3e}")
    assert mx <= MAX_REL and mean <= MEAN_REL


# ---------------------------------------------------------------------------------------------
# fused QKV: per-head RMS norm + rotary embedding of Q and K in the epilogue
# ---------------------------------------------------------------------------------------------
def _qkv_tables(M, heads, seed):
    rng = np.random.default_rng(seed)
    q_w = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    k_w = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    pos = np.arange(M, dtype=np.float64)[:, None]
    freq = 10000.0 ** (-np.arange(64, dtype=np.float64) / 64.0)[None, :]
    ang = pos * freq + rng.uniform(-0.1, 0.1, (M, 64))
    return q_w, k_w, np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _run_qkv(gpu, layer, x_bits, heads, tables):
    import torch
    import quantized_gemm_amd as q
    q_w, k_w, cs, sn = tables
    x = to_dev_bf16(x_bits, gpu)
    qact, ascale, t = q.svdq_quantize_act(x, layer.inv, layer.l1t)
    y = q.svdq_linear_w4a4_qkv(qact, ascale, layer.qw, layer.sw, t, layer.l2t, layer.bias, heads,
                               to_dev(q_w, gpu), to_dev(k_w, gpu), to_dev(cs, gpu), to_dev(sn, gpu))
    y_plain = q.svdq_linear_w4a4(qact, ascale, layer.qw, layer.sw, t, layer.l2t, layer.bias)
    torch.cuda.synchronize()
    return bf16_to_np(y), bf16_to_np(y_plain)


def _check_qkv_epilogue(y, y_plain, heads, tables):
    """The epilogue against the oracle applied to the kernel's own plain output: within one bf16
    ulp everywhere (float32 on the GPU, float64 in the oracle, one bf16 rounding each), V identical."""
    q_w, k_w, cs, sn = tables
    ref = oracle.qkv_norm_rope(y_plain, heads, q_w, k_w, cs, sn)
    ok = within_one_bf16_ulp(y, ref, abs_floor=2.0 ** -16 * float(np.abs(ref).max()))
    assert ok.all(), f"QKV epilogue beyond one bf16 ulp at {np.argwhere(~ok)[:5]}"
    say(f"  Q/K exact fraction {np.mean(y[:, :2 * heads * 128] == ref[:, :2 * heads * 128]):.6f}")
    assert np.array_equal(y[:, 2 * heads * 128:], y_plain[:, 2 * heads * 128:])


def test_qkv_norm_rope_small_ragged(gpu):
    M, K, heads, r = 200, 256, 2, 16
    say(f"[qkv] M={M} K={K} heads={heads} r={r}")
    p = random_w4a4_problem(M, K, 3 * heads * 128, r, seed=91)
    tables = _qkv_tables(M, heads, seed=92)
    y, y_plain = _run_qkv(gpu, Layer(p, gpu), p["x_bits"], heads, tables)
    _check_qkv_epilogue(y, y_plain, heads, tables)
    # and the whole chain against the oracle's
    ref = oracle.qkv_norm_rope(p["y"], heads, *tables)
    mx, mean = tolerance_report(y, ref)
    say(f"  QKV max|err|/max|ref| = {mx:.3e}, mean rel = {mean:.3e}")
    assert mx <= MAX_REL and mean <= MEAN_REL


# (M, K, heads, rank): one token and one head with no low-rank branch, a ragged token count with a
# rank between instantiation steps, and the largest rank with a partial last row tile
@pytest.mark.parametrize("M,K,heads,rank", [(1, 64, 1, 0), (77, 448, 1, 48), (130, 320, 3, 256)])
def test_qkv_norm_rope_ranks_and_ragged_tokens(gpu, M, K, heads, rank):
    say(f"[qkv] M={M} K={K} heads={heads} r={rank}")
    p = random_w4a4_problem(M, K, 3 * heads * 128, rank, seed=94 + rank)
    tables = _qkv_tables(M, heads, seed=95 + rank)
    y, y_plain = _run_qkv(gpu, Layer(p, gpu), p["x_bits"], heads, tables)
    _check_qkv_epilogue(y, y_plain, heads, tables)
    mx, mean = tolerance_report(y, oracle.qkv_norm_rope(p["y"], heads, *tables))
    say(f"  QKV max|err|/max|ref| = {mx:.3e}, mean rel = {mean:.3e}")
    assert mx <= MAX_REL and mean <= MEAN_REL


@pytest.mark.timeout(600)
def test_qkv_norm_rope_flux_shape(gpu):
    """FLUX attention: M 4608, K 3072, 24 heads of 128 (N 9216), rank 32."""
    p = w4a4_problem("qkv_r32")
    heads = p["cfg"].N // (3 * 128)
    say(f"[qkv] FLUX shape, heads={heads}")
    tables = _qkv_tables(p["cfg"].M, heads, seed=93)
    y, y_plain = _run_qkv(gpu, Layer(p, gpu), p["x_bits"], heads, tables)
    _check_qkv_epilogue(y, y_plain, heads, tables)


# ---------------------------------------------------------------------------------------------
# W4A16 projection
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("M,with_bias", [(16, False), (16, True), (1, False), (5, True), (33, False)])
def test_w4a16_parity(gpu, M, with_bias):
    import torch
    import quantized_gemm_amd as q
    say(f"[w4a16 parity] M={M} bias={with_bias}")
    p = w4a16_problem("awq", M=M, with_bias=with_bias)
    qw, s = q.svdq_pack_weights(q.SVDQ_FMT_W4A16_BF16SCALE, p["w"])
    assert np.array_equal(synth.f32_from_bf16_bits(s), p["scales"])
    x = to_dev_bf16(p["x_bits"], gpu)
    b = None if p["bias"] is None else to_dev_bf16(synth.bf16_bits_from_f32(p["bias"]), gpu)
    y = q.awq_linear_w4a16(x, to_dev(qw, gpu), to_dev_bf16(s, gpu), b)
    y2 = q.awq_linear_w4a16(x, to_dev(qw, gpu), to_dev_bf16(s, gpu), b)
    torch.cuda.synchronize()
    mx, mean = tolerance_report(bf16_to_np(y), p["y"])
    say(f"  Y max|err|/max|Y| = {mx:.3e}, mean rel = {mean:.3e}")
    assert mx <= MAX_REL and mean <= MEAN_REL
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


# (M, K, N, kx, kw): the adaLN projection, an odd group count with several row tiles, a three-pass grid
W4A16_EXACT = [(16, 3072, 18432, -2, -6), (5, 1600, 2000, 0, -3), (40, 1024, 8192, -4, 1), (2, 192, 45104, 3, -9)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("M,K,N,kx,kw", W4A16_EXACT, ids=[f"M{m}K{k}N{n}" for m, k, n, _, _ in W4A16_EXACT])
def test_w4a16_exact_with_grid_inputs(gpu, M, K, N, kx, kw):
    """Kernel (c) checked bit for bit. Activations are integers in [-8, 8] times 2^kx, weights codes in
    [-7, 7] times 2^kw with a +-7 in every group (so the bf16 scale is exactly 2^kw), the bias an
    integer times 2^(kx+kw). Then every step is exact: the bf16 products x (128 + u) and their float32
    sums (per group at most 136 * 512 + 64 * 8 * 143 units of 2^kx), the correction -136 * sum x, the
    power-of-two rescale and the running sum over K (at most 8 * 7 * K units of 2^(kx+kw)), and the
    bias add, all below 2^24 units. Y must be exactly bf16(x @ w + b)."""
    import torch
    import quantized_gemm_amd as q
    say(f"[w4a16 exact] M={M} K={K} N={N} 2^{kx} 2^{kw}")
    assert 8 * 7 * K + 50 < 2 ** 24
    rng = np.random.default_rng(M + K + N)
    xi = rng.integers(-8, 9, size=(M, K))
    code = rng.integers(-7, 8, size=(K // 64, 64, N))
    code[:, 17, :] = 7 * np.where(rng.random((K // 64, N)) < 0.5, -1, 1)
    code = code.reshape(K, N)
    bi = rng.integers(-50, 51, size=N)
    x = np.ldexp(xi.astype(np.float64), kx).astype(np.float32)
    w = np.ldexp(code.astype(np.float64), kw).astype(np.float32)
    b = np.ldexp(bi.astype(np.float64), kx + kw).astype(np.float32)
    xb, bb = synth.bf16_bits_from_f32(x), synth.bf16_bits_from_f32(b)
    assert np.array_equal(synth.f32_from_bf16_bits(xb), x) and np.array_equal(synth.f32_from_bf16_bits(bb), b)
    qw, sc = q.svdq_pack_weights(q.SVDQ_FMT_W4A16_BF16SCALE, w)
    assert np.all(synth.f32_from_bf16_bits(sc) == np.float32(2.0 ** kw))
    gy = Guarded((M, N), torch.bfloat16, gpu)
    y = q.awq_linear_w4a16(to_dev_bf16(xb, gpu), to_dev(qw, gpu), to_dev_bf16(sc, gpu), to_dev_bf16(bb, gpu),
                           gy.tensor)
    gy.check("y")
    ref = oracle.bf16_round(np.ldexp((xi.astype(np.float64) @ code.astype(np.float64)) + bi, kx + kw))
    got = bf16_to_np(y)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} outputs differ, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("M,K,N", [(20, 448, 592), (16, 6400, 96), (300, 192, 256), (3, 64, 16),
                                   (3, 128, 24576), (2, 192, 45104)])
def test_w4a16_shapes(gpu, M, K, N):
    """Odd group counts (unpaired last group), K longer than one chunk of the waves' slices,
    several row tiles, column-tile counts that leave blocks with fewer tiles, the smallest shape,
    and more column tiles than one pass over K holds per block (N = 24576: two passes of the
    256-block grid; N = 45104: 11 or 12 tiles per block, three passes, odd group count)."""
    import torch
    import quantized_gemm_amd as q
    say(f"[w4a16 shapes] M={M} K={K} N={N}")
    x_bits = synth.random_bf16((M, K), seed=K + N)
    w = oracle.bf16_round(synth.random_f32((K, N), seed=K * N + 1, scale=0.02))
    b = oracle.bf16_round(synth.random_f32((N,), seed=N + 7, scale=0.01))
    codes, s_ref = oracle.quantize_weights_w4a16(w)
    _, y_ref = oracle.awq_linear(synth.f32_from_bf16_bits(x_bits), codes, s_ref, b)
    qw, s = q.svdq_pack_weights(q.SVDQ_FMT_W4A16_BF16SCALE, w)
    gy = Guarded((M, N), torch.bfloat16, gpu)
    y = q.awq_linear_w4a16(to_dev_bf16(x_bits, gpu), to_dev(qw, gpu), to_dev_bf16(s, gpu),
                           to_dev_bf16(synth.bf16_bits_from_f32(b), gpu), gy.tensor)
    gy.check("y")
    mx, mean = tolerance_report(bf16_to_np(y), y_ref)
    say(f"  Y max|err|/max|Y| = {mx:.3e}, mean rel = {mean:.3e}")
    assert mx <= MAX_REL and mean <= MEAN_REL


# ---------------------------------------------------------------------------------------------
# the unfused form timed by bench.py --naive-vs-fused computes the same layer
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "attn"])
def test_naive_unfused_layer_matches_oracle(gpu, name):
    """bench.py's naive form (r = 0 kernels + separate bf16 down / up projections) against the
    oracle's naive form, which mirrors its two extra bf16 roundings (diag(inv) L1 rounded to bf16,
    since the down projection reads X itself, and the 4-bit branch's output rounded to bf16 before
    T L2 is added): the layer's bars, 1e-2 max and 2e-3 mean relative error. It is not the product
    path; the fused kernels are checked against the fused oracle."""
    import torch
    import quantized_gemm_amd as q
    import bench
    say(f"[naive layer] {name}")
    p = w4a4_problem(name)
    M, K = p["x"].shape
    N = p["resid"].shape[1]
    qw, sw = q.svdq_pack_weights(q.SVDQ_FMT_W4A4_F32SCALE, p["resid"])
    l1s = to_dev(p["inv"][:, None].astype(np.float64) * p["l1"], gpu).to(torch.bfloat16)
    l2 = to_dev(np.ascontiguousarray(p["l2"]), gpu).to(torch.bfloat16)
    x = to_dev_bf16(p["x_bits"], gpu)
    qact = torch.empty((K // 64, M, 32), dtype=torch.uint8, device=gpu)
    asc = torch.empty((K // 64, M), dtype=torch.float32, device=gpu)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=gpu)
    bias = None if p["bias_bits"] is None else to_dev_bf16(p["bias_bits"], gpu)
    bench.naive_low_rank_layer(q, x, to_dev(p["inv"], gpu), l1s, l2, to_dev(qw, gpu), to_dev(sw, gpu), bias,
                               qact, asc, y)
    torch.cuda.synchronize()
    ref = oracle.svdq_layer_naive(p["x"], p["inv"], p["l1"], p["l2"], p["resid"], p["bias"])
    mx, mean = tolerance_report(bf16_to_np(y), ref["y"])
    say(f"  Y max|err|/max|Y| = {mx:.3e}, mean rel = {mean:.3e}")
    assert mx <= MAX_REL and mean <= MEAN_REL

