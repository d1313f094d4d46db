"""GPU parity of the MXFP4 variant (E2M1 codes, E8M0 block-32 scales) against the CPU oracle,
through the C ABI (needs an MI355X).

Bar: codes and E8M0 scales bit-exact; T within one bf16 ulp; Y (bf16) with
max|err| <= 1e-2 * max|Y_ref| and sum|err| / sum|Y_ref| <= 2e-3 (the INT4 layer's bar: the
quantization is identical on both sides, only the float32 accumulation order differs).
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from guard import Guarded
from problems import decode_mx_codes, decode_mx_scales, mxfp4_problem, tolerance_report, within_one_bf16_ulp

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


def to_dev_bf16(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def to_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bf16_to_np(t):
    import torch
    return synth.f32_from_bf16_bits(t.view(torch.int16).cpu().numpy().view(np.uint16))


def run_layer(p, dev, rows=None):
    import torch
    import quantized_gemm_amd as q
    r = p["cfg"].rank
    qw, sw = q.svdq_pack_weights(q.SVDQ_FMT_MXFP4_E8M0SCALE, p["resid"])
    l1t = l2t = None
    if r:
        a, b = q.svdq_pack_lowrank(p["l1"], p["l2"])
        l1t, l2t = to_dev_bf16(a, dev), to_dev_bf16(b, dev)
    xb = p["x_bits"] if rows is None else p["x_bits"][:rows]
    M, K = xb.shape
    N = p["resid"].shape[1]
    gq, gs = Guarded((K // 64, M, 32), torch.uint8, dev), Guarded((K // 64, M, 2), torch.uint8, dev)
    gt = Guarded((M, r), torch.bfloat16, dev) if r else None
    gy = Guarded((M, N), torch.bfloat16, dev)
    qact, ascale, t = q.svdq_quantize_act_mxfp4(to_dev_bf16(xb, dev), to_dev(p["inv"], dev), l1t, gq.tensor,
                                                gs.tensor, gt.tensor if r else None)
    y = q.svdq_linear_mxfp4(qact, ascale, to_dev(qw, dev), to_dev(sw, dev), t, l2t, to_dev_bf16(p["bias_bits"], dev),
                            gy.tensor)
    for g, what in ((gq, "qact"), (gs, "ascale"), (gt, "lora_act"), (gy, "y")):
        if g is not None:
            g.check(what)
    return qact, ascale, t, y


def check(p, qact, ascale, t, y, rows=None):
    M, K = p["x"].shape
    M = M if rows is None else rows
    assert np.array_equal(decode_mx_codes(qact.cpu().numpy(), M, K), p["qa"][:M]), "E2M1 activation codes differ"
    assert np.array_equal(decode_mx_scales(ascale.cpu().numpy(), M, K), p["sa"][:M]), "E8M0 activation scales differ"
    if p["cfg"].rank:
        tg, tr = bf16_to_np(t), p["t"][:M]
        ok = within_one_bf16_ulp(tg, tr, abs_floor=2.0 ** -16 * float(np.abs(tr).max()))
        assert ok.all(), f"T beyond one bf16 ulp at {np.argwhere(~ok)[:5]}"
    mx, mean = tolerance_report(bf16_to_np(y), p["y"][:M])
    say(f"  Y max|err|/max|Y| = {mx:.3e}, mean rel = {mean:.3e}")
    assert mx <= MAX_REL and mean <= MEAN_REL


# (M, K, N, rank): one slab, an odd slab count, several tiles with ragged M and N, ranks 0 to 256,
# the FLUX attention shape, and ragged token counts in the quantizer's 32-token blocks
SHAPES = [(256, 256, 512, 16), (33, 64, 48, 16), (130, 192, 272, 48), (77, 448, 144, 0), (200, 640, 400, 256),
          (4608, 3072, 3072, 32), (4113, 256, 384, 256), (4127, 192, 64, 32)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("M,K,N,rank", SHAPES, ids=[f"M{m}K{k}N{n}r{r}" for m, k, n, r in SHAPES])
def test_mxfp4_layer_parity(gpu, M, K, N, rank):
    say(f"[mxfp4] M={M} K={K} N={N} r={rank}")
    p = mxfp4_problem(M, K, N, rank, seed=M + K + N + rank)
    check(p, *run_layer(p, gpu))


@pytest.mark.parametrize("rows", [1, 7, 17, 129])
def test_mxfp4_ragged_token_counts(gpu, rows):
    p = mxfp4_problem(256, 256, 512, 16, seed=3)
    check(p, *run_layer(p, gpu, rows=rows), rows=rows)


def test_mxfp4_zero_residual(gpu):
    p = mxfp4_problem(96, 256, 128, 16, seed=5, resid_zero=True)
    check(p, *run_layer(p, gpu))


def test_mxfp4_activation_edge_values(gpu):
    """Ties of the E2M1 rounding, saturation, zero and subnormal blocks, huge values: codes and scales
    bit-exact."""
    import torch
    import quantized_gemm_amd as q
    rng = np.random.default_rng(41)
    M, K = 40, 256
    x = (rng.standard_normal((M, K)) * 3).astype(np.float32)
    x[2] = 0.0
    x[3, :32] = np.array([6, 4, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -5, -0.25, -0.75] + [1] * 20, np.float32)
    x[4, :32] = np.array([7.75, 7, 6.5, -7.5] + [2] * 28, np.float32)                   # saturation
    x[5, 32:64] = np.float32(2.0 ** -130) * rng.integers(-9, 10, 32).astype(np.float32)
    x[6, :] *= 1e4
    x[7, :32] = -0.0
    xb = synth.bf16_bits_from_f32(x)
    xv = synth.f32_from_bf16_bits(xb)
    for inv in (np.ones(K, np.float32), (1.0 / rng.uniform(0.5, 3, K)).astype(np.float32)):
        qa, sa, _ = oracle.quantize_activations_mxfp4(xv, inv, None)
        qact, ascale, _ = q.svdq_quantize_act_mxfp4(to_dev_bf16(xb, gpu), to_dev(inv, gpu), None)
        torch.cuda.synchronize()
        assert np.array_equal(decode_mx_codes(qact.cpu().numpy(), M, K), qa)
        assert np.array_equal(decode_mx_scales(ascale.cpu().numpy(), M, K), sa)


# (M, K, N, sa, sw): ragged token and column counts; every activation block scale 2^sa, every weight
# block scale 2^sw
EXACT_SHAPES = [(200, 512, 272, -3, -5), (33, 3072, 48, 2, -7), (4127, 192, 64, 0, 0)]


@pytest.mark.parametrize("M,K,N,sa,sw", EXACT_SHAPES, ids=[f"M{m}K{k}N{n}" for m, k, n, _, _ in EXACT_SHAPES])
def test_mxfp4_product_exact_with_grid_inputs(gpu, M, K, N, sa, sw):
    """Inputs that are E2M1 values times one power of two per operand, with a +-6 in every block of 32,
    so the rule reproduces them exactly (scale 2^s, element x / 2^s). Every product is a multiple of
    2^(sa+sw-2) and |sum| <= 36 K of 2^(sa+sw), fewer than 2^24 quarter-units for these K, so the
    matrix instruction's float32 sums are exact in any order: Y must be exactly
    bf16(sum_k x_k w_k), the float64 product rounded once."""
    import torch
    import quantized_gemm_amd as q
    say(f"[mxfp4 exact] M={M} K={K} N={N} 2^{sa} 2^{sw}")
    rng = np.random.default_rng(M + K + N)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6])
    a = grid[rng.integers(0, len(grid), size=(M, K))]
    b = grid[rng.integers(0, len(grid), size=(K, N))]
    a.reshape(M, K // 32, 32)[:, :, 3] = 6 * np.where(rng.random((M, K // 32)) < 0.5, -1, 1)
    b.reshape(K // 32, 32, N)[:, 11, :] = 6 * np.where(rng.random((K // 32, N)) < 0.5, -1, 1)
    x = np.ldexp(a, sa).astype(np.float32)
    w = np.ldexp(b, sw).astype(np.float32)
    xb = synth.bf16_bits_from_f32(x)
    assert np.array_equal(synth.f32_from_bf16_bits(xb), x)
    pw, psw = q.svdq_pack_weights(q.SVDQ_FMT_MXFP4_E8M0SCALE, w)
    assert np.all(psw == sw + 127)
    gq, gs = Guarded((K // 64, M, 32), torch.uint8, gpu), Guarded((K // 64, M, 2), torch.uint8, gpu)
    gy = Guarded((M, N), torch.bfloat16, gpu)
    qact, ascale, _ = q.svdq_quantize_act_mxfp4(to_dev_bf16(xb, gpu), None, None, gq.tensor, gs.tensor, None)
    y = q.svdq_linear_mxfp4(qact, ascale, to_dev(pw, gpu), to_dev(psw, gpu), None, None, None, gy.tensor)
    for g, what in ((gq, "qact"), (gs, "ascale"), (gy, "y")):
        g.check(what)
    assert np.all(ascale.cpu().numpy() == sa + 127), "activation scales differ"
    assert np.array_equal(oracle.e2m1_decode(decode_mx_codes(qact.cpu().numpy(), M, K)), a), "codes differ"
    ref = oracle.bf16_round((a.astype(np.float64) @ b.astype(np.float64)) * 2.0 ** (sa + sw))
    got = bf16_to_np(y)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} outputs differ, first at {bad[:3].tolist()}"
