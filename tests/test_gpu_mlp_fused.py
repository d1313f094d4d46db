"""The MLP pair fused across its boundary (svdq_linear_w4a4_gelu_quant): the up projection's
epilogue runs the down layer's activation step on the GELU output instead of storing it.

Checked against the oracle applied to the GELU output H that the GPU computes (the unfused
svdq_linear_w4a4_gelu, whose epilogue produces the same H): the down layer's INT4 codes and scales
bit-exact, its T within one bf16 ulp, and the down layer's Y within the layer bar.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from guard import Guarded
from problems import decode_qact, random_w4a4_problem, tolerance_report, within_one_bf16_ulp

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


# (M, D, F, r_up, r_down): one tile column pair, a ragged token count with a half last column tile
# (F % 128 == 64) and no up-projection branch, and the FLUX MLP pair
CASES = [(256, 256, 512, 16, 16), (100, 128, 320, 0, 32), (4608, 3072, 12288, 32, 32)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("M,D,F,ru,rd", CASES, ids=[f"M{m}D{d}F{f}r{a}-{b}" for m, d, f, a, b in CASES])
def test_gelu_quant_matches_oracle_on_gpu_intermediate(gpu, M, D, F, ru, rd):
    import torch
    import quantized_gemm_amd as q
    say(f"[mlp fused] M={M} D={D} F={F} r_up={ru} r_down={rd}")
    up = random_w4a4_problem(M, D, F, ru, seed=81 + M)
    qw1, sw1 = q.svdq_pack_weights(q.SVDQ_FMT_W4A4_F32SCALE, up["resid"])
    qw1, sw1 = to_dev(qw1, gpu), to_dev(sw1, gpu)
    l1t1 = l2t1 = None
    if ru:
        a, b = q.svdq_pack_lowrank(up["l1"], up["l2"])
        l1t1, l2t1 = to_dev_bf16(a, gpu), to_dev_bf16(b, gpu)
    bias1 = to_dev_bf16(up["bias_bits"], gpu)
    qa1, sa1, t1 = q.svdq_quantize_act(to_dev_bf16(up["x_bits"], gpu), to_dev(up["inv"], gpu), l1t1)
    # the GPU's own GELU output (not used by the fused path; the reference input of the oracle)
    h = q.svdq_linear_w4a4(qa1, sa1, qw1, sw1, t1, l2t1, bias1, activation="gelu_tanh")
    torch.cuda.synchronize()
    h_gpu = bf16_to_np(h)
    # the down layer, prepared from that intermediate
    w_dn = synth.random_f32((F, D), seed=82, scale=0.02)
    b_dn = oracle.bf16_round(synth.random_f32((D,), seed=83, scale=0.01))
    d_dn = oracle.svdq_decompose(h_gpu, w_dn, rd)
    inv2 = to_dev(d_dn["inv"], gpu)
    l1t2 = l2t2 = None
    if rd:
        a, b = q.svdq_pack_lowrank(d_dn["l1_bf16"], d_dn["l2_bf16"])
        l1t2, l2t2 = to_dev_bf16(a, gpu), to_dev_bf16(b, gpu)
    gq, gs = Guarded((F // 64, M, 32), torch.uint8, gpu), Guarded((F // 64, M), torch.float32, gpu)
    gt = Guarded((M, rd), torch.bfloat16, gpu) if rd else None
    qa2, sa2, t2 = q.svdq_linear_w4a4_gelu_quant(qa1, sa1, qw1, sw1, t1, l2t1, bias1, inv2, l1t2, gq.tensor, gs.tensor,
                                                 gt.tensor if rd else None)
    for g, what in ((gq, "qact_next"), (gs, "ascale_next"), (gt, "lora_act_next")):
        if g is not None:
            g.check(what)
    ref = oracle.svdq_layer(h_gpu, d_dn["inv"], d_dn["l1_bf16"], d_dn["l2_bf16"], d_dn["resid"], b_dn)
    assert np.array_equal(decode_qact(qa2.cpu().numpy(), M, F), ref["qa"]), "next-layer codes differ"
    assert np.array_equal(sa2.cpu().numpy().view(np.uint32), np.ascontiguousarray(ref["sa"]).view(np.uint32)), \
        "next-layer scales differ"
    if rd:
        tg = bf16_to_np(t2)
        ok = within_one_bf16_ulp(tg, ref["t"], abs_floor=2.0 ** -16 * float(np.abs(ref["t"]).max()))
        assert ok.all(), f"T beyond one bf16 ulp at {np.argwhere(~ok)[:5]}"
        say(f"  T exact fraction {np.mean(tg == ref['t']):.6f}")
    # the same as the unfused quantizer on the stored intermediate
    qa3, sa3, t3 = q.svdq_quantize_act(h, inv2, l1t2)
    torch.cuda.synchronize()
    assert torch.equal(qa2, qa3) and torch.equal(sa2.view(torch.int32), sa3.view(torch.int32))
    # and the down layer from the fused outputs
    qw2, sw2 = q.svdq_pack_weights(q.SVDQ_FMT_W4A4_F32SCALE, d_dn["resid"])
    y = q.svdq_linear_w4a4(qa2, sa2, to_dev(qw2, gpu), to_dev(sw2, gpu), t2, l2t2,
                           to_dev_bf16(synth.bf16_bits_from_f32(b_dn), gpu))
    torch.cuda.synchronize()
    mx, mean = tolerance_report(bf16_to_np(y), ref["y"])
    say(f"  Y = down(H) max|err|/max|Y| = {mx:.3e}, mean rel = {mean:.3e}")
    assert mx <= MAX_REL and mean <= MEAN_REL


def test_gelu_quant_rejects_bad_workspace(gpu):
    import torch
    import quantized_gemm_amd as q
    lib = q.load_library()
    assert lib.svdq_gelu_quant_workspace_bytes(4608, 12288, 32) == 96 * 4608 * 32 * 4
    assert lib.svdq_gelu_quant_workspace_bytes(100, 320, 32) == 3 * 100 * 32 * 4
    assert lib.svdq_gelu_quant_workspace_bytes(100, 336, 32) == 0          # N % 64 != 0
    up = random_w4a4_problem(64, 128, 256, 0, seed=5)
    qw, sw = q.svdq_pack_weights(q.SVDQ_FMT_W4A4_F32SCALE, up["resid"])
    qa, sa, _ = q.svdq_quantize_act(to_dev_bf16(up["x_bits"], gpu), to_dev(up["inv"], gpu), None)
    inv2 = torch.ones(256, dtype=torch.float32, device=gpu)
    l1t2 = torch.zeros((16, 256), dtype=torch.bfloat16, device=gpu)
    small = torch.empty(16, dtype=torch.uint8, device=gpu)
    with pytest.raises(q.SvdqError):
        q.svdq_linear_w4a4_gelu_quant(qa, sa, to_dev(qw, gpu), to_dev(sw, gpu), None, None, None, inv2, l1t2,
                                      workspace=small)
