"""The no-allocation entry point svdq_linear_w4a4_gelu_quant_noalloc against the workspace entry
point svdq_linear_w4a4_gelu_quant, through the C ABI: the same kernels, so the next layer's codes,
scales and T must be bit-identical. Two calls in a row, the second with a smaller input (the scratch
keeps the first call's contents), and a size beyond the scratch rejected before any launch."""
import numpy as np
import pytest

import synth
from problems import random_w4a4_problem

pytestmark = pytest.mark.gpu


def to_dev_bf16(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def to_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _layer(M, D, F, ru, rd, seed, dev):
    import torch
    import quantized_gemm_amd as q
    up = random_w4a4_problem(M, D, F, ru, seed=seed)
    qw, sw = q.svdq_pack_weights(q.SVDQ_FMT_W4A4_F32SCALE, up["resid"])
    l1t = l2t = None
    if ru:
        a, b = q.svdq_pack_lowrank(up["l1"], up["l2"])
        l1t, l2t = to_dev_bf16(a, dev), to_dev_bf16(b, dev)
    qa, sa, t = q.svdq_quantize_act(to_dev_bf16(up["x_bits"], dev), to_dev(up["inv"], dev), l1t)
    rng = np.random.default_rng(seed)
    inv2 = torch.from_numpy((1.0 / rng.uniform(0.5, 2.0, F)).astype(np.float32)).to(dev)
    l1n = torch.from_numpy(synth.random_bf16((rd, F), seed=seed + 1, scale=0.05).view(np.int16)).to(dev).view(
        torch.bfloat16) if rd else None
    return (qa, sa, to_dev(qw, dev), to_dev(sw, dev), t, l2t, to_dev_bf16(up["bias_bits"], dev), inv2, l1n)


def test_noalloc_matches_workspace_entry_point():
    import torch
    import quantized_gemm_amd as q
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    dev = torch.device("cuda:0")
    q.load_library()
    q.svdq_check_device()
    for (M, D, F, ru, rd, seed) in [(256, 256, 512, 16, 32, 91), (100, 128, 320, 0, 16, 92)]:
        args = _layer(M, D, F, ru, rd, seed, dev)
        qa_w, sa_w, t_w = q.svdq_linear_w4a4_gelu_quant(*args)
        qa_n = torch.full((F // 64, M, 32), 0xA5, dtype=torch.uint8, device=dev)
        sa_n = torch.full((F // 64, M), -1.0, dtype=torch.float32, device=dev)
        t_n = torch.full((M, rd), -1.0, dtype=torch.bfloat16, device=dev)
        q.svdq_linear_w4a4_gelu_quant_noalloc(*args, qa_n, sa_n, t_n)
        torch.cuda.synchronize()
        assert torch.equal(qa_n, qa_w), (M, F)
        assert torch.equal(sa_n.view(torch.int32), sa_w.view(torch.int32)), (M, F)
        assert torch.equal(t_n.view(torch.int16), t_w.view(torch.int16)), (M, F)
    # beyond the scratch: the size check comes first, so the library returns SVDQ_ERR_SHAPE without
    # touching a pointer or launching anything (the address values below are never dereferenced)
    lib = q.load_library()
    assert lib.svdq_gelu_quant_workspace_bytes(8192, 16384, 256) > 64 << 20
    fake = 1 << 12
    st = lib.svdq_linear_w4a4_gelu_quant_noalloc(fake, fake, fake, fake, None, None, 0, None, 8192, 16384, 64, fake,
                                                  fake, 256, fake, fake, fake, None)
    assert st == -2, st
