"""CPU tests of the C ABI library: symbol exports, argument validation, and the host packer
checked bit for bit against the oracle (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))
HEADER = os.path.join(os.path.dirname(HERE), "include", "svdq.h")

q = pytest.importorskip("quantized_gemm_amd")


@pytest.fixture(scope="module")
def lib():
    try:
        return q.load_library()
    except RuntimeError as e:
        pytest.fail(str(e))


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\**([a-z_0-9]+)\(", text, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert {"svdq_quantize_act", "svdq_linear_w4a4", "awq_linear_w4a16", "svdq_pack_weights",
            "svdq_pack_lowrank", "svdq_debug_group_sums"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.svdq_abi_version() == 1


# ---------------------------------------------------------------------------------------------
# decoders written from the layout description in include/svdq.h
# ---------------------------------------------------------------------------------------------
def decode_w4a4(packed: np.ndarray, rows: int, K: int) -> np.ndarray:
    """Group-major: (group g, row) -> 32 bytes at (g*rows + row)*32, byte b = codes of
    k = 64g + 2b (low nibble) and 64g + 2b + 1 (high nibble), two's complement -> int8 [rows, K]."""
    G = K // 64
    out = np.empty((rows, K), np.int16)
    flat = packed.reshape(-1)
    for g in range(G):
        for r in range(rows):
            blk = flat[(g * rows + r) * 32:(g * rows + r) * 32 + 32].astype(np.int16)
            out[r, 64 * g + 0:64 * g + 64:2] = blk & 0xF
            out[r, 64 * g + 1:64 * g + 64:2] = (blk >> 4) & 0xF
    out[out >= 8] -= 16
    return out.astype(np.int8)


def decode_w4a16(packed: np.ndarray, K: int, N: int) -> np.ndarray:
    """W4A16 layout -> int8 codes [K, N]: per column tile, group pairs in 1 KiB blocks with 16
    bytes per lane (8 per group); an unpaired last group is a 512-byte block, 8 bytes per lane."""
    G = K // 64
    flat = packed.reshape(-1)
    shifts = [0, 16, 4, 20, 8, 24, 12, 28]
    codes = np.empty((K, N), np.int8)
    for n in range(N):
        t, i = divmod(n, 16)
        for k in range(K):
            g, kk = divmod(k, 64)
            h, rem = divmod(kk, 32)
            j, s = divmod(rem, 8)
            lane = i + 16 * j
            if G % 2 == 1 and g == G - 1:
                off = t * G * 512 + g * 512 + 8 * lane
            else:
                off = t * G * 512 + (g - g % 2) * 512 + 16 * lane + 8 * (g % 2)
            w = int(flat[off + 4 * h:off + 4 * h + 4].view(np.uint32)[0])
            codes[k, n] = ((w >> shifts[s]) & 0xF) - 8
    return codes


def test_pack_w4a4_bit_exact_vs_oracle(lib):
    rng = np.random.default_rng(21)
    K, N = 256, 48
    r = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    r[64:128, 5] = 0.0                                     # zero group
    r[128:192, 7] = np.float32(3e-44) * rng.standard_normal(64).astype(np.float32)  # subnormal scale
    r[:, 9] *= 1e3
    qw, sw = q.svdq_pack_weights(q.SVDQ_FMT_W4A4_F32SCALE, r)
    oc, os_ = oracle.quantize_weights_w4a4(r)
    assert np.array_equal(sw, os_)
    codes = decode_w4a4(qw, N, K).T
    assert np.array_equal(codes, oc)
    assert codes.min() >= -8 and codes.max() <= 7


def test_pack_w4a4_on_layer_residual(lib):
    cfg = synth.CONFIGS["tiny"]
    inp = synth.make_layer_inputs(cfg)
    x = synth.f32_from_bf16_bits(inp["x"])
    w = synth.f32_from_bf16_bits(inp["w"])
    d = oracle.svdq_decompose(x, w, cfg.rank)
    qw, sw = q.svdq_pack_weights(q.SVDQ_FMT_W4A4_F32SCALE, d["resid"])
    oc, os_ = oracle.quantize_weights_w4a4(d["resid"])
    assert np.array_equal(sw, os_)
    assert np.array_equal(decode_w4a4(qw, cfg.N, cfg.K).T, oc)


@pytest.mark.parametrize("K", [128, 192])
def test_pack_w4a16_bit_exact_vs_oracle(lib, K):
    rng = np.random.default_rng(22)
    N = 32
    w = oracle.bf16_round((rng.standard_normal((K, N)) * 0.02).astype(np.float32))
    w[:64, 3] = 0.0
    qw, s = q.svdq_pack_weights(q.SVDQ_FMT_W4A16_BF16SCALE, w)
    oc, os_ = oracle.quantize_weights_w4a16(w)
    assert np.array_equal(synth.f32_from_bf16_bits(s), os_)
    assert np.array_equal(decode_w4a16(qw, K, N), oc)


def test_pack_lowrank_bit_exact(lib):
    rng = np.random.default_rng(23)
    K, N, r = 128, 64, 32
    l1 = rng.standard_normal((K, r)).astype(np.float32)
    l2 = rng.standard_normal((r, N)).astype(np.float32)
    l1t, l2t = q.svdq_pack_lowrank(l1, l2)
    # decode the L1t operand blocks (layout in include/svdq.h)
    flat = synth.f32_from_bf16_bits(l1t.reshape(-1))
    G = K // 64
    dec = np.empty((K, r), np.float32)
    for c in range(r // 16):
        for g in range(G):
            for hh in range(2):
                for lane in range(64):
                    i, jl = lane % 16, lane // 16
                    for e in range(8):
                        dec[64 * g + 32 * hh + 8 * jl + e, 16 * c + i] = flat[(((c * G + g) * 2 + hh) * 64 + lane) * 8 + e]
    assert np.array_equal(dec, oracle.bf16_round(l1))
    assert np.array_equal(synth.f32_from_bf16_bits(l2t), oracle.bf16_round(l2).T)


def test_product_prep_matches_oracle_prep():
    from quantized_gemm_amd import prep
    cfg = synth.CONFIGS["tiny"]
    inp = synth.make_layer_inputs(cfg)
    x = synth.f32_from_bf16_bits(inp["x"])
    w = synth.f32_from_bf16_bits(inp["w"])
    d = oracle.svdq_decompose(x, w, cfg.rank)
    p = prep.decompose(x, w, cfg.rank)
    assert np.array_equal(p["inv_smooth"], d["inv"])
    # the same LAPACK routine on the same matrix: identical factors
    assert np.array_equal(p["l1"], d["l1_bf16"]) and np.array_equal(p["l2"], d["l2_bf16"])
    assert np.array_equal(p["resid"], d["resid"])


def test_product_prep_reuses_the_svd_across_ranks():
    from quantized_gemm_amd import prep
    cfg = synth.CONFIGS["tiny"]
    inp = synth.make_layer_inputs(cfg)
    x = synth.f32_from_bf16_bits(inp["x"])
    w = synth.f32_from_bf16_bits(inp["w"])
    first = prep.decompose(x, w, 32)
    for r in (16, 48):
        fresh, reused = prep.decompose(x, w, r), prep.decompose(x, w, r, svd=first["svd"])
        for key in ("inv_smooth", "l1", "l2", "resid"):
            assert np.array_equal(fresh[key], reused[key]), (r, key)
    assert prep.decompose(x, w, 0)["svd"] is None


# ---------------------------------------------------------------------------------------------
# argument validation (checked before any HIP call, so it runs without a GPU)
# ---------------------------------------------------------------------------------------------
P = 0x10000  # a 16-byte-aligned dummy address; never dereferenced on the error paths below
ODD = 0x10008


def test_packer_validation(lib):
    assert lib.svdq_pack_weights(7, P, 64, 16, P, P) == -4
    assert lib.svdq_pack_weights(0, None, 64, 16, P, P) == -1
    assert lib.svdq_pack_weights(0, P, 65, 16, P, P) == -2
    assert lib.svdq_pack_weights(1, P, 64, 8, P, P) == -2
    assert lib.svdq_pack_lowrank(P, P, 64, 16, 8, P, P) == -3
    assert lib.svdq_pack_lowrank(P, P, 64, 16, 272, P, P) == -3
    assert lib.svdq_packed_weight_bytes(0, 64, 16) == 512
    assert lib.svdq_scale_bytes(0, 128, 16) == 128 and lib.svdq_scale_bytes(1, 128, 16) == 64
    assert lib.svdq_scale_bytes(3, 128, 16) == 0 and lib.svdq_packed_weight_bytes(0, 100, 16) == 0


def test_device_entry_validation(lib):
    # svdq_quantize_act(x, M, K, inv, l1t, r, qact, ascale, lora, stream)
    assert lib.svdq_quantize_act(None, 16, 64, None, None, 0, P, P, None, None) == -1
    assert lib.svdq_quantize_act(ODD, 16, 64, None, None, 0, P, P, None, None) == -1
    assert lib.svdq_quantize_act(P, 0, 64, None, None, 0, P, P, None, None) == -2
    assert lib.svdq_quantize_act(P, 16, 96, None, None, 0, P, P, None, None) == -2
    assert lib.svdq_quantize_act(P, 1 << 27, 64, None, None, 0, P, P, None, None) == -2   # row limit
    assert lib.svdq_quantize_act(P, 16, 64, None, P, 24, P, P, P, None) == -3
    assert lib.svdq_quantize_act(P, 16, 64, None, P, 0, P, P, None, None) == -3
    assert lib.svdq_quantize_act(P, 16, 64, None, P, 32, P, P, None, None) == -3
    # svdq_linear_w4a4(qa, sa, qw, sw, lora, l2t, r, bias, y, M, N, K, stream)
    assert lib.svdq_linear_w4a4(P, P, P, P, None, None, 0, None, None, 16, 16, 64, None) == -1
    assert lib.svdq_linear_w4a4(P, P, P, P, None, None, 0, None, P, 16, 24, 64, None) == -2
    assert lib.svdq_linear_w4a4(P, P, P, P, None, None, 0, None, P, 16, 16, 0, None) == -2
    assert lib.svdq_linear_w4a4(P, P, P, P, None, None, 0, None, P, 16, 1 << 27, 64, None) == -2
    assert lib.svdq_linear_w4a4(P, P, P, P, P, None, 32, None, P, 16, 16, 64, None) == -3
    assert lib.svdq_linear_w4a4(P, P, P, P, None, None, 0, ODD, P, 16, 16, 64, None) == -1
    # the fused-QKV form: norm / rotary tables required, N = 3 * heads * 128
    assert lib.svdq_linear_w4a4_qkv(P, P, P, P, None, None, 0, None, P, 16, 384, 64, 1, None, P, P, P, None) == -1
    assert lib.svdq_linear_w4a4_qkv(P, P, P, P, None, None, 0, None, P, 16, 384, 64, 1, P, P, P, ODD, None) == -1
    assert lib.svdq_linear_w4a4_qkv(P, P, P, P, None, None, 0, None, P, 16, 384, 64, 2, P, P, P, P, None) == -2
    assert lib.svdq_linear_w4a4_qkv(P, P, P, P, None, None, 0, None, P, 16, 384, 64, 0, P, P, P, P, None) == -2
    # the GELU form validates exactly like the plain one
    assert lib.svdq_linear_w4a4_gelu(P, P, P, P, None, None, 0, None, None, 16, 16, 64, None) == -1
    assert lib.svdq_linear_w4a4_gelu(P, P, P, P, None, None, 0, None, P, 16, 24, 64, None) == -2
    assert lib.svdq_linear_w4a4_gelu(P, P, P, P, P, None, 32, None, P, 16, 16, 64, None) == -3
    # awq_linear_w4a16(x, qw, scales, bias, y, M, N, K, stream)
    assert lib.awq_linear_w4a16(P, None, P, None, P, 16, 16, 64, None) == -1
    assert lib.awq_linear_w4a16(P, P, P, None, P, 16, 17, 64, None) == -2
    # svdq_debug_group_sums(qa, qw, M, N, K, m0, n0, tm, tn, out, stream)
    assert lib.svdq_debug_group_sums(P, P, 16, 16, 64, 8, 0, 16, 16, P, None) == -2
    assert lib.svdq_debug_group_sums(P, P, 16, 16, 64, 0, 0, 0, 16, P, None) == -2


def test_valid_arguments_without_gpu_report_arch(lib):
    """With valid arguments the next check is the device; this container has no GPU."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert lib.svdq_check_device() == -5
    assert lib.svdq_quantize_act(P, 16, 64, None, None, 0, P, P, None, None) == -5
    assert lib.svdq_linear_w4a4(P, P, P, P, None, None, 0, None, P, 16, 16, 64, None) == -5
    assert lib.svdq_linear_w4a4_gelu(P, P, P, P, None, None, 0, None, P, 16, 16, 64, None) == -5
    assert lib.svdq_linear_w4a4_qkv(P, P, P, P, None, None, 0, None, P, 16, 384, 64, 1, P, P, P, P, None) == -5
    assert lib.awq_linear_w4a16(P, P, P, None, P, 16, 16, 64, None) == -5


@pytest.mark.slow
def test_pack_full_up_shape_bit_exact_vs_oracle(lib):
    """The weights of the FLUX MLP up projection (K 3072, N 12288: 37.7M codes), packed by the library
    in both 4-bit formats and decoded with the documented layouts (vectorised decoder: group-major
    records, low nibble = even k), bit-exact against the oracle."""
    from problems import decode_mx_codes, decode_mx_scales, decode_qact
    cfg = synth.CONFIGS["up"]
    inp = synth.make_layer_inputs(cfg, M=64)
    w = synth.f32_from_bf16_bits(inp["w"])
    w[:, :3] *= 1e3                                         # columns with large groups
    w[:64, 3] = 0.0                                         # a zero group
    K, N = w.shape
    qw, sw = q.svdq_pack_weights(q.SVDQ_FMT_W4A4_F32SCALE, w)
    oc, os_ = oracle.quantize_weights_w4a4(w)
    assert np.array_equal(sw.view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(decode_qact(qw, N, K), np.ascontiguousarray(oc.T))
    qm, sm = q.svdq_pack_weights(q.SVDQ_FMT_MXFP4_E8M0SCALE, w)
    mc, ms = oracle.quantize_weights_mxfp4(w)
    assert np.array_equal(decode_mx_codes(qm, N, K), mc)
    assert np.array_equal(decode_mx_scales(sm, N, K), ms)
