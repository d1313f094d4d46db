"""Shared test fixtures: synthetic layer problems prepared and evaluated by the oracle, plus the
independent decoders / encoders of the packed layouts documented in include/svdq.h.

Only the oracle produces expected values here; the GPU path's outputs are compared against them.
"""
from __future__ import annotations

import functools

import numpy as np

import oracle
import synth


@functools.lru_cache(maxsize=2)
def _raw(name: str, M: int):
    """Drawn inputs and the SVD of the smoothed weight, shared by every rank of one layer."""
    cfg = synth.CONFIGS[name]
    inp = synth.make_layer_inputs(cfg, M=M)
    x = synth.f32_from_bf16_bits(inp["x"])
    w = synth.f32_from_bf16_bits(inp["w"])
    _, lam_prime = oracle.smoothing_factors(x, w)
    svd = np.linalg.svd(lam_prime[:, None] * w.astype(np.float64), full_matrices=False)
    return inp, x, w, svd


@functools.lru_cache(maxsize=3)
def w4a4_problem(name: str, M: int = None, rank: int = None):
    """Inputs + oracle results for one W4A4 configuration (optionally with another M or rank)."""
    cfg = synth.CONFIGS[name]
    if rank is not None:
        cfg = cfg.with_rank(rank)
    inp, x, w, svd = _raw(name, M)
    b = synth.f32_from_bf16_bits(inp["bias"]) if inp["bias"] is not None else None
    d = oracle.svdq_decompose(x, w, cfg.rank, svd=svd)
    out = oracle.svdq_layer(x, d["inv"], d["l1_bf16"], d["l2_bf16"], d["resid"], b)
    return {"cfg": cfg, "x_bits": inp["x"], "x": x, "bias_bits": inp["bias"], "bias": b,
            "inv": d["inv"], "l1": d["l1_bf16"], "l2": d["l2_bf16"], "resid": d["resid"], **out}


def random_w4a4_problem(M: int, K: int, N: int, rank: int, seed: int):
    """A W4A4 layer of arbitrary shape from seeded N(0,1) activations (with a few outlier
    channels), N(0, 0.02) weights and N(0, 0.01) bias, prepared and evaluated by the oracle."""
    cfg = synth.LayerConfig(f"rand{M}x{K}x{N}", M, K, N, rank, seed=seed, n_outliers=max(1, K // 100),
                            outlier_scale=30.0)
    inp = synth.make_layer_inputs(cfg)
    x = synth.f32_from_bf16_bits(inp["x"])
    w = synth.f32_from_bf16_bits(inp["w"])
    b = synth.f32_from_bf16_bits(inp["bias"])
    d = oracle.svdq_decompose(x, w, rank)
    out = oracle.svdq_layer(x, d["inv"], d["l1_bf16"], d["l2_bf16"], d["resid"], b)
    return {"cfg": cfg, "x_bits": inp["x"], "x": x, "bias_bits": inp["bias"], "bias": b,
            "inv": d["inv"], "l1": d["l1_bf16"], "l2": d["l2_bf16"], "resid": d["resid"], **out}


@functools.lru_cache(maxsize=4)
def w4a16_problem(name: str = "awq", M: int = None, with_bias: bool = False):
    cfg = synth.CONFIGS[name]
    inp = synth.make_layer_inputs(cfg, M=M)
    x = synth.f32_from_bf16_bits(inp["x"])
    w = synth.f32_from_bf16_bits(inp["w"])
    b = None
    if with_bias:
        b = oracle.bf16_round(synth.random_f32((cfg.N,), seed=cfg.seed + 100, scale=0.01))
    codes, s = oracle.quantize_weights_w4a16(w)
    y64, y = oracle.awq_linear(x, codes, s, b)
    return {"cfg": cfg, "x_bits": inp["x"], "x": x, "w": w, "bias": b, "codes": codes, "scales": s,
            "y64": y64, "y": y}


def decode_qact(packed: np.ndarray, rows: int, K: int) -> np.ndarray:
    """Group-major packed codes (the 32 bytes of (group g, row) at (g*rows + row)*32; byte b holds
    k = 64g + 2b in its low nibble and 64g + 2b + 1 in its high nibble, two's complement)
    -> int8 [rows, K]."""
    G = K // 64
    b = np.asarray(packed, dtype=np.uint8).reshape(G, rows, 32).astype(np.int16)
    out = np.empty((rows, G, 64), np.int16)
    out[:, :, 0::2] = (b & 0xF).transpose(1, 0, 2)
    out[:, :, 1::2] = ((b >> 4) & 0xF).transpose(1, 0, 2)
    out[out >= 8] -= 16
    return out.reshape(rows, K).astype(np.int8)


def bf16_bits(a_f32: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_from_f32(a_f32)


def tolerance_report(y: np.ndarray, y_ref: np.ndarray):
    """(max|err| / max|Y_ref|, sum|err| / sum|Y_ref|) in float64."""
    y = y.astype(np.float64)
    y_ref = y_ref.astype(np.float64)
    err = np.abs(y - y_ref)
    return float(err.max() / np.abs(y_ref).max()), float(err.sum() / np.abs(y_ref).sum())


def within_one_bf16_ulp(a: np.ndarray, b: np.ndarray, abs_floor: float) -> np.ndarray:
    """Elementwise: bf16 values a and b are equal, adjacent, or both within abs_floor of each other."""
    ab = synth.bf16_bits_from_f32(a).astype(np.int32)
    bb = synth.bf16_bits_from_f32(b).astype(np.int32)
    same_sign = (ab >> 15) == (bb >> 15)
    adjacent = same_sign & (np.abs(ab - bb) <= 1)
    return adjacent | (np.abs(a.astype(np.float64) - b.astype(np.float64)) <= abs_floor)


def decode_mx_codes(packed: np.ndarray, rows: int, K: int) -> np.ndarray:
    """MXFP4 codes in the group-major record (byte b of (slab g, row) holds k = 64g + 2b in bits 0-3
    and 64g + 2b + 1 in bits 4-7) -> uint8 4-bit codes [rows, K]."""
    G = K // 64
    b = np.asarray(packed, dtype=np.uint8).reshape(G, rows, 32)
    out = np.empty((rows, G, 64), np.uint8)
    out[:, :, 0::2] = (b & 0xF).transpose(1, 0, 2)
    out[:, :, 1::2] = (b >> 4).transpose(1, 0, 2)
    return out.reshape(rows, K)


def decode_mx_scales(scales: np.ndarray, rows: int, K: int) -> np.ndarray:
    """E8M0 bytes [K/64, rows, 2] (block 2g + h of a row at (g*rows + row)*2 + h) -> uint8 [rows, K/32]."""
    s = np.asarray(scales, dtype=np.uint8).reshape(K // 64, rows, 2)
    return np.ascontiguousarray(s.transpose(1, 0, 2).reshape(rows, K // 32))


def mxfp4_problem(M: int, K: int, N: int, rank: int, seed: int, resid_zero: bool = False):
    """A seeded MXFP4 layer (same input recipe as the INT4 layers) prepared and evaluated by the oracle."""
    cfg = synth.LayerConfig(f"mx{M}x{K}x{N}", M, K, N, rank, seed=seed, n_outliers=max(1, K // 100),
                            outlier_scale=30.0)
    inp = synth.make_layer_inputs(cfg)
    x = synth.f32_from_bf16_bits(inp["x"])
    w = synth.f32_from_bf16_bits(inp["w"])
    b = synth.f32_from_bf16_bits(inp["bias"])
    d = oracle.svdq_decompose(x, w, rank)
    resid = np.zeros_like(d["resid"]) if resid_zero else d["resid"]
    out = oracle.svdq_layer_mxfp4(x, d["inv"], d["l1_bf16"], d["l2_bf16"], resid, b)
    return {"cfg": cfg, "x_bits": inp["x"], "x": x, "bias_bits": inp["bias"], "bias": b, "inv": d["inv"],
            "l1": d["l1_bf16"], "l2": d["l2_bf16"], "resid": resid, **out}
