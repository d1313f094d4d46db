"""Thin ctypes binding of ``libsvdq.so`` (the C ABI in include/svdq.h).

Argument marshalling only: every step of the layer runs in the library's HIP kernels (device
entry points) or its C++ packer (host entry points). Functions carry the C names; device entry
points take torch tensors on the current HIP device and enqueue on the current torch stream
unless a stream handle is given. There is no fallback: a missing library or a non-gfx950 device
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libsvdq.so")
_lib = None

SVDQ_OK = 0
SVDQ_FMT_W4A4_F32SCALE = 0
SVDQ_FMT_W4A16_BF16SCALE = 1
SVDQ_FMT_MXFP4_E8M0SCALE = 2
GROUP = 64

_vp, _i64, _int, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t

_SIGNATURES = {
    "svdq_status_string": (ctypes.c_char_p, [_int]),
    "svdq_abi_version": (_int, []),
    "svdq_check_device": (_int, []),
    "svdq_packed_weight_bytes": (_sz, [_int, _i64, _i64]),
    "svdq_scale_bytes": (_sz, [_int, _i64, _i64]),
    "svdq_pack_weights": (_int, [_int, _vp, _i64, _i64, _vp, _vp]),
    "svdq_pack_lowrank": (_int, [_vp, _vp, _i64, _i64, _int, _vp, _vp]),
    "svdq_quantize_act": (_int, [_vp, _i64, _i64, _vp, _vp, _int, _vp, _vp, _vp, _vp]),
    "svdq_linear_w4a4": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _int, _vp, _vp, _i64, _i64, _i64, _vp]),
    "svdq_linear_w4a4_gelu": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _int, _vp, _vp, _i64, _i64, _i64, _vp]),
    "svdq_linear_w4a4_qkv": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _int, _vp, _vp, _i64, _i64, _i64, _int, _vp, _vp,
                                    _vp, _vp, _vp]),
    "awq_linear_w4a16": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "svdq_debug_group_sums": (_int, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _vp, _vp]),
    "svdq_bench_unit_peak": (_int, [_int, _int, _int, _vp, _vp, _vp]),
    "svdq_gelu_quant_workspace_bytes": (_sz, [_i64, _i64, _int]),
    "svdq_linear_w4a4_gelu_quant": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _int, _vp, _i64, _i64, _i64, _vp, _vp, _int,
                                           _vp, _vp, _vp, _vp, _sz, _vp]),
    "svdq_linear_w4a4_gelu_quant_noalloc": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _int, _vp, _i64, _i64, _i64, _vp,
                                                   _vp, _int, _vp, _vp, _vp, _vp]),
    "svdq_quantize_act_mxfp4": (_int, [_vp, _i64, _i64, _vp, _vp, _int, _vp, _vp, _vp, _vp]),
    "svdq_linear_mxfp4": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _int, _vp, _vp, _i64, _i64, _i64, _vp]),
}


class SvdqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"HIP library not built: {_LIB_PATH} is missing "
                               "(run quantized_gemm_amd/build.py or __graft_entry__.build())")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load_library().svdq_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != SVDQ_OK:
        raise SvdqError(fn, status)


def svdq_abi_version() -> int:
    return load_library().svdq_abi_version()


def svdq_check_device() -> None:
    _check("svdq_check_device", load_library().svdq_check_device())


# ------------------------------------------------------------------------------------------------
# Host packer (numpy in, numpy out)
# ------------------------------------------------------------------------------------------------
def _np_ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _aligned_empty(nbytes: int, dtype) -> np.ndarray:
    raw = np.empty(nbytes + 64, dtype=np.uint8)
    off = (-raw.ctypes.data) % 64
    return raw[off:off + nbytes].view(dtype)


def svdq_pack_weights(fmt: int, w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Pack a float32 [K, N] weight; returns (qweight uint8 [K*N/2], scales [K/64, N])."""
    lib = load_library()
    w = np.ascontiguousarray(w, dtype=np.float32)
    K, N = w.shape
    qbytes = lib.svdq_packed_weight_bytes(fmt, K, N)
    sbytes = lib.svdq_scale_bytes(fmt, K, N)
    if qbytes == 0 or sbytes == 0:
        _check("svdq_pack_weights", lib.svdq_pack_weights(fmt, None, K, N, None, None) or -2)
    q = _aligned_empty(qbytes, np.uint8)
    sdt = {SVDQ_FMT_W4A4_F32SCALE: np.float32, SVDQ_FMT_W4A16_BF16SCALE: np.uint16}.get(fmt, np.uint8)
    s = _aligned_empty(sbytes, sdt)
    _check("svdq_pack_weights", lib.svdq_pack_weights(fmt, _np_ptr(w), K, N, _np_ptr(q), _np_ptr(s)))
    if fmt == SVDQ_FMT_MXFP4_E8M0SCALE:
        return q, s.reshape(K // GROUP, N, 2)
    return q, s.reshape(K // GROUP, N)


def svdq_pack_lowrank(l1: np.ndarray, l2: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """float32 L1 [K, r], L2 [r, N] -> bf16 bits of L1 in the MFMA operand-block order of
    include/svdq.h (r*K values, shaped (r, K) for its size only) and of L2^T [N, r]."""
    l1 = np.ascontiguousarray(l1, dtype=np.float32)
    l2 = np.ascontiguousarray(l2, dtype=np.float32)
    K, r = l1.shape
    r2, N = l2.shape
    if r2 != r:
        raise ValueError("L1 [K, r] and L2 [r, N] disagree on r")
    l1t = _aligned_empty(r * K * 2, np.uint16).reshape(r, K)
    l2t = _aligned_empty(N * r * 2, np.uint16).reshape(N, r)
    _check("svdq_pack_lowrank", load_library().svdq_pack_lowrank(_np_ptr(l1), _np_ptr(l2), K, N, r,
                                                                 _np_ptr(l1t), _np_ptr(l2t)))
    return l1t, l2t


# ------------------------------------------------------------------------------------------------
# Device entry points (torch tensors on the current HIP device)
# ------------------------------------------------------------------------------------------------
def _dev_ptr(t, name: str, dtypes, shape=None) -> int:
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    return t.data_ptr()


def _stream(stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _bf16():
    import torch
    return (torch.bfloat16, torch.int16, torch.uint16)


def svdq_quantize_act(x, inv_smooth, l1t, qact=None, ascale=None, lora_act=None, stream=None):
    """Kernel (a). x bf16 [M, K]; inv_smooth float32 [K] or None; l1t bf16 [r, K] or None.

    Returns (qact uint8 [M, K/2], ascale float32 [K/64, M], lora_act bf16 [M, r] or None).
    """
    import torch
    M, K = x.shape
    r = 0 if l1t is None else l1t.shape[0]
    dev = x.device
    if qact is None:
        qact = torch.empty((K // GROUP, M, 32), dtype=torch.uint8, device=dev)  # group-major codes
    if ascale is None:
        ascale = torch.empty((K // GROUP, M), dtype=torch.float32, device=dev)
    if r and lora_act is None:
        lora_act = torch.empty((M, r), dtype=torch.bfloat16, device=dev)
    st = load_library().svdq_quantize_act(
        _dev_ptr(x, "x", _bf16()), M, K, _dev_ptr(inv_smooth, "inv_smooth", (torch.float32,), (K,)),
        _dev_ptr(l1t, "l1t", _bf16(), (r, K) if r else None), r,
        _dev_ptr(qact, "qact", (torch.uint8,), (K // GROUP, M, 32)),
        _dev_ptr(ascale, "ascale", (torch.float32,), (K // GROUP, M)),
        _dev_ptr(lora_act, "lora_act", _bf16(), (M, r)) if r else None, _stream(stream))
    _check("svdq_quantize_act", st)
    return qact, ascale, (lora_act if r else None)


def svdq_linear_w4a4(qact, ascale, qweight, wscale, lora_act, l2t, bias, y=None, stream=None, activation=None):
    """Kernel (b). qact uint8 [K/64, M, 32] (group-major codes), ascale float32 [K/64, M],
    qweight uint8 (K*N/2 bytes, group-major), wscale float32 [K/64, N]. Returns y bf16 [M, N].
    activation: None, or "gelu_tanh" for the MLP up projection (svdq_linear_w4a4_gelu)."""
    if activation not in (None, "gelu_tanh"):
        raise ValueError(f"unknown activation {activation!r}")
    fn = "svdq_linear_w4a4" if activation is None else "svdq_linear_w4a4_gelu"
    import torch
    G, M = ascale.shape
    K = G * GROUP
    N = wscale.shape[1]
    if qact.numel() != M * K // 2:
        raise ValueError("qact size does not match K*M/2")
    r = 0 if l2t is None else l2t.shape[1]
    if qweight.numel() != N * K // 2:
        raise ValueError("qweight size does not match [N, K/2]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=qact.device)
    st = getattr(load_library(), fn)(
        _dev_ptr(qact, "qact", (torch.uint8,)), _dev_ptr(ascale, "ascale", (torch.float32,), (K // GROUP, M)),
        _dev_ptr(qweight, "qweight", (torch.uint8,)), _dev_ptr(wscale, "wscale", (torch.float32,), (K // GROUP, N)),
        _dev_ptr(lora_act, "lora_act", _bf16(), (M, r)) if r else None,
        _dev_ptr(l2t, "l2t", _bf16(), (N, r)) if r else None, r,
        _dev_ptr(bias, "bias", _bf16(), (N,)), _dev_ptr(y, "y", _bf16(), (M, N)), M, N, K, _stream(stream))
    _check(fn, st)
    return y


def svdq_linear_w4a4_qkv(qact, ascale, qweight, wscale, lora_act, l2t, bias, heads, q_norm_w, k_norm_w, rope_cos,
                         rope_sin, y=None, stream=None):
    """Kernel (b) for a fused QKV projection (N = 3 * heads * 128) with the per-head RMS norm of Q
    and K (weights float32 [128]) and the rotary embedding (rope_cos / rope_sin float32 [M, 64])
    in its epilogue. Returns y bf16 [M, N]."""
    import torch
    G, M = ascale.shape
    K = G * GROUP
    N = wscale.shape[1]
    if qact.numel() != M * K // 2:
        raise ValueError("qact size does not match K*M/2")
    r = 0 if l2t is None else l2t.shape[1]
    if qweight.numel() != N * K // 2:
        raise ValueError("qweight size does not match [N, K/2]")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=qact.device)
    f32 = (torch.float32,)
    st = load_library().svdq_linear_w4a4_qkv(
        _dev_ptr(qact, "qact", (torch.uint8,)), _dev_ptr(ascale, "ascale", f32, (K // GROUP, M)),
        _dev_ptr(qweight, "qweight", (torch.uint8,)), _dev_ptr(wscale, "wscale", f32, (K // GROUP, N)),
        _dev_ptr(lora_act, "lora_act", _bf16(), (M, r)) if r else None,
        _dev_ptr(l2t, "l2t", _bf16(), (N, r)) if r else None, r,
        _dev_ptr(bias, "bias", _bf16(), (N,)), _dev_ptr(y, "y", _bf16(), (M, N)), M, N, K, int(heads),
        _dev_ptr(q_norm_w, "q_norm_w", f32, (128,)), _dev_ptr(k_norm_w, "k_norm_w", f32, (128,)),
        _dev_ptr(rope_cos, "rope_cos", f32, (M, 64)), _dev_ptr(rope_sin, "rope_sin", f32, (M, 64)),
        _stream(stream))
    _check("svdq_linear_w4a4_qkv", st)
    return y


def awq_linear_w4a16(x, qweight, scales, bias, y=None, stream=None):
    """Kernel (c). x bf16 [M, K]; qweight uint8 (W4A16 block layout); scales bf16 [K/64, N]."""
    import torch
    M, K = x.shape
    N = scales.shape[1]
    if qweight.numel() != N * K // 2:
        raise ValueError("qweight size does not match K*N/2")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    st = load_library().awq_linear_w4a16(
        _dev_ptr(x, "x", _bf16()), _dev_ptr(qweight, "qweight", (torch.uint8,)),
        _dev_ptr(scales, "scales", _bf16(), (K // GROUP, N)), _dev_ptr(bias, "bias", _bf16(), (N,)),
        _dev_ptr(y, "y", _bf16(), (M, N)), M, N, K, _stream(stream))
    _check("awq_linear_w4a16", st)
    return y


def svdq_debug_group_sums(qact, qweight, N: int, m0: int, n0: int, tm: int, tn: int, out=None, stream=None):
    """Exact per-group integer sums P[g, m0+i, n0+j] of the W4A4 product: int32 [K/64, tm, tn].
    qact uint8 [K/64, M, 32]."""
    import torch
    if qact.dim() != 3 or qact.shape[2] != 32:
        raise ValueError(f"qact must be [K/64, M, 32], got {tuple(qact.shape)}")
    G, M, _ = qact.shape
    K = G * GROUP
    if qweight.numel() != N * K // 2:
        raise ValueError("qweight size does not match [N, K/2]")
    if out is None:
        out = torch.empty((K // GROUP, tm, tn), dtype=torch.int32, device=qact.device)
    st = load_library().svdq_debug_group_sums(
        _dev_ptr(qact, "qact", (torch.uint8,)), _dev_ptr(qweight, "qweight", (torch.uint8,)), M, N, K, m0, n0, tm, tn,
        _dev_ptr(out, "out", (torch.int32,), (K // GROUP, tm, tn)), _stream(stream))
    _check("svdq_debug_group_sums", st)
    return out


SVDQ_BENCH_KINDS = {"mfma_i8_32x32x32": (0, 2 * 32 * 32 * 32), "mfma_bf16_32x32x16": (1, 2 * 32 * 32 * 16),
                    "mfma_f32_32x32x1_2b": (2, 2 * 2 * 32 * 32), "valu_fma_f32": (3, 2 * 64),
                    "mix_i8_fma": (4, 2 * 32 * 32 * 32)}


def svdq_bench_unit_peak(kind: str, blocks: int, iters: int, clocks, sink, stream=None) -> None:
    """Launch the unit microbenchmark (include/svdq_bench.h): clocks uint64-compatible int64
    device tensor [blocks, 2], sink int32 device tensor [256]."""
    import torch
    code = SVDQ_BENCH_KINDS[kind][0]
    st = load_library().svdq_bench_unit_peak(code, int(blocks), int(iters),
                                             _dev_ptr(clocks, "clocks", (torch.int64,), (blocks, 2)),
                                             _dev_ptr(sink, "sink", (torch.int32,), (256,)), _stream(stream))
    if st != 0:
        raise RuntimeError(f"svdq_bench_unit_peak failed with {st}")


def svdq_quantize_act_mxfp4(x, inv_smooth, l1t, qact=None, ascale=None, lora_act=None, stream=None):
    """Kernel (a) of the MXFP4 variant. Returns (qact uint8 [K/64, M, 32] E2M1 codes, ascale uint8
    [K/64, M, 2] E8M0 bytes, lora_act bf16 [M, r] or None)."""
    import torch
    M, K = x.shape
    r = 0 if l1t is None else l1t.shape[0]
    dev = x.device
    if qact is None:
        qact = torch.empty((K // GROUP, M, 32), dtype=torch.uint8, device=dev)
    if ascale is None:
        ascale = torch.empty((K // GROUP, M, 2), dtype=torch.uint8, device=dev)
    if r and lora_act is None:
        lora_act = torch.empty((M, r), dtype=torch.bfloat16, device=dev)
    st = load_library().svdq_quantize_act_mxfp4(
        _dev_ptr(x, "x", _bf16()), M, K, _dev_ptr(inv_smooth, "inv_smooth", (torch.float32,), (K,)),
        _dev_ptr(l1t, "l1t", _bf16(), (r, K) if r else None), r,
        _dev_ptr(qact, "qact", (torch.uint8,), (K // GROUP, M, 32)),
        _dev_ptr(ascale, "ascale", (torch.uint8,), (K // GROUP, M, 2)),
        _dev_ptr(lora_act, "lora_act", _bf16(), (M, r)) if r else None, _stream(stream))
    _check("svdq_quantize_act_mxfp4", st)
    return qact, ascale, (lora_act if r else None)


def svdq_linear_mxfp4(qact, ascale, qweight, wscale, lora_act, l2t, bias, y=None, stream=None):
    """Kernel (b) of the MXFP4 variant. qact uint8 [K/64, M, 32], ascale uint8 [K/64, M, 2],
    qweight uint8 (K*N/2 bytes), wscale uint8 [K/64, N, 2]. Returns y bf16 [M, N]."""
    import torch
    G, M, _ = ascale.shape
    K = G * GROUP
    N = wscale.shape[1]
    if qact.numel() != M * K // 2:
        raise ValueError("qact size does not match K*M/2")
    if qweight.numel() != N * K // 2:
        raise ValueError("qweight size does not match [N, K/2]")
    r = 0 if l2t is None else l2t.shape[1]
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=qact.device)
    u8 = (torch.uint8,)
    st = load_library().svdq_linear_mxfp4(
        _dev_ptr(qact, "qact", u8), _dev_ptr(ascale, "ascale", u8, (G, M, 2)), _dev_ptr(qweight, "qweight", u8),
        _dev_ptr(wscale, "wscale", u8, (G, N, 2)), _dev_ptr(lora_act, "lora_act", _bf16(), (M, r)) if r else None,
        _dev_ptr(l2t, "l2t", _bf16(), (N, r)) if r else None, r, _dev_ptr(bias, "bias", _bf16(), (N,)),
        _dev_ptr(y, "y", _bf16(), (M, N)), M, N, K, _stream(stream))
    _check("svdq_linear_mxfp4", st)
    return y


def svdq_linear_w4a4_gelu_quant(qact, ascale, qweight, wscale, lora_act, l2t, bias, inv_next, l1t_next, qact_next=None,
                                ascale_next=None, lora_act_next=None, workspace=None, stream=None):
    """The MLP up projection with its GELU and the next layer's activation step fused into the
    epilogue (H is not stored). Returns (qact_next uint8 [N/64, M, 32], ascale_next float32 [N/64, M],
    lora_act_next bf16 [M, r_next] or None)."""
    import torch
    G, M = ascale.shape
    K = G * GROUP
    N = wscale.shape[1]
    if qact.numel() != M * K // 2:
        raise ValueError("qact size does not match K*M/2")
    if qweight.numel() != N * K // 2:
        raise ValueError("qweight size does not match [N, K/2]")
    r = 0 if l2t is None else l2t.shape[1]
    rn = 0 if l1t_next is None else l1t_next.shape[0]
    dev = qact.device
    lib = load_library()
    if qact_next is None:
        qact_next = torch.empty((N // GROUP, M, 32), dtype=torch.uint8, device=dev)
    if ascale_next is None:
        ascale_next = torch.empty((N // GROUP, M), dtype=torch.float32, device=dev)
    if rn and lora_act_next is None:
        lora_act_next = torch.empty((M, rn), dtype=torch.bfloat16, device=dev)
    need = lib.svdq_gelu_quant_workspace_bytes(M, N, rn)
    if rn and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    f32 = (torch.float32,)
    st = lib.svdq_linear_w4a4_gelu_quant(
        _dev_ptr(qact, "qact", (torch.uint8,)), _dev_ptr(ascale, "ascale", f32, (G, M)),
        _dev_ptr(qweight, "qweight", (torch.uint8,)), _dev_ptr(wscale, "wscale", f32, (G, N)),
        _dev_ptr(lora_act, "lora_act", _bf16(), (M, r)) if r else None,
        _dev_ptr(l2t, "l2t", _bf16(), (N, r)) if r else None, r, _dev_ptr(bias, "bias", _bf16(), (N,)), M, N, K,
        _dev_ptr(inv_next, "inv_next", f32, (N,)), _dev_ptr(l1t_next, "l1t_next", _bf16(), (rn, N)) if rn else None,
        rn, _dev_ptr(qact_next, "qact_next", (torch.uint8,), (N // GROUP, M, 32)),
        _dev_ptr(ascale_next, "ascale_next", f32, (N // GROUP, M)),
        _dev_ptr(lora_act_next, "lora_act_next", _bf16(), (M, rn)) if rn else None,
        _dev_ptr(workspace, "workspace", (torch.uint8,)) if rn else None,
        int(workspace.numel()) if rn else 0, _stream(stream))
    _check("svdq_linear_w4a4_gelu_quant", st)
    return qact_next, ascale_next, (lora_act_next if rn else None)


def svdq_linear_w4a4_gelu_quant_noalloc(qact, ascale, qweight, wscale, lora_act, l2t, bias, inv_next, l1t_next,
                                        qact_next, ascale_next, lora_act_next=None, stream=None):
    """svdq_linear_w4a4_gelu_quant with the library's per-device scratch instead of a workspace; the
    caller passes every output (nothing is allocated here or in the library)."""
    import torch
    G, M = ascale.shape
    K = G * GROUP
    N = wscale.shape[1]
    if qact.numel() != M * K // 2:
        raise ValueError("qact size does not match K*M/2")
    if qweight.numel() != N * K // 2:
        raise ValueError("qweight size does not match [N, K/2]")
    r = 0 if l2t is None else l2t.shape[1]
    rn = 0 if l1t_next is None else l1t_next.shape[0]
    f32 = (torch.float32,)
    st = load_library().svdq_linear_w4a4_gelu_quant_noalloc(
        _dev_ptr(qact, "qact", (torch.uint8,)), _dev_ptr(ascale, "ascale", f32, (G, M)),
        _dev_ptr(qweight, "qweight", (torch.uint8,)), _dev_ptr(wscale, "wscale", f32, (G, N)),
        _dev_ptr(lora_act, "lora_act", _bf16(), (M, r)) if r else None,
        _dev_ptr(l2t, "l2t", _bf16(), (N, r)) if r else None, r, _dev_ptr(bias, "bias", _bf16(), (N,)), M, N, K,
        _dev_ptr(inv_next, "inv_next", f32, (N,)), _dev_ptr(l1t_next, "l1t_next", _bf16(), (rn, N)) if rn else None,
        rn, _dev_ptr(qact_next, "qact_next", (torch.uint8,), (N // GROUP, M, 32)),
        _dev_ptr(ascale_next, "ascale_next", f32, (N // GROUP, M)),
        _dev_ptr(lora_act_next, "lora_act_next", _bf16(), (M, rn)) if rn else None, _stream(stream))
    _check("svdq_linear_w4a4_gelu_quant_noalloc", st)
    return qact_next, ascale_next, (lora_act_next if rn else None)
