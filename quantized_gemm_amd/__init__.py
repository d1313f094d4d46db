"""MI355X (gfx950) SVDQuant W4A4 + low-rank linear and W4A16 projection.

The compute lives in ``lib/libsvdq.so`` (hand-written HIP kernels + a C++ host packer, C ABI in
``include/svdq.h``); this package is its thin Python binding plus the offline decomposition that
turns a dense weight into the layer's inputs (``prep``).
"""
from .binding import (  # noqa: F401
    GROUP, SVDQ_FMT_W4A16_BF16SCALE, SVDQ_FMT_W4A4_F32SCALE, SVDQ_OK, SvdqError, awq_linear_w4a16, library_path,
    load_library, status_string, svdq_abi_version, svdq_check_device, svdq_debug_group_sums, svdq_linear_w4a4,
    svdq_linear_w4a4_qkv, svdq_pack_lowrank, svdq_pack_weights, svdq_quantize_act, SVDQ_BENCH_KINDS,
    svdq_bench_unit_peak, SVDQ_FMT_MXFP4_E8M0SCALE, svdq_quantize_act_mxfp4, svdq_linear_mxfp4,
    svdq_linear_w4a4_gelu_quant, svdq_linear_w4a4_gelu_quant_noalloc,
)
