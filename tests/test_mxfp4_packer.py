"""The host packer's MXFP4 format against the oracle (CPU, through the C ABI): codes and E8M0
scales bit-exact, decoded with the layout include/svdq.h documents."""
import numpy as np
import pytest

import oracle
import quantized_gemm_amd as q
from problems import decode_mx_codes, decode_mx_scales


@pytest.fixture(scope="module")
def lib():
    return q.load_library()


@pytest.mark.parametrize("K,N", [(64, 16), (192, 48), (256, 512), (3072, 128)])
def test_pack_mxfp4_bit_exact_vs_oracle(lib, K, N):
    rng = np.random.default_rng(K + N)
    w = (rng.standard_normal((K, N)) * rng.uniform(1e-3, 10, (1, N))).astype(np.float32)
    w[:32, 0] = 0.0                                      # an all-zero block
    w[32:64, 1] = np.float32(1e-41)                       # subnormal block
    w[:32, 2] = np.array([6, 4, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -5] + [1] * 22, np.float32)   # ties
    qw, sw = q.svdq_pack_weights(q.SVDQ_FMT_MXFP4_E8M0SCALE, w)
    assert sw.shape == (K // 64, N, 2) and sw.dtype == np.uint8
    oc, os_ = oracle.quantize_weights_mxfp4(w)
    assert np.array_equal(decode_mx_codes(qw, N, K), oc)
    assert np.array_equal(decode_mx_scales(sw, N, K), os_)


def test_mxfp4_sizes(lib):
    assert lib.svdq_packed_weight_bytes(q.SVDQ_FMT_MXFP4_E8M0SCALE, 256, 48) == 256 * 48 // 2
    assert lib.svdq_scale_bytes(q.SVDQ_FMT_MXFP4_E8M0SCALE, 256, 48) == 256 // 32 * 48
    assert lib.svdq_scale_bytes(3, 256, 48) == 0
