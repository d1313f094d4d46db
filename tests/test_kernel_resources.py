"""Register budgets of the GPU kernels, as the compiler reported them in the build (no GPU needed).

Every kernel is written to fit its registers without private (scratch) memory: a spill turns
register traffic into memory traffic on the hot path, and in the W4A4 GEMM it also adds HBM writes.
The build records the compiler's kernel-resource-usage figures next to the library; no kernel may
use scratch, and the GEMM must keep the occupancy its design assumes (two 256-thread blocks per CU,
i.e. two waves per SIMD).
"""
import os

import pytest

from quantized_gemm_amd import build as qbuild


@pytest.fixture(scope="module")
def resources():
    if not os.path.exists(qbuild.RESOURCES):
        pytest.fail(f"{qbuild.RESOURCES} missing: build the library first (quantized_gemm_amd/build.py)")
    rows = []
    for line in open(qbuild.RESOURCES):
        if line.startswith("#") or not line.strip():
            continue
        src, name, vgpr, agpr, scratch, occ = line.split()
        rows.append((src, name, int(vgpr), int(agpr), int(scratch), int(occ)))
    return rows


def test_every_kernel_instantiation_reported(resources):
    count = lambda src: sum(1 for r in resources if r[0] == src)
    # quantizer, for INT4 and for MXFP4: one 16-token-block instantiation per rank r = 16 q,
    # q = 0..16, a 32-token-block one per rank r > 0 and a 24-token-block one per rank r = 32, 48, 64
    assert count("quant_act.hip") == (17 + 16 + 3) * 2
    # GEMM: the debug dump and the down-projection partial sum in the dispatch unit, and the
    # 17 ranks x 4 epilogues in the generated units
    assert count("w4a4_gemm.hip") == 2
    gemm = [r for r in resources if r[0].startswith("w4a4_inst_") and "w4a4_gemm_kernel" in r[1]]
    assert len(gemm) == 17 * 4
    assert len({r[1] for r in gemm}) == 17 * 4
    assert count("mxfp4_gemm.hip") == 17
    assert count("w4a16_gemv.hip") == 1


def test_no_kernel_uses_scratch(resources):
    spills = [r for r in resources if r[4] != 0]
    assert not spills, f"kernels using scratch memory: {spills}"


def test_gemm_keeps_two_waves_per_simd(resources):
    for r in resources:
        if r[0].startswith("w4a4_inst_") or r[0] == "mxfp4_gemm.hip":
            assert r[5] >= 2, r
