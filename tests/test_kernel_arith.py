"""Host checks of arithmetic identities the GPU kernels rely on (no GPU needed).

The activation quantizer computes the group scale absmax / 7 without a division: q1 = absmax *
RN(1/7) followed by one FMA residual and one FMA correction. The kernels are only bit-exact with
the oracle's IEEE quotient if that identity holds for every possible absmax (a non-negative finite
float), so it is checked exhaustively here in C (float32 arithmetic, round to nearest, subnormals
preserved).
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "div7_exhaustive.c")


@pytest.fixture(scope="module")
def div7_binary(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    out = str(tmp_path_factory.mktemp("native") / "div7_exhaustive")
    # -ffp-contract=off: no fused operations other than the explicit fmaf calls
    subprocess.run([cc, "-O2", "-ffp-contract=off", "-fno-fast-math", SRC, "-o", out, "-lm"], check=True)
    return out


def test_div7_identity_every_float(div7_binary):
    r = subprocess.run([div7_binary, "1"], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert "checked 2139095040 values, 0 mismatches" in r.stdout
