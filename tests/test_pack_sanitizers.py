"""The host packer (pack.cpp) built with AddressSanitizer and UndefinedBehaviorSanitizer on the CPU
and driven through every entry point: valid shapes of each format into exact-size buffers, edge
values, and invalid arguments (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def sanitized_driver(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no C++ compiler")
    out = str(tmp_path_factory.mktemp("native") / "pack_sanitize")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fno-fast-math",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "quantized_gemm_amd", "csrc", "pack.cpp"), os.path.join(HERE, "native", "pack_sanitize.cpp"),
           "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


def test_packer_under_asan_and_ubsan(sanitized_driver):
    # verify_asan_link_order=0: the driver may run under a preloaded library of the environment
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sanitized_driver], capture_output=True, text=True, timeout=300, env=env)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "pack_sanitize: 0 failures" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
