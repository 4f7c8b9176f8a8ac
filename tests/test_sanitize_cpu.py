"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no GPU code built):

  * the C ABI's validation and size arithmetic (gated_delta_rule_gdr_amd/csrc/gdr2_api.hip
    compiled as plain C++ against launch stand-ins that touch no memory), every entry point with
    valid arguments, rejected arguments and sizes whose products overflow 64 bits;
  * the fp64 oracle (oracle/gdr2_oracle.c), every entry point on ragged shapes, with its
    by-construction identities (decode steps == forward, KDA == GDR-2 with tied gates).

Each driver exits non-zero on a failed expectation; the sanitizers abort on their first report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="2")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=ENV)
    assert r.returncode == 0, f"{' '.join(cmd)} failed ({r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_abi_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_san")
    _run(["g++", "-std=c++17", "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "gated_delta_rule_gdr_amd", "csrc"),
          *SAN, os.path.join(ROOT, "gated_delta_rule_gdr_amd", "csrc", "gdr2_api.hip"),
          os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", exe], ROOT)
    out = _run([exe], ROOT)
    assert out.strip().startswith("ok"), out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c99", "-fopenmp", *SAN, os.path.join(ROOT, "oracle", "gdr2_oracle.c"),
          os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm", "-o", exe], ROOT)
    out = _run([exe], ROOT)
    assert out.strip().startswith("ok"), out
