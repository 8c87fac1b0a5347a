"""Host code under the address and undefined-behaviour sanitizers (CPU only).

Two host-side parts are built with gcc / g++ and -fsanitize=address,undefined
(no recovery, so the first report fails the run) and driven through edge
cases by the drivers in tests/sanitize/:

- the CPU oracle (oracle/ck4_oracle.c): every function on small inputs in
  exactly sized heap buffers, with zero rows, saturating and subnormal E4M3
  scales, all group sizes and the +-49 K accumulator bound at K = 131072;
- the C ABI's validation layer (int4_w4a4_quantized_amd/csrc/ck4_api.cpp)
  with the HIP runtime queries and the kernel launchers replaced by stand-ins,
  in three device modes (no device, a gfx950, another GPU): each entry point
  with valid arguments and with null, misaligned, short-stride, unsupported
  and int64-limit arguments. A refusal must return its documented status and
  launch nothing; a valid call launches exactly its kernels, and only on a
  gfx950. No device code is built or run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not found")


def test_oracle_under_sanitizers(tmp_path):
    _need("gcc")
    exe = tmp_path / "oracle_driver"
    subprocess.run(["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", *SAN,
                    os.path.join(ROOT, "oracle", "ck4_oracle.c"), os.path.join(ROOT, "tests", "sanitize",
                                                                               "oracle_driver.c"),
                    "-o", str(exe), "-lm"], check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle driver ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr


@pytest.mark.parametrize("mode", ["none", "gfx950", "other"])
def test_abi_validation_under_sanitizers(tmp_path_factory, mode):
    _need("g++")
    d = tmp_path_factory.getbasetemp() / "abi_san"
    exe = d / "abi_driver"
    if not exe.exists():
        d.mkdir(exist_ok=True)
        subprocess.run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                        "-I", os.path.join(ROOT, "include"),
                        "-I", os.path.join(ROOT, "int4_w4a4_quantized_amd", "csrc"), *SAN,
                        os.path.join(ROOT, "int4_w4a4_quantized_amd", "csrc", "ck4_api.cpp"),
                        os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", str(exe)],
                       check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe), mode], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
