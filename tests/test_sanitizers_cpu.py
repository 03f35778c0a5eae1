"""Host-side AddressSanitizer / UndefinedBehaviorSanitizer builds (CPU only).

1. The oracle (oracle/fp4_oracle.c, plain C) built with gcc and both
   sanitizers and driven over every grid, scale format, block, rounding
   mode and input type (tests/helpers/oracle_sanitize_driver.c).
2. The C-ABI library's host code (api.cpp) built with both sanitizers on
   its host pass only, linked with stand-ins for the kernel launchers
   (tests/helpers/abi_sanitize_stubs.cpp, which abort if reached), and
   driven through argument checks that must reject each call before any
   launch (tests/helpers/abi_sanitize_driver.cpp).  No GPU is needed.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HELPERS = os.path.join(ROOT, "tests", "helpers")
CSRC = os.path.join(ROOT, "fp4_block_scaled_quantize_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=1", "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", "-pthread", "-ffp-contract=off", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "fp4_oracle.c"), os.path.join(HELPERS, "oracle_sanitize_driver.c"),
          "-lm", "-o", exe])
    r = _run([exe], env={**os.environ, **SAN_ENV}, timeout=300)
    assert "ok" in r.stdout


def _hipcc():
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def test_abi_host_code_under_asan_ubsan(tmp_path):
    clangxx = "/opt/rocm/llvm/bin/clang++"
    hiplib = "/opt/rocm/lib"
    if not os.path.exists(_hipcc()) or not os.path.exists(clangxx):
        pytest.skip("no ROCm toolchain")
    # sanitizers on the host pass only (-Xarch_host before each), the
    # device pass of api.cpp (its static scratch array) built as usual
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I", INCLUDE, "-I", CSRC, *host_san]
    objs = []
    for src in (os.path.join(CSRC, "api.cpp"), os.path.join(HELPERS, "abi_sanitize_stubs.cpp"),
                os.path.join(HELPERS, "abi_sanitize_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([_hipcc(), *common, "-x", "hip", "-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "abi_san")
    link_san = ["-fsanitize=address,undefined"]
    _run([clangxx, *link_san, *objs, "-L", hiplib, "-Wl,-rpath," + hiplib, "-lamdhip64", "-o", exe])
    r = _run([exe], env={**os.environ, **SAN_ENV}, timeout=300)
    assert "ok" in r.stdout
