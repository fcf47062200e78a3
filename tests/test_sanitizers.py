"""The oracle and the C ABI's host-side argument checks built with
AddressSanitizer and UndefinedBehaviorSanitizer and run on the CPU.

  * oracle/dash_oracle.c with tests/sanitize/oracle_driver.c (gcc): every
    oracle entry point on small seeded inputs, valid and invalid, with leak
    detection;
  * csrc/api.cpp (host code instrumented, device code as usual) linked with
    the other objects of the library build and tests/sanitize/abi_driver.cpp
    (clang++): every entry point with arguments it must reject, and the
    sizing helpers.  Nothing reaches a GPU.
A sanitizer report or a wrong status fails the test.  (A planted one-past-
the-end write in a copy of the oracle's summary loop is reported as a
heap-buffer-overflow by the same build.)
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "sparse_hierarchical_attention_block_amd", "csrc")
OBJS = os.path.join(ROOT, "_build", "dash")
ROCM = "/opt/rocm"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall", "-Wno-unknown-pragmas",
          os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "dash_oracle.c"),
          "-lm", "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "oracle driver: ok" in r.stdout


def test_abi_host_checks_under_sanitizers(tmp_path):
    others = ["summarize", "route", "route_tile", "route_long", "attend", "decode", "backward",
              "peaks"]
    objs = [os.path.join(OBJS, o + ".o") for o in others]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("the library's objects are not built (python "
                    "sparse_hierarchical_attention_block_amd/build.py)")
    api = str(tmp_path / "api_san.o")
    # host code instrumented, device code compiled as usual
    _run([os.path.join(ROCM, "bin", "hipcc"), "-O1", "-g", "-std=c++17", "-fPIC",
          "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-x", "hip", "-c",
          os.path.join(CSRC, "api.cpp"), "-o", api])
    clang = os.path.join(ROCM, "lib", "llvm", "bin", "clang++")
    drv = str(tmp_path / "abi_driver.o")
    exe = str(tmp_path / "abi_san")
    _run([clang, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
          "-c", os.path.join(SAN, "abi_driver.cpp"), "-o", drv])
    _run([clang, "-fsanitize=address,undefined", drv, api, *objs,
          "-L" + os.path.join(ROCM, "lib"), "-Wl,-rpath," + os.path.join(ROCM, "lib"),
          "-lamdhip64", "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "abi driver: ok" in r.stdout
