"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

Three programs under tests/sanitize/ are built with the sanitizers and run:

* oracle_driver.c with the C oracle: quantize-append in each layout, attention with each
  Jensen form, window scores, budget and gather lists;
* host_driver.cpp against the library, with the C-ABI layer (argument checks, planners,
  workspace sizing, window budget) built with host-side sanitizers and linked with the
  library's kernel objects. Every call it makes is answered or rejected before a launch;
* decode_checker.cpp: the decode kernel's own walk and indexing over exact-size buffers,
  and its value tile's layout (each row and channel position written once per step).

A report from either sanitizer makes the program exit non-zero (halt_on_error), which
fails the test with the report in the message.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n-> %d\n%s%s" % (" ".join(cmd), r.returncode, r.stdout, r.stderr[-6000:])
    return r


def test_oracle_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_san")
    _run([gcc, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-ffp-contract=off",
          os.path.join(ROOT, "oracle", "kvq_oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "0 failures" in r.stdout


def test_library_host_code_under_sanitizers(tmp_path):
    from bit_kv_cache_pack_amd import build as B
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    kernel_srcs = [s for s in B.SOURCES if s != "api.hip"]
    objs = [os.path.join(B.OBJ_DIR, os.path.splitext(s)[0] + ".o") for s in kernel_srcs]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    api_obj = str(tmp_path / "api_san.o")
    _run([hipcc, "--offload-arch=" + B.ARCH, "-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer",
          "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + san +
         ["-I", B.INCLUDE, "-I", B.CSRC, "-c", os.path.join(B.CSRC, "api.hip"), "-o", api_obj])
    exe = str(tmp_path / "host_san")
    _run([hipcc, "--offload-arch=" + B.ARCH, "-g"] + san + ["-I", B.INCLUDE, "-x", "c++",
         os.path.join(SAN, "host_driver.cpp"), "-x", "none", api_obj] + objs + ["-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "0 failures" in r.stdout


def test_decode_kernel_accesses_in_bounds(tmp_path):
    """The decode kernel's walk and index functions (csrc/decode_walk.cuh, which the kernel
    itself calls) run on the host for every workgroup, wave, step and lane of real launch
    plans, over exact-size host buffers under the sanitizers: every access inside its
    buffer and inside its step's rows, every token walked once, and the configurations the
    kernel is not built for refused."""
    from bit_kv_cache_pack_amd import build as B
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    objs = [os.path.join(B.OBJ_DIR, os.path.splitext(s)[0] + ".o") for s in B.SOURCES]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    exe = str(tmp_path / "decode_checker")
    _run([hipcc, "--offload-arch=" + B.ARCH, "-g", "-O1", "-std=c++17"] + san +
         ["-I", B.INCLUDE, "-I", B.CSRC, "-x", "hip", os.path.join(SAN, "decode_checker.cpp"), "-x", "none"] +
         objs + ["-o", exe])
    r = _run([exe], env=ENV, timeout=600)
    assert " 0 failures" in r.stdout
