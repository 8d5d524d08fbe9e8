"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The oracle (oracle/oracle.c) is built a second time with both sanitizers
  and run on small edge cases (an empty sequence, a window, an unmasked
  ragged chunk, sinks NULL / -inf / large, bf16 and fp32) in a process with
  the sanitizer runtime preloaded; its outputs must equal those of the
  normal build bit for bit.
* The library's host code (csrc/api.cpp: argument checks, launch shapes,
  workspace sizing) is built with both sanitizers on its host pass and
  linked with the other objects into tests/sanitize/abi_driver.cpp, which
  calls every entry point with arguments the host checks reject (or with
  nothing to enqueue) and checks the status codes.

A sanitizer report aborts the process, which fails the test.
"""
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
ORACLE_SRC = os.path.join(ROOT, "oracle", "oracle.c")
CSRC = os.path.join(ROOT, "gqa_paged_attention_amd", "csrc")
BUILD = os.path.join(ROOT, "gqa_paged_attention_amd", "_build")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(map(str, cmd))}\n{res.stdout}\n{res.stderr}"
    return res


def _oracle_lib(path, sanitize):
    flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"] if sanitize else ["-O2"]
    _run(["gcc", *flags, "-fopenmp", "-fPIC", "-shared", ORACLE_SRC, "-o", str(path), "-lm"])


def test_oracle_under_asan_and_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc is not available")
    libasan = _run(["gcc", "-print-file-name=libasan.so"]).stdout.strip()
    plain, san = tmp_path / "liboracle.so", tmp_path / "liboracle_san.so"
    _oracle_lib(plain, False)
    _oracle_lib(san, True)
    script = os.path.join(HERE, "oracle_cases.py")
    _run([sys.executable, script, str(plain), str(tmp_path / "plain.npz")])
    env = dict(os.environ, LD_PRELOAD=libasan, **SAN_ENV)
    res = _run([sys.executable, script, str(san), str(tmp_path / "san.npz")], env=env)
    assert "cases ok" in res.stdout
    a, b = np.load(tmp_path / "plain.npz"), np.load(tmp_path / "san.npz")
    assert sorted(a.files) == sorted(b.files) and a.files
    for k in a.files:
        assert np.array_equal(a[k], b[k]), k


def test_abi_host_checks_under_asan_and_ubsan(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)):
        pytest.skip("ROCm compilers are not available")
    objs = [os.path.join(BUILD, s + ".o") for s in ("append.hip", "decode.hip", "prefill.hip",
                                                     "rows_f32.hip")]
    if not all(os.path.exists(o) for o in objs):
        pytest.fail("the library's objects are not built (python -m gqa_paged_attention_amd.build)")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    api = tmp_path / "api_san.o"
    # sanitizers on the host pass only (the device code is built as usual)
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
          *inc, "-x", "hip", "-c", os.path.join(CSRC, "api.cpp"), "-o", str(api)])
    drv = tmp_path / "driver.o"
    _run([CLANGXX, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", *inc, "-c",
          os.path.join(HERE, "abi_driver.cpp"), "-o", str(drv)])
    exe = tmp_path / "abi_driver"
    _run([CLANGXX, "-fsanitize=address,undefined", str(drv), str(api), *objs,
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)])
    res = _run([str(exe)], env=dict(os.environ, **SAN_ENV))
    assert "ok: 0 failed" in res.stdout, res.stdout
