"""CPU sanitizer runs (no GPU needed).

1. The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
   (gcc), running every oracle pin.
2. The library's host side -- argument validation of every entry point
   (hq_api.hip) and the width split of non-power-of-two rotations
   (hq_paley.hip) -- built host-only with the same sanitizers (hipcc, no
   device code; the kernel launchers are stand-ins from
   tests/hostcheck/launch_stubs.hip), running the ABI contract tests.

Each run is a child process with the sanitizer runtime preloaded (Python
itself is not instrumented); any report fails the run.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hadamard_rotation_amd", "csrc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _runtime(compiler: list[str], name: str) -> str:
    p = subprocess.run(compiler + [f"-print-file-name={name}"], capture_output=True,
                       text=True).stdout.strip()
    if not p or not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip(f"sanitizer runtime {name} not found")
    return p


def _run_child(code: str, preload: str, tmp) -> subprocess.CompletedProcess:
    env = dict(os.environ, LD_PRELOAD=preload, PYTHONPATH=ROOT, **SAN_ENV)
    script = os.path.join(str(tmp), "child.py")
    with open(script, "w") as f:
        f.write(code)
    return subprocess.run([sys.executable, script], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=900)


def _check(r: subprocess.CompletedProcess):
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]


def test_oracle_pins_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not found")
    lib = os.path.join(str(tmp_path), "liboracle_san.so")
    subprocess.check_call([gcc, "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-pthread",
                           "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined",
                           os.path.join(ROOT, "oracle", "hq_oracle.c"), "-o", lib, "-lm"])
    code = f"""
import sys
from oracle import oracle as O
O._LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider",
                      "tests/test_oracle_pins.py", "tests/test_oracle_paley.py",
                      "tests/test_oracle_attention.py"]))
"""
    r = _run_child(code, _runtime([gcc], "libasan.so"), tmp_path)
    _check(r)
    assert " passed" in r.stdout


def test_abi_validation_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    clang = "/opt/rocm/lib/llvm/bin/clang"
    if not os.path.exists(clang):
        pytest.skip("ROCm clang not found")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    flags = ["--offload-host-only", "-O1", "-g", "-std=c++17", "-fPIC",
             "-fno-omit-frame-pointer", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
    srcs = [os.path.join(CSRC, "hq_api.hip"), os.path.join(CSRC, "hq_paley.hip"),
            os.path.join(ROOT, "tests", "hostcheck", "launch_stubs.hip")]
    objs = []
    for src in srcs:
        obj = os.path.join(str(tmp_path), os.path.basename(src) + ".o")
        subprocess.check_call([hipcc, *flags, *san, "-c", src, "-o", obj])
        objs.append(obj)
    lib = os.path.join(str(tmp_path), "libhq_hostcheck.so")
    subprocess.check_call([hipcc, "--offload-host-only", "-shared", "-fPIC", *san, *objs,
                           "-o", lib])
    code = f"""
import sys
from hadamard_rotation_amd import binding as B
B.load({lib!r})
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", "tests/test_abi.py",
                      "-k", "not product_package"]))
"""
    r = _run_child(code, _runtime([clang], "libclang_rt.asan-x86_64.so"), tmp_path)
    _check(r)
    assert " passed" in r.stdout
