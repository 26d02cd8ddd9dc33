"""Host-side sanitizer builds, CPU only.

* The oracle built with gcc's AddressSanitizer and UndefinedBehaviorSanitizer (undefined
  behaviour fatal) runs its pins (``test_oracle.py``) in a child process.
* The C-ABI library with its host code built with clang's AddressSanitizer and
  UndefinedBehaviorSanitizer (the gfx950 device code is compiled as usual) runs the host ABI
  tests (``test_abi_host.py``: exports, argument validation, the selector, installed
  choices) in a child process.

The sanitized builds go to ``tests/_build`` (not tracked) and are rebuilt when their sources
change.  Leak detection is off: the Python interpreter itself keeps memory until exit.
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "tests", "_build")
CSRC = os.path.join(ROOT, "dense_fp16_gemm_fp32_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _digest(paths, flags) -> str:
    h = hashlib.sha256(" ".join(flags).encode())
    for p in sorted(paths):
        with open(p, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _cached_build(name, sources, flags, cmd):
    """Runs cmd (a list ending in the output path placeholder OUT) unless a build of the
    same sources and flags exists; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    out = os.path.join(BUILD, "%s_%s.so" % (name, _digest(sources, flags)))
    if not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        r = subprocess.run([c if c != "OUT" else tmp for c in cmd], stdout=subprocess.PIPE,
                           stderr=subprocess.STDOUT, text=True)
        assert r.returncode == 0, r.stdout[-4000:]
        os.replace(tmp, out)
    return out


def _runtime(compiler: list) -> str:
    path = subprocess.run(compiler + ["-print-file-name=" + (
        "libasan.so" if compiler[0] == "gcc" else "libclang_rt.asan-x86_64.so")],
        stdout=subprocess.PIPE, text=True, check=True).stdout.strip()
    assert os.path.isabs(path) and os.path.exists(path), path
    return path


def _run_pytest(args, env_extra):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *args], cwd=ROOT, env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=900)
    print(r.stdout[-3000:])
    return r


def test_oracle_pins_under_asan_and_ubsan():
    import oracle
    flags = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"]
    lib = _cached_build("liboracle_gemm_asan_ubsan", [oracle.SOURCE], flags,
                        oracle.compile_command(oracle.SOURCE, "OUT", flags))
    r = _run_pytest([os.path.join("tests", "test_oracle.py")],
                    {"ORACLE_LIB": lib, "LD_PRELOAD": _runtime(["gcc"])})
    assert r.returncode == 0, "oracle pins failed under ASan/UBSan"
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stdout
    assert "runtime error" not in r.stdout


PLUGIN = '''
import os
def pytest_configure(config):
    import dense_fp16_gemm_fp32_amd as g
    g.LIBRARY = os.environ["MI355GEMM_SANITIZED_LIBRARY"]
'''


def test_c_abi_host_code_under_asan_and_ubsan():
    sources = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [
        os.path.join(ROOT, "include", "mi355gemm.h")]
    # every sanitizer flag applies to the host compilation only (-Xarch_host before each)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = [os.path.join(ROCM, "bin", "hipcc"), "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-fPIC", "-shared", "-mcode-object-version=5",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I" + os.path.join(ROOT, "include"), "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           *san, os.path.join(CSRC, "mi355gemm.hip"), "-o", "OUT"]
    lib = _cached_build("libmi355gemm_host_asan_ubsan", sources, san, cmd)
    os.makedirs(BUILD, exist_ok=True)
    with open(os.path.join(BUILD, "sanitized_library.py"), "w") as fh:
        fh.write(PLUGIN)
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    r = _run_pytest(["-p", "sanitized_library", os.path.join("tests", "test_abi_host.py")],
                    {"MI355GEMM_SANITIZED_LIBRARY": lib, "LD_PRELOAD": _runtime([clang]),
                     "PYTHONPATH": BUILD + os.pathsep + os.environ.get("PYTHONPATH", "")})
    assert r.returncode == 0, "host ABI tests failed under ASan/UBSan"
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stdout
    assert "runtime error" not in r.stdout
