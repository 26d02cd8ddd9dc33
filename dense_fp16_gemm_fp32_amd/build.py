"""Build the gfx950 HIP library ``libmi355gemm.so`` in-tree with hipcc, and two
measurement aids that are not part of it: the ``bandwidth_probe`` executable (per-CU LDS,
LDS-DMA and L2 throughput) and ``libmi355gemm_phases.so``, the same library built with
MI355_PHASE_CLOCK=1 so the direct kernel records per-workgroup phase timestamps (read by
``python -m dense_fp16_gemm_fp32_amd.phases``).

``python -m dense_fp16_gemm_fp32_amd.build`` or ``build()`` always recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", "mi355gemm.hip")]
HEADERS = [os.path.join(PKG, "csrc", "gemm_common.hpp"), os.path.join(PKG, "csrc", "gemm_direct.hpp"), os.path.join(PKG, "csrc", "gemm_staged.hpp"), os.path.join(PKG, "csrc", "gemm_narrow.hpp"), os.path.join(PKG, "csrc", "gemm_pingpong.hpp"), os.path.join(PKG, "csrc", "tuned_table.inc"), os.path.join(PKG, "csrc", "vector_add.hpp"), os.path.join(PKG, "csrc", "softmax.hpp"), os.path.join(PKG, "csrc", "attention.hpp"), os.path.join(ROOT, "include", "mi355gemm.h")]
LIBRARY = os.path.join(PKG, "libmi355gemm.so")
PHASE_LIBRARY = os.path.join(PKG, "libmi355gemm_phases.so")
PROBE_SOURCE = os.path.join(PKG, "csrc", "bandwidth_probe.hip")
PROBE = os.path.join(PKG, "bandwidth_probe")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"


def compile_command(output: str = LIBRARY, extra: list[str] | None = None) -> list[str]:
    return [
        os.path.join(ROCM, "bin", "hipcc"),
        "--offload-arch=" + ARCH,
        "-O3", "-std=c++17", "-fPIC", "-shared",
        "-mcode-object-version=5",
        # packed fp32 VALU forms stay off: the compiler may not form v_pk_*_f32 here
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I" + os.path.join(ROOT, "include"),
        "-Wl,-rpath," + os.path.join(ROCM, "lib"),
        *(extra or []),
        *SOURCES,
        "-o", output,
    ]


def probe_command(output: str = PROBE) -> list[str]:
    return [
        os.path.join(ROCM, "bin", "hipcc"),
        "--offload-arch=" + ARCH,
        "-O3", "-std=c++17",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wl,-rpath," + os.path.join(ROCM, "lib"),
        PROBE_SOURCE,
        "-o", output,
    ]


def _run_hipcc(cmd: list[str], tmp: str, output: str, verbose: bool) -> str:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature flag and says so; that
    # warning is expected, anything else is shown.
    lines = [l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if r.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError("hipcc failed (%d)" % r.returncode)
    if lines and verbose:
        print("\n".join(lines))
    os.replace(tmp, output)
    return output


def build_probe(output: str = PROBE, verbose: bool = False) -> str:
    tmp = output + ".tmp%d" % os.getpid()
    return _run_hipcc(probe_command(tmp), tmp, output, verbose)


def build_phase_clock(output: str = PHASE_LIBRARY, verbose: bool = False) -> str:
    tmp = output + ".tmp%d" % os.getpid()
    return _run_hipcc(compile_command(tmp, ["-DMI355_PHASE_CLOCK=1"]), tmp, output, verbose)


def build(output: str = LIBRARY, verbose: bool = False) -> str:
    tmp = output + ".tmp%d" % os.getpid()
    cmd = compile_command(tmp)
    return _run_hipcc(cmd, tmp, output, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_probe(verbose=True))
    print(build_phase_clock(verbose=True))
