"""Ahead-of-time build of the HIP library for gfx950 (hipcc, no JIT).

``python -m moe_matmul_amd.build`` compiles ``csrc/nvfp4_grouped_gemm.hip``
into ``moe_matmul_amd/libnvfp4_grouped_gemm.so`` next to this file, and the
mainloop measurement kernels ``csrc/mainloop_probe.hip`` into
``moe_matmul_amd/libnvfp4_mainloop_probe.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", "nvfp4_grouped_gemm.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libnvfp4_grouped_gemm.so")
# measurement kernels behind the mainloop choice (not part of the GEMM)
PROBE_SOURCES = [os.path.join(HERE, "csrc", "mainloop_probe.hip")]
PROBE_LIB = os.path.join(HERE, "libnvfp4_mainloop_probe.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 instructions: hipcc otherwise forms v_pk_*_f32 from float code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the library)")


def build(verbose: bool = False) -> str:
    """Compile the library and the probe library (always, even if built copies
    exist); return the library's path."""
    _compile(SOURCES, LIB, verbose)
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


def _compile(sources, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *sources, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    if verbose:
        noise = "is not a recognized feature for this target"
        out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
        if out.strip():
            print(out)
    os.replace(tmp, lib)


if __name__ == "__main__":
    print(build(verbose=True))
