"""Build the HIP library in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "va.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libva.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
              shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libva.so)")


def compile_flags():
    # Packed fp32 ops are turned off for all device code (-packed-fp32-ops).
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
            "-I", INCLUDE, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall"]


# The same source with the phase timestamps of the FP8 paged kernel compiled in
# (va_set_stamp_buffer); a diagnostic library, loaded only by bench.py --stamps.
LIB_STAMPS = os.path.join(HERE, "libva_stamps.so")


def build(verbose: bool = False, extra=(), out: str = LIB) -> str:
    """Compile csrc/va.hip into `out` (default paged_gqa_attention_va_amd/libva.so;
    always recompiles)."""
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc()] + compile_flags() + list(extra) + [SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def build_stamps(verbose: bool = False) -> str:
    """Compile the diagnostic libva_stamps.so (-DVA_STAMPS)."""
    return build(verbose=verbose, extra=("-DVA_STAMPS",), out=LIB_STAMPS)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_stamps(verbose=True))
