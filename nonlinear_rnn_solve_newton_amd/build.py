"""Build the HIP C-ABI library libpararnn.so for gfx950 (in-tree).

Two compiler passes: the device pass compiles the kernels for gfx950 into an
offload bundle, with packed fp32 instructions (v_pk_*_f32) switched off; the
host pass compiles the launch code and embeds that bundle. The target-feature
flag goes to the device pass only, where it exists.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "libpararnn.so"
# measurement kernels for the device ceilings bench.py reports (not the solver)
CEIL_LIB = PKG / "libceilings.so"
ARCH = "gfx950"

COMMON_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-Wall"]
# no packed fp32 (v_pk_*_f32) instructions in the device code
DEVICE_FLAGS = ["--cuda-device-only", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
HOST_FLAGS = ["--cuda-host-only", "-fPIC", "-shared"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return str(Path(rocm) / "bin" / "hipcc")


def build_one(src: Path, out: Path, verbose: bool = False, extra_flags=(), host_flags=()) -> Path:
    """Compile one .hip source into a shared library at `out`; host_flags go to
    the host pass only (e.g. a sanitizer build of the host code)."""
    tmp = out.with_name(out.name + ".tmp")
    with tempfile.TemporaryDirectory() as td:
        fatbin = Path(td) / (src.stem + ".hipfb")
        dev = [hipcc(), *COMMON_FLAGS, *DEVICE_FLAGS, *extra_flags, str(src), "-o", str(fatbin)]
        host = [hipcc(), *COMMON_FLAGS, *HOST_FLAGS, *extra_flags, *host_flags, "-Xclang", "-fcuda-include-gpubinary",
                "-Xclang", str(fatbin), str(src), "-o", str(tmp)]
        for cmd in (dev, host):
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, extra_flags=()) -> Path:
    build_one(CSRC / "ceilings.hip", CEIL_LIB, verbose, extra_flags)
    return build_one(CSRC / "pararnn.hip", LIB, verbose, extra_flags)


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
