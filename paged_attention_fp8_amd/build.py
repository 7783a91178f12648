"""Build libpafp8.so (HIP, gfx950) in-tree.

    python -m paged_attention_fp8_amd.build [--asm OUT_DIR]

Compiles every csrc/*.hip into one shared library next to this file (with
--asm, also writes each source's device assembly into OUT_DIR).  Packed
FP32 instructions are disabled (-packed-fp32-ops) and no fast-math flag is
used, so fp32 division stays correctly rounded.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpafp8.so")
ARCH = os.environ.get("PAFP8_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def common_flags():
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False) -> str:
    """Compile the library (always; this is the does-it-build check)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *common_flags(), "-shared", "-o", tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def emit_asm(out_dir: str) -> None:
    """Device assembly of every source (for inspecting register use and ISA)."""
    os.makedirs(out_dir, exist_ok=True)
    for src in sources():
        name = os.path.splitext(os.path.basename(src))[0]
        subprocess.run([hipcc(), *common_flags(), "--cuda-device-only", "-S", "-o",
                        os.path.join(out_dir, name + ".s"), src], check=True)


if __name__ == "__main__":
    if "--asm" in sys.argv:
        i = sys.argv.index("--asm")
        if i + 1 >= len(sys.argv):
            sys.exit("--asm needs an output directory")
        emit_asm(os.path.abspath(sys.argv[i + 1]))
    print(build(verbose=True))
