"""Build the CARVE HIP library (libcarve.so) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libcarve.so")
SOURCES = [os.path.join(PKG, "csrc", "carve_lib.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions stay off for every kernel in this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the kernels post-process every
    # product with vector ALU code, which cannot read accumulation registers
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
    "-I", os.path.join(PKG, "csrc"),
]


# Host-side sanitizers for the C ABI layer (argument checks, shape contract,
# dispatch): AddressSanitizer and UndefinedBehaviorSanitizer on the host pass
# only; the device code is built as usual. The result is a separate library,
# loaded in place of libcarve.so by pointing CARVE_LIB_PATH at it, with the
# ASan runtime preloaded into the Python process.
SANITIZE_LIB = os.path.join(PKG, "libcarve_asan.so")
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def build_library(verbose: bool = True, sanitize: bool = False) -> str:
    out = SANITIZE_LIB if sanitize else LIB
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *(SANITIZE_FLAGS if sanitize else []), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build_library(sanitize="--sanitize" in sys.argv[1:])
    sys.exit(0)
