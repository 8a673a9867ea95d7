"""Builds libwkv7.so (the HIP kernels and the C ABI) in-tree, for gfx950 only."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libwkv7.so")
SOURCES = ["wkv7_api.hip", "wkv7_step.hip", "wkv7_chunk.hip", "wkv7_tail.hip", "wkv7_bwd.hip", "wkv7_bwdc.hip"]
ARCH = "gfx950"

# -packed-fp32-ops: no packed fp32 math is emitted for any kernel of this library.
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile every source into libwkv7.so.  Always recompiles.  Returns the path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = [hipcc()] + HIPCC_FLAGS + (extra_flags or []) + ["-I", os.path.join(ROOT, "include")] + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless.
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
