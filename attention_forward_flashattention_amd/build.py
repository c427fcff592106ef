"""Build the HIP library ``libattn_fwd.so`` (forward, backward and alpha-entmax kernels) for gfx950
with hipcc (in-tree)."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f) for f in ("attn_fwd.hip", "attn_bwd.hip", "attn_entmax.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn_fwd.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the attention library)")


def build(extra_flags=()) -> str:
    """Compile the library; always recompiles.  Returns the path of the .so."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, *SRCS, "-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
