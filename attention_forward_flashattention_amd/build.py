"""Build the HIP library ``libattn_fwd.so`` (forward, backward and alpha-entmax kernels) for gfx950
with hipcc (in-tree).

The library carries the sha256 of the sources it was built from (``attn_source_sha()``), so a
caller can tell a library built from other sources than the ones beside it."""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SRCS = [os.path.join(CSRC, f) for f in ("attn_fwd.hip", "attn_bwd.hip", "attn_entmax.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn_fwd.so")
OBJ_DIR = os.path.join(PKG, "_build")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def source_files():
    """Every file the library is compiled from: the kernel sources, their private header and the
    public headers, in a fixed order."""
    files = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith((".hip", ".h"))]
    files += [os.path.join(INCLUDE, f) for f in sorted(os.listdir(INCLUDE)) if f.endswith(".h")]
    return files


def source_sha(extra_flags=()) -> str:
    """sha256[:16] over the compile flags and the (relative path, bytes) of every source file."""
    h = hashlib.sha256()
    h.update(" ".join([*HIPCC_FLAGS, *extra_flags]).encode())
    for f in source_files():
        h.update(os.path.relpath(f, ROOT).encode() + b"\0")
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the attention library)")


def build(extra_flags=()) -> str:
    """Compile the library (the three sources in parallel, then one link); always recompiles.
    Returns the path of the .so."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    sha = source_sha(extra_flags)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
        cmd = [cc, *HIPCC_FLAGS, *extra_flags, f'-DATTN_SOURCE_SHA="{sha}"', "-I", INCLUDE, "-c", src,
               "-o", obj]
        subprocess.check_call(cmd)
        return obj

    with ThreadPoolExecutor(max_workers=len(SRCS)) as ex:
        objs = list(ex.map(compile_one, SRCS))
    tmp = LIB + ".tmp"
    subprocess.check_call([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
