"""Build libmoe.so (HIP for gfx950) in-tree with hipcc.

    python -m quantized_expert_mlp_amd.build

Every call compiles from source (hipcc cross-compiles without a GPU).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["moe_api.cpp", "routing.hip", "gemv.hip", "gemv_mxfp4.hip", "gemv_tiled.hip", "gemm.hip",
           "misc.hip"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe)")


FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # keep hipcc from forming packed-fp32 VALU instructions (the device pass
    # honours it; the host pass prints HOST_FEATURE_NOTE and ignores it, and
    # the driver cannot forward a -Xclang pair to the device pass alone)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
]
HOST_FEATURE_NOTE = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"


def _diagnostics(stderr: str) -> str:
    """The compiler's messages without the host pass's note about the
    device-only feature flag above (one per file; every other line kept)."""
    return "\n".join(l for l in stderr.splitlines() if l.strip() != HOST_FEATURE_NOTE)


def build(verbose: bool = False) -> str:
    cc = hipcc()
    out_dir = os.path.join(PKG, "_build")
    os.makedirs(out_dir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"]
        cmd = [cc] + FLAGS + ["-I", INCLUDE, "-I", CSRC] + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, _diagnostics(r.stderr)))
        msg = _diagnostics(r.stderr)
        if msg.strip():
            print("%s:\n%s" % (src, msg), file=sys.stderr)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
