"""Build libqkvfront.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqkvfront.so")
SOURCES = [os.path.join(CSRC, "qkvf_api.cpp"), os.path.join(CSRC, "qkvf_kernels.hip"),
           os.path.join(CSRC, "qkvf_attn2.hip"), os.path.join(CSRC, "qkvf_layer_front.hip"),
           os.path.join(CSRC, "qkvf_stream.hip"),
           os.path.join(CSRC, "qkvf_route.hip")]
HEADERS = [os.path.join(ROOT, "include", "qkvf.h"), os.path.join(CSRC, "qkvf_internal.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Per-source device options: attn2 keeps its MFMA operands and results in
# VGPRs (no copies between accumulation and vector registers).
EXTRA_FLAGS = {
    "qkvf_attn2.hip": ["-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form"],
}
# hipcc's host pass does not know the packed-fp32 feature and says so
_NOISE = "'-packed-fp32-ops' is not a recognized feature"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if _NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source to an object (with its own extra options), link
    the shared library next to this file, then swap it in."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory(prefix="qkvf_build_") as d:
        objs = []
        for src in SOURCES:
            name = os.path.basename(src)
            obj = os.path.join(d, name + ".o")
            _run([hipcc, *HIPCC_FLAGS, *EXTRA_FLAGS.get(name, []), *inc, "-c", src, "-o", obj],
                 verbose)
            objs.append(obj)
        _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
