"""Build libmi_attn.so in-tree with hipcc for gfx950.

Run as ``python -m tiled_attention_forward_02_amd.build`` or call build().
The shared library lands next to this file, where the binding loads it.
"""

from __future__ import annotations

import ctypes
import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
# Each source with its own extra device flags. The backward's dK/dV kernel
# keeps two fp32 accumulators and the K, V fragments live; left to its
# heuristics the compiler gives its MFMAs accumulators in AGPRs and copies
# them to VGPRs and back on every loop iteration, so the VGPR form is forced
# there (the forward is unaffected: it is compiled on its own). At d = 256
# those accumulators need the AGPRs (they exceed the 256 VGPRs), so the d = 256
# backward is a translation unit of its own, built without the flag.
SOURCES = (
    ("attn_fwd.hip", ()),
    ("attn_bwd.hip", ("-mllvm", "-amdgpu-mfma-vgpr-form=1")),
    ("attn_bwd256.hip", ()),
)
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG_DIR, "libmi_attn.so")
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmi_attn)")


COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # NaN-free max/min on the device side only (no canonicalising moves)
    "-Xarch_device", "-fno-honor-nans",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE,
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that note is noise
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def _check_links(path):
    """Refuse a library with unresolved symbols. A kernel whose host stub the
    compiler did not emit leaves its launch undefined without any diagnostic;
    the library then fails only when loaded."""
    try:
        ctypes.CDLL(path, mode=os.RTLD_NOW)
    except OSError as e:
        os.unlink(path)
        raise RuntimeError(f"built library does not load: {e}") from None


def build(verbose=False):
    """Compile the HIP sources into libmi_attn.so (always recompiles)."""
    with tempfile.TemporaryDirectory(prefix="mi_attn_build_") as tmpdir:
        objs = []
        for name, extra in SOURCES:
            obj = os.path.join(tmpdir, name + ".o")
            _run([hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, name), "-o", obj], verbose)
            objs.append(obj)
        tmp = LIB + ".tmp"
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    _check_links(tmp)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
