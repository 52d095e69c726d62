"""Build libdattn.so (HIP, gfx950) in-tree.

    python -m deberta_disentangled_attention_amd.build

Packed-FP32 VALU instructions are disabled for the device code
(-packed-fp32-ops); the host pass warns that it does not know that target
feature, which is harmless.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libdattn.so")
SOURCES = ["dattn_api.hip", "dattn_fwd.hip", "dattn_bwd.hip", "fast_f32.hip", "pack.hip", "rel_bucket.hip",
           "relproj.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdattn.so)")


def compile_command(out: str = LIB_PATH, extra=()) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        f"-I{os.path.join(PKG_DIR, '..', 'include')}",
        *extra,
        "-o", out,
        *[os.path.join(CSRC, s) for s in SOURCES],
    ]


def build(verbose: bool = True, out: str = LIB_PATH, extra=()) -> str:
    """Compile the library (always recompiles) and return its path."""
    tmp = out + ".tmp"
    cmd = compile_command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass reports the device-only feature as unknown; drop that noise
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    # optional: output path, then extra compiler flags (e.g. -DNAME=VALUE)
    if len(sys.argv) > 1:
        build(out=os.path.abspath(sys.argv[1]), extra=sys.argv[2:])
    else:
        build()
