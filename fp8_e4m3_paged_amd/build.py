"""Build libkvfp8.so (gfx950) in-tree with hipcc.

    python -m fp8_e4m3_paged_amd.build [--verbose]

Compiles every HIP source under csrc/ into one shared library next to this
file. Packed-fp32 instruction selection is switched off for the device code.
fp32 division keeps HIP's default correctly rounded lowering (no fast-math),
which the FP8 encoder relies on.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvfp8.so")
SOURCES = ["kv_cache_ops.hip", "decode_attn.hip", "ingest.hip", "gemv.hip", "kvfp8_api.hip", "page_pool.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def command(out: str = LIB, extra=()) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-I", os.path.join(os.path.dirname(HERE), "include"),
        *extra,
        "-o", out,
        *[os.path.join(CSRC, s) for s in SOURCES],
    ]


def build(verbose: bool = False, extra=()) -> str:
    """Compile the library; raises CalledProcessError on failure. Returns its path."""
    tmp = LIB + ".tmp"
    cmd = command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise subprocess.CalledProcessError(res.returncode, cmd, res.stdout, res.stderr)
    if verbose and (res.stdout or res.stderr):
        # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
        sys.stderr.write(res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv)
    print(LIB)
