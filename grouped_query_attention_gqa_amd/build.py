"""Build libgqa.so for gfx950 with hipcc (in-tree, next to this file).

    python -m grouped_query_attention_gqa_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libgqa.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["api.hip", "decode.hip", "decode_wide.hip", "device_info.hip", "prefill.hip", "prefill_bwd.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgqa.so)")


def command(out: str = LIB_PATH):
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed-FP32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-Wl,--no-undefined",
        "-I", INCLUDE, "-I", CSRC,
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out,
    ]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into ``libgqa.so``; always recompiles."""
    tmp = LIB_PATH + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l and "ignoring feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
