"""Build libsparse_mla.so in-tree with hipcc for gfx950.

    python sparse_top_mla_prefill_amd/build.py [--verbose]

(run as a file: importing the package loads the library this script replaces)

All HIP code is compiled with the packed-fp32 feature disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsparse_mla.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["attn.hip", "decode.hip", "narrow.hip", "narrow_fp8.hip", "roles.hip", "pack.hip",
           "fp8qk.hip", "api.cpp"]
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile every source into libsparse_mla.so (always recompiles). Returns the path."""
    cmd = [HIPCC, *FLAGS, *(extra_flags or []), *[os.path.join(CSRC, s) for s in SOURCES],
           "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless.
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
