"""The LDS-DMA inline assembly in attn.hip, decode.hip and the narrow kernel writes M0 (global_load_lds takes its
LDS base there). M0 is a reserved register, so clang may not honour it as a clobber; the
kernels are safe only while no compiled code keeps a value in M0 across those statements.
This test compiles every HIP source for gfx950 to assembly and checks that M0 appears only
inside inline-assembly blocks, so a compiler change that starts using M0 fails here."""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "sparse_top_mla_prefill_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", ["attn.hip", "decode.hip", "narrow.hip", "narrow_fp8.hip",
                                 "fp8qk.hip", "pack.hip"])
def test_m0_only_in_inline_asm(src):
    tmp = tempfile.mkdtemp(prefix="m0guard_")
    try:
        out = os.path.join(tmp, "k.s")
        cmd = [HIPCC, "--offload-arch=gfx950", "--cuda-device-only", "-S", "-O3", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), os.path.join(CSRC, src), "-o", out]
        res = subprocess.run(cmd, capture_output=True, text=True, cwd=tmp)
        assert res.returncode == 0, res.stderr[-2000:]
        in_asm = False
        bad, ours = [], 0
        for ln in open(out):
            s = ln.strip()
            if s.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if s.startswith(";;#ASMEND"):
                in_asm = False
                continue
            if in_asm:
                ours += bool(re.search(r"\bm0\b", s))
                continue
            if s.startswith(";") or s.startswith("."):
                continue
            if re.search(r"\bm0\b", s):
                bad.append(s)
        assert not bad, f"{src}: compiled code uses M0 outside inline asm: {bad[:5]}"
        if src in ("attn.hip", "decode.hip", "narrow.hip", "narrow_fp8.hip"):
            assert ours > 0, f"{src}: no LDS-DMA statement found (the scan would be vacuous)"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
