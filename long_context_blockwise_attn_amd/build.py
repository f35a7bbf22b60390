"""Builds libbwattn.so (HIP, gfx950) in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 only and linked into one
shared library next to this file.  The library exports the C-ABI declared in
include/bwattn.h.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbwattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["prep.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_decode.hip", "attn_f32.hip", "packed_ce.hip", "bwattn.cpp"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    # no packed fp32 instructions (v_pk_*_f32) anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# MFMA accumulators in VGPRs for the bf16 kernels, whose softmax reads the
# score accumulators directly; they fit in 256 VGPRs and spill nothing to
# AGPRs.  The fp32 kernels keep the compiler's default AGPR accumulators:
# their dQ and dK/dV kernels need more than 256 registers per lane, and with
# the VGPR form they reload MFMA operands from AGPR spill slots 2 wait states
# before the MFMA, the pattern of the only build of these sources that gave
# results differing from call to call (tests/test_isa_guards.py checks every
# kernel's assembly for it).
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
AGPR_ACCUMULATORS = {"attn_f32.hip"}


def _flags(src: str) -> list:
    lang = [] if src.endswith(".hip") else ["-x", "hip"]
    form = [] if src in AGPR_ACCUMULATORS else VGPR_FORM
    return COMMON + form + lang


def device_asm_flags(src: str) -> list:
    """The flags of `src`'s build for its gfx950 assembly (add -S, the source
    and -o): the compiled kernels themselves, for reading."""
    return _flags(src) + ["--offload-device-only"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, src + ".o")
    cmd = [HIPCC] + _flags(src) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
