"""Builds ``libkvc.so`` (the gfx950 HIP kernels and the C ABI of include/kvc.h).

Each ``csrc/*.hip`` file is compiled with hipcc for gfx950 in parallel, then linked
into one shared library under ``sparse_decode_amd/_build``.  Packed-fp32 VALU
instructions are disabled for every translation unit.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(OUT_DIR, "libkvc.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results straight into arch VGPRs: no v_accvgpr_read per element
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # no kernel produces or propagates NaN (masked logits are -inf, bf16 rounding and
    # selection keys are integer operations): IEEE mode off drops the NaN
    # canonicalisation of every min/max operand
    "-fno-honor-nans", "-mno-amdgpu-ieee",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    "-Wno-unused-result",
]


# The C ABI layer validates host arguments, NaN included: it keeps IEEE semantics
# (under -fno-honor-nans a comparison may assume its operand is not NaN).
KERNEL_ONLY_FLAGS = ("-fno-honor-nans", "-mno-amdgpu-ieee")
HOST_CHECKED_SOURCES = ("kvc_api.hip",)


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    flags = COMMON_FLAGS
    if os.path.basename(src) in HOST_CHECKED_SOURCES:
        flags = [f for f in COMMON_FLAGS if f not in KERNEL_ONLY_FLAGS]
    cmd = [HIPCC, *flags, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, res.stdout, res.stderr))
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if ln.strip() and noise not in ln]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compiles every HIP source and links libkvc.so; returns its path."""
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    extra = list(extra or [])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), srcs))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (res.stdout, res.stderr))
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
