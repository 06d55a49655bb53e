"""Build libhq.so (the C-ABI library of gfx950 HIP kernels) in-tree with hipcc.

Every translation unit is compiled for gfx950 only, with packed-fp32 code
generation switched off, then linked into one shared library next to this
file.  ``build()`` always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhq.so")
PROBE_LIB = os.path.join(PKG, "libhq_probe.so")
OBJDIR = os.path.join(ROOT, "_build")
SOURCES = ["hq_host.cpp", "quant_pack.hip", "decode_attn.hip", "select_vertical.hip",
           "prefill_attn.hip"]
PROBE_SOURCES = ["stream_probe.hip"]                # measurement helper, its own library

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# device code only: -fno-honor-nans (kernel inputs are finite by contract, so
# fmaxf/fminf need no canonicalising v_max per operand and chains fold into
# v_max3_f32); the host's argument checks keep their NaN tests
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Wno-unused-function", "-Xarch_device", "-fno-honor-nans",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


# per-file device flags: the decode scan keeps its MFMA accumulators in
# VGPRs (the online softmax rescales them with VALU instructions, and in
# AGPRs every block paid for copies between the two register files)
FILE_FLAGS = {"decode_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip() and verbose:
        print(out)
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    shutil.move(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile and link libhq.so (and the benchmark's libhq_probe.so);
    returns the path of libhq.so."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
