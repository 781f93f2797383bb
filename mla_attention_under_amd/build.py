"""Ahead-of-time build of libmla.so for gfx950 (hipcc, in-tree).

Each source compiles to an object in parallel under ``_build/``; the objects
link into ``libmla.so`` next to this file, replaced atomically so a running
process never sees a half-written library.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmla.so")
SOURCES = ["mla_host.cpp", "mla_pack.hip", "mla_gemm.hip", "mla_attn.hip", "mla_decode.hip", "mla_rope.hip", "mla_attn_bwd.hip",
           "mla_peak.hip"]
ARCH = "gfx950"

# -packed-fp32-ops keeps the compiler from emitting packed fp32 VALU forms.
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source additions. The attention backward's four-wave kernel keeps about
# 330 values live at one wave per SIMD; with the default MFMA register form the
# compiler parks its dk / dv accumulators in AGPRs and copies them through
# VGPRs every step (about 350 v_accvgpr moves per step), while the VGPR form
# leaves them in place.
FILE_FLAGS = {"mla_attn_bwd.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form=1"]}


def _hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libmla.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
