"""Build the gfx950 shared library libtpshard.so in-tree with hipcc.

    python -m megatron_tensor_layer_amd.build

Compiles every source under csrc/ (in parallel) and links them into
megatron_tensor_layer_amd/libtpshard.so.  Always recompiles.
"""
from __future__ import annotations

import os
import pathlib
import shutil
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
CSRC = PKG / "csrc"
BUILD = PKG.parent / "_build"
LIB = PKG / "libtpshard.so"

SOURCES = ["gemv.hip", "gemv_fp8.hip", "splitk.hip", "rowstream.hip", "gemm.hip", "reduce.hip", "norm.hip", "attn_core.hip", "attn_decode.hip", "probe.hip", "workspace.hip", "tpshard_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function",
    # never emit packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmds):
    procs = [(c, subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
             for c in cmds]
    failed = []
    for c, p in procs:
        out, _ = p.communicate()
        # the host pass does not know the packed-fp32 target feature: harmless
        out = "\n".join(l for l in out.splitlines()
                        if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
        if out.strip():
            print(out, file=sys.stderr)
        if p.returncode != 0:
            failed.append(" ".join(c))
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(failed))


def build(verbose: bool = False) -> pathlib.Path:
    if shutil.which(HIPCC) is None and not pathlib.Path(HIPCC).exists():
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    BUILD.mkdir(exist_ok=True)
    objs, cmds = [], []
    for src in SOURCES:
        obj = BUILD / (src + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([HIPCC, *FLAGS, *lang, "-c", str(CSRC / src), "-o", str(obj)])
    if verbose:
        for c in cmds:
            print(" ".join(c))
    _run(cmds)
    tmp = LIB.with_suffix(".so.tmp")
    _run([[HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
