"""Compile the HIP kernels and the C ABI into one shared library for gfx950.

    python -m scaled_dot_product_18_amd.build [--verbose]

Produces ``scaled_dot_product_18_amd/libsdpa18.so`` in-tree, and beside it
``libmfmapeak.so``, the matrix-core throughput microbenchmark that
``bench.py --mfma-peak`` runs (not part of the attention library). Every
translation unit is compiled with packed fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass
warns that it does not know the feature, which is harmless.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libsdpa18.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

PEAK_SOURCE = "mfma_peak.hip"
PEAK_LIB_PATH = os.path.join(PKG_DIR, "libmfmapeak.so")
SOURCES = ["attn_api.cpp", "attn_fwd_bf16.hip", "attn_fwd_bf16_pp.hip", "attn_fwd_ppk.hip", "attn_fwd_fp8_pp.hip",
           "attn_fwd_mfma.hip", "attn_fwd_f32.hip", "attn_fwd_splitkv.hip", "attn_bwd.hip", "attn_bwd_f32.hip"]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    if os.path.exists(path):
        return path
    found = shutil.which("hipcc")
    if not found:
        raise RuntimeError("hipcc not found (set ROCM_PATH)")
    return found


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I" + INCLUDE, "-I" + CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-command-line-argument"]


def build(verbose: bool = False, out_dir: str | None = None) -> str:
    """Compile every source and link libsdpa18.so; returns the library path."""
    hipcc = _hipcc()
    obj_dir = os.path.join(out_dir or os.path.join(ROOT, "_build"), "obj")
    os.makedirs(obj_dir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(obj_dir, src + ".o")
        lang = ["-x", "hip"]
        cmd = [hipcc, *common_flags(), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        noise = "is not a recognized feature for this target"
        err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
        if res.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
        return obj

    def link(objs, path):
        tmp = path + ".tmp"
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp, *objs]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stderr}")
        os.replace(tmp, path)
        if verbose:
            print(f"built {path}")

    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES + [PEAK_SOURCE]))
    link(objs[:-1], LIB_PATH)
    link(objs[-1:], PEAK_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv)
