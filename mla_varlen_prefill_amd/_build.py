"""Builds libmla_prefill.so (all HIP sources of csrc/) in-tree for gfx950 with hipcc.

Usage: ``python -m mla_varlen_prefill_amd._build`` (or ``__graft_entry__.build()``). It always
recompiles. Packed-FP32 instruction selection is switched off for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libmla_prefill.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["abi.hip", "plan.hip", "dense_fwd.hip", "sparse_fwd.hip", "combine.hip", "latent_ctx.hip"]
# Calibration kernels used by the benchmark harness only (measured MFMA and HBM rates).
CALIB_SOURCE = "calib.hip"
CALIB_PATH = os.path.join(PKG_DIR, "libmla_calib.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmla_prefill.so)")


def compile_flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wno-unused-command-line-argument",
    ]


def build(verbose: bool = False, extra_flags=None) -> str:
    cc = hipcc()
    obj_dir = os.path.join(PKG_DIR, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    objs = []
    procs = []
    for src in SOURCES + [CALIB_SOURCE]:
        obj = os.path.join(obj_dir, src.replace(".hip", ".o"))
        cmd = [cc, *compile_flags(), *(extra_flags or []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if src != CALIB_SOURCE:
            objs.append(obj)
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        text = "\n".join(l for l in out.decode(errors="replace").splitlines()
                         if "packed-fp32-ops" not in l)
        if pr.returncode != 0:
            failed.append(src)
            sys.stderr.write(f"--- {src}\n{text}\n")
        elif verbose and text.strip():
            print(text)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB_PATH + ".tmp"
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB_PATH)
    calib_tmp = CALIB_PATH + ".tmp"
    subprocess.run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC",
                    os.path.join(obj_dir, CALIB_SOURCE.replace(".hip", ".o")), "-o", calib_tmp], check=True)
    os.replace(calib_tmp, CALIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
