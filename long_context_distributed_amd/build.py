"""Builds libmeshattn.so (C ABI + gfx950 HIP kernels) in the package directory.

    python -m long_context_distributed_amd.build          # build
    python -m long_context_distributed_amd.build --asm    # also keep gfx950 assembly in _build/

Every source is compiled with hipcc for gfx950 only.  Packed FP32 VALU
instructions are switched off for all device code.
"""
import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmeshattn.so")

SOURCES = ["api.cpp", "block_list.cpp", "plan.cpp", "tile_fwd_bf16.hip", "tile_fwd_f32.hip", "lse_merge.hip",
           "tile_bwd_bf16.hip", "bwd_delta.hip"]
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build")
    return path


def _compile(src, asm):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc(), f"--offload-arch={ARCH}", *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if asm and src.endswith(".hip"):
        cmd += ["-save-temps=obj"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "not a recognized feature for this target"
    err = "\n".join(x for x in res.stderr.splitlines() if noise not in x)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{err}")
    return obj, err


def build(asm=False, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda s: _compile(s, asm), SOURCES))
    for (_, err), src in zip(results, SOURCES):
        if verbose and err.strip():
            print(f"[{src}]\n{err}", file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
           *[o for o, _ in results]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libmeshattn.so failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", action="store_true", help="keep gfx950 assembly under _build/")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(asm=a.asm, verbose=a.verbose))


if __name__ == "__main__":
    main()
