"""Build libpkv.so (HIP kernels for gfx950 + host runtime) in-tree with hipcc.

    python -m prefill_slot_mapping_amd.build [--debug]

Compiles every source under csrc/ to an object file in _build/ and links
prefill_slot_mapping_amd/libpkv.so. Always recompiles (the build check runs on every call).
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(os.path.dirname(PKG_DIR), "_build")
LIB_PATH = os.path.join(PKG_DIR, "libpkv.so")
ARCH = "gfx950"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

DEVICE_SOURCES = ["write_kv.hip", "decode.hip", "decode_mfma.hip", "merge.hip",
                  "prefill.hip", "noalloc.hip"]
HOST_SOURCES = ["allocator.cpp", "api.cpp", "planner.cpp", "scheduler.cpp"]

# Packed-FP32 instructions are disabled for all device code: the compiler may not form
# v_pk_{add,mul,fma}_f32 from ordinary float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source extras. decode.hip, decode_mfma.hip: no floating-point operation there sees a NaN
# (bad rows are written as a NaN bit pattern through an integer select), which lets maxima fuse
# with their DPP lane permutes. decode.hip: no implicit contraction of a multiply and an add into
# an FMA (every FMA is written out).
SOURCE_FLAGS = {"decode.hip": ["-fno-honor-nans", "-ffp-contract=off"],
                "decode_mfma.hip": ["-fno-honor-nans"]}


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libpkv.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(debug: bool = False, verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    opt = ["-O1", "-g"] if debug else ["-O3"]
    common = ["-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", *opt,
              f"-I{os.path.join(os.path.dirname(PKG_DIR), 'include')}"]
    cmds = []
    objs = []
    for src in DEVICE_SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".", "_") + ".o")
        cmds.append([cc, "-x", "hip", f"--offload-arch={ARCH}", *common, *DEVICE_FLAGS,
                     *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".", "_") + ".o")
        cmds.append([cc, "-x", "c++", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", *common, "-c",
                     os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB_PATH + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--debug", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    path = build(debug=args.debug, verbose=args.verbose)
    print(path)


if __name__ == "__main__":
    sys.exit(main())
