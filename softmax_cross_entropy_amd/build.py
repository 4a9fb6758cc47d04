"""Build the HIP library libce_mi355x.so in-tree for gfx950 with hipcc.

    python -m softmax_cross_entropy_amd.build [--jobs N] [--verbose]

The translation units are compiled in parallel to objects under
softmax_cross_entropy_amd/_build/ and linked into
softmax_cross_entropy_amd/libce_mi355x.so (loaded by the ctypes binding).
"""

from __future__ import annotations

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
BUILD = os.path.join(PKG, "_build")
LIB_NAME = "libce_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["ce_api.hip", "ce_linear.hip", "ce_inst_f32.hip", "ce_inst_bf16.hip",
           "ce_inst_f32_wide.hip", "ce_inst_bf16_wide.hip", "ce_inst_f32_gbf16.hip",
           "ce_inst_nograd.hip", "ce_stream.hip", "ce_shard.hip"]
# rocBLAS runs the products of the linear layer fused with the cross-entropy.
LINK_FLAGS = ["-lrocblas", "-Wl,-rpath,/opt/rocm/lib"]

# -ffp-contract=off: every fused multiply-add in the kernels is written out
# explicitly, so a value computed in two places (e.g. the target logit and
# the same element in the vector loop) rounds identically.
# The packed-fp32 target feature is switched off: no v_pk_{add,mul,fma}_f32.
COMMON_FLAGS = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
    "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(jobs: int = 0, verbose: bool = False) -> str:
    """Compile every translation unit and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([cc, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    n = jobs or min(len(cmds), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=n) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB_PATH + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, *LINK_FLAGS, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


# Build with AddressSanitizer and UndefinedBehaviorSanitizer on the host code
# for the host-side checks of the C ABI (argument validation, planning,
# workspace layout): each sanitizer flag applies to the host pass only, the
# device code is the ordinary build's. Only CPU checks load this library.
SAN_DIR = os.path.join(BUILD, "host_san")
SAN_LIB = os.path.join(SAN_DIR, "libce_host_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def build_host_sanitized(jobs: int = 0, verbose: bool = False) -> str:
    """The library with its host code under ASan and UBSan; returns its path. A program that loads it must be linked with the same
    sanitizers (it provides their runtime)."""
    os.makedirs(SAN_DIR, exist_ok=True)
    cc = hipcc()
    flags = [*COMMON_FLAGS, *SAN_FLAGS]
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(SAN_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
    n = jobs or min(len(cmds), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=n) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = SAN_LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, *LINK_FLAGS, "-o", tmp],
         verbose)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--host-sanitized", action="store_true",
                    help="build only the host-side ASan/UBSan library for the ABI checks")
    a = ap.parse_args(argv)
    path = build_host_sanitized(a.jobs, a.verbose) if a.host_sanitized else build(a.jobs,
                                                                                  a.verbose)
    print(path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
