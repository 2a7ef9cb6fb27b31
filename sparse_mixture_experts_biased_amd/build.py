"""Build the HIP library libmoe_mi355x.so in-tree with hipcc for gfx950.

    python -m sparse_mixture_experts_biased_amd.build [-j N] [--sanitize]

Object files go to _build/ at the repository root; the shared library is
written next to this file, where the Python binding loads it.

--sanitize builds libmoe_mi355x_san.so instead (objects in _build_san/): the
host code under AddressSanitizer and UndefinedBehaviorSanitizer, the device
code unchanged.  The binding loads it when MOE_LIB names it; the process needs
the ASan runtime preloaded (see sanitizer_env()).
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
BUILD = os.path.join(ROOT, "_build")
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["api.cpp", "route.hip", "permute.hip", "swiglu_f32.hip", "swiglu_bf16.hip",
           "combine.hip", "bias.hip", "backward.hip", "calib.hip"]

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build the library")
    return exe


# host-only sanitizers: each flag applies to the host compilation alone
SAN_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
             "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer "
             "-shared-libsan").split()
SAN_BUILD = os.path.join(ROOT, "_build_san")
SAN_LIB_PATH = os.path.join(PKG, "libmoe_mi355x_san.so")


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON_FLAGS + \
        list(extra)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def is_stale(lib_path: str) -> bool:
    """True when lib_path is missing or older than a source it is built from."""
    if not os.path.exists(lib_path):
        return True
    t = os.path.getmtime(lib_path)
    srcs = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + \
        [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))]
    return any(os.path.getmtime(f) > t for f in srcs)


def build(jobs: int = 8, verbose: bool = False, sanitize: bool = False) -> str:
    build_dir = SAN_BUILD if sanitize else BUILD
    lib_path = SAN_LIB_PATH if sanitize else LIB_PATH
    extra = SAN_FLAGS if sanitize else []
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, 16))) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), SOURCES))
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs + extra
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


def sanitizer_env() -> dict:
    """Environment for a Python process that loads the sanitized library: the
    ASan runtime preloaded (Python itself is not instrumented), leak checks
    off (the interpreter keeps its allocations), MOE_LIB set."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    rt = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(rt) or not os.path.exists(rt):
        raise RuntimeError("the ASan runtime of the HIP toolchain was not found")
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", MOE_LIB=SAN_LIB_PATH)
    return env


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", "--jobs", type=int, default=8)
    ap.add_argument("--sanitize", action="store_true",
                    help="host code under ASan + UBSan, into libmoe_mi355x_san.so")
    args = ap.parse_args(argv)
    build(args.jobs, verbose=True, sanitize=args.sanitize)


if __name__ == "__main__":
    sys.exit(main())
