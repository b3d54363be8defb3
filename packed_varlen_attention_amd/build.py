"""Build libh3.so for gfx950 with hipcc, in-tree.

    python -m packed_varlen_attention_amd.build [--jobs N] [--verbose] [--sanitize]

Each .hip source under csrc/ is compiled to an object under _build/ (in
parallel), then linked into packed_varlen_attention_amd/libh3.so.  Device code
is built with packed-fp32 instructions disabled.

--sanitize builds a host-checking variant instead, _build/sanitize/libh3.so:
the host code (argument validation, workspace carving, launch set-up) with
AddressSanitizer and UndefinedBehaviorSanitizer, the device code unchanged.
It is for CPU runs of the host-side tests (load it with H3_LIBRARY=<path> and
the ASan runtime in LD_PRELOAD); it is never what the GPU runs.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libh3.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results land in VGPRs unless register pressure moves them; without
    # this, one-wave-per-SIMD kernels put every accumulator in AGPRs and copy
    # the softmax inputs back out on every tile.
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # Nothing on the kernels' path propagates NaN through min/max (pad rows are
    # never read; masked keys are -inf), so max needs no quieting instructions.
    # Device code only: the host pass keeps its NaN checks of the arguments.
    "-Xarch_device", "-fno-honor-nans",
    "-I" + os.path.join(ROOT, "include"),
]


# Host-only sanitizer flags: each -fsanitize applies to the host pass alone.
SANITIZE_FLAGS = ["-O1", "-g",
                  "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SANITIZE_LINK = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-shared-libasan"]
SANITIZE_DIR = os.path.join(BUILD_DIR, "sanitize")


def asan_runtime() -> str:
    """Path of the clang ASan shared runtime that the sanitizer build links."""
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    hits = sorted(glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("clang ASan runtime not found under %s" % root)
    return hits[-1]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libh3.so)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, verbose: bool, sanitize: bool = False) -> str:
    out_dir = SANITIZE_DIR if sanitize else BUILD_DIR
    obj = os.path.join(out_dir, os.path.splitext(os.path.basename(src))[0] + ".o")
    flags = [f for f in COMMON_FLAGS if f != "-O3"] + SANITIZE_FLAGS if sanitize else COMMON_FLAGS
    cmd = [hipcc()] + flags + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature: drop that warning only
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(jobs: int = 0, verbose: bool = False, sanitize: bool = False) -> str:
    out_dir = SANITIZE_DIR if sanitize else BUILD_DIR
    lib_path = os.path.join(SANITIZE_DIR, "libh3.so") if sanitize else LIB_PATH
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize), srcs))
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + \
        (SANITIZE_LINK if sanitize else []) + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, lib_path)
    return lib_path


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--sanitize", action="store_true",
                    help="host ASan + UBSan variant under _build/sanitize/ (CPU runs of the host tests only)")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose, a.sanitize))


if __name__ == "__main__":
    main()
