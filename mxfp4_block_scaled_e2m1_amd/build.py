"""Build libmxfp4.so (the HIP kernels and the C-ABI) for gfx950 with hipcc.

Usage: python -m mxfp4_block_scaled_e2m1_amd.build [--jobs N]
The library is written next to this file so that it travels with the source tree.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmxfp4.so")
SOURCES = ["mx_api.hip", "gemm.hip", "gemm_nv.hip", "decode.hip", "elementwise.hip", "route.hip", "pack.hip", "fp8_linear.hip",
           "probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # no packed-fp32 instructions are generated (see the notes of the kernels)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE-correct fp32 division and square root (the NVFP4 quantiser divides)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Wno-inline-asm",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libmxfp4")


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the C-ABI layer
# (argument checks, workspace carving, runner, profiler): every flag applies to
# the host compilation only (device code is built as usual). The library is
# loaded into a process that preloads the compiler's ASan runtime.
SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]
BUILD_SAN = os.path.join(HERE, "_build_san")
LIB_SAN = os.path.join(BUILD_SAN, "libmxfp4_san.so")


def asan_runtime() -> str:
    """The compiler's shared ASan runtime (to preload into a process that loads
    the sanitized library)."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    hits = sorted(glob.glob(os.path.join(root, "..", "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")) +
                  glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found")
    return os.path.realpath(hits[0])


def build(jobs: int = 4, verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every source and link the library (in place next to this file),
    or, with sanitize, the host-sanitized copy under _build_san/."""
    out_dir = BUILD_SAN if sanitize else BUILD
    lib = LIB_SAN if sanitize else LIB
    extra = SANITIZE_FLAGS if sanitize else []
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()

    def compile_one(src: str) -> str:
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        cmd = [cc, *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = lib + ".tmp"
    link_extra = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-shared-libasan"] if sanitize else []
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--sanitize", action="store_true", help="host ASan + UBSan copy under _build_san/")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose, a.sanitize))
    sys.exit(0)
