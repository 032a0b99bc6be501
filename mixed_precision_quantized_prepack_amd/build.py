"""Build libw4.so (the HIP library behind the C ABI in include/w4.h) for gfx950.

    python -m mixed_precision_quantized_prepack_amd.build [-j JOBS] [-v]
    python -m mixed_precision_quantized_prepack_amd.build --sanitize

Each source is compiled separately (in parallel) into _build/ and linked into
mixed_precision_quantized_prepack_amd/libw4.so.  Always recompiles.

--sanitize builds _build/sanitize/libw4_sanitize.so: the host code of the C ABI
(w4_api.cpp: argument validation, planning, schedule table, options) compiled
with AddressSanitizer and UndefinedBehaviorSanitizer (host side only; the GPU
code is unchanged), linked with the kernels' objects of the last plain build.
It is loaded through W4_LIBRARY with the sanitizer runtime preloaded, for the
CPU tests of the ABI (tests/test_sanitized_abi.py); it is not for GPU runs.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libw4.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
    # packed fp32 arithmetic is kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the grouped kernels' fold reads every accumulator
    # with VALU instructions, which cannot take AGPR operands
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]

SOURCES = ["w4_api.cpp", "w4_prepack_quant.hip", "w4_gemm.hip", "w4_gemm_stream.hip", "w4_gemm_pingpong.hip"]


def _compile(src: str, verbose: bool, build_dir: str, extra) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *extra]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{msgs}")
    if msgs.strip() and verbose:
        print(msgs, flush=True)
    return obj


def build(jobs: int = 4, verbose: bool = False, extra_flags=(), out_path: str = LIB_PATH) -> str:
    """Compile and link.  ``extra_flags`` (e.g. tuning -D defines) and
    ``out_path`` allow side builds for experiments; the defaults build the
    library the package loads."""
    build_dir = BUILD_DIR if out_path == LIB_PATH else out_path + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, list(extra_flags)), SOURCES))
    tmp = out_path + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libw4.so failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, out_path)
    return out_path


SANITIZE_DIR = os.path.join(BUILD_DIR, "sanitize")
SANITIZE_LIB = os.path.join(SANITIZE_DIR, "libw4_sanitize.so")
# host-side only (each sanitizer flag applies to the host compilation)
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-g"]


def sanitizer_runtime() -> str:
    """The shared AddressSanitizer runtime of the host compiler (to preload)."""
    r = subprocess.run([HIPCC, "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"the AddressSanitizer runtime was not found ({path!r})")
    return path


def build_sanitized(verbose: bool = False) -> str:
    """w4_api.cpp with host sanitizers, linked with the kernel objects in
    _build/ (built first if missing)."""
    kernel_srcs = [s for s in SOURCES if s.endswith(".hip")]
    kernel_objs = [os.path.join(BUILD_DIR, s + ".o") for s in kernel_srcs]
    if not all(os.path.exists(o) for o in kernel_objs):
        build(verbose=verbose)
    os.makedirs(SANITIZE_DIR, exist_ok=True)
    api_obj = _compile("w4_api.cpp", verbose, SANITIZE_DIR, SANITIZE_FLAGS)
    tmp = SANITIZE_LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libasan", *SANITIZE_FLAGS[:4],
           "-o", tmp, api_obj, *kernel_objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {SANITIZE_LIB} failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, SANITIZE_LIB)
    return SANITIZE_LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", "--jobs", type=int, default=4)
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--sanitize", action="store_true", help="build the host-sanitized ABI library instead")
    a = ap.parse_args(argv)
    print(build_sanitized(a.verbose) if a.sanitize else build(a.jobs, a.verbose))
    return 0


if __name__ == "__main__":
    sys.exit(main())
