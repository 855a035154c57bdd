"""Build libhymba_hh.so for gfx950 with hipcc (in-tree).

    python -m hybrid_attention_ssm_amd.csrc.build [--jobs N] [--asan]

Compiles every translation unit of this directory to an object under _build/
and links them into hybrid_attention_ssm_amd/libhymba_hh.so.  Always rebuilds.

--asan (a check of the host code): builds _build/libhymba_hh_asan.so, whose
host code (the C ABI: validation, workspace layout, launch sequence) is
compiled with AddressSanitizer; the GPU code is compiled as usual.  A process
that loads it needs the ASan runtime preloaded (asan_runtime()).
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libhymba_hh.so")
SOURCES = ["hh_api.cpp", "gemm.hip", "attention.hip", "scan.hip", "branches.hip", "norm.hip", "decode.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-I" + os.path.join(ROOT, "include"),
    # never emit packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str, build: str) -> str:
    obj = os.path.join(build, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-x", "hip", "-c", os.path.join(HERE, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def asan_runtime() -> str:
    """Path of clang's shared ASan runtime (to LD_PRELOAD)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang++"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def build_asan(jobs: int = 8, verbose: bool = False) -> str:
    """_build/libhymba_hh_asan.so: host code under AddressSanitizer."""
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    asan_dir = os.path.join(build_dir, "asan")
    os.makedirs(asan_dir, exist_ok=True)
    # the sanitizer applies to the host side only (-Xarch_host before it)
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]

    def comp(src):
        obj = os.path.join(asan_dir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *CFLAGS, *host_san, "-x", "hip", "-c", os.path.join(HERE, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (asan) failed for {src}:\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(comp, SOURCES))
    lib = os.path.join(build_dir, "libhymba_hh_asan.so")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan", "-fsanitize=address",
           *objs, "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (asan) failed:\n{r.stderr}")
    if verbose:
        print(f"built {lib}")
    return lib


def build(jobs: int = 8, verbose: bool = False) -> str:
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--asan", action="store_true", help="build _build/libhymba_hh_asan.so instead")
    args = ap.parse_args()
    (build_asan if args.asan else build)(args.jobs, verbose=True)
    sys.exit(0)
