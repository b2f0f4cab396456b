"""Compile the HIP library ``libwsgemv.so`` for gfx950 (in-tree).

Each source is compiled with hipcc to an object file, then linked into one
shared library next to this file.  Run ``python -m
weight_streaming_gemv_decode_amd.build``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
REPO = os.path.dirname(HERE)
INCLUDE = os.path.join(REPO, "include")
LIB = os.path.join(HERE, "libwsgemv.so")
BUILD_DIR = os.path.join(REPO, "_build")

SOURCES = ["api.cpp", "dense.hip", "w4.hip", "conv1d.hip", "topk.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 instructions (v_pk_*_f32) are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-I", INCLUDE, "-I", CSRC]


def _compile(src: str) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so.
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = False) -> str:
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host code checked by AddressSanitizer and UndefinedBehaviorSanitizer (the
# device code is unchanged).  Each -fsanitize flag applies to the host pass only.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime, to preload into a
    process that loads the sanitizer build."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def build_sanitized(out_dir: str) -> str:
    """libwsgemv.so in out_dir with the host code (the C ABI, argument
    validation, launch planning, plan creation) built under the sanitizers;
    kernels as in build().  CPU tests load it through WSGEMV_LIB."""
    os.makedirs(out_dir, exist_ok=True)

    def one(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *SANITIZE_HOST, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        return obj
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(one, SOURCES))
    lib = os.path.join(out_dir, "libwsgemv.so")
    subprocess.run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *SANITIZE_HOST, *objs, "-o", lib], check=True)
    return lib


def clean() -> None:
    if os.path.isdir(BUILD_DIR):
        shutil.rmtree(BUILD_DIR)


if __name__ == "__main__":
    build(verbose=True)
