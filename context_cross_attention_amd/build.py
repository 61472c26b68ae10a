"""Build libgdpa.so (HIP kernels + C ABI) for gfx950, in-tree.

    python -m context_cross_attention_amd.build             # the library
    python -m context_cross_attention_amd.build --sanitize  # + _build/libgdpa_asan.so

Compiles every source under csrc/ with hipcc into objects under _build/ and
links them into context_cross_attention_amd/libgdpa.so.  `--sanitize` also builds
a copy whose host code of the C ABI (gdpa_api.cpp: argument validation, workspace
planning, the stream cache) carries AddressSanitizer and UndefinedBehaviorSanitizer
checks, for CPU-only tests of the boundary (the device code is unchanged).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgdpa.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # Packed fp32 VALU forms stay off: the compiler would otherwise emit them from
    # plain float code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]
SOURCES = ["gdpa_sched.hip", "gdpa_fwd.hip", "gdpa_fwd_res.hip", "gdpa_bwd.hip", "gdpa_bwd_res.hip",
           "gdpa_bwd_dq.hip", "gdpa_gemm.hip", "gdpa_pma.hip", "gdpa_api.cpp"]
# Per-source extra flags.  The seed pooling kernels touch their MFMA results with
# VALU code every block (softmax, bf16 packing, rescale); with the VGPR form of
# MFMA the compiler keeps them in VGPRs instead of copying them out of AGPRs.
EXTRA_FLAGS = {"gdpa_pma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


SAN_LIB = os.path.join(BUILD, "libgdpa_asan.so")
CLANGXX = os.environ.get("CLANGXX", "/opt/rocm/llvm/bin/clang++")
# Host-only sanitizer flags: each one is prefixed so that no device code is built with it.
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def san_runtime() -> str:
    """The clang AddressSanitizer runtime that a process loading SAN_LIB must preload."""
    r = subprocess.run([CLANGXX, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def build_sanitized(verbose: bool = True) -> str:
    """_build/libgdpa_asan.so: gdpa_api.cpp with host sanitizers, the kernels as built."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        if src == "gdpa_api.cpp":
            obj = os.path.join(BUILD, "gdpa_api_asan.o")
            cmd = [HIPCC, "-x", "hip", *CFLAGS, *SAN_HOST, "-g", "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed for {src} (sanitized):\n{r.stderr}")
        elif not os.path.exists(obj):
            _compile(src)
        objs.append(obj)
    # The host link pulls in clang's shared sanitizer runtimes; the objects already hold
    # their device code.
    cmd = [CLANGXX, "-shared", "-fPIC", "-shared-libsan", "-fsanitize=address,undefined", "-o", SAN_LIB, *objs,
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


if __name__ == "__main__":
    build()
    if "--sanitize" in sys.argv[1:]:
        build_sanitized()
