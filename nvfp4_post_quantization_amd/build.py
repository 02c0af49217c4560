"""Build the HIP library libnvfp4mi.so for gfx950, in-tree.

Every source under csrc/ is compiled by hipcc to an object in _build/ (in
parallel) and linked into nvfp4_post_quantization_amd/libnvfp4mi.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libnvfp4mi.so")
SOURCES = ["api.hip", "quant.hip", "hessian.hip", "sweep.hip", "cast.hip", "fp8.hip", "rotate.hip", "linear.hip",
           "probe.hip", "sweep_stats.hip"]
ARCH = os.environ.get("NVFP4MI_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    # keep packed fp32 VALU forms out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]
# hipBLASLt serves the plain bf16 GEMM of the QuantLinear forward
LINK = ["-L/opt/rocm/lib", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile all sources and link libnvfp4mi.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp, *LINK]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host-sanitizer build of the argument-validation layer: api.hip compiled with
# AddressSanitizer and UndefinedBehaviorSanitizer on its host code only
# (-Xarch_host before each -fsanitize=; device code is built as usual), linked
# with the other objects of the regular build.  Loaded with the clang ASan
# runtime preloaded; tests/test_abi_sanitized.py runs the C-ABI validation
# tests against it.  No GPU is needed: validation fails before any HIP call.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_LIB = os.path.join(BUILD, "san", "libnvfp4mi_san.so")


def asan_runtime() -> str:
    """Path of the clang ASan runtime that the sanitized library needs preloaded."""
    clang = os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "llvm", "bin", "clang")
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang ASan runtime not found")
    return path


def build_sanitized(verbose: bool = False) -> str:
    """Build SAN_LIB (the regular objects must exist: build() first)."""
    others = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "api.hip"]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"regular objects missing ({missing[0]}): run build() first")
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    obj = os.path.join(os.path.dirname(SAN_LIB), "api_san.o")
    cmds = [
        [_hipcc(), *[f for f in FLAGS if f != "-O3"], "-O1", "-g", *SAN_FLAGS, "-c", os.path.join(CSRC, "api.hip"),
         "-o", obj],
        [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", obj, *others, "-o", SAN_LIB,
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", *LINK],
    ]
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitizer build failed:\n{r.stderr}")
    return SAN_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
