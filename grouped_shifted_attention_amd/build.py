"""Build libs2attn.so (the C-ABI library) in-tree for gfx950.

Usage: ``python -m grouped_shifted_attention_amd.build [-v]``.  Compiles each
source with hipcc into ``_build/`` at the repository root (objects are kept
out of git) and links the shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libs2attn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# Race-check build: the same sources with S2A_DEBUG_BARRIERS, which turns every
# LDS hand-over into a full drain-and-barrier; its results must equal the
# normal build's bit for bit (tests/test_gpu_race_check.py).
DEBUG_LIB_PATH = os.path.join(PKG, "libs2attn_debugbarriers.so")

SOURCES = ["api.cpp", "fwd.hip", "bwd.hip", "bwd_delta.hip", "rope.hip", "lora_qkv.hip", "lora_bwd.hip"]
HEADERS = ["device_common.hpp", "kernels.hpp", "staging.hpp", "lora_kernels.hpp"]

ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # Keep the compiler from forming packed-FP32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libs2attn.so")
    return path


def _compile(src: str, verbose: bool, extra=(), build_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(build_dir, src + ".o")
    cmd = [hipcc()] + CFLAGS + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns about the device-only feature flag; drop that line.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{err}")
    if verbose and err.strip():
        print(err, flush=True)
    return obj


def build(verbose: bool = False, defines=(), out_path: str = LIB_PATH, build_dir: str = BUILD_DIR) -> str:
    """Compile every source and link libs2attn.so; returns the library path.

    ``defines`` are extra -D options (kernel configuration macros);
    ``out_path`` / ``build_dir`` let configuration variants build side by side.
    """
    os.makedirs(build_dir, exist_ok=True)
    extra = [f"-D{d}" for d in defines]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, extra, build_dir), SOURCES))
    tmp = out_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {LIB_NAME} failed:\n{r.stderr}")
    os.replace(tmp, out_path)
    return out_path


def build_all(verbose: bool = False) -> list:
    """The product library and the race-check build next to it."""
    return [build(verbose),
            build(verbose, defines=("S2A_DEBUG_BARRIERS",), out_path=DEBUG_LIB_PATH,
                  build_dir=os.path.join(ROOT, "_build", "debugbarriers"))]


if __name__ == "__main__":
    print(build_all(verbose="-v" in sys.argv[1:]))
