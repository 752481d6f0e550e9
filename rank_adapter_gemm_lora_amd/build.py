"""Compile the HIP library for gfx950 (MI355X) in-tree.

    python -m rank_adapter_gemm_lora_amd.build

writes ``rank_adapter_gemm_lora_amd/librank_adapter_gemm_lora_amd.so``; objects go
to ``_build/``.  Every source is compiled each time (no staleness checks), in
parallel.  All HIP code is built with packed fp32 instructions disabled.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "librank_adapter_gemm_lora_amd.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = ["lora_api.cpp", "seg_build.hip", "shrink.hip", "expand.hip", "decode.hip", "pool.hip",
           "merge.hip", "residency.cpp"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC,
         "-Wall", "-Wno-unused-function"]


# Host code checked by AddressSanitizer and UndefinedBehaviorSanitizer (the
# GPU code is built as usual): a CPU-only test build, see build_sanitized().
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-g"]


def _compile(src: str, build_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def _build(lib_path: str, build_dir: str, extra=(), verbose: bool = False) -> str:
    os.makedirs(build_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), SOURCES))
    tmp = lib_path + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *extra, *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


def build(verbose: bool = False) -> str:
    return _build(LIB_PATH, BUILD_DIR, verbose=verbose)


def build_sanitized(lib_path: str, verbose: bool = False) -> str:
    """The library with its host code under ASan and UBSan, for CPU-only checks
    of the host logic (a process loading it needs the ASan runtime preloaded:
    sanitizer_runtime())."""
    return _build(lib_path, os.path.join(BUILD_DIR, "sanitized"), SANITIZE_HOST, verbose=verbose)


def sanitizer_runtime() -> str:
    """Path of the compiler's shared ASan runtime (to preload)."""
    res = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True)
    path = res.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        import glob
        hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        if not hits:
            raise RuntimeError("no ASan runtime found")
        path = hits[0]
    return path


if __name__ == "__main__":
    build(verbose=True)
