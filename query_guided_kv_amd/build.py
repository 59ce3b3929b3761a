"""Build libkvsel.so in-tree with hipcc for gfx950.

Usage: ``python -m query_guided_kv_amd.build`` (or ``build()`` from Python).
Every HIP source is compiled on its own (in parallel) into ``_build/`` and the
objects are linked into ``query_guided_kv_amd/libkvsel.so``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvsel.so")

SOURCES = ["api.cpp", "reposition.hip", "score.hip", "score_mfma.hip", "aggregate.hip",
           "aggregate_mfma.hip", "topk.hip", "gather.hip", "decode.hip", "index_attn.hip", "noalloc.hip"]

ARCH = os.environ.get("KVSEL_ARCH", "gfx950")


def hipcc() -> str:
    env = os.environ.get("HIPCC")
    if env:
        return env
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc") or ""):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def compile_flags() -> list:
    # packed fp32 VALU ops are disabled on purpose: the compiler would form
    # v_pk_{add,mul,fma}_f32 from plain float code otherwise.  No kernel makes
    # or tests a NaN (masked logits are -inf), so device code is built with
    # -fno-honor-nans: fmaxf then skips the quieting of its operands.  Host
    # code keeps IEEE comparisons (argument checks reject NaN).
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Xarch_device", "-fno-honor-nans",
            "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + compile_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libkvsel.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def asan_runtime() -> str:
    """The compiler's AddressSanitizer runtime (to preload into a process that
    loads the sanitizer build)."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the AddressSanitizer runtime of hipcc was not found")
    return path


def build_asan(out_dir: str) -> str:
    """The same library with its HOST code built under AddressSanitizer
    (device code as in build(); sanitizers are not used on the GPU), into
    out_dir; returns the library path.  Load it in a process that preloads
    asan_runtime()."""
    os.makedirs(out_dir, exist_ok=True)
    flags = [f for f in compile_flags() if f != "-O3"] + \
        "-O1 -g -Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()

    def one(src: str) -> str:
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        r = subprocess.run([hipcc()] + flags + ["-c", os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(one, SOURCES))
    lib = os.path.join(out_dir, "libkvsel_asan.so")
    r = subprocess.run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", lib] + objs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
