"""Build libmoe.so (the HIP library, gfx950 only) in-tree with hipcc.

Each .hip translation unit is compiled separately (in parallel) and the
objects are linked into ``sparse_mixture_experts_top2_amd/libmoe.so``.
Packed fp32 instructions are disabled for device code (``-packed-fp32-ops``).
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["abi.hip", "route.hip", "dispatch.hip", "combine.hip", "experts_f32.hip",
           "experts_bf16.hip", "gemm_gateup.hip", "gemm_down.hip", "gemm_bt.hip", "gemm_dw.hip",
           "experts_w8.hip", "backward.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def compile_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
            f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + compile_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def build_host_sanitized(out_dir: str) -> str:
    """The host side of every unit with AddressSanitizer and
    UndefinedBehaviorSanitizer (device code is not built: the library then
    serves only calls that return from their argument checks, which is what
    the CPU tests make).  The sanitizer flags go to the host compilation
    only.  Returns the path of the shared library."""
    os.makedirs(out_dir, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    flags = [f"--offload-arch={ARCH}", "--offload-host-only", "-O1", "-g",
             "-fno-omit-frame-pointer", "-std=c++17", "-fPIC", "-fvisibility=hidden",
             f"-I{INCLUDE}", f"-I{CSRC}"] + san

    def one(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        res = subprocess.run([hipcc()] + flags + ["-c", os.path.join(CSRC, src), "-o", obj],
                             capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc (host, sanitized) failed on {src}:\n{res.stderr}")
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(one, SOURCES))
    # Host-only objects name the device code bundles that a full build
    # embeds; define each as an empty offload bundle (no code objects).
    nm = subprocess.run(["nm", "-u"] + objs, capture_output=True, text=True, check=True).stdout
    names = sorted(set(re.findall(r"\b(__hip_fatbin_[0-9a-f]+)\b", nm)))
    stub = os.path.join(out_dir, "empty_bundles.c")
    with open(stub, "w") as fh:
        for n in names:
            fh.write(f'__attribute__((aligned(4096), used)) const char {n}[32] = '
                     '"__CLANG_OFFLOAD_BUNDLE__";\n')
    stub_obj = stub[:-2] + ".o"
    subprocess.run(["gcc", "-c", "-fPIC", stub, "-o", stub_obj], check=True)
    objs.append(stub_obj)
    lib = os.path.join(out_dir, "libmoe_host_sanitized.so")
    subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libasan"]
                   + san + objs + ["-o", lib], check=True)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
