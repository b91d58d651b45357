"""Builds libtv.so in-tree with hipcc for gfx950.

Usage: ``python -m tree_attention_verification_tv_amd.build``. The library is
written next to this file; object files go to ``_build/`` at the repository
root.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libtv.so")

ARCH = "gfx950"
SOURCES = ["tv_tree.hip", "tv_typical.hip", "tv_draft.hip", "tv_attn_f32.hip", "tv_attn_bf16.hip", "tv_layout.hip",
           "tv_api.cpp"]
# Packed fp32 arithmetic is switched off for device code (host passes only
# warn that they do not know the feature).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build libtv.so")
    return path


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = [f"--offload-arch={ARCH}", *DEVICE_FLAGS]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stdout}\n{res.stderr}")
    return obj


def _llvm_tool(name: str) -> str:
    for d in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin"), "/opt/rocm/llvm/bin"):
        path = os.path.join(d, name)
        if os.path.exists(path):
            return path
    path = shutil.which(name)
    if path is None:
        raise RuntimeError(f"{name} not found (ROCm's LLVM tools are needed to read the built code object)")
    return path


def kernel_private_segments(lib_path: str = LIB_PATH) -> dict:
    """Per-lane private (scratch) bytes of every kernel in the library's
    gfx950 code object, from the code object's AMDGPU metadata (the
    .hip_fatbin bundle, unbundled, then its notes): {kernel symbol: bytes}."""
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    notes = []
    with tempfile.TemporaryDirectory() as tmp:
        fatbin = os.path.join(tmp, "fatbin.bin")
        res = subprocess.run([_llvm_tool("llvm-objcopy"), f"--dump-section=.hip_fatbin={fatbin}", lib_path,
                              os.path.join(tmp, "lib.stripped")], capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"llvm-objcopy failed on {lib_path}:\n{res.stderr}")
        with open(fatbin, "rb") as f:
            data = f.read()
        # one bundle per translation unit, concatenated (with padding)
        starts = [m.start() for m in re.finditer(re.escape(magic), data)]
        for i, a in enumerate(starts):
            bundle, co = os.path.join(tmp, f"b{i}.bin"), os.path.join(tmp, f"co{i}.o")
            with open(bundle, "wb") as f:
                f.write(data[a:starts[i + 1] if i + 1 < len(starts) else len(data)])
            res = subprocess.run([_llvm_tool("clang-offload-bundler"), "--unbundle", "--type=o",
                                  f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}", f"--input={bundle}",
                                  f"--output={co}"], capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError(f"clang-offload-bundler failed on bundle {i} of {lib_path}:\n{res.stderr}")
            res = subprocess.run([_llvm_tool("llvm-readelf"), "--notes", co], capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError(f"llvm-readelf failed on code object {i}:\n{res.stderr}")
            notes.append(res.stdout)
    out = {}
    for text in notes:
        name = None
        for line in text.splitlines():
            m = re.match(r"\s*\.name:\s+(\S+)", line)
            if m:
                name = m.group(1)
                continue
            m = re.match(r"\s*\.private_segment_fixed_size:\s+(\d+)", line)
            if m and name is not None:
                out[name] = int(m.group(1))
                name = None
    return out


def check_no_scratch(lib_path: str = LIB_PATH) -> None:
    """Raises if any kernel uses private (scratch) memory. The attention
    kernels issue register loads from inline assembly and wait for them by
    hand; a register spill between such a load and its wait would store a
    value that has not arrived, so no kernel may spill."""
    seg = kernel_private_segments(lib_path)
    if not seg:
        raise RuntimeError(f"no kernel metadata found in {lib_path}")
    bad = {k: v for k, v in seg.items() if v}
    if bad:
        raise RuntimeError("kernels with private (scratch) memory, i.e. register spills: " +
                           ", ".join(f"{k} ({v} B/lane)" for k, v in sorted(bad.items())))


def build_library(verbose: bool = False) -> str:
    """Compiles every source and links libtv.so (after checking that no
    kernel spills registers); returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libtv.so failed:\n{res.stdout}\n{res.stderr}")
    check_no_scratch(tmp)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
