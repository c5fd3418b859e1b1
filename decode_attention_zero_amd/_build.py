"""Builds the HIP library ``libdkv.so`` in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libdkv.so")
SOURCES = ["proj.hip", "fresh.hip", "attn_split.hip", "attn_combine.hip", "window.hip", "gemm.hip", "probe.hip",
           "runtime.hip", "noalloc.hip", "append.hip"]
# Host-only C++ (the CPU attention comparator), built with the system compiler.
HOST_SOURCES = ["cpu_attention.cpp"]
HEADERS = [os.path.join(CSRC, "cpu_attention.h"), os.path.join(CSRC, "dkv_internal.h"), os.path.join(CSRC, "device_common.h"), os.path.join(CSRC, "mfma_tile.h"), os.path.join(INCLUDE, "dkv.h"),
           os.path.join(INCLUDE, "dkv_probe.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-fopenmp-simd", "-ffp-contract=fast", "-fno-math-errno",
              "-Wall", "-I", INCLUDE, "-I", CSRC]
ARCH = "gfx950"
# Packed fp32 instructions are switched off for every HIP source.
COMMON_FLAGS = ["-O3", "-std=c++17", "--offload-arch=" + ARCH, "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC]


def sources() -> list[str]:
    return [os.path.join(CSRC, s) for s in SOURCES]


def build_library(out: str = LIBRARY, verbose: bool = False) -> str:
    """Compiles every HIP source into one shared library (always recompiles)."""
    tmp = out + ".tmp%d" % os.getpid()
    objects = []
    try:
        for src in HOST_SOURCES:
            obj = "%s.%s.o" % (tmp, os.path.splitext(src)[0])
            cmd = [CXX] + HOST_FLAGS + ["-c", "-o", obj, os.path.join(CSRC, src)]
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError("host compiler failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
            objects.append(obj)
        cmd = [HIPCC] + COMMON_FLAGS + ["-shared", "-o", tmp] + sources() + ["-x", "none"] + objects + ["-pthread"]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
        if verbose:
            print(res.stderr)
        os.replace(tmp, out)
    finally:
        for obj in objects:
            if os.path.exists(obj):
                os.remove(obj)
    return out


def device_assembly(source: str = "attn_split.hip") -> str:
    """gfx950 assembly of one source (for inspecting this library's own code)."""
    cmd = [HIPCC] + COMMON_FLAGS + ["--cuda-device-only", "-S", "-o", "-",
                                    os.path.join(CSRC, source)]
    return subprocess.run(cmd, capture_output=True, text=True, check=True).stdout
