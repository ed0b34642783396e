"""Compile the HIP library (libfusedproj.so) for gfx950 with hipcc, in-tree.

Each source is compiled to an object in parallel (fusion_residual_add_amd/_build/),
then the objects are linked into fusion_residual_add_amd/libfusedproj.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["fp_rows.hip", "fp_tiled.hip", "fp_stream.hip", "fp_stream_bf16.hip", "fp_stream_f16.hip",
           "fp_stream_i8.hip", "fp_stream_i4.hip", "fp_stream_mx.hip", "fp_stream_f8.hip", "fp_pack.hip", "fp_prefill_bf16.hip", "fp_prefill_f16.hip", "fp_prefill_i8.hip", "fp_prefill_i4.hip", "fp_prefill_mx.hip", "fp_gemm8.hip", "fp_gemm16.hip",
           "fp_noalloc.hip", "fp_api.cpp"]
LIB = os.path.join(PKG, "libfusedproj.so")
OBJDIR = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from emitting packed-fp32 VALU forms
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, src + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + res.stdout + res.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, LIB)
    return LIB


SANITIZED = ["fp_api.cpp", "fp_noalloc.hip"]   # the host code of the C ABI


def build_host_sanitized(out: str) -> str:
    """The library with its C-ABI host code (argument validation, planning,
    workspace layout, the static scratch lookup) compiled with AddressSanitizer
    and UndefinedBehaviorSanitizer, host side only, linked with the objects of
    build(); load it into a process whose first library is clang's ASan runtime.
    Device code is not instrumented."""
    if not all(os.path.exists(os.path.join(OBJDIR, s + ".o")) for s in SOURCES):
        build()
    sdir = os.path.join(OBJDIR, "host_sanitized")
    os.makedirs(sdir, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-Xarch_host", "-g"]
    objs = []
    for src in SOURCES:
        if src in SANITIZED:
            obj = os.path.join(sdir, src + ".o")
            res = subprocess.run([HIPCC, *FLAGS, *san, "-c", os.path.join(CSRC, src), "-o", obj],
                                 capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n" + res.stdout + res.stderr)
            objs.append(obj)
        else:
            objs.append(os.path.join(OBJDIR, src + ".o"))
    res = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                          "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", *objs, "-o", out],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("sanitized link failed:\n" + res.stdout + res.stderr)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
