"""Builds libgret.so (the HIP library) in place for gfx950, and
libgret_stream.so (the streaming kernels the benchmark measures HBM with).

Every source is compiled with hipcc for gfx950 only; packed fp32 vector ops are
disabled for device code. Objects go to ``_build/`` next to this file, the
shared libraries next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgret.so")
STREAM_LIB = os.path.join(HERE, "libgret_stream.so")
STREAM_SOURCES = ["gret_stream.hip"]
SOURCES = ["gret_api.cpp", "gret_decode.hip", "gret_prefill_f32.hip", "gret_prefill_bf16.hip",
           "gret_prefill_c64.hip", "gret_epilogue.hip", "gret_xattn.hip", "gret_proj.hip", "gret_swa.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [_hipcc(), "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
           f"--offload-arch={ARCH}", "-I", os.path.join(HERE, "..", "include")]
    if src.endswith(".hip"):
        cmd += ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    else:
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed for %s" % src)
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("link of %s failed" % os.path.basename(lib))
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + STREAM_SOURCES
    jobs = min(len(srcs), max(1, (os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in STREAM_SOURCES], STREAM_LIB)
    if verbose:
        print("built", LIB, "and", STREAM_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
