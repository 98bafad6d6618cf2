"""ctypes wrapper around the fp64 gated-retention oracle (``gret_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.

The oracle is the plain recurrence of the page "YOCO 完全拆解：Decoder-Decoder
架构如何让 KV Cache 只存一次", section "路线二：Multi-Head Gated Retention"
(state decayed by the per-position head gate, plus the key/value outer
product; output = query times the updated state), carried in double precision.
Inputs are passed exactly as the GPU reads them: float32 arrays, or bf16 bit
patterns held in uint16 arrays; they are widened to double inside the C code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gret_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgret_oracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16 = 0, 1


def build_oracle(force: bool = True) -> str:
    """Compile ``gret_oracle.c`` with gcc (OpenMP, IEEE semantics: no fast-math)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build_oracle()
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.gret_oracle_prefill_f64.argtypes = [vp, vp, vp, ci, vp, vp, vp, vp, vp, ci, vp,
                                                i64, i64, i64, i64, ci]
        lib.gret_oracle_prefill_f64.restype = ci
        lib.gret_oracle_decode_f64.argtypes = [vp, vp, vp, ci, vp, vp, vp, i64, i64, i64, ci]
        lib.gret_oracle_decode_f64.restype = ci
        lib.gret_oracle_max_threads.argtypes = []
        lib.gret_oracle_max_threads.restype = ci
        _lib = lib
        return lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("oracle inputs must be float32 or uint16 (bf16 bits), got %s" % a.dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data


def oracle_max_threads() -> int:
    return int(_load().gret_oracle_max_threads())


def oracle_prefill_f64(q, k, v, log_gamma, state_in=None, *, want_out=True, compare=None,
                       nthreads=0):
    """Run the recurrence over every head.

    q, k: [..., N, dk]; v: [..., N, dv]; log_gamma: [..., N] float32;
    state_in: [..., dk, dv] float32 or float64 or None (widened exactly to float64).
    Leading dims are flattened to heads.
    compare: optional array shaped like the output (float32 or bf16 bits); when
    given, returns per-head (max |compare - ref|, max |ref|) statistics.
    Returns (out_f64 or None, state_f64, stats or None).
    """
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    lg = np.ascontiguousarray(log_gamma, dtype=np.float32)
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise TypeError("q, k, v must share one dtype")
    lead = q.shape[:-2]
    N, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:-1] != q.shape[:-1] or lg.shape != lead + (N,):
        raise ValueError("shape mismatch")
    BH = int(np.prod(lead)) if lead else 1
    s_in = None
    if state_in is not None:
        if state_in.dtype not in (np.float32, np.float64):
            raise TypeError("state_in must be float32 or float64")
        s_in = np.ascontiguousarray(state_in, dtype=np.float64)
        if s_in.shape != lead + (dk, dv):
            raise ValueError("state_in shape mismatch")
    state = np.empty(lead + (dk, dv), dtype=np.float64)
    out = np.empty(lead + (N, dv), dtype=np.float64) if want_out else None
    stats = None
    cmp_code = 0
    if compare is not None:
        compare = np.ascontiguousarray(compare)
        cmp_code = _dtype_code(compare)
        if compare.shape != lead + (N, dv):
            raise ValueError("compare shape mismatch")
        stats = np.empty((BH, 2), dtype=np.float64)
    rc = _load().gret_oracle_prefill_f64(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(lg), _ptr(s_in),
                                         _ptr(state), _ptr(out), _ptr(compare), cmp_code,
                                         _ptr(stats), BH, N, dk, dv, int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle prefill failed (rc=%d)" % rc)
    return out, state, stats


def oracle_decode_f64(q, k, v, log_gamma, state, *, nthreads=0):
    """One recurrent step for every head; ``state`` (float64) is updated in place.

    q, k: [..., dk]; v: [..., dv]; log_gamma: [...] float32; state [..., dk, dv] float64.
    Returns out [..., dv] float64.
    """
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    lg = np.ascontiguousarray(log_gamma, dtype=np.float32)
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise TypeError("q, k, v must share one dtype")
    if state.dtype != np.float64 or not state.flags.c_contiguous:
        raise TypeError("state must be a C-contiguous float64 array")
    lead = q.shape[:-1]
    dk, dv = q.shape[-1], v.shape[-1]
    if k.shape != q.shape or v.shape[:-1] != lead or lg.shape != lead or \
            state.shape != lead + (dk, dv):
        raise ValueError("shape mismatch")
    BH = int(np.prod(lead)) if lead else 1
    out = np.empty(lead + (dv,), dtype=np.float64)
    rc = _load().gret_oracle_decode_f64(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(lg), _ptr(state),
                                        _ptr(out), BH, dk, dv, int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle decode failed (rc=%d)" % rc)
    return out
