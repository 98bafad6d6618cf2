"""Python binding of libgret (gated retention on AMD gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/gret.h``. PyTorch supplies the
device memory and the current HIP stream. There is no CPU fallback; if the
library is not built, every call raises.

Functions mirror the C ABI names:
  gret_prefill(q, k, v, log_gamma, state_in=None, chunk=64, out=None,
               state_out=None, workspace=None) -> (out, state_out)
  gret_prefill_noalloc(q, k, v, log_gamma, state_in=None, chunk=64, out=None,
                       state_out=None) -> (out, state_out)
  gret_prefill_gated(q, k, v, log_gamma, gate, state_in=None, norm_weight=None,
                     norm_bias=None, norm_eps=1e-5, chunk=64, out=None,
                     state_out=None, workspace=None) -> (out, state_out)
  gret_decode_step(q, k, v, log_gamma, state_in, out=None, state_out=None) -> out
  gret_decode_step_gated(q, k, v, log_gamma, state_in, gate, norm_weight=None,
                         norm_bias=None, norm_eps=1e-5, out=None,
                         state_out=None) -> out
  gret_prefill_workspace_bytes(B, H, N, dk, dv, chunk, dtype) -> int
  gret_cross_attention_decode(q, k_cache, v_cache, lengths=None, scale=None,
                              out=None, workspace=None) -> out
  gret_cross_attention_workspace_bytes(B, Hq, Hkv, L, d) -> int
  gret_head_projection(x, w_key, w_gamma=None, key_scale=1.0, temperature=16.0,
                       H=None, k_out=None, log_gamma=None) -> (k_out, log_gamma)
  gret_swa_prefill(q, k, v, window, scale=None, out=None, k_ring=None,
                   v_ring=None) -> out
  gret_swa_decode_step(q, k_new, v_new, k_ring, v_ring, positions, scale=None,
                       out=None, workspace=None) -> out
  gret_swa_decode_workspace_bytes(B, Hq, Hkv, window, d) -> int
  gret_status_string(status) -> str
The gated variants add the output epilogue (per-head GroupNorm, optional
per-channel affine [H, dv] in fp32, element-wise swish(gate)).
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgret.so")

GRET_DTYPE_F32 = 0
GRET_DTYPE_BF16 = 1
GRET_OK = 0

_lock = threading.Lock()
_lib = None


class GretError(RuntimeError):
    """A libgret call returned a nonzero status."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s" % (where, gret_status_string(status)))


def load_library():
    """Load libgret.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libgret.so is not built (%s); run __graft_entry__.build() or "
                               "python -m yoco_gated_retention_amd.build" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        vp, i64, ci, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        lib.gret_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci,
                                     vp, sz, vp]
        lib.gret_prefill.restype = ci
        lib.gret_prefill_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                             i64, ci, vp]
        lib.gret_prefill_noalloc.restype = ci
        lib.gret_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, ci, vp]
        lib.gret_decode_step.restype = ci
        lib.gret_prefill_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, ci,
                                                     ctypes.POINTER(sz)]
        lib.gret_prefill_workspace_bytes.restype = ci
        fl = ctypes.c_float
        lib.gret_prefill_gated.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, fl, vp, vp, i64, i64,
                                           i64, i64, i64, i64, ci, vp, sz, vp]
        lib.gret_prefill_gated.restype = ci
        lib.gret_decode_step_gated.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, fl, vp, vp, i64,
                                               i64, i64, i64, ci, vp]
        lib.gret_decode_step_gated.restype = ci
        lib.gret_cross_attention_workspace_bytes.argtypes = [i64, i64, i64, i64, i64,
                                                             ctypes.POINTER(sz)]
        lib.gret_cross_attention_workspace_bytes.restype = ci
        lib.gret_cross_attention_decode.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                                    fl, ci, vp, sz, vp]
        lib.gret_cross_attention_decode.restype = ci
        lib.gret_head_projection.argtypes = [vp, vp, vp, fl, fl, vp, vp, i64, i64, i64, i64, i64,
                                             ci, vp]
        lib.gret_head_projection.restype = ci
        lib.gret_swa_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, fl,
                                         ci, vp]
        lib.gret_swa_prefill.restype = ci
        lib.gret_swa_decode_workspace_bytes.argtypes = [i64, i64, i64, i64, i64,
                                                        ctypes.POINTER(sz)]
        lib.gret_swa_decode_workspace_bytes.restype = ci
        lib.gret_swa_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                             fl, ci, vp, sz, vp]
        lib.gret_swa_decode_step.restype = ci
        lib.gret_status_string.argtypes = [ci]
        lib.gret_status_string.restype = ctypes.c_char_p
        _lib = lib
        return lib


def gret_status_string(status: int) -> str:
    return load_library().gret_status_string(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GRET_DTYPE_BF16
    if t.dtype == torch.float32:
        return GRET_DTYPE_F32
    raise TypeError("q, k, v must be bfloat16 or float32, got %s" % t.dtype)


def _check_dev(name, t, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor" % name)
    if device is not None and t.device != device:
        raise ValueError("%s must be on %s (q's device), got %s" % (name, device, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))


def _check_tensors(specs, device):
    """specs: (name, tensor or None, exact shape or None, dtype or None). Every
    shape is checked before anything else, so a wrong-sized buffer is rejected
    before any device or library call; then dtype, device (q's GPU) and
    contiguity. The kernels take every size from q and v, so an undersized
    output, state or ring buffer would otherwise be written out of bounds."""
    for name, t, shape, _ in specs:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % name)
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape),
                                                               tuple(t.shape)))
    for name, t, _, dtype in specs:
        if t is not None:
            _check_dev(name, t, dtype, device)


def _check_workspace(workspace, device):
    if workspace is not None:
        _check_dev("workspace", workspace, None, device)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _call(device, fn, *args):
    """Calls a library entry point with q's device current (the library asks
    the runtime for the current device's compute-unit count)."""
    if device.index is None or device.index == torch.cuda.current_device():
        return fn(*args)
    with torch.cuda.device(device):
        return fn(*args)


def _bytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def gret_prefill_workspace_bytes(B, H, N, dk, dv, chunk, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(torch.empty(0, dtype=dtype))
    n = ctypes.c_size_t(0)
    st = load_library().gret_prefill_workspace_bytes(B, H, N, dk, dv, chunk, code,
                                                     ctypes.byref(n))
    if st != GRET_OK:
        raise GretError(st, "gret_prefill_workspace_bytes")
    return int(n.value)


def _prefill_shapes(q, v):
    for name, t in (("q", q), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % name)
    if q.dim() != 4 or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,H,N,dk] and v [B,H,N,dv]")
    B, H, N, dk = q.shape
    return B, H, N, dk, v.shape[3]


def _prefill_setup(q, k, v, log_gamma, state_in, chunk, out, state_out, workspace, extra=()):
    B, H, N, dk, dv = _prefill_shapes(q, v)
    dev = q.device
    _check_tensors([("q", q, None, None), ("k", k, q.shape, q.dtype), ("v", v, None, q.dtype),
                    ("log_gamma", log_gamma, (B, H, N), torch.float32),
                    ("state_in", state_in, (B, H, dk, dv), torch.float32),
                    ("out", out, (B, H, N, dv), q.dtype),
                    ("state_out", state_out, (B, H, dk, dv), torch.float32)] + list(extra), dev)
    _check_workspace(workspace, dev)
    code = _dtype_code(q)
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=dev)
    if state_out is None:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    need = gret_prefill_workspace_bytes(B, H, N, dk, dv, chunk, code)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    return (B, H, N, dk, dv, code, out, state_out, workspace, _bytes(workspace))


def _epilogue_specs(gate, shape, dtype, norm_weight, norm_bias, H, dv):
    if gate is None:
        raise ValueError("gate is required")
    return [("gate", gate, shape, dtype), ("norm_weight", norm_weight, (H, dv), torch.float32),
            ("norm_bias", norm_bias, (H, dv), torch.float32)]


def gret_prefill(q, k, v, log_gamma, state_in=None, chunk=64, out=None, state_out=None,
                 workspace=None):
    """Chunkwise prefill. q, k [B,H,N,dk]; v [B,H,N,dv]; log_gamma [B,H,N] fp32;
    state_in [B,H,dk,dv] fp32 or None. Returns (out [B,H,N,dv], state_out)."""
    lib = load_library()
    B, H, N, dk, dv, code, out, state_out, workspace, ws_bytes = _prefill_setup(
        q, k, v, log_gamma, state_in, chunk, out, state_out, workspace)
    st = _call(q.device, lib.gret_prefill, _ptr(q), _ptr(k), _ptr(v), _ptr(log_gamma),
               _ptr(state_in), _ptr(out), _ptr(state_out), B, H, N, dk, dv, chunk, code,
               _ptr(workspace), ws_bytes, _stream(q.device))
    if st != GRET_OK:
        raise GretError(st, "gret_prefill")
    return out, state_out


def gret_prefill_noalloc(q, k, v, log_gamma, state_in=None, chunk=64, out=None, state_out=None):
    """gret_prefill without a workspace, for callers that cannot allocate device
    memory: the library's fixed per-GPU scratch (GRET_NOALLOC_SCRATCH_BYTES) holds
    the partial states. Pass out and state_out to allocate nothing at all.
    Calls that overlap in time on one GPU race on the scratch."""
    lib = load_library()
    B, H, N, dk, dv = _prefill_shapes(q, v)
    dev = q.device
    _check_tensors([("q", q, None, None), ("k", k, q.shape, q.dtype), ("v", v, None, q.dtype),
                    ("log_gamma", log_gamma, (B, H, N), torch.float32),
                    ("state_in", state_in, (B, H, dk, dv), torch.float32),
                    ("out", out, (B, H, N, dv), q.dtype),
                    ("state_out", state_out, (B, H, dk, dv), torch.float32)], dev)
    code = _dtype_code(q)
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=dev)
    if state_out is None:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    st = _call(dev, lib.gret_prefill_noalloc, _ptr(q), _ptr(k), _ptr(v), _ptr(log_gamma),
               _ptr(state_in), _ptr(out), _ptr(state_out), B, H, N, dk, dv, chunk, code,
               _stream(dev))
    if st != GRET_OK:
        raise GretError(st, "gret_prefill_noalloc")
    return out, state_out


def gret_prefill_gated(q, k, v, log_gamma, gate, state_in=None, norm_weight=None, norm_bias=None,
                       norm_eps=1e-5, chunk=64, out=None, state_out=None, workspace=None):
    """Chunkwise prefill followed by the output epilogue: out = swish(gate) *
    GroupNorm_per_head(retention output). gate [B,H,N,dv] in q's dtype;
    norm_weight, norm_bias [H,dv] fp32 or None. Returns (out, state_out)."""
    lib = load_library()
    B, H, N, dk, dv = _prefill_shapes(q, v)
    extra = _epilogue_specs(gate, (B, H, N, dv), q.dtype, norm_weight, norm_bias, H, dv)
    B, H, N, dk, dv, code, out, state_out, workspace, ws_bytes = _prefill_setup(
        q, k, v, log_gamma, state_in, chunk, out, state_out, workspace, extra)
    st = _call(q.device, lib.gret_prefill_gated, _ptr(q), _ptr(k), _ptr(v), _ptr(log_gamma),
               _ptr(state_in), _ptr(gate), _ptr(norm_weight), _ptr(norm_bias), float(norm_eps),
               _ptr(out), _ptr(state_out), B, H, N, dk, dv, chunk, code, _ptr(workspace),
               ws_bytes, _stream(q.device))
    if st != GRET_OK:
        raise GretError(st, "gret_prefill_gated")
    return out, state_out


def _decode_shapes(q, v):
    for name, t in (("q", q), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % name)
    if q.dim() != 3 or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("q, k must be [B,H,dk] and v [B,H,dv]")
    B, H, dk = q.shape
    return B, H, dk, v.shape[2]


def _decode_setup(q, k, v, log_gamma, state_in, out, state_out, extra=()):
    B, H, dk, dv = _decode_shapes(q, v)
    dev = q.device
    if state_out is None:
        if state_in is None:
            raise ValueError("state_out is required when state_in is None")
        state_out = state_in
    _check_tensors([("q", q, None, None), ("k", k, q.shape, q.dtype), ("v", v, None, q.dtype),
                    ("log_gamma", log_gamma, (B, H), torch.float32),
                    ("state_in", state_in, (B, H, dk, dv), torch.float32),
                    ("state_out", state_out, (B, H, dk, dv), torch.float32),
                    ("out", out, (B, H, dv), q.dtype)] + list(extra), dev)
    _dtype_code(q)
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=dev)
    return B, H, dk, dv, out, state_out


def gret_decode_step(q, k, v, log_gamma, state_in, out=None, state_out=None):
    """One recurrent step. q, k [B,H,dk]; v [B,H,dv]; log_gamma [B,H] fp32;
    state_in [B,H,dk,dv] fp32 (or None = zero). state_out defaults to state_in
    (in-place update). Returns out [B,H,dv]."""
    lib = load_library()
    B, H, dk, dv, out, state_out = _decode_setup(q, k, v, log_gamma, state_in, out, state_out)
    st = _call(q.device, lib.gret_decode_step, _ptr(q), _ptr(k), _ptr(v), _ptr(log_gamma),
               _ptr(state_in), _ptr(out), _ptr(state_out), B, H, dk, dv, _dtype_code(q),
               _stream(q.device))
    if st != GRET_OK:
        raise GretError(st, "gret_decode_step")
    return out


def gret_decode_step_gated(q, k, v, log_gamma, state_in, gate, norm_weight=None, norm_bias=None,
                           norm_eps=1e-5, out=None, state_out=None):
    """One recurrent step with the output epilogue fused into its store:
    out = swish(gate) * GroupNorm_per_head(q S). gate [B,H,dv] in q's dtype."""
    lib = load_library()
    B, H, dk, dv = _decode_shapes(q, v)
    extra = _epilogue_specs(gate, (B, H, dv), q.dtype, norm_weight, norm_bias, H, dv)
    B, H, dk, dv, out, state_out = _decode_setup(q, k, v, log_gamma, state_in, out, state_out,
                                                 extra)
    st = _call(q.device, lib.gret_decode_step_gated, _ptr(q), _ptr(k), _ptr(v), _ptr(log_gamma),
               _ptr(state_in), _ptr(gate), _ptr(norm_weight), _ptr(norm_bias), float(norm_eps),
               _ptr(out), _ptr(state_out), B, H, dk, dv, _dtype_code(q), _stream(q.device))
    if st != GRET_OK:
        raise GretError(st, "gret_decode_step_gated")
    return out


def gret_cross_attention_workspace_bytes(B, Hq, Hkv, L, d) -> int:
    n = ctypes.c_size_t(0)
    st = load_library().gret_cross_attention_workspace_bytes(B, Hq, Hkv, L, d, ctypes.byref(n))
    if st != GRET_OK:
        raise GretError(st, "gret_cross_attention_workspace_bytes")
    return int(n.value)


def gret_cross_attention_decode(q, k_cache, v_cache, lengths=None, scale=None, out=None,
                                workspace=None):
    """Decode attention of q [B,Hq,d] over the global KV cache k_cache, v_cache
    [B,Hkv,L,d] (bf16), GQA with Hq / Hkv query heads per KV head; lengths: int32
    [B] on the GPU or None (all L); scale defaults to d^-1/2. Returns out
    [B,Hq,d] bf16."""
    lib = load_library()
    for name, t in (("q", q), ("k_cache", k_cache)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % name)
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B,Hq,d] and the caches [B,Hkv,L,d]")
    B, Hq, d = q.shape
    _, Hkv, L, _ = k_cache.shape
    dev = q.device
    _check_tensors([("q", q, None, torch.bfloat16),
                    ("k_cache", k_cache, (B, Hkv, L, d), torch.bfloat16),
                    ("v_cache", v_cache, (B, Hkv, L, d), torch.bfloat16),
                    ("lengths", lengths, (B,), torch.int32),
                    ("out", out, (B, Hq, d), torch.bfloat16)], dev)
    _check_workspace(workspace, dev)
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=dev)
    if workspace is None:
        need = gret_cross_attention_workspace_bytes(B, Hq, Hkv, L, d)
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = _call(dev, lib.gret_cross_attention_decode, _ptr(q), _ptr(k_cache), _ptr(v_cache),
               _ptr(lengths), _ptr(out), B, Hq, Hkv, L, d, float(scale), GRET_DTYPE_BF16,
               _ptr(workspace), _bytes(workspace), _stream(dev))
    if st != GRET_OK:
        raise GretError(st, "gret_cross_attention_decode")
    return out


def gret_head_projection(x, w_key, w_gamma=None, key_scale=1.0, temperature=16.0, H=None,
                         k_out=None, log_gamma=None):
    """Head-major projection of x [B,N,D] (bf16) by w_key [H*dk, D], times
    key_scale -> k_out [B,H,N,dk] bf16; with w_gamma [H, D] also the log-gate
    log(sigmoid(x w_gamma^T)) / temperature -> log_gamma [B,H,N] fp32 (else
    None). H is taken from w_gamma, or must be given without it."""
    lib = load_library()
    for name, t in (("x", x), ("w_key", w_key)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % name)
    if x.dim() != 3 or w_key.dim() != 2 or w_key.shape[1] != x.shape[2]:
        raise ValueError("x must be [B,N,D] and w_key [H*dk, D]")
    B, N, D = x.shape
    if w_gamma is not None:
        if not isinstance(w_gamma, torch.Tensor):
            raise TypeError("w_gamma must be a torch.Tensor")
        if w_gamma.dim() != 2 or w_gamma.shape[1] != D:
            raise ValueError("w_gamma must be [H, D]")
        if H is not None and H != w_gamma.shape[0]:
            raise ValueError("H does not match w_gamma")
        H = w_gamma.shape[0]
    elif log_gamma is not None:
        raise ValueError("log_gamma needs w_gamma")
    if H is None or H < 1 or w_key.shape[0] % H != 0:
        raise ValueError("w_key must have H * dk rows")
    dk = w_key.shape[0] // H
    dev = x.device
    _check_tensors([("x", x, None, torch.bfloat16), ("w_key", w_key, None, torch.bfloat16),
                    ("w_gamma", w_gamma, None, torch.bfloat16),
                    ("k_out", k_out, (B, H, N, dk), torch.bfloat16),
                    ("log_gamma", log_gamma, (B, H, N), torch.float32)], dev)
    if k_out is None:
        k_out = torch.empty((B, H, N, dk), dtype=torch.bfloat16, device=dev)
    if w_gamma is not None and log_gamma is None:
        log_gamma = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    st = _call(dev, lib.gret_head_projection, _ptr(x), _ptr(w_key), _ptr(w_gamma),
               float(key_scale), float(temperature), _ptr(k_out), _ptr(log_gamma), B, N, D, H,
               dk, GRET_DTYPE_BF16, _stream(dev))
    if st != GRET_OK:
        raise GretError(st, "gret_head_projection")
    return k_out, log_gamma


def gret_swa_prefill(q, k, v, window, scale=None, out=None, k_ring=None, v_ring=None):
    """Sliding-window causal attention of q [B,Hq,N,d] over k, v [B,Hkv,N,d]
    (bf16) with `window` positions per query; fills k_ring, v_ring
    [B,Hkv,window,d] with the last positions when given. Returns out."""
    lib = load_library()
    for name, t in (("q", q), ("k", k)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % name)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B,Hq,N,d] and k, v [B,Hkv,N,d]")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if (k_ring is None) != (v_ring is None):
        raise ValueError("give both rings or neither")
    window = int(window)
    dev = q.device
    _check_tensors([("q", q, None, torch.bfloat16), ("k", k, (B, Hkv, N, d), torch.bfloat16),
                    ("v", v, (B, Hkv, N, d), torch.bfloat16),
                    ("out", out, (B, Hq, N, d), torch.bfloat16),
                    ("k_ring", k_ring, (B, Hkv, window, d), torch.bfloat16),
                    ("v_ring", v_ring, (B, Hkv, window, d), torch.bfloat16)], dev)
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty_like(q)
    st = _call(dev, lib.gret_swa_prefill, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(k_ring),
               _ptr(v_ring), B, Hq, Hkv, N, d, window, float(scale), GRET_DTYPE_BF16,
               _stream(dev))
    if st != GRET_OK:
        raise GretError(st, "gret_swa_prefill")
    return out


def gret_swa_decode_workspace_bytes(B, Hq, Hkv, window, d) -> int:
    n = ctypes.c_size_t(0)
    st = load_library().gret_swa_decode_workspace_bytes(B, Hq, Hkv, window, d, ctypes.byref(n))
    if st != GRET_OK:
        raise GretError(st, "gret_swa_decode_workspace_bytes")
    return int(n.value)


def gret_swa_decode_step(q, k_new, v_new, k_ring, v_ring, positions, scale=None, out=None,
                         workspace=None):
    """One decode step of sliding-window attention: k_new, v_new [B,Hkv,d] go
    into ring slot positions[b] mod window (rings [B,Hkv,window,d], updated in
    place), then q [B,Hq,d] attends over the valid slots. positions: int32 [B]
    on the GPU. Returns out [B,Hq,d] bf16."""
    lib = load_library()
    for name, t in (("q", q), ("k_ring", k_ring)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % name)
    if q.dim() != 3 or k_ring.dim() != 4:
        raise ValueError("q must be [B,Hq,d] and the rings [B,Hkv,window,d]")
    B, Hq, d = q.shape
    _, Hkv, window, _ = k_ring.shape
    dev = q.device
    _check_tensors([("q", q, None, torch.bfloat16),
                    ("k_new", k_new, (B, Hkv, d), torch.bfloat16),
                    ("v_new", v_new, (B, Hkv, d), torch.bfloat16),
                    ("k_ring", k_ring, (B, Hkv, window, d), torch.bfloat16),
                    ("v_ring", v_ring, (B, Hkv, window, d), torch.bfloat16),
                    ("positions", positions, (B,), torch.int32),
                    ("out", out, (B, Hq, d), torch.bfloat16)], dev)
    _check_workspace(workspace, dev)
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        need = gret_swa_decode_workspace_bytes(B, Hq, Hkv, window, d)
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = _call(dev, lib.gret_swa_decode_step, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_ring),
               _ptr(v_ring), _ptr(positions), _ptr(out), B, Hq, Hkv, window, d, float(scale),
               GRET_DTYPE_BF16, _ptr(workspace), _bytes(workspace), _stream(dev))
    if st != GRET_OK:
        raise GretError(st, "gret_swa_decode_step")
    return out
