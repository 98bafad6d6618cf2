"""C-ABI contract checks that need no GPU: the library loads, exports every
symbol include/gret.h declares, and rejects bad arguments before touching the
HIP runtime (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import yoco_gated_retention_amd as gret

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gret.h")

OK, NULL, SHAPE, UNSUP, ALIAS, HIP, WORKSPACE, VALUE, SCRATCH = range(9)
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def lib():
    return gret.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gret_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"gret_prefill", "gret_decode_step", "gret_prefill_workspace_bytes",
            "gret_status_string", "gret_prefill_gated", "gret_decode_step_gated"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(9):
        assert gret.gret_status_string(s).startswith(
            ["GRET_OK", "GRET_ERR_NULL", "GRET_ERR_SHAPE", "GRET_ERR_UNSUPPORTED",
             "GRET_ERR_ALIAS", "GRET_ERR_HIP", "GRET_ERR_WORKSPACE", "GRET_ERR_VALUE",
             "GRET_ERR_SCRATCH"][s])
    assert gret.gret_status_string(99) == "unknown gret status"


def ws_bytes(lib, B, H, N, dk, dv, chunk, dtype):
    n = ctypes.c_size_t(12345)
    st = lib.gret_prefill_workspace_bytes(B, H, N, dk, dv, chunk, dtype, ctypes.byref(n))
    return st, n.value


def test_workspace_query(lib):
    assert ws_bytes(lib, 1, 2, 512, 64, 64, 64, F32) == (OK, 0)
    st, n = ws_bytes(lib, 1, 24, 524288, 128, 128, 64, BF16)
    assert st == OK and n % 256 == 0 and 0 < n < 256 << 20
    assert ws_bytes(lib, 1, 2, 512, 96, 64, 64, BF16)[0] == UNSUP
    assert ws_bytes(lib, 1, 2, 512, 64, 64, 32, BF16)[0] == UNSUP
    assert ws_bytes(lib, 0, 2, 512, 64, 64, 64, BF16)[0] == SHAPE
    assert ws_bytes(lib, 1, 2, 512, 64, 64, 64, 7)[0] == UNSUP
    assert lib.gret_prefill_workspace_bytes(1, 1, 1, 64, 64, 64, 1, None) == NULL


# Fake, well-aligned device addresses: validation must reject every call below
# before any HIP call, so nothing is ever dereferenced.
BASE = 1 << 40
MB = 1 << 20


def P(i):
    return ctypes.c_void_p(BASE + i * 256 * MB)


def prefill(lib, q=P(0), k=P(1), v=P(2), lg=P(3), si=None, out=P(4), so=P(5), B=1, H=2, N=512,
            dk=64, dv=64, chunk=64, dtype=BF16, ws=P(6), wsb=1 << 30):
    return lib.gret_prefill(q, k, v, lg, si, out, so, B, H, N, dk, dv, chunk, dtype, ws, wsb, None)


def decode(lib, q=P(0), k=P(1), v=P(2), lg=P(3), si=P(5), out=P(4), so=P(5), B=2, H=3, dk=64,
           dv=64, dtype=BF16):
    return lib.gret_decode_step(q, k, v, lg, si, out, so, B, H, dk, dv, dtype, None)


def test_prefill_validation(lib):
    assert prefill(lib, q=None) == NULL
    assert prefill(lib, lg=None) == NULL
    assert prefill(lib, out=None) == NULL
    assert prefill(lib, N=0) == SHAPE
    assert prefill(lib, B=-1) == SHAPE
    assert prefill(lib, B=1 << 40, H=1 << 20) == SHAPE
    assert prefill(lib, dk=32) == UNSUP
    assert prefill(lib, dv=256) == UNSUP
    assert prefill(lib, chunk=100) == UNSUP
    assert prefill(lib, dtype=3) == UNSUP
    assert prefill(lib, q=ctypes.c_void_p(BASE + 8)) == UNSUP  # not 16-byte aligned
    assert prefill(lib, ws=None) == WORKSPACE
    assert prefill(lib, wsb=16) == WORKSPACE
    assert prefill(lib, ws=ctypes.c_void_p(BASE + 6 * 256 * MB + 16)) == WORKSPACE


def test_prefill_aliasing(lib):
    # out on top of q
    assert prefill(lib, out=P(0)) == ALIAS
    # out overlapping the tail of v (v is 1*2*512*64*2 bytes = 128 KiB)
    assert prefill(lib, out=ctypes.c_void_p(BASE + 2 * 256 * MB + 64 * 1024)) == ALIAS
    # states partially overlapping
    assert prefill(lib, si=P(5), so=ctypes.c_void_p(BASE + 5 * 256 * MB + 4096)) == ALIAS
    # state_out on top of k
    assert prefill(lib, so=P(1)) == ALIAS
    # workspace on top of state_in
    assert prefill(lib, si=P(7), ws=P(7)) == ALIAS


def test_prefill_noalloc_validation(lib):
    # the variant without a workspace validates like gret_prefill and, for
    # these rejected calls, returns before any HIP call
    def call(q=P(0), out=P(4), so=P(5), si=None, B=1, H=2, N=512, dk=64, dv=64, chunk=64,
             dtype=BF16):
        return lib.gret_prefill_noalloc(q, P(1), P(2), P(3), si, out, so, B, H, N, dk, dv, chunk,
                                        dtype, None)
    assert call(q=None) == NULL
    assert call(out=None) == NULL
    assert call(N=0) == SHAPE
    assert call(dk=32) == UNSUP
    assert call(chunk=100) == UNSUP
    assert call(dtype=3) == UNSUP
    assert call(out=P(0)) == ALIAS
    assert call(si=P(6), so=ctypes.c_void_p(BASE + 6 * 256 * MB + 4096)) == ALIAS


def test_decode_validation(lib):
    assert decode(lib, so=None) == NULL
    assert decode(lib, v=None) == NULL
    assert decode(lib, H=0) == SHAPE
    assert decode(lib, dk=100) == UNSUP
    assert decode(lib, dtype=2) == UNSUP
    assert decode(lib, out=P(5)) == ALIAS           # out on the state
    assert decode(lib, out=P(2)) == ALIAS           # out on v
    assert decode(lib, so=ctypes.c_void_p(BASE + 5 * 256 * MB + 1024)) == ALIAS  # partial
    assert decode(lib, so=P(0)) == ALIAS            # state_out on q


def prefill_gated(lib, gate=P(8), w=None, b=None, eps=1e-5, out=P(4), dtype=BF16, **kw):
    a = dict(q=P(0), k=P(1), v=P(2), lg=P(3), si=None, so=P(5), B=1, H=2, N=512, dk=64, dv=64,
             chunk=64, ws=P(6), wsb=1 << 30)
    a.update(kw)
    return lib.gret_prefill_gated(a["q"], a["k"], a["v"], a["lg"], a["si"], gate, w, b,
                                  ctypes.c_float(eps), out, a["so"], a["B"], a["H"], a["N"],
                                  a["dk"], a["dv"], a["chunk"], dtype, a["ws"], a["wsb"], None)


def decode_gated(lib, gate=P(8), w=None, b=None, eps=1e-5, out=P(4), **kw):
    a = dict(q=P(0), k=P(1), v=P(2), lg=P(3), si=P(5), so=P(5), B=2, H=3, dk=64, dv=64,
             dtype=BF16)
    a.update(kw)
    return lib.gret_decode_step_gated(a["q"], a["k"], a["v"], a["lg"], a["si"], gate, w, b,
                                      ctypes.c_float(eps), out, a["so"], a["B"], a["H"],
                                      a["dk"], a["dv"], a["dtype"], None)


@pytest.mark.parametrize("call", [prefill_gated, decode_gated])
def test_gated_validation(lib, call):
    assert call(lib, gate=None) == NULL
    assert call(lib, eps=-1.0) == VALUE
    assert call(lib, eps=float("nan")) == VALUE
    assert call(lib, eps=float("inf")) == VALUE
    assert call(lib, gate=ctypes.c_void_p(BASE + 8 * 256 * MB + 8)) == UNSUP
    assert call(lib, w=ctypes.c_void_p(BASE + 9 * 256 * MB + 2)) == UNSUP
    assert call(lib, gate=P(4)) == ALIAS                       # gate on out
    assert call(lib, w=P(9), out=ctypes.c_void_p(BASE + 9 * 256 * MB + 256)) == ALIAS
    assert call(lib, b=P(5)) == ALIAS                          # bias on the state
    assert call(lib, out=None) == NULL
    # the plain rules still apply
    assert call(lib, dk=32) == UNSUP


def xattn(lib, q=P(0), k=P(1), v=P(2), lens=None, out=P(4), B=2, Hq=24, Hkv=8, L=4096, d=128,
          scale=0.088, dtype=BF16, ws=P(6), wsb=1 << 30):
    return lib.gret_cross_attention_decode(q, k, v, lens, out, B, Hq, Hkv, L, d,
                                           ctypes.c_float(scale), dtype, ws, wsb, None)


def test_cross_attention_validation(lib):
    n = ctypes.c_size_t(0)
    assert lib.gret_cross_attention_workspace_bytes(2, 24, 8, 4096, 128, ctypes.byref(n)) == OK
    assert 0 < n.value < 64 << 20 and n.value % 256 == 0
    assert lib.gret_cross_attention_workspace_bytes(2, 24, 8, 4096, 128, None) == NULL
    assert xattn(lib, q=None) == NULL
    assert xattn(lib, L=0) == SHAPE
    assert xattn(lib, B=1, Hq=1, Hkv=1, L=1 << 34) == SHAPE  # more ranges than the merge takes
    # caches longer than 2^23 positions are split into ranges that fit 32-bit offsets
    assert lib.gret_cross_attention_workspace_bytes(1, 8, 8, (1 << 24) + 5, 128,
                                                    ctypes.byref(n)) == OK
    assert xattn(lib, d=96) == UNSUP
    assert xattn(lib, Hq=25) == UNSUP                 # not a multiple of Hkv
    assert xattn(lib, Hq=136) == UNSUP                # 17 query heads per KV head
    assert xattn(lib, dtype=F32) == UNSUP
    assert xattn(lib, scale=float("nan")) == VALUE
    assert xattn(lib, k=ctypes.c_void_p(BASE + 1 * 256 * MB + 8)) == UNSUP
    assert xattn(lib, lens=ctypes.c_void_p(BASE + 7 * 256 * MB + 2)) == UNSUP
    assert xattn(lib, ws=None) == WORKSPACE
    assert xattn(lib, wsb=64) == WORKSPACE
    assert xattn(lib, out=P(1)) == ALIAS              # out on the key cache
    assert xattn(lib, ws=P(2)) == ALIAS               # workspace on the value cache


def proj(lib, x=P(0), wk=P(1), wg=P(2), scale=0.088, tau=16.0, k=P(4), lg=P(5), B=1, N=1000,
         D=3072, H=24, dk=128, dtype=BF16):
    return lib.gret_head_projection(x, wk, wg, ctypes.c_float(scale), ctypes.c_float(tau), k, lg,
                                    B, N, D, H, dk, dtype, None)


def test_head_projection_validation(lib):
    assert proj(lib, x=None) == NULL
    assert proj(lib, k=None) == NULL
    assert proj(lib, lg=None) == NULL                  # gate weights without the output
    assert proj(lib, wg=None) == NULL                  # output without the gate weights
    assert proj(lib, N=0) == SHAPE
    assert proj(lib, D=65536 + 128) == SHAPE
    assert proj(lib, D=3000) == UNSUP                  # not a multiple of 128
    assert proj(lib, dk=72) == UNSUP
    assert proj(lib, dk=272) == UNSUP
    assert proj(lib, H=257, dk=16) == UNSUP            # gate heads beyond one tile
    assert proj(lib, dtype=F32) == UNSUP
    assert proj(lib, tau=0.0) == VALUE
    assert proj(lib, tau=float("inf")) == VALUE
    assert proj(lib, scale=float("nan")) == VALUE
    assert proj(lib, x=ctypes.c_void_p(BASE + 8)) == UNSUP
    assert proj(lib, k=P(0)) == ALIAS                  # keys written over x
    assert proj(lib, lg=P(1)) == ALIAS                 # log-gates over the key weights
    assert proj(lib, lg=ctypes.c_void_p(BASE + 4 * 256 * MB + 1000 * 3072 * 2 - 256)) == ALIAS


def swa_pre(lib, q=P(0), k=P(1), v=P(2), out=P(3), rk=P(4), rv=P(5), B=1, Hq=24, Hkv=8, N=4096,
            d=128, window=1024, scale=0.088, dtype=BF16):
    return lib.gret_swa_prefill(q, k, v, out, rk, rv, B, Hq, Hkv, N, d, window,
                                ctypes.c_float(scale), dtype, None)


def swa_dec(lib, q=P(0), kn=P(1), vn=P(2), rk=P(3), rv=P(4), pos=P(5), out=P(6), B=4, Hq=24,
            Hkv=8, window=1024, d=128, scale=0.088, dtype=BF16, ws=P(7), wsb=1 << 30):
    return lib.gret_swa_decode_step(q, kn, vn, rk, rv, pos, out, B, Hq, Hkv, window, d,
                                    ctypes.c_float(scale), dtype, ws, wsb, None)


def test_swa_validation(lib):
    assert swa_pre(lib, q=None) == NULL
    assert swa_pre(lib, rk=None) == NULL              # one ring without the other
    assert swa_pre(lib, N=0) == SHAPE
    assert swa_pre(lib, window=0) == SHAPE
    assert swa_pre(lib, window=(1 << 23) + 1) == SHAPE
    assert swa_pre(lib, d=96) == UNSUP
    assert swa_pre(lib, Hq=25) == UNSUP
    assert swa_pre(lib, dtype=F32) == UNSUP
    assert swa_pre(lib, scale=float("inf")) == VALUE
    assert swa_pre(lib, q=ctypes.c_void_p(BASE + 8)) == UNSUP
    assert swa_pre(lib, out=P(1)) == ALIAS            # out over the keys
    assert swa_pre(lib, rk=P(2)) == ALIAS             # key ring over the values
    assert swa_pre(lib, rv=P(4)) == ALIAS             # the rings on each other
    n = ctypes.c_size_t(0)
    assert lib.gret_swa_decode_workspace_bytes(4, 24, 8, 1024, 128, ctypes.byref(n)) == OK
    assert n.value % 256 == 0 and n.value >= 256
    assert lib.gret_swa_decode_workspace_bytes(4, 24, 8, 1024, 128, None) == NULL
    assert swa_dec(lib, pos=None) == NULL
    assert swa_dec(lib, window=0) == SHAPE
    assert swa_dec(lib, Hq=8 * 17) == UNSUP           # more than 16 query heads per KV head
    assert swa_dec(lib, pos=ctypes.c_void_p(BASE + 5 * 256 * MB + 2)) == UNSUP
    assert swa_dec(lib, ws=None) == WORKSPACE
    assert swa_dec(lib, wsb=256) == WORKSPACE
    assert swa_dec(lib, out=P(3)) == ALIAS            # out over the key ring
    assert swa_dec(lib, ws=P(4)) == ALIAS             # workspace over the value ring
    assert swa_dec(lib, rk=P(0)) == ALIAS             # key ring over q
    assert swa_dec(lib, scale=float("nan")) == VALUE


def test_launch_size_limits(lib):
    # Shapes whose launches would need more than 2^31 - 1 workgroups, or whose
    # sizes pass 2^50 elements, are rejected before anything is enqueued.
    assert prefill(lib, B=1 << 27, H=1, N=1) == SHAPE          # combine: 16 per head
    assert prefill(lib, B=(1 << 27) - 1, H=1, N=1, ws=None) == WORKSPACE  # the limit itself
    assert decode(lib, B=1 << 27, H=1) == SHAPE
    assert prefill_gated(lib, B=1, H=1 << 20, N=1 << 20) == SHAPE  # epilogue: 2^34 row groups
    assert xattn(lib, B=1 << 28, Hq=4, Hkv=4, L=1) == SHAPE     # combine: B*Hq = 2^30
    assert swa_pre(lib, B=1 << 17, Hq=1, Hkv=1, N=1 << 23, d=64) == SHAPE  # 2^32 query tiles
    assert swa_pre(lib, B=1 << 30, Hq=1 << 10, Hkv=1 << 10, N=1 << 23) == SHAPE  # > 2^50


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(gret, "_lib", None)
    monkeypatch.setattr(gret, "LIB_PATH", "/nonexistent/libgret.so")
    with pytest.raises(RuntimeError, match="not built"):
        gret.load_library()
