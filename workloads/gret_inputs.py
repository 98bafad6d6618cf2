"""Seeded synthetic workloads for gated retention.

Workloads follow the value distributions of the method as described on the page
"YOCO 完全拆解：Decoder-Decoder 架构如何让 KV Cache 只存一次": one scalar gate per
head and position, gamma = sigmoid(u)^(1/16) (section "路线二：Multi-Head Gated
Retention" with the temperature 16 of section "单 token Decode 的实现骨架"), keys
already scaled by d^(-1/2), at the 3B model's mixer width of 24 heads x 128
(section "用 3B 配置手算一遍").

Recipe (one PCG64 stream per (batch, head), seed = the workload's "seed", child i
of SeedSequence(seed) for flattened head i):
  draw order per head: u[N] -> q[N,dk] -> k[N,dk] -> v[N,dv] -> sharp mask[N]
  (only when the workload forces sharp forgetting) -> S0[dk,dv] (only when the
  workload has an initial state) -> decode tokens (u, q, k, v per step).
  Normals are float32 ziggurat draws; q and k are scaled by dk^-0.5 in float32
  (variance 1/dk), v is unit normal; S0 is 0.1 * normal (variance 0.01).
  log_gamma = float32(-softplus(-u) / 16) evaluated in float64, i.e. the log of
  sigmoid(u)^(1/16); sharp positions get float32(ln 0.1).
  bf16 storage uses round-to-nearest-even of the float32 value; arrays hold
  the bf16 bit patterns as uint16.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

LN_SHARP_GAMMA = np.float32(np.log(0.1))

# The workloads, by name. "chunks" lists the chunk sizes exercised; "seed" is
# the root of each workload's seeded streams (one stream per head).
CONFIGS = {
    "tiny_f32": dict(name="tiny_f32_b1h2_n512_d64", B=1, H=2, N=512, dk=64, dv=64, dtype="f32",
                     chunks=(64,), s0_std=0.0, sharp_frac=0.0, decode_steps=16, seed=1001),
    "prefill_32k": dict(name="prefill_b1h24_n32768_d128", B=1, H=24, N=32768, dk=128, dv=128,
                        dtype="bf16", chunks=(64, 128, 256), s0_std=0.0, sharp_frac=0.0,
                        decode_steps=0, seed=1002),
    "prefill_512k": dict(name="prefill_b1h24_n524288_d128_sharp1pct", B=1, H=24, N=524288,
                         dk=128, dv=128, dtype="bf16", chunks=(64, 128, 256), s0_std=0.0,
                         sharp_frac=0.01, decode_steps=0, seed=1003),
    "prefill_1m": dict(name="prefill_b1h24_n1048576_d128_s0", B=1, H=24, N=1048576, dk=128,
                       dv=128, dtype="bf16", chunks=(64, 128, 256), s0_std=0.1, sharp_frac=0.0,
                       decode_steps=0, seed=1004),
    "decode_b256": dict(name="decode_b256h24_d128_1000steps", B=256, H=24, N=0, dk=128, dv=128,
                        dtype="bf16", chunks=(), s0_std=0.1, sharp_frac=0.0, decode_steps=1000,
                        seed=1005),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def _rng(seed: int, head: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(head,))))


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def _log_gamma(u: np.ndarray) -> np.ndarray:
    # log(sigmoid(u)^(1/16)) = -softplus(-u)/16, in float64, stored as float32.
    return (-np.logaddexp(0.0, -u.astype(np.float64)) / 16.0).astype(np.float32)


def gate_log_gamma(u: np.ndarray) -> np.ndarray:
    """The workloads' log-gates from gate logits u drawn elsewhere (for
    inputs drawn on the device): float32(-softplus(-u) / 16)."""
    return _log_gamma(np.asarray(u))


def _draw_token_block(rng, n, dk, dv, dtype):
    u = rng.standard_normal(n, dtype=np.float32)
    q = rng.standard_normal((n, dk), dtype=np.float32)
    q *= np.float32(1.0 / np.sqrt(dk))
    k = rng.standard_normal((n, dk), dtype=np.float32)
    k *= np.float32(1.0 / np.sqrt(dk))
    v = rng.standard_normal((n, dv), dtype=np.float32)
    return _log_gamma(u), _store(q, dtype), _store(k, dtype), _store(v, dtype)


def prefill_head(cfg: dict, head: int, N: int | None = None, dtype: str | None = None,
                 decode_steps: int | None = None):
    """Draw one flattened head's inputs (see the module recipe).

    Returns dict(log_gamma[N], q[N,dk], k[N,dk], v[N,dv], s0[dk,dv] or None,
    dec=list of (log_gamma, q, k, v) single-token tuples).
    """
    N = cfg["N"] if N is None else N
    dtype = cfg["dtype"] if dtype is None else dtype
    steps = cfg["decode_steps"] if decode_steps is None else decode_steps
    dk, dv = cfg["dk"], cfg["dv"]
    rng = _rng(cfg["seed"], head)
    lg, q, k, v = _draw_token_block(rng, N, dk, dv, dtype)
    if cfg["sharp_frac"] > 0.0:
        mask = rng.random(N) < cfg["sharp_frac"]
        lg[mask] = LN_SHARP_GAMMA
    s0 = None
    if cfg["s0_std"] > 0.0:
        s0 = rng.standard_normal((dk, dv), dtype=np.float32) * np.float32(cfg["s0_std"])
    dec = []
    if steps:
        dlg, dq, dk_, dv_ = _draw_token_block(rng, steps, dk, dv, dtype)
        dec = [(dlg[t], dq[t], dk_[t], dv_[t]) for t in range(steps)]
    return dict(log_gamma=lg, q=q, k=k, v=v, s0=s0, dec=dec)


def _workers(n):
    env = os.environ.get("GRET_GEN_THREADS")
    if env:
        return max(1, int(env))
    try:
        cpus = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cpus = os.cpu_count() or 1
    return max(1, min(n, cpus, 16))


def make_prefill_inputs(workload: str, *, N: int | None = None, B: int | None = None,
                        H: int | None = None, dtype: str | None = None,
                        decode_steps: int | None = None, heads=None):
    """Draw a whole prefill workload (optionally at a reduced N / B / H).

    ``heads``: optional iterable of flattened head indices to draw; other heads
    are left zero (used when only a sample of heads is checked).
    Returns dict(q, k, v [B,H,N,d] (uint16 bf16 bits or float32), log_gamma
    [B,H,N] float32, s0 [B,H,dk,dv] float32 or None, dec_* arrays [steps,B,H,...]).
    """
    cfg = CONFIGS[workload]
    B = cfg["B"] if B is None else B
    H = cfg["H"] if H is None else H
    N = cfg["N"] if N is None else N
    dtype = cfg["dtype"] if dtype is None else dtype
    steps = cfg["decode_steps"] if decode_steps is None else decode_steps
    dk, dv = cfg["dk"], cfg["dv"]
    st = np.uint16 if dtype == "bf16" else np.float32
    q = np.zeros((B, H, N, dk), st)
    k = np.zeros((B, H, N, dk), st)
    v = np.zeros((B, H, N, dv), st)
    lg = np.zeros((B, H, N), np.float32)
    s0 = np.zeros((B, H, dk, dv), np.float32) if cfg["s0_std"] > 0.0 else None
    dlg = np.zeros((steps, B, H), np.float32)
    dq = np.zeros((steps, B, H, dk), st)
    dkk = np.zeros((steps, B, H, dk), st)
    dvv = np.zeros((steps, B, H, dv), st)
    todo = list(range(B * H)) if heads is None else sorted(set(int(x) for x in heads))

    def one(x):
        b, h = divmod(x, H)
        d = prefill_head(cfg, x, N=N, dtype=dtype, decode_steps=steps)
        q[b, h], k[b, h], v[b, h], lg[b, h] = d["q"], d["k"], d["v"], d["log_gamma"]
        if s0 is not None:
            s0[b, h] = d["s0"]
        for t, (a, qq, kk, vv) in enumerate(d["dec"]):
            dlg[t, b, h], dq[t, b, h], dkk[t, b, h], dvv[t, b, h] = a, qq, kk, vv

    with ThreadPoolExecutor(_workers(len(todo))) as ex:
        list(ex.map(one, todo))
    return dict(q=q, k=k, v=v, log_gamma=lg, s0=s0, dec_log_gamma=dlg, dec_q=dq, dec_k=dkk,
                dec_v=dvv, B=B, H=H, N=N, dk=dk, dv=dv, dtype=dtype)


# Gates near 1: the temperature on the page keeps gamma close to 1 so that the
# state forgets slowly (section "路线二：Multi-Head Gated Retention"). This
# regime draws the gate logit from N(4, 1): gamma = sigmoid(u)^(1/16) has mean
# about 0.998 and the mean log-gate is about -0.0018.
SLOW_DECAY_SEED = 1013
SLOW_DECAY_LOGIT_MEAN = 4.0


def slow_decay_log_gamma(B: int, H: int, N: int, seed: int = SLOW_DECAY_SEED) -> np.ndarray:
    """log_gamma [B,H,N] float32 with u ~ N(4, 1) per (head, position), one PCG64
    stream per flattened head (child i of SeedSequence(seed)); same mapping
    from u to the log-gate as every other workload."""
    lg = np.empty((B, H, N), np.float32)

    def one(x):
        b, h = divmod(x, H)
        u = _rng(seed, x).standard_normal(N, dtype=np.float32) + np.float32(SLOW_DECAY_LOGIT_MEAN)
        lg[b, h] = _log_gamma(u)

    with ThreadPoolExecutor(_workers(B * H)) as ex:
        list(ex.map(one, range(B * H)))
    return lg


def make_decode_inputs(workload: str = "decode_b256", *, B: int | None = None, H: int | None = None,
                       steps: int | None = None, heads=None):
    """Batched decode workload: initial state [B,H,dk,dv] (std cfg s0_std) and a
    pool of ``steps`` single tokens per (sequence, head).

    Per flattened head stream: S0[dk,dv] first, then u[steps] -> q -> k -> v.
    Returns dict(state [B,H,dk,dv] f32, log_gamma [steps,B,H] f32,
    q,k [steps,B,H,dk], v [steps,B,H,dv] (uint16 bf16 bits or float32)).
    """
    cfg = CONFIGS[workload]
    B = cfg["B"] if B is None else B
    H = cfg["H"] if H is None else H
    steps = cfg["decode_steps"] if steps is None else steps
    dk, dv, dtype = cfg["dk"], cfg["dv"], cfg["dtype"]
    st = np.uint16 if dtype == "bf16" else np.float32
    state = np.zeros((B, H, dk, dv), np.float32)
    lg = np.zeros((steps, B, H), np.float32)
    q = np.zeros((steps, B, H, dk), st)
    k = np.zeros((steps, B, H, dk), st)
    v = np.zeros((steps, B, H, dv), st)
    todo = list(range(B * H)) if heads is None else sorted(set(int(x) for x in heads))

    def one(x):
        b, h = divmod(x, H)
        rng = _rng(cfg["seed"], x)
        state[b, h] = rng.standard_normal((dk, dv), dtype=np.float32) * np.float32(cfg["s0_std"])
        a, qq, kk, vv = _draw_token_block(rng, steps, dk, dv, dtype)
        lg[:, b, h], q[:, b, h], k[:, b, h], v[:, b, h] = a, qq, kk, vv

    with ThreadPoolExecutor(_workers(len(todo))) as ex:
        list(ex.map(one, todo))
    return dict(state=state, log_gamma=lg, q=q, k=k, v=v, B=B, H=H, dk=dk, dv=dv, steps=steps,
                dtype=dtype)


def make_projection_inputs(seed: int, B: int, N: int, D: int, H: int, dk: int,
                           gate: bool = True):
    """Hidden states x [B, N, D] ~ N(0, 1) and linear-layer weights ~ N(0, 1/D)
    (keys [H*dk, D], gate [H, D]), all rounded to bf16 (uint16 bits). With
    these scales every projected value is ~ N(0, 1), the gate logits included."""
    rng = np.random.default_rng(seed)
    s = np.float32(1.0 / np.sqrt(D))
    x = f32_to_bf16_bits(rng.standard_normal((B, N, D), dtype=np.float32))
    wk = f32_to_bf16_bits(rng.standard_normal((H * dk, D), dtype=np.float32) * s)
    wg = f32_to_bf16_bits(rng.standard_normal((H, D), dtype=np.float32) * s) if gate else None
    return x, wk, wg


def make_attention_inputs(seed: int, B: int, Hq: int, Hkv: int, N: int, d: int):
    """Queries [B, Hq, N, d] and keys, values [B, Hkv, N, d], all ~ N(0, 1) and
    rounded to bf16 (uint16 bits): the shapes of a sliding-window layer."""
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, N, d), dtype=np.float32))
    k = f32_to_bf16_bits(rng.standard_normal((B, Hkv, N, d), dtype=np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((B, Hkv, N, d), dtype=np.float32))
    return q, k, v
