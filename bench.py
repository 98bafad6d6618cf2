"""Benchmark: gated-retention prefill (512K positions, 24 heads x 128) and
batched decode on one MI355X, with roofline and CPU-oracle baselines.

One bench step = one chunkwise prefill of the long-prompt workload
(B=1, H=24, N=524288, dk=dv=128, bf16 inputs, fp32 log-gates, 1% of positions
forced to gamma=0.1). The decode workload (256 sequences x 24 heads, fp32
state 384 MiB, 1000 consecutive steps with fresh tokens) is timed after it and
reported in the same JSON line. Inputs are seeded synthetic data already
resident in HBM when timing starts.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--chunk C]
                       [--skip-cpu] [--skip-peaks] [--skip-gated]
                       [--only prefill|decode|xattn|proj|swa]
       python bench.py --calibrate-copy
       python bench.py --summarize-pmc FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR [MFMA_DIR]

HBM traffic: the figures recorded in profiles/gret_prefill_decode_hbm_traffic.json (rocprofv3
FETCH_SIZE / WRITE_SIZE per dispatch, scaled by what the same counters read for
a plain copy of known size) are reported only while the kernel sources hash to
the values recorded with them; otherwise traffic is null. The matrix-core
utilisation recorded there (rocprofv3's MfmaUtil: busy cycles of the MFMA
units over active cycles x SIMDs, per dispatch of the dominant kernel) follows
the same rule.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix
METRIC = "gRet prefill tokens/s @N=512K, 24h×128; decode steps/s; % of roofline"
DEFAULT_CHUNK = 64


CSRC = os.path.join(ROOT, "yoco_gated_retention_amd", "csrc")
# Sources whose change invalidates recorded counter figures, per entry point.
KERNEL_SOURCES = {
    "prefill": ["gret_prefill_c64.hip", "gret_prefill_bf16.hip", "gret_prefill_common.h",
                "gret_api.cpp", "gret_segments.h", "gret_internal.h", "gret_device.h"],
    "decode": ["gret_decode.hip", "gret_internal.h", "gret_device.h"],
    "decode_gated": ["gret_decode.hip", "gret_internal.h", "gret_device.h"],
    "xattn": ["gret_xattn.hip", "gret_internal.h", "gret_device.h"],
    "prefill_gated": ["gret_prefill_c64.hip", "gret_prefill_common.h", "gret_api.cpp",
                      "gret_segments.h", "gret_internal.h", "gret_device.h"],
    "epilogue": ["gret_epilogue.hip", "gret_internal.h", "gret_device.h"],
    "proj": ["gret_proj.hip", "gret_internal.h", "gret_device.h"],
    "swa": ["gret_swa.hip", "gret_internal.h", "gret_device.h"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gret_prefill_decode_hbm_traffic.json")


def sources_sha256(which):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[which]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def recorded_traffic(which):
    """HBM bytes per entry-point call from the committed counter summary, or
    None when it is missing or was taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[which]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_sha256(which):
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def recorded_mfma(which, kernel):
    """rocprofv3 MfmaUtil (percent) of the named kernel of an entry point from
    the committed counter summary, or None (missing, or other sources)."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[which]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_sha256(which):
        return None
    for name, k in rec.get("kernels", {}).items():
        if kernel in name and "mfma_util_pct" in k:
            return k["mfma_util_pct"]
    return None


def short_kernel_name(name):
    name = name.replace("(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    return name.split("(")[0]


def kernel_group(name):
    if "proj_kernel" in name:
        return "proj"
    if "swa_prefill" in name or "swa_ring_fill" in name:
        return "swa"
    if "xattn" in name:
        return "xattn"
    if "output_gate" in name:
        return "epilogue"
    if "decode" in name:
        # the gated instantiation (template flag true; rocprofv3 may leave bf16
        # instantiations mangled, where the flag reads Lb1E)
        return "decode_gated" if ("Lb1E" in name or ", true>" in name) else "decode"
    if "prefill" in name and ("Lb1E" in name or ", true>" in name):
        return "prefill_gated"
    if "prefill" in name or "combine" in name:
        return "prefill"
    return "other:" + name.split("(")[0][:60]


def pmc_per_dispatch(d, counter):
    """Per kernel name: (dispatches, mean counter value per dispatch) from a
    rocprofv3 --pmc csv output directory."""
    acc = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = r["Kernel_Name"]
                n, tot = acc.get(key, (0, 0.0))
                acc[key] = (n + 1, tot + float(r["Counter_Value"]))
    return {k: (n, tot / n) for k, (n, tot) in acc.items()}


def summarize_pmc(fetch_dir, write_dir, cfetch_dir, cwrite_dir, mfma_dir=None):
    """Scales FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by the plain-copy
    calibration and sums them per entry-point call (the prefill is three
    launches: main, combine, prefix). With mfma_dir (a run of MfmaUtil and
    SQ_INSTS_VALU_MFMA_MOPS_BF16), each kernel also gets its matrix-core
    utilisation and the bf16 matrix flops the hardware counted."""
    copy_bytes = 1 << 30  # --calibrate-copy: 1 GiB read and 1 GiB written per copy
    cf = [v for k, (n, v) in pmc_per_dispatch(cfetch_dir, "FETCH_SIZE").items() if "copy" in k]
    cw = [v for k, (n, v) in pmc_per_dispatch(cwrite_dir, "WRITE_SIZE").items() if "copy" in k]
    if not cf or not cw:
        raise SystemExit("no copy kernel found in the calibration runs")
    f_scale = copy_bytes / (max(cf) * 1024.0)
    w_scale = copy_bytes / (max(cw) * 1024.0)
    out = {"calibration": {"copy_bytes": copy_bytes, "fetch_kib": max(cf), "write_kib": max(cw),
                           "fetch_scale": f_scale, "write_scale": w_scale}}
    fetch = pmc_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = pmc_per_dispatch(write_dir, "WRITE_SIZE")
    util = pmc_per_dispatch(mfma_dir, "MfmaUtil") if mfma_dir else {}
    mops = pmc_per_dispatch(mfma_dir, "SQ_INSTS_VALU_MFMA_MOPS_BF16") if mfma_dir else {}
    for which in ("prefill", "prefill_gated", "decode", "decode_gated", "xattn", "epilogue",
                  "proj", "swa"):
        names = sorted(k for k in fetch if kernel_group(k) == which)
        if not names:
            continue
        if which == "prefill_gated":
            # the combine launch is shared by the plain and the gated prefill
            names += sorted(k for k in fetch if "prefill_combine" in k)
        kern = {}
        for k in names:
            kern[short_kernel_name(k)] = {
                "dispatches": fetch[k][0], "fetch_kib": fetch[k][1],
                "write_kib": write.get(k, (0, float("nan")))[1],
                "fetch_bytes": fetch[k][1] * 1024.0 * f_scale,
                "write_bytes": write.get(k, (0, 0.0))[1] * 1024.0 * w_scale}
            if k in util:
                kern[short_kernel_name(k)]["mfma_util_pct"] = util[k][1]
            if k in mops:
                # one MOPS unit is 512 flops
                kern[short_kernel_name(k)]["mfma_bf16_flops"] = mops[k][1] * 512.0
        out[which] = {"sources_sha256": sources_sha256(which), "kernels": kern,
                      "fetch_bytes": sum(x["fetch_bytes"] for x in kern.values()),
                      "write_bytes": sum(x["write_bytes"] for x in kern.values())}
    print(json.dumps(out, indent=1))


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def prefill_algorithmic(B, H, N, dk, dv, chunk, state_in):
    """Bytes that must cross HBM (inputs read once, outputs written once) and
    the flops of the chunkwise form at this chunk size (causal tiles only)."""
    esz = 2
    per_tok = (2 * dk + dv) * esz + dv * esz + 4
    state = B * H * dk * dv * 4 * (2 if state_in else 1)
    nbytes = B * H * N * per_tok + state
    flops = B * H * N * ((chunk + 1) * (dk + dv) + 4 * dk * dv)
    return nbytes, flops


def decode_algorithmic(B, H, dk, dv):
    nbytes = 2 * B * H * dk * dv * 4 + B * H * (2 * dk + 2 * dv) * 2 + 4 * B * H
    flops = 5 * B * H * dk * dv
    return nbytes, flops


def host_cpus():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_threads():
    """Oracle threads: the cores this process may run on, at most 16 (the
    host share of one GPU)."""
    return max(1, min(host_cpus(), 16))


def cpu_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return {"model": model, "logical_cpus": os.cpu_count(), "cpus_available": host_cpus(),
            "oracle_threads": cpu_threads()}


def to_dev(a, dev):
    import torch

    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def time_calls(fn, steps, warmup, warm_s=0.0):
    """Runs fn warmup times (and, with warm_s > 0, keeps calling it until warm_s
    seconds have passed: a short call after an idle stretch, such as a CPU
    leg, otherwise runs on clocks that are still ramping up), synchronises,
    then times `steps` back-to-back calls on the current stream with one HIP
    event before each call and one after the last. Returns (mean ms over the
    block, median ms of the calls, per-call ms)."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if warm_s > 0:
        t0 = time.time()
        while time.time() - t0 < warm_s:
            for _ in range(8):
                fn()
            torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(steps):
        ev[i].record(stream)
        fn()
    ev[steps].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return ev[0].elapsed_time(ev[steps]) / steps, float(np.median(per)), per


class DevicePrefill:
    """One prefill workload resident on the device, with its output, state and
    workspace allocated once (outside any timed region)."""

    def __init__(self, gret, d, dev, log_gamma=None):
        import torch

        self.gret = gret
        self.q, self.k, self.v = to_dev(d["q"], dev), to_dev(d["k"], dev), to_dev(d["v"], dev)
        self.lg = to_dev(d["log_gamma"] if log_gamma is None else log_gamma, dev)
        self.si = None if d.get("s0") is None else to_dev(d["s0"], dev)
        self.B, self.H, self.N, self.dk = d["q"].shape
        self.dv = d["v"].shape[3]
        dt = self.q.dtype
        self.out = torch.empty((self.B, self.H, self.N, self.dv), dtype=dt, device=dev)
        self.so = torch.empty((self.B, self.H, self.dk, self.dv), dtype=torch.float32, device=dev)
        self.code = 1 if dt == torch.bfloat16 else 0
        self.ws = {}

    def set_log_gamma(self, lg, dev):
        self.lg = to_dev(lg, dev)

    def workspace(self, chunk):
        import torch

        if chunk not in self.ws:
            need = self.gret.gret_prefill_workspace_bytes(self.B, self.H, self.N, self.dk, self.dv,
                                                          chunk, self.code)
            self.ws[chunk] = torch.empty(max(need, 1), dtype=torch.uint8, device=self.q.device)
        return self.ws[chunk]

    def call(self, chunk):
        ws = self.workspace(chunk)
        return lambda: self.gret.gret_prefill(self.q, self.k, self.v, self.lg, self.si, chunk=chunk,
                                              out=self.out, state_out=self.so, workspace=ws)

    def time(self, chunk, steps, warmup, warm_s=0.0):
        return time_calls(self.call(chunk), steps, warmup, warm_s)

    def free(self):
        import torch

        self.q = self.k = self.v = self.lg = self.si = self.out = self.so = None
        self.ws = {}
        torch.cuda.empty_cache()


def prefill_roofline(B, H, N, dk, dv, chunk, state_in, ms, kernel, measured_gbs=None,
                     measured_seg_gbs=None):
    nbytes, flops = prefill_algorithmic(B, H, N, dk, dv, chunk, state_in)
    achieved = nbytes / (ms * 1e-3) / 1e9
    r = {"kernel": kernel, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": nbytes,
         "algorithmic_flops_per_launch": flops, "mfma_tflops": flops / (ms * 1e-3) / 1e12,
         "mfma_frac": flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
    if measured_gbs:
        r["peak_measured"] = measured_gbs
        r["frac_measured"] = achieved / measured_gbs
    if measured_seg_gbs:
        r["peak_measured_segmented"] = measured_seg_gbs
        r["frac_measured_segmented"] = achieved / measured_seg_gbs
    return r


def time_prefill_gated(dp, chunk, steps, warmup, dev, seed=3003):
    """Plain and gated prefill on the same resident inputs (gate: seeded normal,
    bf16; affine: seeded, fp32). At chunk 64 the prefill kernels apply the
    output epilogue in their output store (the gate tile streams into LDS
    beside the other tiles); at 128 and 256 an in-place pass rewrites the
    output. The difference of the two call times is the epilogue's cost."""
    import torch

    B, H, N, dk, dv = dp.B, dp.H, dp.N, dp.dk, dp.dv
    g = torch.Generator(device=dev).manual_seed(seed)
    gate = (2.0 * torch.randn((B, H, N, dv), generator=g, device=dev)).to(torch.bfloat16)
    w = 1.0 + 0.2 * torch.randn((H, dv), generator=g, device=dev)
    b = 0.2 * torch.randn((H, dv), generator=g, device=dev)
    ws = dp.workspace(chunk)
    plain = time_calls(dp.call(chunk), steps, warmup)[1]
    gated = time_calls(lambda: dp.gret.gret_prefill_gated(
        dp.q, dp.k, dp.v, dp.lg, gate, state_in=dp.si, norm_weight=w, norm_bias=b, chunk=chunk,
        out=dp.out, state_out=dp.so, workspace=ws), steps, warmup)[1]
    del gate, w, b
    torch.cuda.empty_cache()
    rows = B * H * N
    epi_ms = gated - plain
    res = {"workload": "prefill_gated (same inputs) + per-head GroupNorm + swish gate",
           "ms_per_call": gated, "plain_ms_per_call": plain, "tokens_per_s": B * N / (gated * 1e-3),
           "timing": "median of %d calls each" % steps, "fused": chunk == 64}
    if chunk == 64:
        # the plain prefill's bytes plus the gate rows and the affine
        nbytes = prefill_algorithmic(B, H, N, dk, dv, chunk, dp.si is not None)[0] + \
            rows * dv * 2 + 2 * H * dv * 4
        achieved = nbytes / (gated * 1e-3) / 1e9
        res["epilogue"] = {"ms": epi_ms, "where": "in the prefill kernels' output store"}
        res["roofline"] = {"kernel": "prefill_main_c64_kernel<128,128,true> + combine + prefix",
                           "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                           "algorithmic_bytes_per_launch": nbytes,
                           "traffic": recorded_traffic("prefill_gated")}
        return res
    epi_bytes = rows * dv * 2 * 3 + 2 * H * dv * 4
    achieved = epi_bytes / (epi_ms * 1e-3) / 1e9 if epi_ms > 0 else None
    res["epilogue"] = {"ms": epi_ms, "algorithmic_bytes": epi_bytes,
                       "roofline": {"kernel": "output_gate_kernel (in-place pass)", "bound": "hbm",
                                    "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                    "frac": None if achieved is None else achieved / HBM_PEAK_GBS,
                                    "traffic": recorded_traffic("epilogue")}}
    return res


STREAM_LIB = os.path.join(ROOT, "yoco_gated_retention_amd", "libgret_stream.so")


def bench_stream_ceiling(dp, reps=5, all_variants=None):
    """Measured HBM ceiling for the prefill's access mix: three read streams and
    one write stream of one workload-sized array each (the prefill's own q, k,
    v and output buffers), 16 bytes per lane, swept over the cache policy of
    loads and stores, rows per lane (unroll) and workgroups per CU; the same mix
    in the prefill's own pattern (each CU streams its own contiguous segment,
    loads through LDS); plus the read-only, write-only and copy rates of the
    grid-stride kernels. Median of `reps` runs per variant; the best variant of
    each mix is reported."""
    import ctypes

    import torch

    lib = ctypes.CDLL(STREAM_LIB)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.gret_stream_run.argtypes = [ci, ci, ci, ci, ci, ci, vp, vp, vp, vp, i64, vp]
    lib.gret_stream_run.restype = ci
    lib.gret_stream_segmented_run.argtypes = [ci, ci, ci, ci, vp, vp, vp, vp, i64, vp]
    lib.gret_stream_segmented_run.restype = ci
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nbytes = dp.q.numel() * dp.q.element_size()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    a, b, c, o = ptr(dp.q), ptr(dp.k), ptr(dp.v), ptr(dp.out)
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run(reads, write, nl, ns, u, w):
        def f():
            rc = lib.gret_stream_run(reads, write, nl, ns, u, w * cus, a, b, c, o, nbytes, sp)
            if rc != 0:
                raise RuntimeError("gret_stream_run failed: %d" % rc)
        return time_calls(f, reps, 2)[1]

    def sweep(reads, write, pols, unrolls=(1, 2, 4, 8), per_cu=(1, 2, 4, 8)):
        """Best variant overall and the best rate of each cache-policy pair."""
        moved = nbytes * (reads + (1 if write else 0))
        top, by_pol = None, {}
        table = []
        for (nl, ns) in pols:
            for u in unrolls:
                for w in per_cu:
                    ms = run(reads, write, nl, ns, u, w)
                    gbs = moved / (ms * 1e-3) / 1e9
                    key = "%s_loads+%s_stores" % ("nt" if nl else "default", "nt" if ns else "wb")
                    by_pol[key] = max(by_pol.get(key, 0.0), gbs)
                    table.append([nl, ns, u, w, round(gbs, 1)])
                    if top is None or gbs > top["GB/s"]:
                        top = {"GB/s": gbs, "ms": ms, "nt_load": nl, "nt_store": ns, "unroll": u,
                               "workgroups_per_cu": w}
        if all_variants is not None:
            all_variants.append({"reads": reads, "write": write,
                                 "columns": ["nt_load", "nt_store", "unroll", "wg_per_cu", "GB/s"],
                                 "rows": table})
        return top, by_pol

    res = {"array_bytes": nbytes, "timing": "median of %d runs per variant" % reps,
           "kernel": "stream_kernel (libgret_stream.so): 16 B per lane, grid-stride, persistent"}
    res["read3_write1"], res["read3_write1_by_policy"] = sweep(3, 1, [(1, 0), (0, 1), (0, 0),
                                                                      (1, 1)])
    # the prefill's own pattern: one workgroup per CU streaming its own segment
    # through LDS (one segment per CU, as the prefill's one workgroup per CU)
    seg_rows, seg_top = [], None
    for (nl, ns) in [(1, 0), (1, 1), (0, 0), (0, 1)]:
        for depth in (2, 3, 4, 6):
            def f(depth=depth, nl=nl, ns=ns):
                rc = lib.gret_stream_segmented_run(depth, nl, ns, cus, a, b, c, o, nbytes, sp)
                if rc != 0:
                    raise RuntimeError("gret_stream_segmented_run failed: %d" % rc)
            ms = time_calls(f, reps, 2)[1]
            gbs = 4 * nbytes / (ms * 1e-3) / 1e9
            seg_rows.append([nl, ns, depth, round(gbs, 1)])
            if seg_top is None or gbs > seg_top["GB/s"]:
                seg_top = {"GB/s": gbs, "ms": ms, "nt_load": nl, "nt_store": ns, "depth": depth,
                           "workgroups": cus}
    res["read3_write1_segmented"] = seg_top
    if all_variants is not None:
        all_variants.append({"reads": 3, "write": 1, "segmented": True,
                             "columns": ["nt_load", "nt_store", "depth", "GB/s"], "rows": seg_rows})
    res["read3"] = sweep(3, 0, [(1, 0), (0, 0)])[0]
    res["copy"] = sweep(1, 1, [(1, 0), (0, 1), (0, 0), (1, 1)])[0]
    res["write"] = sweep(0, 1, [(0, 0), (0, 1)], unrolls=(4,))[0]
    return res


def bench_gemm_peak(dev, n=8192, reps=10):
    """Measured matrix-core rate: torch's library bf16 GEMM of n x n x n."""
    import torch

    g = torch.Generator(device=dev).manual_seed(1)
    a = torch.randn((n, n), generator=g, device=dev).to(torch.bfloat16)
    b = torch.randn((n, n), generator=g, device=dev).to(torch.bfloat16)
    c = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
    ms = time_calls(lambda: torch.matmul(a, b, out=c), reps, 3)[1]
    del a, b, c
    torch.cuda.empty_cache()
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    return {"TFLOP/s": tf, "ms": ms, "shape": "%dx%dx%d bf16 (torch.matmul)" % (n, n, n),
            "frac_of_spec": tf / BF16_PEAK_TFLOPS}


def bench_decode_gated(gret, dev, d, reps=1, seed=4004):
    """1000 gated decode steps (epilogue fused into the step) on the decode
    workload, fresh seeded gate values per step."""
    import torch

    B, H, dk, dv = d["B"], d["H"], d["dk"], d["dv"]
    steps = d["q"].shape[0]
    state = to_dev(d["state"], dev)
    q, k, v, lg = (to_dev(d[x], dev) for x in ("q", "k", "v", "log_gamma"))
    g = torch.Generator(device=dev).manual_seed(seed)
    gate = (2.0 * torch.randn((steps, B, H, dv), generator=g, device=dev)).to(torch.bfloat16)
    w = 1.0 + 0.2 * torch.randn((H, dv), generator=g, device=dev)
    b = 0.2 * torch.randn((H, dv), generator=g, device=dev)
    out = torch.empty((B, H, dv), dtype=torch.bfloat16, device=dev)

    def run():
        for t in range(steps):
            gret.gret_decode_step_gated(q[t], k[t], v[t], lg[t], state, gate[t], norm_weight=w,
                                        norm_bias=b, out=out)

    run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / (reps * steps)
    nbytes = decode_algorithmic(B, H, dk, dv)[0] + B * H * dv * 2 + 2 * H * dv * 4
    achieved = nbytes / (us * 1e-6) / 1e9
    del state, q, k, v, lg, gate, out
    torch.cuda.empty_cache()
    return {"workload": "decode_gated_b256h24_d128_1000steps", "steps_per_s": 1e6 / us,
            "us_per_step": us,
            "roofline": {"kernel": "decode_step_kernel (gated)", "bound": "hbm",
                         "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS,
                         "traffic": recorded_traffic("decode_gated"),
                         "algorithmic_bytes_per_launch": nbytes}}


def bench_cross_attention(gret, dev, B, L, reps=20, Hq=24, Hkv=8, d=128, seed=5005,
                          cpu_seconds=0.0):
    """Cross-Decoder decode attention over a global KV cache of L positions per
    sequence (seeded normal q, K, V in bf16; all positions valid)."""
    import torch

    g = torch.Generator(device=dev).manual_seed(seed)
    q = torch.randn((B, Hq, d), generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn((B, Hkv, L, d), generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn((B, Hkv, L, d), generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(gret.gret_cross_attention_workspace_bytes(B, Hq, Hkv, L, d),
                     dtype=torch.uint8, device=dev)

    def call():
        gret.gret_cross_attention_decode(q, k, v, None, None, out=out, workspace=ws)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / reps
    nbytes = B * Hkv * L * d * 2 * 2 + 2 * B * Hq * d * 2
    achieved = nbytes / (us * 1e-6) / 1e9
    res = {"workload": "cross_attention_decode_b%d_l%d_hq%d_hkv%d_d%d" % (B, L, Hq, Hkv, d),
           "calls_per_s": 1e6 / us, "us_per_call": us,
           "roofline": {"kernel": "xattn_split_kernel + xattn_combine_kernel", "bound": "hbm",
                        "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": achieved / HBM_PEAK_GBS, "traffic": recorded_traffic("xattn"),
                        "algorithmic_bytes_per_launch": nbytes}}
    if cpu_seconds > 0:
        import oracle

        # the oracle on one sequence's share (host copies of the bf16 bits)
        qh = q[:1].view(torch.int16).cpu().numpy().view(np.uint16)
        n_cpu = min(L, 65536)
        kh = k[:1, :, :n_cpu].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        vh = v[:1, :, :n_cpu].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.time()
        reps_cpu = 0
        while time.time() - t0 < cpu_seconds:
            oracle.oracle_cross_attention_f64(qh, kh, vh)
            reps_cpu += 1
        dt = time.time() - t0
        res["cpu_baseline"] = {"value": reps_cpu * n_cpu / dt, "unit": "cached positions/s",
                               "cores": 1, "kind": "oracle",
                               "sample": "one sequence, all 24 query heads, first %d positions, "
                                         "%d calls in %.1f s" % (n_cpu, reps_cpu, dt)}
    del q, k, v, out, ws
    torch.cuda.empty_cache()
    return res


def bench_projection(gret, dev, B=1, N=524288, D=3072, H=24, dk=128, reps=10, seed=7007,
                     cpu_seconds=0.0):
    """Key and log-gate projection of the prefill workload's tokens (hidden size
    3072, 24 heads of 128, gate): x ~ N(0, 1), weights ~ N(0, 1/D), bf16, drawn
    on the device by a seeded generator. Also times torch's library GEMM on the
    same product (token-major output, no scaling, no log-gate, no head-major
    layout) as context."""
    import torch

    g = torch.Generator(device=dev).manual_seed(seed)
    x = torch.randn((B, N, D), generator=g, device=dev).to(torch.bfloat16)
    wk = (torch.randn((H * dk, D), generator=g, device=dev) * D ** -0.5).to(torch.bfloat16)
    wg = (torch.randn((H, D), generator=g, device=dev) * D ** -0.5).to(torch.bfloat16)
    k = torch.empty((B, H, N, dk), dtype=torch.bfloat16, device=dev)
    lg = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def timed(f):
        for _ in range(2):
            f()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms = timed(lambda: gret.gret_head_projection(x, wk, wg, key_scale=dk ** -0.5,
                                                 temperature=16.0, k_out=k, log_gamma=lg))
    wcat = torch.cat([wk, wg], 0)
    x2 = x.view(B * N, D)
    lib_ms = timed(lambda: torch.matmul(x2, wcat.t()))
    flops = 2 * B * N * D * (H * dk + H)
    nbytes = B * N * D * 2 + (H * dk + H) * D * 2 + B * N * H * (dk * 2 + 4)
    tf = flops / (ms * 1e-3) / 1e12
    res = {"workload": "key_gate_projection_b%d_n%d_d%d_h%d_dk%d" % (B, N, D, H, dk),
           "ms_per_call": ms, "tokens_per_s": B * N / (ms * 1e-3),
           "library_gemm_ms": lib_ms,
           "roofline": {"kernel": "proj_kernel", "bound": "mfma", "achieved": tf,
                        "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": tf / BF16_PEAK_TFLOPS, "traffic": recorded_traffic("proj"),
                        "mfma_busy_pct": recorded_mfma("proj", "proj_kernel"),
                        "algorithmic_flops_per_launch": flops,
                        "algorithmic_bytes_per_launch": nbytes}}
    if cpu_seconds > 0:
        import oracle
        from threadpoolctl import threadpool_limits

        threads = cpu_threads()
        n_cpu = 512
        xh = x[:, :n_cpu].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        wkh = wk.view(torch.int16).cpu().numpy().view(np.uint16)
        wgh = wg.view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.time()
        calls = 0
        with threadpool_limits(threads):
            while time.time() - t0 < cpu_seconds:
                oracle.oracle_head_projection_f64(xh, wkh, wgh, key_scale=dk ** -0.5,
                                                  temperature=16.0)
                calls += 1
        dt = time.time() - t0
        res["cpu_baseline"] = {"value": calls * n_cpu / dt, "unit": "tokens/s", "cores": threads,
                               "kind": "oracle",
                               "sample": "first %d tokens, all 24 heads and the gate, %d calls "
                                         "in %.1f s (fp64)" % (n_cpu, calls, dt)}
    del x, wk, wg, k, lg, wcat
    torch.cuda.empty_cache()
    return res


def bench_swa(gret, dev, B=1, H=24, N=524288, d=128, W=1024, Bd=256, reps=10, seed=9009,
              cpu_seconds=0.0, decode=True):
    """Sliding-window-attention Self-Decoder: prefill of the prefill workload's
    shape (24 heads of 128, window 1024, q, k, v ~ N(0, 1) bf16 drawn on the
    device) with the ring fill, and decode steps of 256 sequences over full
    rings of 1024 positions."""
    import torch

    g = torch.Generator(device=dev).manual_seed(seed)
    q = torch.randn((B, H, N, d), generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn((B, H, N, d), generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn((B, H, N, d), generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty_like(q)
    rk = torch.empty((B, H, W, d), dtype=torch.bfloat16, device=dev)
    rv = torch.empty_like(rk)
    stream = torch.cuda.current_stream()

    def timed(f, n):
        for _ in range(2):
            f()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms = timed(lambda: gret.gret_swa_prefill(q, k, v, W, out=out, k_ring=rk, v_ring=rv), reps)
    keys = B * H * (W * (W + 1) // 2 + (N - W) * W)  # (query, key) pairs inside the windows
    flops = 4 * d * keys
    tf = flops / (ms * 1e-3) / 1e12
    res = {"prefill": {"workload": "swa_prefill_b%d_h%d_n%d_d%d_w%d" % (B, H, N, d, W),
                       "ms_per_call": ms, "tokens_per_s": B * N / (ms * 1e-3),
                       "roofline": {"kernel": "swa_prefill_kernel + swa_ring_fill_kernel",
                                    "bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS,
                                    "unit": "TFLOP/s", "frac": tf / BF16_PEAK_TFLOPS,
                                    "traffic": recorded_traffic("swa"),
                                    "mfma_busy_pct": recorded_mfma("swa", "swa_prefill_kernel"),
                                    "algorithmic_flops_per_launch": flops,
                                    "algorithmic_bytes_per_launch": 4 * B * H * N * d * 2}}}
    if cpu_seconds > 0:
        import oracle

        n_cpu = 2048
        qh = q[:1, :1, :n_cpu].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        kh = k[:1, :1, :n_cpu].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        vh = v[:1, :1, :n_cpu].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.time()
        calls = 0
        while time.time() - t0 < cpu_seconds:
            oracle.oracle_swa_prefill_f64(qh, kh, vh, W)
            calls += 1
        dt = time.time() - t0
        res["prefill"]["cpu_baseline"] = {
            "value": calls * n_cpu / dt, "unit": "token-heads/s", "cores": cpu_threads(),
            "kind": "oracle",
            "sample": "one head, first %d positions, %d calls in %.1f s (fp64)" % (n_cpu, calls, dt)}
    del q, k, v, out, rk, rv
    torch.cuda.empty_cache()
    if not decode:
        return res

    rk = torch.randn((Bd, H, W, d), generator=g, device=dev).to(torch.bfloat16)
    rv = torch.randn((Bd, H, W, d), generator=g, device=dev).to(torch.bfloat16)
    qd = torch.randn((Bd, H, d), generator=g, device=dev).to(torch.bfloat16)
    kn = torch.randn((Bd, H, d), generator=g, device=dev).to(torch.bfloat16)
    vn = torch.randn((Bd, H, d), generator=g, device=dev).to(torch.bfloat16)
    pos = torch.full((Bd,), 4 * W + 7, dtype=torch.int32, device=dev)
    od = torch.empty_like(qd)
    ws = torch.empty(gret.gret_swa_decode_workspace_bytes(Bd, H, H, W, d), dtype=torch.uint8,
                     device=dev)
    us = 1000.0 * timed(lambda: gret.gret_swa_decode_step(qd, kn, vn, rk, rv, pos, out=od,
                                                          workspace=ws), 50)
    nbytes = 2 * Bd * H * W * d * 2 + 2 * Bd * H * d * 2 * 2
    achieved = nbytes / (us * 1e-6) / 1e9
    res["decode"] = {"workload": "swa_decode_b%d_h%d_d%d_w%d" % (Bd, H, d, W),
                     "us_per_step": us, "steps_per_s": 1e6 / us,
                     "roofline": {"kernel": "swa_append_kernel + xattn_split_kernel (one range "
                                            "per ring here, so no xattn_combine_kernel launch)",
                                  "bound": "hbm",
                                  "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                                  "algorithmic_bytes_per_launch": nbytes}}
    del rk, rv, qd, kn, vn, od, ws
    torch.cuda.empty_cache()
    return res


def bench_decode(gret, dev, steps_total, reps, warmup_reps):
    import torch

    from workloads import make_decode_inputs

    t0 = time.time()
    d = make_decode_inputs("decode_b256", steps=steps_total)
    log("decode inputs generated in %.1f s" % (time.time() - t0))
    B, H, dk, dv = d["B"], d["H"], d["dk"], d["dv"]
    state = to_dev(d["state"], dev)
    q, k, v, lg = (to_dev(d[x], dev) for x in ("q", "k", "v", "log_gamma"))
    out = torch.empty((B, H, dv), dtype=torch.bfloat16, device=dev)

    def run():
        for t in range(steps_total):
            gret.gret_decode_step(q[t], k[t], v[t], lg[t], state, out=out)

    for _ in range(warmup_reps):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    us_per_step = e0.elapsed_time(e1) * 1000.0 / (reps * steps_total)
    nbytes, flops = decode_algorithmic(B, H, dk, dv)
    achieved = nbytes / (us_per_step * 1e-6) / 1e9
    res = {
        "workload": "decode_b256h24_d128_1000steps",
        "steps_per_s": 1e6 / us_per_step,
        "us_per_step": us_per_step,
        "timed_steps": reps * steps_total,
        "roofline": {"kernel": "decode_step_kernel", "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": recorded_traffic("decode"),
                     "algorithmic_bytes_per_launch": nbytes},
    }
    del state, q, k, v, lg, out
    torch.cuda.empty_cache()
    return res, d


def cpu_prefill_baseline(d, budget_s, threads=None, piece=65536, label=None):
    """The oracle's fp64 recurrence over all heads of a prefill workload, on
    consecutive pieces of `piece` positions (state carried between them), until
    about budget_s seconds have passed; a workload finished early is started
    again. The oracle computes every output row; only keeping them (an fp64 copy
    of the whole output) is left out."""
    import oracle

    threads = cpu_threads() if threads is None else threads
    B, H, N = d["q"].shape[:3]
    s0 = d.get("s0")
    state = s0
    pos, done, dt = 0, 0, 0.0
    while dt < budget_s:
        sl = {x: np.ascontiguousarray(d[x][:, :, pos:pos + piece])
              for x in ("q", "k", "v", "log_gamma")}
        t0 = time.time()
        _, state, _ = oracle.oracle_prefill_f64(sl["q"], sl["k"], sl["v"], sl["log_gamma"],
                                                state_in=state, want_out=False, nthreads=threads)
        dt += time.time() - t0
        n = sl["q"].shape[2]
        done += n
        pos += n
        if pos >= N:
            pos, state = 0, s0
    return {"value": B * done / dt, "unit": "tokens/s", "cores": min(threads, B * H),
            "kind": "oracle",
            "sample": "%s: %d positions of all %d heads (fp64 recurrence in pieces of %d; every "
                      "output computed, not kept, %.1f s on %d thread%s)" % (
                          label or "prefill", done, B * H, piece, dt, threads,
                          "" if threads == 1 else "s")}


def cpu_decode_baseline(d, budget_s):
    """The oracle's fp64 decode step on all heads, consecutive steps of the
    decode workload until about budget_s seconds have passed."""
    import oracle

    threads = cpu_threads()
    s = d["state"].astype(np.float64)
    steps = d["q"].shape[0]
    n, dt = 0, 0.0
    while n < steps and dt < budget_s:
        t0 = time.time()
        oracle.oracle_decode_f64(d["q"][n], d["k"][n], d["v"][n], d["log_gamma"][n], s,
                                 nthreads=threads)
        dt += time.time() - t0
        n += 1
    B, H = d["B"], d["H"]
    return {"value": n / dt, "unit": "steps/s", "cores": min(threads, B * H), "kind": "oracle",
            "sample": "first %d of the %d steps, all %dx%d heads (fp64, %.1f s)" % (
                n, steps, B, H, dt)}


def bench_prefill_legs(gret, dev, args):
    """Every prefill leg: the headline workload (512K positions x 24 heads) with
    its roofline against the spec and the measured stream ceiling, the same
    workload with gates near 1, the chunk sweeps, the 1M workload with an
    initial state, the fp32 tiny workload, the gated (epilogue) prefill, the
    measured peaks and the CPU-oracle baselines."""
    import torch

    from workloads import CONFIGS, make_prefill_inputs, slow_decay_log_gamma

    res = {}
    chunk = args.chunk
    kern = "gret_prefill (main + combine + prefix launches)"
    cfg = CONFIGS["prefill_512k"]
    t0 = time.time()
    d3 = make_prefill_inputs("prefill_512k")
    log("prefill inputs generated in %.1f s" % (time.time() - t0))
    B, H, N, dk, dv = 1, cfg["H"], cfg["N"], cfg["dk"], cfg["dv"]
    dp = DevicePrefill(gret, d3, dev)
    ms, med, per = dp.time(chunk, args.steps, args.warmup)
    peaks = {}
    if not args.skip_peaks:
        peaks["hbm_stream"] = bench_stream_ceiling(dp)
        log("stream ceiling 3 reads + 1 write: %.0f GB/s (%s); segmented, through LDS: %.0f GB/s"
            % (peaks["hbm_stream"]["read3_write1"]["GB/s"],
               json.dumps(peaks["hbm_stream"]["read3_write1_by_policy"]),
               peaks["hbm_stream"]["read3_write1_segmented"]["GB/s"]))
        peaks["bf16_gemm"] = bench_gemm_peak(dev)
        log("bf16 GEMM: %.0f TFLOP/s" % peaks["bf16_gemm"]["TFLOP/s"])
    meas = peaks["hbm_stream"]["read3_write1"]["GB/s"] if peaks else None
    meas_seg = peaks["hbm_stream"]["read3_write1_segmented"]["GB/s"] if peaks else None
    roof = prefill_roofline(B, H, N, dk, dv, chunk, False, ms, kern, meas, meas_seg)
    roof["traffic"] = recorded_traffic("prefill")
    roof["mfma_busy_pct"] = recorded_mfma("prefill", "prefill_main_c64_kernel")
    if peaks:
        roof["mfma_peak_measured"] = peaks["bf16_gemm"]["TFLOP/s"]
        roof["mfma_frac_measured"] = roof["mfma_tflops"] / peaks["bf16_gemm"]["TFLOP/s"]
    res.update({
        "value": B * N / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
        "ms_median": med, "ms_min": min(per), "ms_max": max(per),
        "config": {"workload": cfg["name"], "B": B, "H": H, "N": N, "dk": dk, "dv": dv,
                   "chunk": chunk, "log_gamma": "fp32", "state": "fp32", "inputs": "bf16"},
        "roofline": roof, "measured_peaks": peaks or None})
    log("prefill chunk=%d: %.3f ms/step (median %.3f), %.3e tokens/s, %.0f GB/s (%.1f%% of HBM "
        "peak%s)" % (chunk, ms, med, res["value"], roof["achieved"], 100 * roof["frac"],
                     "" if not meas else ", %.1f%% / %.1f%% of the measured grid-stride / "
                     "segmented stream ceilings" % (100 * roof["frac_measured"],
                                                    100 * roof["frac_measured_segmented"])))

    n_rep = max(10, args.steps // 2)
    if args.headline:
        if not args.skip_gated:
            res["prefill_gated"] = time_prefill_gated(dp, chunk, n_rep, 2, dev)
        dp.free()
        return res

    # gates near 1 (u ~ N(4, 1)), same q, k, v
    dp.set_log_gamma(slow_decay_log_gamma(B, H, N), dev)
    _, med_slow, _ = dp.time(chunk, n_rep, 2)
    res["prefill_slow_decay"] = {
        "workload": cfg["name"] + "_gate_logit_n4_1",
        "log_gamma": "u ~ N(4, 1), mean log-gate -0.0018 (gamma ~ 0.998), no sharp positions",
        "ms_median": med_slow, "tokens_per_s": B * N / (med_slow * 1e-3),
        "ratio_to_standard_median": med_slow / med,
        "roofline": prefill_roofline(B, H, N, dk, dv, chunk, False, med_slow, kern, meas,
                                     meas_seg),
        "timing": "median of %d calls" % n_rep}
    log("prefill, gates near 1: %.3f ms (%.2fx the standard regime)" % (med_slow, med_slow / med))
    dp.set_log_gamma(d3["log_gamma"], dev)

    # chunk sizes at 512K
    sweep = []
    for ch in (64, 128, 256):
        _, m, _ = dp.time(ch, n_rep, 2)
        sweep.append({"chunk": ch, "ms_median": m, "tokens_per_s": B * N / (m * 1e-3),
                      "roofline": prefill_roofline(B, H, N, dk, dv, ch, False, m, kern, meas,
                                                    meas_seg)})
        if ch != chunk:
            dp.ws.pop(ch, None)  # keep one workspace resident at a time
    res["prefill_512k_chunk_sweep"] = sweep
    log("512K chunk sweep (ms): %s" % ", ".join("%d: %.3f" % (x["chunk"], x["ms_median"])
                                                 for x in sweep))
    if not args.skip_gated:
        gp = time_prefill_gated(dp, chunk, n_rep, 2, dev)
        res["prefill_gated"] = gp
        log("prefill gated: %.3f ms/call (plain %.3f; epilogue %.3f ms)" % (
            gp["ms_per_call"], gp["plain_ms_per_call"], gp["epilogue"]["ms"]))
    dp.free()
    del dp
    if not args.skip_cpu:
        res["cpu_baseline"] = cpu_prefill_baseline(d3, args.cpu_seconds, label=cfg["name"])
        log("cpu baseline: %s" % json.dumps(res["cpu_baseline"]))
    del d3

    # configuration 2: 32K positions, chunk sizes 64 / 128 / 256
    c2 = CONFIGS["prefill_32k"]
    d2 = make_prefill_inputs("prefill_32k")
    dp2 = DevicePrefill(gret, d2, dev)
    sw2 = []
    for ch in (64, 128, 256):
        _, m, _ = dp2.time(ch, 20, 3, warm_s=0.25)
        sw2.append({"chunk": ch, "ms_median": m, "tokens_per_s": c2["N"] / (m * 1e-3),
                    "roofline": prefill_roofline(1, c2["H"], c2["N"], c2["dk"], c2["dv"], ch,
                                                 False, m, kern, meas, meas_seg)})
    dp2.free()
    res["prefill_32k_chunk_sweep"] = {"workload": c2["name"],
                                      "timing": "median of 20 calls after 0.25 s of warm-up calls",
                                      "chunks": sw2}
    log("32K chunk sweep (ms): %s" % ", ".join("%d: %.4f" % (x["chunk"], x["ms_median"])
                                                for x in sw2))
    if not args.skip_cpu:
        res["prefill_32k_chunk_sweep"]["cpu_baseline_1thread"] = cpu_prefill_baseline(
            d2, args.cpu_seconds, threads=1, piece=2048, label=c2["name"])
    del d2

    # configuration 4: 1M positions, nonzero initial state
    c4 = CONFIGS["prefill_1m"]
    t0 = time.time()
    d4 = make_prefill_inputs("prefill_1m")
    log("1M inputs generated in %.1f s" % (time.time() - t0))
    dp4 = DevicePrefill(gret, d4, dev)
    _, m4, per4 = dp4.time(chunk, 10, 2)
    dp4.free()
    del dp4, d4
    res["prefill_1m"] = {"workload": c4["name"], "chunk": chunk, "ms_median": m4,
                         "ms_min": min(per4), "tokens_per_s": c4["N"] / (m4 * 1e-3),
                         "timing": "median of 10 calls",
                         "roofline": prefill_roofline(1, c4["H"], c4["N"], c4["dk"], c4["dv"],
                                                      chunk, True, m4, kern, meas, meas_seg)}
    log("1M prefill: %.3f ms (%.1f%% of HBM peak)" % (
        m4, 100 * res["prefill_1m"]["roofline"]["frac"]))

    # configuration 1: fp32, 2 heads x 512, then 16 decode steps
    res["tiny_f32"] = bench_tiny_f32(gret, dev, args)
    torch.cuda.empty_cache()
    return res


def bench_tiny_f32(gret, dev, args):
    """The fp32 tier: prefill of 2 heads x 512 (chunk 64) and the 16 decode steps
    that follow, on the GPU; the oracle on one host thread beside it."""
    import torch

    import oracle
    from workloads import CONFIGS, make_prefill_inputs

    c1 = CONFIGS["tiny_f32"]
    d = make_prefill_inputs("tiny_f32")
    dp = DevicePrefill(gret, d, dev)
    _, m, _ = dp.time(64, 20, 3, warm_s=0.25)
    steps = c1["decode_steps"]
    toks = [[to_dev(d[x][t], dev) for x in ("dec_q", "dec_k", "dec_v", "dec_log_gamma")]
            for t in range(steps)]
    state = dp.so.clone()
    out = torch.empty((1, c1["H"], c1["dv"]), dtype=torch.float32, device=dev)

    def decode_all():
        for t in range(steps):
            gret.gret_decode_step(*toks[t], state, out=out)

    _, md, _ = time_calls(decode_all, 10, 2, warm_s=0.25)
    dp.free()
    res = {"workload": c1["name"], "prefill_ms_median": m, "tokens_per_s": c1["N"] / (m * 1e-3),
           "decode_us_per_step": 1000.0 * md / steps, "timing": "median of 20 prefills; median "
           "of 10 runs of the 16 decode steps (each after 0.25 s of warm-up calls)"}
    if not args.skip_cpu:
        t0, n = time.time(), 0
        while time.time() - t0 < 2.0:
            _, s, _ = oracle.oracle_prefill_f64(d["q"], d["k"], d["v"], d["log_gamma"],
                                                want_out=False, nthreads=1)
            for t in range(steps):
                oracle.oracle_decode_f64(d["dec_q"][t], d["dec_k"][t], d["dec_v"][t],
                                         d["dec_log_gamma"][t], s, nthreads=1)
            n += 1
        dt = time.time() - t0
        res["cpu_baseline_1thread"] = {
            "value": n * c1["N"] / dt, "unit": "tokens/s (prefill + 16 decode steps)",
            "cores": 1, "kind": "oracle",
            "sample": "the whole workload %d times in %.1f s" % (n, dt)}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--chunk", type=int, default=DEFAULT_CHUNK)
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "xattn", "proj", "swa", "stream"],
                    default=None)
    ap.add_argument("--decode-reps", type=int, default=1)
    ap.add_argument("--headline", action="store_true",
                    help="prefill: only the 512K workload at --chunk (and its gated form), so that "
                         "per-kernel profiler averages cover that one workload")
    ap.add_argument("--skip-peaks", action="store_true",
                    help="skip the measured HBM stream ceiling and the library GEMM rate")
    ap.add_argument("--no-swa-decode", action="store_true",
                    help="skip the sliding-window decode timing (it runs on the cross-attention "
                         "kernels, whose counter runs should see only the cross-attention calls)")
    ap.add_argument("--skip-gated", action="store_true",
                    help="skip the gated (output epilogue) prefill and decode timings")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of each CPU-oracle baseline")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR", default=None,
                    help="print HBM traffic per call from rocprofv3 --pmc output directories "
                         "(FETCH_SIZE run, WRITE_SIZE run, the two --calibrate-copy runs, and "
                         "optionally a MfmaUtil + SQ_INSTS_VALU_MFMA_MOPS_BF16 run)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 1 GiB (x3) to calibrate the HBM "
                         "traffic counters")
    args = ap.parse_args()
    if args.summarize_pmc:
        if len(args.summarize_pmc) not in (4, 5):
            ap.error("--summarize-pmc takes 4 or 5 directories")
        summarize_pmc(*args.summarize_pmc)
        return
    if args.calibrate_copy:
        import torch

        src = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": src.numel() * 2,
                          "calibrate_copy_bytes_written": dst.numel() * 2, "copies": 3}))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (heads and "
              "sequences shard across GPUs without communication, each GPU running these "
              "kernels on its share). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import yoco_gated_retention_amd as gret
    from workloads import CONFIGS, make_prefill_inputs

    gret.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic (seeded; value distributions of the pages' gRet gate)"}

    result["host_cpu"] = cpu_info()
    if args.only == "stream":
        # the stream ceiling alone, every variant, on arrays of the 512K workload's size
        import types

        n = CONFIGS["prefill_512k"]["N"] * CONFIGS["prefill_512k"]["H"] * 128
        arr = types.SimpleNamespace(**{x: torch.empty(n, dtype=torch.bfloat16, device=dev)
                                       for x in ("q", "k", "v", "out")})
        table = []
        st = bench_stream_ceiling(arr, all_variants=table)
        st["variants"] = table
        result.update({"value": st["read3_write1"]["GB/s"], "unit": "GB/s",
                       "config": {"workload": "stream_3read_1write_%d_bytes" % st["array_bytes"]},
                       "measured_peaks": {"hbm_stream": st}})
    if args.only in (None, "prefill"):
        result.update(bench_prefill_legs(gret, dev, args))

    if args.only in (None, "xattn"):
        xa = [bench_cross_attention(gret, dev, 1, 524288,
                                    cpu_seconds=0.0 if args.skip_cpu else 3.0),
              bench_cross_attention(gret, dev, 16, 32768)]
        result["cross_attention"] = xa
        for x in xa:
            log("cross attention %s: %.1f us/call, %.0f GB/s (%.1f%%)" % (
                x["workload"], x["us_per_call"], x["roofline"]["achieved"],
                100 * x["roofline"]["frac"]))
        if args.only == "xattn":
            result.update({"value": xa[0]["calls_per_s"], "unit": "calls/s",
                           "ms_per_step": xa[0]["us_per_call"] / 1000.0,
                           "config": {"workload": xa[0]["workload"]},
                           "roofline": xa[0]["roofline"]})
    if args.only in (None, "proj"):
        pj = bench_projection(gret, dev, cpu_seconds=0.0 if args.skip_cpu else 3.0)
        result["projection"] = pj
        log("key/gate projection: %.3f ms/call, %.0f TFLOP/s (%.1f%% of bf16 peak); library "
            "GEMM without the epilogue %.3f ms" % (pj["ms_per_call"], pj["roofline"]["achieved"],
                                                    100 * pj["roofline"]["frac"],
                                                    pj["library_gemm_ms"]))
        if args.only == "proj":
            result.update({"value": pj["tokens_per_s"], "unit": "tokens/s",
                           "ms_per_step": pj["ms_per_call"],
                           "config": {"workload": pj["workload"]}, "roofline": pj["roofline"]})
    if args.only in (None, "swa"):
        sw = bench_swa(gret, dev, cpu_seconds=0.0 if args.skip_cpu else 3.0,
                       decode=not args.no_swa_decode)
        result["swa"] = sw
        log("swa prefill: %.3f ms/call, %.0f TFLOP/s (%.1f%% of bf16 peak)" % (
            sw["prefill"]["ms_per_call"], sw["prefill"]["roofline"]["achieved"],
            100 * sw["prefill"]["roofline"]["frac"]))
        if "decode" in sw:
            log("swa decode: %.1f us/step, %.0f GB/s (%.1f%%)" % (
                sw["decode"]["us_per_step"], sw["decode"]["roofline"]["achieved"],
                100 * sw["decode"]["roofline"]["frac"]))
        if args.only == "swa":
            result.update({"value": sw["prefill"]["tokens_per_s"], "unit": "tokens/s",
                           "ms_per_step": sw["prefill"]["ms_per_call"],
                           "config": {"workload": sw["prefill"]["workload"]},
                           "roofline": sw["prefill"]["roofline"]})
    if args.only in (None, "decode"):
        dec, dd = bench_decode(gret, dev, CONFIGS["decode_b256"]["decode_steps"], args.decode_reps, 1)
        if not args.skip_cpu:
            dec["cpu_baseline"] = cpu_decode_baseline(dd, args.cpu_seconds)
        result["decode"] = dec
        log("decode: %.2f us/step, %.0f steps/s, %.0f GB/s (%.1f%%)" % (
            dec["us_per_step"], dec["steps_per_s"], dec["roofline"]["achieved"],
            100 * dec["roofline"]["frac"]))
        if not args.skip_gated:
            dg = bench_decode_gated(gret, dev, dd)
            result["decode_gated"] = dg
            log("decode gated: %.2f us/step, %.0f steps/s, %.0f GB/s (%.1f%%)" % (
                dg["us_per_step"], dg["steps_per_s"], dg["roofline"]["achieved"],
                100 * dg["roofline"]["frac"]))
        if args.only == "decode":
            result.update({"value": dec["steps_per_s"], "unit": "steps/s",
                           "ms_per_step": dec["us_per_step"] / 1000.0,
                           "config": {"workload": dec["workload"]},
                           "roofline": dec["roofline"]})
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
