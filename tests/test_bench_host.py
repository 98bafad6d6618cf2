"""Host-side logic of bench.py, without a GPU: the algorithmic byte and flop
counts behind the roofline figures, the grouping of kernel names into entry
points, the scaling of rocprofv3 counter tables by the copy calibration, and
the rule that recorded counters are used only for the sources they were taken
on."""
import csv
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_prefill_algorithmic_bytes_and_flops():
    nbytes, flops = bench.prefill_algorithmic(1, 24, 524288, 128, 128, 64, False)
    # per (token, head): q, k, v read and out written in bf16, one fp32 log-gate;
    # plus the fp32 final state of every head
    assert nbytes == 24 * 524288 * ((2 * 128 + 128) * 2 + 128 * 2 + 4) + 24 * 128 * 128 * 4
    assert nbytes == 12_936_806_400
    # per (token, head) at chunk C: (C + 1)(dk + dv) for the causal triangle
    # (scores and P V), 4 dk dv for the cross term and the state update
    assert flops == 24 * 524288 * (65 * 256 + 4 * 128 * 128)
    # an initial state is read as well
    with_state, _ = bench.prefill_algorithmic(1, 24, 524288, 128, 128, 64, True)
    assert with_state - nbytes == 24 * 128 * 128 * 4


def test_decode_algorithmic_bytes():
    nbytes, flops = bench.decode_algorithmic(256, 24, 128, 128)
    # the fp32 state read and written, q, k, v read and out written in bf16,
    # one fp32 log-gate per (sequence, head)
    assert nbytes == 811_622_400
    assert flops == 5 * 256 * 24 * 128 * 128


def test_kernel_names_group_into_entry_points():
    g = bench.kernel_group
    ns = "gret::(anonymous namespace)::"
    assert g("void " + ns + "prefill_main_c64_kernel<128, 128>(" + ns + "Params)") == "prefill"
    assert g(ns + "prefill_prefix_c64_kernel<128, 128>(" + ns + "Params)") == "prefill"
    assert g(ns + "prefill_combine_kernel<128, 128>(" + ns + "Params)") == "prefill"
    assert g(ns + "decode_step_kernel<__bf16, 128, 128, false>(...)") == "decode"
    assert g(ns + "decode_step_kernel<__bf16, 128, 128, true>(...)") == "decode_gated"
    assert g("_ZN4gret12_GLOBAL__N_118decode_step_kernelIDF16bLi128ELi128ELb1EEEvNS0_1PE") == \
        "decode_gated"
    assert g(ns + "xattn_split_kernel<128>(...)") == "xattn"
    assert g(ns + "xattn_combine_kernel<128>(...)") == "xattn"
    assert g(ns + "output_gate_kernel<__bf16, 128>(...)") == "epilogue"
    assert g(ns + "proj_kernel(" + ns + "ProjParams)") == "proj"
    assert g(ns + "swa_prefill_kernel<128>(...)") == "swa"
    assert g(ns + "swa_ring_fill_kernel(...)") == "swa"
    assert g("at::native::elementwise_kernel<...>").startswith("other:")


def _pmc_dir(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (kernel, counter, value) in enumerate(rows):
            w.writerow([i, kernel, counter, value])
    return path


def test_summarize_pmc_scales_by_the_copy_calibration(tmp_path, capsys):
    main = "gret::prefill_main_c64_kernel<128, 128>(Params)"
    comb = "gret::prefill_combine_kernel<128, 128>(Params)"
    copy = "copy_kernel(float4 const*, float4*, long)"
    fetch = _pmc_dir(str(tmp_path / "f"), [(main, "FETCH_SIZE", 100.0), (main, "FETCH_SIZE", 300.0),
                                           (comb, "FETCH_SIZE", 10.0)])
    write = _pmc_dir(str(tmp_path / "w"), [(main, "WRITE_SIZE", 50.0), (main, "WRITE_SIZE", 50.0),
                                           (comb, "WRITE_SIZE", 5.0)])
    # the counters read half of the copy's 1 GiB for FETCH_SIZE and all of it for WRITE_SIZE
    cf = _pmc_dir(str(tmp_path / "cf"), [(copy, "FETCH_SIZE", 524288.0)])
    cw = _pmc_dir(str(tmp_path / "cw"), [(copy, "WRITE_SIZE", 1048576.0)])
    mf = _pmc_dir(str(tmp_path / "m"), [(main, "MfmaUtil", 16.0), (main, "MfmaUtil", 17.0),
                                        (main, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1000.0)])
    bench.summarize_pmc(fetch, write, cf, cw, mf)
    out = json.loads(capsys.readouterr().out)
    assert out["calibration"]["fetch_scale"] == 2.0 and out["calibration"]["write_scale"] == 1.0
    pre = out["prefill"]
    assert pre["sources_sha256"] == bench.sources_sha256("prefill")
    # per call: the mean over dispatches of each kernel, summed over the kernels
    assert pre["fetch_bytes"] == (200.0 + 10.0) * 1024 * 2.0
    assert pre["write_bytes"] == (50.0 + 5.0) * 1024 * 1.0
    k = pre["kernels"]["gret::prefill_main_c64_kernel<128, 128>"]
    assert k["dispatches"] == 2 and k["mfma_util_pct"] == 16.5
    assert k["mfma_bf16_flops"] == 1000.0 * 512
    assert "decode" not in out  # no dispatches of it in these tables


def test_summarize_pmc_gated_prefill_takes_only_the_prefill_combine(tmp_path, capsys):
    gmain = "gret::prefill_main_c64_kernel<128, 128, true>(Params)"
    comb = "gret::prefill_combine_kernel<128, 128>(Params)"
    xcomb = "gret::xattn_combine_kernel<128>(XParams)"
    copy = "copy_kernel(float4 const*, float4*, long)"
    rows = [(gmain, 400.0), (comb, 10.0), (xcomb, 7.0)]
    fetch = _pmc_dir(str(tmp_path / "f"), [(k, "FETCH_SIZE", v) for k, v in rows])
    write = _pmc_dir(str(tmp_path / "w"), [(k, "WRITE_SIZE", v) for k, v in rows])
    cf = _pmc_dir(str(tmp_path / "cf"), [(copy, "FETCH_SIZE", 524288.0)])
    cw = _pmc_dir(str(tmp_path / "cw"), [(copy, "WRITE_SIZE", 1048576.0)])
    bench.summarize_pmc(fetch, write, cf, cw)
    out = json.loads(capsys.readouterr().out)
    gated = out["prefill_gated"]["kernels"]
    assert sorted(gated) == ["gret::prefill_combine_kernel<128, 128>",
                             "gret::prefill_main_c64_kernel<128, 128, true>"]
    assert out["prefill_gated"]["fetch_bytes"] == (400.0 + 10.0) * 1024 * 2.0
    assert out["xattn"]["fetch_bytes"] == 7.0 * 1024 * 2.0


def test_recorded_counters_need_matching_sources(tmp_path, monkeypatch):
    rec = {"prefill": {"sources_sha256": bench.sources_sha256("prefill"),
                       "fetch_bytes": 10.0, "write_bytes": 3.0,
                       "kernels": {"gret::prefill_main_c64_kernel<128, 128>":
                                   {"mfma_util_pct": 16.5}}},
           "decode": {"sources_sha256": "0" * 64, "fetch_bytes": 1.0, "write_bytes": 1.0,
                      "kernels": {}}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.recorded_traffic("prefill") == 13.0
    assert bench.recorded_mfma("prefill", "prefill_main_c64_kernel") == 16.5
    assert bench.recorded_traffic("decode") is None      # taken on other sources
    assert bench.recorded_traffic("swa") is None         # never recorded


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout + r.stderr
