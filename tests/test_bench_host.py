"""Host-side logic of bench.py, on the CPU: the one-GPU contract, the
kernel-trace parser that the rooflines come from, the roofline selection,
and that the committed records still describe the current kernel sources.
No GPU and no oracle: bench.py imports torch and the library only once it
measures."""
from __future__ import annotations

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_block_flops_and_projection_units():
    D, F = bench.D, bench.F
    assert bench.block_flops(1) == 2.0 * (3 * D * D + D * D + D * F + F * D)
    assert bench.block_flops(512, gated=True) == 2.0 * 512 * (3 * D * D + D * D + 2 * D * F + F * D)
    u = bench.proj_units(1)
    # codes (b/8 bytes per weight) + one FP16 scale and zero per 128 weights
    assert u["down"] == {"K": F, "N": D, "bytes": F * D // 2 + 4 * F * D // 128, "flop": 2.0 * F * D}
    assert sum(v["bytes"] for v in u.values()) == 26738688  # the block's packed bytes
    assert bench.proj_units(1, bits=2)["qkv"]["bytes"] == 3 * D * D // 4 + 4 * 3 * D * D // 128


def _write_trace(path, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z",
            "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        t = 1_000_000
        for i, (name, grid, us) in enumerate(rows):
            w.writerow([i + 1, name, grid[0], grid[1], grid[2], t, t + int(us * 1000)])
            t += int(us * 1000) + 500


GEMV = "void qg::(anonymous namespace)::k_gemv<4, 64, 1, 1, 2, true, 1>(unsigned short const*)"
GEMV_D = "void qg::(anonymous namespace)::k_gemv<4, 64, 4, 4, 8, false, 1>(unsigned short const*)"
RING = "void qg::(anonymous namespace)::k_gemm_ring<4, 64, 2, 4, 0, 2>(unsigned short const*)"
RLN = "void qg::(anonymous namespace)::k_reduce_residual_ln<8>(float const*)"
LN = "void qg::(anonymous namespace)::k_layernorm_vec<8>(float const*)"


def test_trace_parser_finds_each_loop_period(tmp_path, monkeypatch):
    """Synthetic trace: packing, 5 decode iterations (one broken by an
    unrelated launch), a live leg, then the prefill loop after its first
    LayerNorm.  Every exact repetition of each loop's period is matched, the
    projections are labelled in order, and the extra launches stay out."""
    rows = [("void qg::k_pack<4>(float const*)", (4096, 1, 1), 30.0)]
    dec = [(GEMV, (196608, 1, 1), 4.0), (GEMV.replace("true", "false"), (65536, 1, 1), 3.0),
           (GEMV, (262144, 1, 1), 4.5), (GEMV_D, (65536, 1, 1), 3.5)]
    for it in range(5):
        rows += [(n, g, us + 0.1 * it) for n, g, us in dec]
        if it == 2:
            rows.append(("void other_kernel()", (64, 1, 1), 9.0))
    rows.append((GEMV_D, (65536, 1, 1), 3.0))  # a live leg's launch
    rows.append((LN, (131072, 1, 1), 5.0))
    pre = [(RING, (196608, 1, 1), 23.0), (RING.replace("64, 2", "32, 2"), (131072, 1, 1), 13.0),
           (RLN, (131072, 1, 1), 6.0), (RING, (262144, 1, 1), 26.0),
           (RING, (65536, 1, 2), 28.0), (RLN, (131072, 1, 1), 5.5)]
    for it in range(3):
        rows += [(n, g, us) for n, g, us in pre]
    trace = tmp_path / "t_kernel_trace.csv"
    _write_trace(trace, rows)
    monkeypatch.setattr(bench, "TRACE_JSON", str(tmp_path / "rt.json"))
    monkeypatch.setattr(bench, "TRACE_MD", str(tmp_path / "rt.md"))
    bench.trace_from(str(trace), "synthetic")
    rec = json.load(open(tmp_path / "rt.json"))
    d = rec["decode"]
    assert d["iterations_matched"] == 5
    assert [e["label"] for e in d["kernels"]] == ["qkv", "out", "up", "down"]
    assert [e["count"] for e in d["kernels"]] == [5] * 4
    assert d["kernels"][0]["avg_us"] == pytest.approx(4.2, abs=2e-3)
    assert d["kernels"][3]["bytes"] == bench.proj_units(1)["down"]["bytes"]
    p = rec["prefill"]
    assert p["iterations_matched"] == 3
    assert [e["label"] for e in p["kernels"]] == ["qkv", "out", "out+k_reduce_residual_ln", "up",
                                                  "down", "down+k_reduce_residual_ln"]
    assert p["kernels"][4]["grid"] == [65536, 1, 2]
    assert p["kernels"][4]["flop"] == bench.proj_units(512)["down"]["flop"]
    assert rec["sources_sha256_16"] == bench.sources_hash()
    md = open(tmp_path / "rt.md").read()
    assert "command: `synthetic`" in md and "| down |" in md


def test_roofline_picks_the_slowest_projection(tmp_path, monkeypatch):
    rec = {"decode": {"kernels": [
        {"label": "qkv", "kernel": GEMV, "avg_us": 4.0, "bytes": 100_000, "K": 1, "N": 1},
        {"label": "up", "kernel": GEMV, "avg_us": 5.0, "bytes": 200_000, "K": 2, "N": 3},
        {"label": "up+x", "kernel": "void x()", "avg_us": 9.0}]},
        "prefill": {"kernels": [
            {"label": "down", "kernel": RING, "avg_us": 20.0, "flop": 2e10, "K": 4, "N": 5},
            {"label": "qkv", "kernel": RING, "avg_us": 10.0, "flop": 1e10, "K": 6, "N": 7},
            {"label": "down+k", "kernel": RLN, "avg_us": 30.0}]}}
    mem = {"block_26.7MB_warm_read_GB/s": 10000.0, "mall_read_128MiB_GB/s": 5000.0}
    dec, pre = bench.roofline_entries(rec, {"GB/s": 1.0}, {"TFLOP/s": 1.0}, mem)
    # a launch without algorithmic bytes (the reduction, LayerNorm) never counts
    assert dec["projection"] == "up" and dec["achieved"] == pytest.approx(40.0)
    assert dec["frac"] == pytest.approx(40.0 / bench.HBM_PEAK_GBS, abs=1e-4)
    assert dec["frac_vs_measured_l2_read"] == pytest.approx(0.004)
    assert dec["bound"] == "l2" and "k_gemv" in dec["kernel"] and "(anonymous" not in dec["kernel"]
    assert pre["projection"] == "down" and pre["achieved"] == pytest.approx(1000.0)
    assert pre["peak"] == 2516.6 and pre["bound"] == "mfma"


def test_committed_records_match_the_kernel_sources():
    """The rooflines use the committed trace and counter records only while
    the kernel sources hash as recorded: they must describe this tree."""
    h = bench.sources_hash()
    for name in ("roofline_trace.json", "loop_kernels.json"):
        rec = json.load(open(os.path.join(ROOT, "profiles", name)))
        assert rec["sources_sha256_16"] == h, name
        assert rec.get("command"), name
    traffic = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))["decode_loop"]
    assert traffic["sources_sha256_16"] == h and traffic["command"]
