#!/usr/bin/env python3
"""Throughput of the weight-only INT4/INT2 quantised GEMM hot path on one MI355X.

A step is one pass of the hot path over one batch of synthetic input: the
INT4 loop block (D=2048: QKV 2048->6144, out 2048->2048, FFN up 2048->8192,
down 8192->2048, group 128) applied for L=8 iterations at M=1 decode through
qg_loop_range -- every GEMM of those iterations, the LayerNorm glue and the
residual epilogues.  Weights are packed once beforehand (they arrive packed at
model load).  The residual h lives in one buffer, like the runtime's FP32
residual stream: each step applies the block's L iterations to the state the
previous step left (the same work whatever the values), so nothing but the
hot path runs inside the timed region.  `value` is the effective weight
bandwidth: steps * L * (packed block bytes: codes + scales + zeros) / wall
time.

The JSON line also carries
  * step_distribution: p10 / p50 / p90 of single steps timed with HIP events
    after the timed region;
  * roofline: the dominant kernel of the step (the FFN down-projection GEMV,
    K=8192, N=2048, the same kernel and grid as inside the loop) timed with
    HIP events on the stream it runs on, over a captured batch of
    back-to-back launches on the same, cache-warm weights, against the
    8 TB/s HBM peak;
  * cpu_baseline: the FP64 CPU oracle timed on the host cores on a bounded
    sample of the same workload (whole L=8 steps for ~10 s);
  * extra: the other measured workloads (single-pass INT4 GEMM over a 535 MB
    rotation pool, cold single-pass block, M=512 prefill TFLOP/s, the INT2
    block, M=16 decode for L=32 and the M=2048 down projection), and as
    context the vendor library's dense FP16 GEMM on the same prefill shapes.
Diagnostics go to stderr; stdout holds the one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense FP16 MFMA
D, F, L_MAIN = 2048, 8192, 8


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def block_flops(M: int, D: int = D, F: int = F, gated: bool = False) -> float:
    return 2.0 * M * (D * 3 * D + D * D + (2 if gated else 1) * D * F + F * D)


def time_loop(qg, torch, blk, h, L, scratch, steps, warmup):
    """`warmup` untimed then `steps` timed calls of qg_loop_range(0, L) on the
    residual h; returns the wall time of the timed calls in seconds."""
    for _ in range(warmup):
        qg.qg_loop_range(blk, h, 0, L, scratch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        qg.qg_loop_range(blk, h, 0, L, scratch)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def graph_leg(torch, launch, count, replays=10):
    """Average duration (s) of one launch among `count` back-to-back launches
    captured in a graph, timed with HIP events around the replays on the
    stream that runs them."""
    launch(0)  # host-side validation and warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(count):
            launch(i)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3 / (replays * count)


def traffic_record(kernel_key: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256(open(os.path.join(ROOT, GEMV_SRC), "rb").read()).hexdigest()[:16]
    e = rec.get(kernel_key)
    if not e or e.get("source_sha256_16") != h:
        return None
    return e.get("hbm_bytes_per_launch")


COPY_BYTES = 256 << 20  # calibration copy: larger than the 256 MB MALL's share it can hold
GEMV_KEY = "gemv_int4_k8192_n2048"
GEMV_SRC = os.path.join("int2_quantized_gemm_amd", "csrc", "kernels_gemv.hip")


def pmc_target(qg, torch, workloads, launches: int = 50):
    """Counter target: the roofline kernel (down-projection GEMV, same weights
    and grid as the roofline leg) launched eagerly `launches` times after a
    warm-up, then `launches` device-to-device copies of COPY_BYTES, the
    calibration kernel of known traffic."""
    dev = "cuda"
    inp = workloads.block(1, seed=0)
    down = qg.qg_pack(inp.W["down"].to(dev), 4)
    u = torch.empty(1, F, dtype=torch.float16, device=dev).normal_()
    y = torch.empty(1, D, dtype=torch.float16, device=dev)
    for _ in range(5):
        qg.qg_gemm_int4(u, down, Y=y)
    torch.cuda.synchronize()
    for _ in range(launches):
        qg.qg_gemm_int4(u, down, Y=y)
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(launches):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"pmc target: {launches} GEMV launches ({down.nbytes()} algorithmic bytes each), "
        f"{launches} copies of {COPY_BYTES} bytes")


def pmc_prefill(qg, torch, workloads, launches: int = 10):
    """Counter target for the MFMA kernels: the M=2048 down projection
    (K=8192 -> N=2048, 128-row ring tiles) and the M=512 FFN up projection
    (K=2048 -> N=8192, 64-row ring tiles), each launched `launches` times
    after a warm-up, then a dense FP16 GEMM of the vendor library (4096^3,
    torch.matmul) whose FLOP rate is known, to calibrate the MFMA-busy
    counter."""
    dev = "cuda"
    for (M, K, N) in ((2048, 8192, 2048), (512, 2048, 8192)):
        W, X = workloads.single_gemm(M, K, N, seed=0)
        p = qg.qg_pack(W.to(dev), 4)
        Xd = X.to(dev)
        Y = torch.empty(M, N, dtype=torch.float16, device=dev)
        for _ in range(3):
            qg.qg_gemm_int4(Xd, p, Y=Y)
        torch.cuda.synchronize()
        for _ in range(launches):
            qg.qg_gemm_int4(Xd, p, Y=Y)
        torch.cuda.synchronize()
    a = torch.randn(4096, 4096, device=dev, dtype=torch.float16)
    b = torch.randn(4096, 4096, device=dev, dtype=torch.float16)
    c = torch.empty(4096, 4096, device=dev, dtype=torch.float16)
    for _ in range(3 + launches):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    log(f"pmc prefill: {launches} launches each of the two ring GEMMs and the dense 4096^3 GEMM")


def traffic_from(fetch_csv: str, write_csv: str, command: str):
    """HBM bytes per launch of the roofline GEMV from two rocprofv3 --pmc runs
    of --pmc-target (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each
    scaled by expected / counted bytes of the calibration copy; written to
    profiles/traffic.json under the kernel source's hash."""
    import csv
    import statistics

    def per_dispatch(path, counter):
        tot = {}
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] != counter:
                continue
            k = (int(row["Dispatch_Id"]), row["Kernel_Name"])
            tot[k] = tot.get(k, 0.0) + float(row["Counter_Value"])
        gemv = [v for (d, n), v in sorted(tot.items()) if "k_gemv" in n]
        copy = [v for (d, n), v in sorted(tot.items()) if "copy" in n.lower()]
        big = max(copy)
        # drop the GEMV warm-up launches and the small host-side copies
        return gemv[5:], [v for v in copy if v > 0.25 * big]

    g_f, c_f = per_dispatch(fetch_csv, "FETCH_SIZE")
    g_w, c_w = per_dispatch(write_csv, "WRITE_SIZE")
    med = statistics.median
    kib = 1024.0
    scale_f = COPY_BYTES / (med(c_f) * kib)
    scale_w = COPY_BYTES / (med(c_w) * kib)
    fetch_b = med(g_f) * kib * scale_f
    write_b = med(g_w) * kib * scale_w
    src = os.path.join(ROOT, GEMV_SRC)
    rec_path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(rec_path)) if os.path.exists(rec_path) else {}
    rec[GEMV_KEY] = {
        "kernel": "k_gemv<4,64,4,2,false,1> (K=8192, N=2048, M=1)",
        "source": GEMV_SRC,
        "source_sha256_16": hashlib.sha256(open(src, "rb").read()).hexdigest()[:16],
        "fetch_kib_per_launch_raw": round(med(g_f), 1),
        "write_kib_per_launch_raw": round(med(g_w), 1),
        "copy_bytes": COPY_BYTES,
        "copy_fetch_kib_raw": round(med(c_f), 1),
        "copy_write_kib_raw": round(med(c_w), 1),
        "scale_fetch": round(scale_f, 4),
        "scale_write": round(scale_w, 4),
        "fetch_bytes_per_launch": int(fetch_b),
        "write_bytes_per_launch": int(write_b),
        "hbm_bytes_per_launch": int(fetch_b + write_b),
        "launches": [len(g_f), len(g_w)],
        "command": command,
    }
    with open(rec_path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec[GEMV_KEY]))


def cpu_baseline(budget_s: float):
    import numpy as np

    import oracle
    import workloads
    inp = workloads.block(1, seed=0)
    ob = oracle.pack_block({k: v.numpy() for k, v in inp.W.items()}, 4, D, F)
    h0 = inp.X.numpy().astype(np.float64)
    block_bytes = sum(p.codes.nbytes + p.scales.nbytes + p.zeros.nbytes
                      for p in (ob.qkv, ob.out, ob.up, ob.down))
    def run(seconds):
        steps, t0 = 0, time.perf_counter()
        while True:
            oracle.loop_range(ob, h0, 0, L_MAIN)
            steps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return steps, el

    cores = oracle.num_threads()
    steps, el = run(budget_s)
    # the same on one core, for about half the budget
    oracle.set_num_threads(1)
    try:
        steps1, el1 = run(budget_s / 2)
    finally:
        oracle.set_num_threads(cores)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": round(steps * L_MAIN * block_bytes / el / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{steps} whole steps of the same workload (INT4 block, M=1, L={L_MAIN}, "
                  f"seed 0) through the FP64 oracle, {el:.1f} s wall",
        "seconds": round(el, 2),
        "single_core": {"value": round(steps1 * L_MAIN * block_bytes / el1 / 1e9, 4),
                        "unit": "GB/s", "steps": steps1, "seconds": round(el1, 2)},
        "cpu_model": model,
    }


def extra_legs(qg, torch, workloads, args):
    out = {}
    dev = "cuda"

    def sync():
        torch.cuda.synchronize()

    # c1: single INT4 GEMM M=1 K=N=2048 over a >= 512 MB rotation pool (HBM,
    # single pass: no copy is re-read before the pool wraps).
    W, X = workloads.single_gemm(1, 2048, 2048, seed=0)
    p = qg.qg_pack(W.to(dev), 4)
    pool = [qg.PackedWeight(4, 2048, 2048, p.codes.clone(), p.scales.clone(), p.zeros.clone())
            for _ in range(240)]
    Xd, Y = X.to(dev), torch.empty(1, 2048, dtype=torch.float16, device=dev)
    per = graph_leg(torch, lambda i: qg.qg_gemm_int4(Xd, pool[i], Y=Y), len(pool), replays=4)
    out["c1_int4_gemm_m1_pool"] = {
        "us_per_call": round(per * 1e6, 3), "GB/s": round(p.nbytes() / per / 1e9, 1),
        "frac_hbm": round(p.nbytes() / per / 1e9 / HBM_PEAK_GBS, 4),
        "pool_MB": round(len(pool) * p.nbytes() / 1e6, 1)}
    del pool
    sync()

    def loop_case(name, bits, M, L, gated=False, per_row=False):
        inp = workloads.block(M, seed=0, gated=gated)
        blk = qg.pack_block(inp.W, bits, D, F, per_row=per_row)
        scratch = qg.alloc_loop_scratch(blk, M)
        h = inp.X.float().to(dev)
        t1 = time_loop(qg, torch, blk, h, L, scratch, 1, 2)
        reps = int(max(3, min(200, 0.3 / max(t1, 1e-6))))
        per = time_loop(qg, torch, blk, h, L, scratch, reps, 1) / reps
        r = {"M": M, "L": L, "bits": bits, "ms_per_call": round(per * 1e3, 4),
             "eff_weight_GB/s": round(L * blk.nbytes() / per / 1e9, 1),
             "TFLOP/s": round(block_flops(M, gated=gated) * L / per / 1e12, 2)}
        if gated:
            r["ffn"] = "swiglu"
        if per_row:
            r["group"] = "per-row (K)"
        r["frac_hbm"] = round(r["eff_weight_GB/s"] / HBM_PEAK_GBS, 4)
        r["frac_mfma"] = round(r["TFLOP/s"] / MFMA_F16_PEAK_TFLOPS, 4)
        out[name] = r

    # c2 cold: L=1 over a rotation pool of 20 distinct blocks (535 MB).
    inp = workloads.block(1, seed=0)
    blk = qg.pack_block(inp.W, 4, D, F)
    copies = []
    for _ in range(20):
        copies.append(qg.Block(D, F, *(qg.PackedWeight(w.bits, w.K, w.N, w.codes.clone(),
                                                      w.scales.clone(), w.zeros.clone())
                                       for w in (blk.qkv, blk.out, blk.up, blk.down))))
    scratch = qg.alloc_loop_scratch(blk, 1)
    h = inp.X.float().to(dev)
    for b in copies:
        qg.qg_loop_range(b, h, 0, 1, scratch)
    sync()
    reps = 5
    t0 = time.perf_counter()
    for _ in range(reps):
        for b in copies:
            qg.qg_loop_range(b, h, 0, 1, scratch)
    sync()
    cold = (time.perf_counter() - t0) / (reps * len(copies))
    out["c2_int4_block_m1_cold_l1"] = {"ms_per_iteration": round(cold * 1e3, 4),
                                       "GB/s": round(blk.nbytes() / cold / 1e9, 1)}
    del copies
    sync()

    loop_case("c3_int4_block_m512_l8", 4, 512, 8)
    loop_case("c4a_int2_block_m1_l16", 2, 1, 16)
    loop_case("c4b_int2_block_m128_l8", 2, 128, 8)
    loop_case("c5a_int4_block_m16_l32", 4, 16, 32)
    # Medium M (batched decode between the skinny and the 128-row tiles).
    loop_case("next3_int4_block_m64_l8", 4, 64, 8)
    # Per-row groups (one scale and zero per output channel): decode.
    loop_case("next3_int4_perrow_block_m1_l8", 4, 1, 8, per_row=True)
    # SwiGLU block (gate projection D x F added): decode and prefill.
    loop_case("next2_int4_gated_block_m1_l8", 4, 1, 8, gated=True)
    loop_case("next2_int4_gated_block_m512_l8", 4, 512, 8, gated=True)

    # c5b: M=2048 single-shot prefill through the down projection K=8192 -> N=2048.
    W, X = workloads.single_gemm(2048, 8192, 2048, seed=0)
    p = qg.qg_pack(W.to(dev), 4)
    Xd, Y = X.to(dev), torch.empty(2048, 2048, dtype=torch.float16, device=dev)
    # 2000 back-to-back launches (~0.2 s, like the loop legs) after the warm
    # replay: a handful of launches after an idle gap runs at lower clocks.
    med = graph_leg(torch, lambda i: qg.qg_gemm_int4(Xd, p, Y=Y), 20, replays=100)
    out["c5b_int4_down_m2048"] = {"us_per_call": round(med * 1e6, 2),
                                  "TFLOP/s": round(2.0 * 2048 * 8192 * 2048 / med / 1e12, 2),
                                  "frac_mfma": round(2.0 * 2048 * 8192 * 2048 / med / 1e12
                                                     / MFMA_F16_PEAK_TFLOPS, 4)}
    del Xd, Y, p
    sync()

    # Measured memory bandwidth, context for the spec peak (not a roofline
    # peak): a device-to-device copy of 1 GiB (single pass through HBM) and of
    # 48 MiB (source and destination MALL-resident after the first pass),
    # bytes read + written per second; eager launches, HIP events.
    def copy_bw(nbytes, reps):
        src = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).random_()
        dst = torch.empty_like(src)
        dst.copy_(src)
        sync()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            dst.copy_(src)
        b.record()
        sync()
        per = a.elapsed_time(b) * 1e-3 / reps
        del src, dst
        return round(2 * nbytes / per / 1e9, 1)
    out["measured_copy_bw_GB/s"] = {"hbm_1GiB": copy_bw(1 << 30, 20),
                                    "mall_48MiB": copy_bw(48 << 20, 400),
                                    "kind": "torch device copy, read + write, context only"}
    sync()

    # Dense FP16 GEMM of the vendor library (torch.matmul -> hipBLASLt) on the
    # same shapes as C3's projections at M = 512 and as C5b: what an
    # unquantised FP16 weight reaches on this chip at these sizes, context for
    # the MFMA fractions above (not part of the measured path).
    def dense(M, K, N):
        a = torch.randn(M, K, device=dev, dtype=torch.float16)
        w = torch.randn(K, N, device=dev, dtype=torch.float16)
        y = torch.empty(M, N, device=dev, dtype=torch.float16)
        t = graph_leg(torch, lambda i: torch.matmul(a, w, out=y), 20, replays=100)
        del a, w, y
        return t
    c3_shapes = {"qkv": (512, D, 3 * D), "out": (512, D, D), "up": (512, D, F), "down": (512, F, D)}
    c3_t = {k: dense(*v) for k, v in c3_shapes.items()}
    c5b_t = dense(2048, 8192, 2048)
    c3_sum = sum(c3_t.values())
    out["dense_fp16_library"] = {
        "kind": "torch.matmul FP16 x FP16 (hipBLASLt), graph-timed, context only",
        "c3_projections_us": {k: round(v * 1e6, 2) for k, v in c3_t.items()},
        "c3_four_projections_TFLOP/s": round(block_flops(512) / c3_sum / 1e12, 1),
        "c3_four_projections_frac_mfma": round(block_flops(512) / c3_sum / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
        "c5b_us": round(c5b_t * 1e6, 2),
        "c5b_TFLOP/s": round(2.0 * 2048 * 8192 * 2048 / c5b_t / 1e12, 1)}
    sync()

    # INT4 -> INT2 tier switch of the measured block: the four projections
    # re-quantised out of place into preallocated INT2 weights.  Each call
    # synchronises (it reports errors), so this is the caller-visible time;
    # bytes = INT4 read + INT2 written (codes, scales and zeros).
    inp = workloads.block(1, seed=0)
    blk4 = qg.pack_block(inp.W, 4, D, F)
    w4s = [blk4.qkv, blk4.out, blk4.up, blk4.down]
    outs = [qg.PackedWeight.empty(w.K, w.N, 2, dev) for w in w4s]
    for w, o in zip(w4s, outs):
        qg.qg_requant_4to2(w, out=o)
    reps = 20
    t0 = time.perf_counter()
    for _ in range(reps):
        for w, o in zip(w4s, outs):
            qg.qg_requant_4to2(w, out=o)
    per = (time.perf_counter() - t0) / reps
    moved = sum(w.nbytes() for w in w4s) + sum(o.nbytes() for o in outs)
    out["next1_requant_int4_to_int2_block"] = {
        "ms_per_block": round(per * 1e3, 4), "bytes_moved": moved,
        "GB/s": round(moved / per / 1e9, 1), "frac_hbm": round(moved / per / 1e9 / HBM_PEAK_GBS, 4)}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--pmc-target", action="store_true",
                    help="only launch the roofline kernel and the calibration copy (for "
                         "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs)")
    ap.add_argument("--pmc-prefill", action="store_true",
                    help="only launch the two ring GEMMs and a dense FP16 GEMM (for rocprofv3 "
                         "--pmc SQ counter runs)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from the two counter runs (no GPU)")
    ap.add_argument("--traffic-command", default="",
                    help="the command lines that produced the counter runs, recorded as is")
    args = ap.parse_args()

    if args.traffic_from:
        traffic_from(args.traffic_from[0], args.traffic_from[1], args.traffic_command)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU: this library has no multi-GPU path "
              f"(--gpus {args.gpus} requested).", file=sys.stderr)
        sys.exit(2)

    import torch

    import int2_quantized_gemm_amd as qg
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"
    torch.cuda.set_device(0)
    if args.pmc_target:
        pmc_target(qg, torch, workloads)
        return
    if args.pmc_prefill:
        pmc_prefill(qg, torch, workloads)
        return

    # ---- main leg: INT4 loop block, M=1, L=8 (decode)
    inp = workloads.block(1, seed=0)
    blk = qg.pack_block(inp.W, 4, D, F, dev)
    scratch = qg.alloc_loop_scratch(blk, 1, dev)
    h = inp.X.float().to(dev)
    el = time_loop(qg, torch, blk, h, L_MAIN, scratch, args.steps, args.warmup)
    assert bool(torch.isfinite(h).all()), "residual became non-finite"
    block_bytes = blk.nbytes()
    value = args.steps * L_MAIN * block_bytes / el / 1e9
    log(f"main: {args.steps} steps in {el * 1e3:.2f} ms -> {value:.1f} GB/s effective")
    # Per-step distribution (after the timed region, so it does not touch
    # `value`): each of `steps` further steps bracketed by HIP events on the
    # stream the loop runs on.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        qg.qg_loop_range(blk, h, 0, L_MAIN, scratch)
        b.record()
    torch.cuda.synchronize()
    step_us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    pct = lambda q: round(step_us[min(len(step_us) - 1, int(q * len(step_us)))], 2)
    step_dist = {"unit": "us per step (L=8 iterations), HIP events", "n": len(step_us),
                 "p10": pct(0.10), "p50": pct(0.50), "p90": pct(0.90)}
    log(f"step distribution: {step_dist}")

    # ---- roofline: the dominant kernel of the step in its loop configuration
    # (down projection: u [1][F] FP16 -> [1][D], the GEMV kernel the loop runs)
    u = torch.empty(1, F, dtype=torch.float16, device=dev).normal_()
    y = torch.empty(1, D, dtype=torch.float16, device=dev)
    avg_s = graph_leg(torch, lambda i: qg.qg_gemm_int4(u, blk.down, Y=y), 200, replays=5)
    down_bytes = blk.down.nbytes()
    achieved = down_bytes / avg_s / 1e9
    traffic = traffic_record(GEMV_KEY)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "kernel": "k_gemv<4,64,4,2,false,1> (FFN down projection, K=8192, N=2048, M=1)",
                "algorithmic_bytes_per_launch": down_bytes,
                "avg_launch_us": round(avg_s * 1e6, 3)}
    log(f"roofline: {roofline}")

    result = {
        "metric": "quant_gemm effective weight GB/s (M=1) and TFLOP/s (M=512), % of roofline",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(el / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "INT4 loop block D=2048 (QKV 2048->6144, out 2048->2048, "
                               "up 2048->8192, down 8192->2048), group 128, M=1 decode, L=8, "
                               "W~N(0,0.02), X~N(0,1) FP16, seed 0",
                   "weights": "int4 asymmetric, FP16 scales/zeros",
                   "accumulate": "f32",
                   "block_bytes": block_bytes,
                   "iterations_per_step": L_MAIN},
        "roofline": roofline,
        "step_distribution": step_dist,
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        log(f"cpu_baseline: {result['cpu_baseline']}")
    if not args.no_extra:
        result["extra"] = extra_legs(qg, torch, workloads, args)
        # reuse gain of the loop: time of one cold (single-pass) iteration over
        # one warm iteration of the main leg
        cold = result["extra"]["c2_int4_block_m1_cold_l1"]["ms_per_iteration"]
        result["extra"]["c2_reuse_gain"] = round(cold / (el / args.steps / L_MAIN * 1e3), 3)
        log(f"extra: {json.dumps(result['extra'])}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
