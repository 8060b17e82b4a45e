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
  * roofline: the slowest kernel of the step (one of the loop's four GEMVs),
    its algorithmic bytes over its average duration inside the loop as
    recorded by `rocprofv3 --kernel-trace` in profiles/roofline_trace.json
    (written by --trace-from from a trace of this script; used while the
    kernel sources still hash as recorded), against the 8 TB/s HBM peak and
    against the measured read bandwidths of the L2 (the block read back to
    back: each XCD's share fits its L2, as in the warm loop; `bound` "l2") and
    of the MALL; the down-projection GEMV's HIP-event period over
    back-to-back graph launches of it on the stream it runs on is reported
    beside it;
  * roofline_prefill: the same for the slowest kernel of the M=512 chunked
    prefill block (C3), in TFLOP/s against the 2516.6 TFLOP/s dense FP16
    MFMA peak;
  * memory: read-only bandwidth of HBM (1 GiB streamed), of the MALL
    (128 MiB, more than the L2s hold) and of the block's 26.7 MB working set
    read back to back (cache-resident);
  * device: name, CUs, memory, and the shader / memory clock levels sampled
    from the driver's sysfs files by a second thread while the decode loop
    runs in an untimed window (the C3 leg carries the same for the prefill
    loop, with its MFMA fraction at the median shader clock beside the
    fraction at the 2.4 GHz spec peak);
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
MFMA_F16_PEAK_TFLOPS = 2516.6  # MI355X dense FP16 MFMA: 256 CUs x 2.4 GHz x 4096 FLOP/clk
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


def traffic_record():
    """Per-projection HBM bytes per launch of the decode loop's GEMVs from the
    committed counter record, if it was taken on the current kernel sources;
    otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get("decode_loop")
    if not rec or rec.get("sources_sha256_16") != sources_hash():
        return None
    return rec


COPY_BYTES = 256 << 20  # calibration copy: as large as the MALL, so it streams through HBM


def pmc_target(qg, torch, workloads, steps: int = 30):
    """Counter target: `steps` steps of the measured decode loop (INT4 block,
    M=1, L=8, the main leg's weights and launch sequence), then 20
    device-to-device copies of COPY_BYTES, the calibration kernel of known
    traffic."""
    dev = "cuda"
    inp = workloads.block(1, seed=0)
    blk = qg.pack_block(inp.W, 4, D, F, dev)
    scratch = qg.alloc_loop_scratch(blk, 1, dev)
    h = inp.X.float().to(dev)
    for _ in range(steps):
        qg.qg_loop_range(blk, h, 0, L_MAIN, scratch)
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(20):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"pmc target: {steps} loop steps ({steps * L_MAIN} iterations), 20 copies of {COPY_BYTES} bytes")


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
    """HBM bytes per launch of each GEMV of the decode loop from two rocprofv3
    --pmc runs of --pmc-target (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch), each scaled by expected / counted bytes of the calibration
    copy.  The loop's four GEMVs are the period of k_gemv dispatches starting
    at the first one; the first two iterations (cold caches) are dropped.
    Written to profiles/traffic.json under the kernel sources' hash."""
    import csv
    import statistics

    def per_dispatch(path, counter):
        tot, sig = {}, {}
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] != counter:
                continue
            d = int(row["Dispatch_Id"])
            tot[d] = tot.get(d, 0.0) + float(row["Counter_Value"])
            sig[d] = (row["Kernel_Name"], int(row["Grid_Size"]))
        ds = sorted(tot)
        gemv = [d for d in ds if "k_gemv" in sig[d][0]]
        period = next(p for p in range(1, len(gemv)) if sig[gemv[p]] == sig[gemv[0]])
        per = [[tot[d] for d in gemv[j::period]][2:] for j in range(period)]
        copy = [tot[d] for d in ds if "copy" in sig[d][0].lower()]
        big = max(copy)
        return per, [sig[gemv[j]] for j in range(period)], [v for v in copy if v > 0.25 * big]

    med = statistics.median
    kib = 1024.0
    f_per, sigs, c_f = per_dispatch(fetch_csv, "FETCH_SIZE")
    w_per, _, c_w = per_dispatch(write_csv, "WRITE_SIZE")
    scale_f = COPY_BYTES / (med(c_f) * kib)
    scale_w = COPY_BYTES / (med(c_w) * kib)
    units = proj_units(1)
    proj = {}
    for j, label in enumerate(PROJ[:len(sigs)]):
        fb, wb = med(f_per[j]) * kib * scale_f, med(w_per[j]) * kib * scale_w
        proj[label] = {"kernel": sigs[j][0][:80], "grid": sigs[j][1],
                       "fetch_kib_raw": round(med(f_per[j]), 1), "write_kib_raw": round(med(w_per[j]), 1),
                       "fetch_bytes": int(fb), "write_bytes": int(wb), "hbm_bytes": int(fb + wb),
                       "algorithmic_bytes": units[label]["bytes"],
                       "ratio_to_algorithmic": round((fb + wb) / units[label]["bytes"], 4),
                       "launches": len(f_per[j])}
    rec_path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = {"decode_loop": {
        "what": "INT4 block M=1 L=8 loop, FETCH_SIZE and WRITE_SIZE per GEMV launch (median), "
                "scaled by the calibration copy",
        "sources_sha256_16": sources_hash(), "copy_bytes": COPY_BYTES,
        "copy_fetch_kib_raw": round(med(c_f), 1), "copy_write_kib_raw": round(med(c_w), 1),
        "scale_fetch": round(scale_f, 4), "scale_write": round(scale_w, 4),
        "projections": proj, "command": command}}
    with open(rec_path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec["decode_loop"]))


# ---- kernel-trace record: per-kernel durations inside the measured loops.

TRACE_JSON = os.path.join(ROOT, "profiles", "roofline_trace.json")
TRACE_MD = os.path.join(ROOT, "profiles", "roofline_trace.md")
CSRC = os.path.join(ROOT, "int2_quantized_gemm_amd", "csrc")
PROJ = ("qkv", "out", "up", "down")


def sources_hash() -> str:
    """Hash of every kernel source: a trace record holds only while it matches."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()[:16]


def proj_units(M: int, bits: int = 4):
    """Algorithmic bytes (codes + scales + zeros) and FLOPs of the block's
    four projections at M rows."""
    shapes = {"qkv": (D, 3 * D), "out": (D, D), "up": (D, F), "down": (F, D)}
    return {k: {"K": K, "N": N, "bytes": N * K * bits // 8 + 4 * N * K // 128,
                "flop": 2.0 * M * N * K} for k, (K, N) in shapes.items()}


def trace_from(trace_csv: str, command: str):
    """Per-kernel durations of the decode loop (M=1) and of the M=512 prefill
    loop, from a `rocprofv3 --kernel-trace` CSV of this script (--no-cpu
    --no-extra --no-clocks).  A loop's kernel sequence is found as the period of
    dispatches that starts at its first kernel (the first k_gemv for decode,
    the first kernel after the first k_layernorm for prefill) and every exact
    repetition of it is collected, so launches outside the loops (the live
    legs, packing) do not mix in.  Writes profiles/roofline_trace.json and
    profiles/roofline_trace.md."""
    import csv
    import statistics
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Dispatch_Id"]))
    disp = [((r["Kernel_Name"], int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]), int(r["Grid_Size_Z"])),
             (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3) for r in rows]

    def loop(first: int, M: int):
        sig0 = disp[first][0]
        period = next(p for p in range(1, len(disp) - first) if disp[first + p][0] == sig0)
        pat = [disp[first + j][0] for j in range(period)]
        per = [[] for _ in pat]
        i, reps = first, 0
        while i + period <= len(disp):
            if all(disp[i + j][0] == pat[j] for j in range(period)):
                for j in range(period):
                    per[j].append(disp[i + j][1])
                i, reps = i + period, reps + 1
            else:
                i += 1
        units = proj_units(M)
        out, gi, prev = [], 0, None
        for sig, ts in zip(pat, per):
            name = sig[0]
            if "k_gemv" in name or "k_gemm" in name:
                label = PROJ[gi]
                gi += 1
                prev = label
            else:
                label = f"{prev}+{name.split('<')[0].split('::')[-1]}"
            e = {"label": label, "kernel": name, "grid": list(sig[1:]), "count": len(ts),
                 "avg_us": round(statistics.mean(ts), 3), "median_us": round(statistics.median(ts), 3),
                 "min_us": round(min(ts), 3), "max_us": round(max(ts), 3)}
            if label in units:
                u = units[label]
                e.update({"M": M, "K": u["K"], "N": u["N"], "bytes": u["bytes"], "flop": u["flop"]})
            out.append(e)
        return {"M": M, "iterations_matched": reps, "kernels": out}

    first_gemv = next(i for i, (sig, _) in enumerate(disp) if "k_gemv" in sig[0])
    first_ln = next(i for i, (sig, _) in enumerate(disp) if "k_layernorm" in sig[0])
    rec = {"command": command, "trace": os.path.basename(trace_csv),
           "sources_sha256_16": sources_hash(),
           "decode": loop(first_gemv, 1), "prefill": loop(first_ln + 1, 512)}
    with open(TRACE_JSON, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    # summary of every kernel of the run (the --stats view) plus the loops
    tot = {}
    for (sig, t) in disp:
        tot.setdefault(sig[0], []).append(t)
    lines = ["# Per-kernel durations: INT4 loop block, M=1 decode (L=8) and M=512 prefill (L=8)", "",
             f"command: `{command}`", "",
             f"Written by `python bench.py --trace-from {os.path.basename(trace_csv)} ...` from the "
             "trace; durations are rocprofv3 kernel-trace start-to-end times (microseconds). "
             f"Kernel sources sha256/16 = `{rec['sources_sha256_16']}`.", ""]
    for part, title in (("decode", "M=1 decode loop, per iteration"),
                        ("prefill", "M=512 prefill loop, per iteration")):
        L = rec[part]
        lines += [f"## {title} ({L['iterations_matched']} iterations matched)", "",
                  "| kernel | launch | calls | avg us | median us | min us | max us | algorithmic | rate |",
                  "|---|---|---|---|---|---|---|---|---|"]
        for e in L["kernels"]:
            if "bytes" in e and part == "decode":
                alg, rate = f"{e['bytes']} B", f"{e['bytes'] / e['avg_us'] / 1e3:.1f} GB/s"
            elif "flop" in e and part == "prefill":
                alg, rate = f"{e['flop'] / 1e9:.2f} GFLOP", f"{e['flop'] / e['avg_us'] / 1e6:.1f} TFLOP/s"
            else:
                alg, rate = "", ""
            lines.append(f"| {e['label']} | `{e['kernel'][:70]}` grid {e['grid']} | {e['count']} | "
                         f"{e['avg_us']} | {e['median_us']} | {e['min_us']} | {e['max_us']} | {alg} | {rate} |")
        lines.append("")
    lines += ["## All kernels of the run", "", "| kernel | calls | total us | avg us |", "|---|---|---|---|"]
    for name, ts in sorted(tot.items(), key=lambda kv: -sum(kv[1]))[:25]:
        lines.append(f"| `{name[:90]}` | {len(ts)} | {sum(ts):.1f} | {statistics.mean(ts):.3f} |")
    with open(TRACE_MD, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({k: rec[k] for k in ("decode", "prefill")})[:2000])


# Loop workloads of the per-kernel breakdown, in launch order:
# (name, bits, M, L).
LOOP_CONFIGS = (("c2_int4_block_m1_l8", 4, 1, 8), ("c4a_int2_block_m1_l16", 2, 1, 16),
                ("c5a_int4_block_m16_l32", 4, 16, 32), ("c4b_int2_block_m128_l8", 2, 128, 8),
                ("c3_int4_block_m512_l8", 4, 512, 8))
LOOPS_JSON = os.path.join(ROOT, "profiles", "loop_kernels.json")
LOOPS_MD = os.path.join(ROOT, "profiles", "loop_kernels.md")


def loops_target(qg, torch, workloads, calls: int = 4):
    """Trace / counter target: each loop workload of LOOP_CONFIGS packed (its
    pack kernels mark where it starts in a trace), one warm-up call, then
    `calls` calls of qg_loop_range; then two calibration kernels: 13 dense
    FP16 4096^3 GEMMs of the vendor library (torch.matmul; a known FLOP rate
    for the MFMA counters) and 20 device copies of COPY_BYTES (known bytes
    for FETCH_SIZE / WRITE_SIZE)."""
    dev = "cuda"
    for name, bits, M, L in LOOP_CONFIGS:
        inp = workloads.block(M, seed=0)
        blk = qg.pack_block(inp.W, bits, D, F, dev)
        scratch = qg.alloc_loop_scratch(blk, M, dev)
        h = inp.X.float().to(dev)
        torch.cuda.synchronize()
        for _ in range(1 + calls):
            qg.qg_loop_range(blk, h, 0, L, scratch)
        torch.cuda.synchronize()
        log(f"loops target: {name}: {1 + calls} calls")
    a = torch.randn(4096, 4096, device=dev, dtype=torch.float16)
    b = torch.randn(4096, 4096, device=dev, dtype=torch.float16)
    c = torch.empty(4096, 4096, device=dev, dtype=torch.float16)
    for _ in range(13):
        torch.matmul(a, b, out=c)
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(20):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("loops target: calibration GEMMs and copies done")


def loop_pattern(disp, first: int, M: int, end: int | None = None):
    """Kernel sequence of one loop iteration starting at dispatch `first` of
    disp = [(signature, value)] (signature = (kernel name, grid...)): the
    period until the first signature recurs; every exact repetition of it in
    disp[first:end] is collected, so launches outside the loop do not mix
    in.  Returns (labels, signatures, per-position value lists, repetitions);
    labels name the projection of each GEMM launch (qkv, out, up, down) and
    `projection+kernel` for the launches that finish one."""
    end = len(disp) if end is None else end
    sig0 = disp[first][0]
    period = next(p for p in range(1, end - first) if disp[first + p][0] == sig0)
    pat = [disp[first + j][0] for j in range(period)]
    per = [[] for _ in pat]
    i, reps = first, 0
    while i + period <= end:
        if all(disp[i + j][0] == pat[j] for j in range(period)):
            for j in range(period):
                per[j].append(disp[i + j][1])
            i, reps = i + period, reps + 1
        else:
            i += 1
    labels, gi, prev = [], 0, None
    for sig in pat:
        name = sig[0]
        if "k_gemv" in name or "k_gemm" in name:
            prev = PROJ[gi % len(PROJ)]
            gi += 1
            labels.append(prev)
        else:
            labels.append(f"{prev}+{name.split('<')[0].split('::')[-1]}")
    return labels, pat, per, reps


def loop_segments(names):
    """[start, end) dispatch ranges of the LOOP_CONFIGS workloads in a
    loops-target run: each begins after its weights' pack kernels, and the
    loop's first iteration begins at its first GEMV (M = 1) or at the first
    launch after its first LayerNorm (M > 1)."""
    starts, loop_seen = [], True
    for i, n in enumerate(names):
        if "k_pack" in n:
            if loop_seen:
                starts.append(i)
            loop_seen = False
        elif "k_gemv" in n or "k_gemm" in n or "k_layernorm" in n:
            loop_seen = True
    assert len(starts) >= len(LOOP_CONFIGS), f"{len(starts)} pack groups in the trace"
    starts = starts[-len(LOOP_CONFIGS):]
    bounds = starts[1:] + [len(names)]
    segs = []
    for (name, bits, M, L), a, b in zip(LOOP_CONFIGS, starts, bounds):
        if M == 1:
            first = next(i for i in range(a, b) if "k_gemv" in names[i])
        else:
            first = next(i for i in range(a, b) if "k_layernorm" in names[i]) + 1
        segs.append((first, b))
    return segs


def loops_from(trace_csv: str, pmc_csvs, command: str):
    """profiles/loop_kernels.json and .md: per loop workload of LOOP_CONFIGS,
    every launch of one iteration with its rocprofv3 kernel-trace duration
    (median over the matched iterations) and, from `rocprofv3 --pmc` runs of
    the same target, the median of each SQ counter per launch and the ratios
    derived from them."""
    import csv
    import statistics
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Dispatch_Id"]))
    disp = [((r["Kernel_Name"], int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]), int(r["Grid_Size_Z"])),
             (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3) for r in rows]
    segs = loop_segments([d[0][0] for d in disp])
    # counters: dispatch -> {counter: value summed over the rows of that dispatch}
    pmc_disp = []
    for path in pmc_csvs:
        per = {}
        for r in csv.DictReader(open(path)):
            d = int(r["Dispatch_Id"])
            e = per.setdefault(d, {"name": r["Kernel_Name"], "grid": int(r["Grid_Size"]), "c": {}})
            e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        pmc_disp.append([per[d] for d in sorted(per)])
    rec = {"command": command, "trace": os.path.basename(trace_csv),
           "counters": [os.path.basename(p) for p in pmc_csvs],
           "sources_sha256_16": sources_hash(), "configs": {}}
    # calibration: the copies (bytes) and the dense GEMM (MFMA counters), the
    # last dispatches of each run
    scale = {}
    dense = {}
    for pd in pmc_disp:
        copies = [e for e in pd if "copy" in e["name"].lower()]
        for cn in ("FETCH_SIZE", "WRITE_SIZE"):
            vals = [e["c"][cn] for e in copies if cn in e["c"]]
            if vals:
                big = max(vals)
                scale[cn] = COPY_BYTES / (statistics.median(v for v in vals if v > 0.25 * big) * 1024.0)
        gemm = [e for e in pd if "qg::" not in e["name"] and "copy" not in e["name"].lower()
                and "fill" not in e["name"].lower()]
        if gemm:
            top = max(set(e["name"] for e in gemm), key=lambda n: sum(e["name"] == n for e in gemm))
            last = [e for e in gemm if e["name"] == top][-10:]
            dense["kernel"] = top.split("(")[0][:60]
            for cn in last[0]["c"]:
                dense.setdefault("counters", {})[cn] = statistics.median(e["c"][cn] for e in last)
    rec["traffic_scale"] = {k: round(v, 4) for k, v in scale.items()}
    for (name, bits, M, L), (first, end) in zip(LOOP_CONFIGS, segs):
        labels, pat, per, reps = loop_pattern(disp, first, M, end)
        units = proj_units(M, bits)
        ks = []
        for lab, sig, ts in zip(labels, pat, per):
            e = {"label": lab, "kernel": sig[0].replace("void ", "")
                 .replace("qg::(anonymous namespace)::", "").split("(")[0], "grid": list(sig[1:]),
                 "median_us": round(statistics.median(ts), 3), "count": len(ts)}
            if lab in units:
                e.update(bytes=units[lab]["bytes"], flop=units[lab]["flop"])
            ks.append(e)
        # the same launches in each counter run
        for pd in pmc_disp:
            pn = [e["name"] for e in pd]
            pf, pe = loop_segments(pn)[[c[0] for c in LOOP_CONFIGS].index(name)]
            pdisp = [((e["name"], e["grid"]), e["c"]) for e in pd]
            _, _, pper, _ = loop_pattern(pdisp, pf, M, pe)
            for e, vals in zip(ks, pper):
                for cn in vals[0]:
                    e.setdefault("counters", {})[cn] = statistics.median(v[cn] for v in vals)
        for e in ks:
            c = e.get("counters", {})
            d = {}
            if "FETCH_SIZE" in c and "FETCH_SIZE" in scale:
                d["fetch_MB"] = round(c["FETCH_SIZE"] * 1024.0 * scale["FETCH_SIZE"] / 1e6, 3)
            if "WRITE_SIZE" in c and "WRITE_SIZE" in scale:
                d["write_MB"] = round(c["WRITE_SIZE"] * 1024.0 * scale["WRITE_SIZE"] / 1e6, 3)
            if c.get("SQ_INSTS_MFMA"):
                d["valu_per_mfma"] = round((c.get("SQ_INSTS_VALU", 0) - c["SQ_INSTS_MFMA"])
                                           / c["SQ_INSTS_MFMA"], 2)
            if c.get("SQ_WAVE_CYCLES"):
                d["wait_share"] = round(c.get("SQ_WAIT_INST_ANY", 0) / c["SQ_WAVE_CYCLES"], 3)
            if c.get("SQ_WAVES"):
                d["valu_per_wave"] = round(c.get("SQ_INSTS_VALU", 0) / c["SQ_WAVES"], 1)
            if c.get("GRBM_GUI_ACTIVE") and c.get("SQ_VALU_MFMA_BUSY_CYCLES"):
                d["mfma_busy"] = round(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (c["GRBM_GUI_ACTIVE"] / 8 * 1024), 3)
            if c.get("SQ_LDS_IDX_ACTIVE"):
                d["lds_bank_conflict_share"] = round(c.get("SQ_LDS_BANK_CONFLICT", 0) / c["SQ_LDS_IDX_ACTIVE"], 3)
            if d:
                e["derived"] = d
        tot = sum(e["median_us"] for e in ks)
        rec["configs"][name] = {"bits": bits, "M": M, "L": L, "iterations_matched": reps,
                                "sum_of_medians_us": round(tot, 2), "kernels": ks}
    if dense:
        c = dense["counters"]
        d = {}
        if c.get("SQ_INSTS_MFMA"):
            d["valu_per_mfma"] = round((c.get("SQ_INSTS_VALU", 0) - c["SQ_INSTS_MFMA"]) / c["SQ_INSTS_MFMA"], 2)
        if c.get("SQ_WAVE_CYCLES"):
            d["wait_share"] = round(c.get("SQ_WAIT_INST_ANY", 0) / c["SQ_WAVE_CYCLES"], 3)
        if c.get("GRBM_GUI_ACTIVE") and c.get("SQ_VALU_MFMA_BUSY_CYCLES"):
            d["mfma_busy"] = round(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (c["GRBM_GUI_ACTIVE"] / 8 * 1024), 3)
        dense["derived"] = d
        rec["dense_fp16_4096_calibration"] = dense
    with open(LOOPS_JSON, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    lines = ["# Per-launch breakdown of the loop workloads (one iteration each)", "",
             f"commands: `{command}`", "",
             "Durations are rocprofv3 kernel-trace start-to-end times (median over the matched "
             "iterations; the trace's own per-dispatch cost makes them slightly longer than the "
             "graph-timed period); counters are medians per launch over the same iterations of "
             "separate `--pmc` runs. Derived: VALU/MFMA = (SQ_INSTS_VALU - SQ_INSTS_MFMA) / "
             "SQ_INSTS_MFMA; wait = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES; MFMA busy = "
             "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs); LDS conflict = "
             "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (cycles); fetch / write MB = FETCH_SIZE / "
             "WRITE_SIZE per launch scaled by the calibration copy. "
             f"Kernel sources sha256/16 = `{rec['sources_sha256_16']}`.", ""]
    for name, cfg in rec["configs"].items():
        lines += [f"## {name} (INT{cfg['bits']}, M={cfg['M']}, L={cfg['L']}; "
                  f"{cfg['iterations_matched']} iterations matched; sum {cfg['sum_of_medians_us']} us)", "",
                  "| launch | kernel | grid | median us | rate | waves | VALU/wave | VALU/MFMA | wait | MFMA busy | LDS conflict | fetch MB | write MB |",
                  "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
        for e in cfg["kernels"]:
            rate = ""
            if "bytes" in e and cfg["M"] <= 16:
                rate = f"{e['bytes'] / e['median_us'] / 1e3:.0f} GB/s"
            elif "flop" in e:
                rate = f"{e['flop'] / e['median_us'] / 1e6:.0f} TFLOP/s"
            c, d = e.get("counters", {}), e.get("derived", {})
            lines.append(f"| {e['label']} | `{e['kernel'][:48]}` | {e['grid']} | {e['median_us']} | {rate} | "
                         f"{int(c['SQ_WAVES']) if 'SQ_WAVES' in c else ''} | {d.get('valu_per_wave', '')} | "
                         f"{d.get('valu_per_mfma', '')} | {d.get('wait_share', '')} | {d.get('mfma_busy', '')} | "
                         f"{d.get('lds_bank_conflict_share', '')} | {d.get('fetch_MB', '')} | {d.get('write_MB', '')} |")
        lines.append("")
    if "dense_fp16_4096_calibration" in rec:
        dd = rec["dense_fp16_4096_calibration"]
        lines += ["## Calibration: the vendor library's dense FP16 GEMM, 4096^3 (torch.matmul)", "",
                  f"`{dd['kernel']}`: " + ", ".join(f"{k} {v}" for k, v in dd["derived"].items()), ""]
    if scale:
        lines += [f"Traffic scale factors from the {COPY_BYTES >> 20} MiB device copies (expected bytes / "
                  f"counted bytes): " + ", ".join(f"{k} x{v:.3f}" for k, v in scale.items()), ""]
    with open(LOOPS_MD, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({k: v["sum_of_medians_us"] for k, v in rec["configs"].items()}))


def trace_record():
    """The committed trace record if it was taken on the current kernel
    sources, else None."""
    if not os.path.exists(TRACE_JSON):
        return None
    rec = json.load(open(TRACE_JSON))
    return rec if rec.get("sources_sha256_16") == sources_hash() else None


def read_bw(torch, bench_lib, nbytes: int, launches: int, replays: int, grid: int = 1024):
    """Read-only bandwidth (GB/s) of qgb_read over one buffer of nbytes,
    graph-timed (the same grid and buffer every launch)."""
    import ctypes as C
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def launch(_):
        st = bench_lib.qgb_read(C.c_void_p(buf.data_ptr()), C.c_size_t(nbytes), grid,
                                C.c_void_p(sink.data_ptr()),
                                C.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0, st
    per = graph_leg(torch, launch, launches, replays=replays)
    del buf
    return round(nbytes / per / 1e9, 1)


def memory_ceilings(torch):
    """Read-only bandwidths: HBM (1 GiB, four times the MALL: every launch
    streams it from HBM), MALL (128 MiB: four times what the eight 4 MB L2s
    hold, half the MALL), and the block's own size read back to back
    (26,738,688 B: its per-XCD share fits an L2)."""
    import ctypes as C
    lib = C.CDLL(os.path.join(ROOT, "int2_quantized_gemm_amd", "libqgbench.so"))
    lib.qgb_read.restype = C.c_int
    lib.qgb_read.argtypes = [C.c_void_p, C.c_size_t, C.c_int, C.c_void_p, C.c_void_p]
    return {"hbm_read_1GiB_GB/s": read_bw(torch, lib, 1 << 30, 4, 5, grid=2048),
            "mall_read_128MiB_GB/s": read_bw(torch, lib, 128 << 20, 20, 10),
            "block_26.7MB_warm_read_GB/s": read_bw(torch, lib, 26738688, 50, 10),
            "kind": "qgb_read (libqgbench.so): 16-byte loads, grid-stride, graph-timed, "
                    "read-only; 1024-workgroup grid (2048 for 1 GiB)"}


def gpu_clocks(pci: str | None = None):
    """Current shader (sclk) and memory (mclk) clock levels of the GPU, read
    from the amdgpu driver's sysfs files (pp_dpm_sclk / pp_dpm_mclk, the
    level marked '*'), for the card at PCI address `pci` if given, else for
    every card; with the dense FP16 MFMA peak at that shader clock (256 CUs x
    4096 FLOP/clk) for comparison with the 2.4 GHz spec peak.  File reads
    only; an empty dict where the files are not readable."""
    import glob
    import re
    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            addr = os.path.basename(os.path.realpath(dev))
            if pci and addr.lower() != pci.lower():
                continue
            rec = {}
            for kind in ("sclk", "mclk"):
                with open(os.path.join(dev, f"pp_dpm_{kind}")) as f:
                    cur = [ln for ln in f.read().splitlines() if ln.rstrip().endswith("*")]
                m = re.search(r"(\d+)\s*Mhz", cur[0], re.I) if cur else None
                rec[f"{kind}_MHz"] = int(m.group(1)) if m else None
            if rec.get("sclk_MHz"):
                rec["mfma_f16_peak_at_sclk_TFLOP/s"] = round(256 * 4096 * rec["sclk_MHz"] / 1e6, 1)
            out[addr] = rec
        except (OSError, IndexError):
            continue
    if pci and not out:  # address not matched: every card's clocks instead
        return gpu_clocks(None)
    return out


def sustained_clocks(torch, step, pci, seconds: float = 0.5):
    """Clock levels sampled every 20 ms by a second thread while the calling
    thread runs `step` back to back for `seconds` (outside any timed region):
    the sustained clocks under the workload, as median and range."""
    import statistics
    import threading
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            for rec in gpu_clocks(pci).values():
                samples.append(rec)
            stop.wait(0.02)

    th = threading.Thread(target=sampler)
    th.start()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        step()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stop.set()
    th.join()
    out = {"samples": len(samples), "steps": n}
    for k in ("sclk_MHz", "mclk_MHz"):
        v = [r[k] for r in samples if r.get(k)]
        if v:
            out[k] = {"median": statistics.median(v), "min": min(v), "max": max(v)}
    if "sclk_MHz" in out:
        out["mfma_f16_peak_at_median_sclk_TFLOP/s"] = round(256 * 4096 * out["sclk_MHz"]["median"] / 1e6, 1)
    return out


def device_pci(torch):
    """PCI address (dddd:bb:dd.f) of GPU 0 where torch reports it, else None."""
    p = torch.cuda.get_device_properties(0)
    if all(hasattr(p, a) for a in ("pci_domain_id", "pci_bus_id", "pci_device_id")):
        return f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
    return None


def device_info(torch):
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""),
            "compute_units": p.multi_processor_count,
            "memory_GiB": round(p.total_memory / 2**30, 1), "pci": device_pci(torch)}


def short_name(kernel: str) -> str:
    """A kernel's template name without namespaces and parameter list."""
    return kernel.replace("void ", "").replace("qg::(anonymous namespace)::", "").split("(")[0]


def loops_record():
    """The committed per-launch breakdown (profiles/loop_kernels.json) if it
    was taken on the current kernel sources, else None."""
    if not os.path.exists(LOOPS_JSON):
        return None
    rec = json.load(open(LOOPS_JSON))
    return rec if rec.get("sources_sha256_16") == sources_hash() else None


def roofline_entries(rec, live_decode, live_prefill, mem):
    """The decode and prefill roofline objects: from the trace record when it
    matches the sources, else from the live HIP-event legs."""
    dec, pre = {}, {}
    if rec is not None:
        gemv = [e for e in rec["decode"]["kernels"] if "bytes" in e]
        k = max(gemv, key=lambda e: e["avg_us"])
        a = k["bytes"] / k["avg_us"] / 1e3
        dec = {"bound": "l2", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(a / HBM_PEAK_GBS, 4),
               "frac_vs_measured_l2_read": round(a / mem["block_26.7MB_warm_read_GB/s"], 4),
               "frac_vs_measured_mall_read": round(a / mem["mall_read_128MiB_GB/s"], 4),
               "kernel": f"{short_name(k['kernel'])} ({k['label']} projection, K={k['K']}, N={k['N']}, M=1)",
               "projection": k["label"],
               "algorithmic_bytes_per_launch": k["bytes"], "avg_launch_us": k["avg_us"],
               "duration_source": "rocprofv3 kernel trace inside the L=8 loop, "
                                  "profiles/roofline_trace.json / .md",
               "per_projection_avg_us": {e["label"]: e["avg_us"] for e in gemv}}
        mm = [e for e in rec["prefill"]["kernels"] if "flop" in e]
        k = max(mm, key=lambda e: e["avg_us"])
        t = k["flop"] / k["avg_us"] / 1e6
        pre = {"bound": "mfma", "achieved": round(t, 1), "peak": MFMA_F16_PEAK_TFLOPS,
               "unit": "TFLOP/s", "frac": round(t / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None,
               "kernel": f"{short_name(k['kernel'])} ({k['label']} projection, M=512, K={k['K']}, "
                         f"N={k['N']})",
               "projection": k["label"],
               "algorithmic_flop_per_launch": k["flop"], "avg_launch_us": k["avg_us"],
               "duration_source": "rocprofv3 kernel trace inside the L=8 loop, "
                                  "profiles/roofline_trace.json / .md",
               "per_projection_avg_us": {e["label"]: e["avg_us"] for e in rec["prefill"]["kernels"]}}
    else:
        dec = {"bound": "l2", "achieved": live_decode["GB/s"], "peak": HBM_PEAK_GBS,
               "unit": "GB/s", "frac": round(live_decode["GB/s"] / HBM_PEAK_GBS, 4),
               "frac_vs_measured_l2_read": round(live_decode["GB/s"] / mem["block_26.7MB_warm_read_GB/s"], 4),
               "frac_vs_measured_mall_read": round(live_decode["GB/s"] / mem["mall_read_128MiB_GB/s"], 4),
               "kernel": live_decode["kernel"], "algorithmic_bytes_per_launch": live_decode["bytes"],
               "avg_launch_us": live_decode["us"],
               "duration_source": "HIP events (no trace record for the current kernel sources)"}
        pre = {"bound": "mfma", "achieved": live_prefill["TFLOP/s"], "peak": MFMA_F16_PEAK_TFLOPS,
               "unit": "TFLOP/s", "frac": round(live_prefill["TFLOP/s"] / MFMA_F16_PEAK_TFLOPS, 4),
               "traffic": None, "kernel": live_prefill["kernel"],
               "algorithmic_flop_per_launch": live_prefill["flop"],
               "avg_launch_us": live_prefill["us"],
               "duration_source": "HIP events (no trace record for the current kernel sources)"}
    dec["live_hip_events"] = live_decode
    pre["live_hip_events"] = live_prefill
    return dec, pre


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


def c3_leg(qg, torch, workloads, clocks: bool = True):
    """INT4 block at M=512 rows (prefill_chunk = 512), L=8 iterations per
    qg_loop_range call (its cached graph), ~0.3 s of calls after a warm-up."""
    inp = workloads.block(512, seed=0)
    blk = qg.pack_block(inp.W, 4, D, F)
    scratch = qg.alloc_loop_scratch(blk, 512)
    h = inp.X.float().to("cuda")
    t1 = time_loop(qg, torch, blk, h, L_MAIN, scratch, 1, 3)
    reps = int(max(5, min(400, 0.3 / max(t1, 1e-6))))
    per = time_loop(qg, torch, blk, h, L_MAIN, scratch, reps, 2) / reps
    tf = block_flops(512) * L_MAIN / per / 1e12
    r = {"M": 512, "L": L_MAIN, "bits": 4, "calls": reps, "ms_per_call": round(per * 1e3, 4),
         "TFLOP/s": round(tf, 2), "frac_mfma": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}
    # clock levels under this workload (its own untimed window), and the
    # fraction against the MFMA peak at the median shader clock seen there
    if not clocks:
        return r
    clk = sustained_clocks(torch, lambda: qg.qg_loop_range(blk, h, 0, L_MAIN, scratch),
                           device_pci(torch))
    r["clocks"] = clk
    if "mfma_f16_peak_at_median_sclk_TFLOP/s" in clk:
        r["frac_mfma_at_median_sclk"] = round(tf / clk["mfma_f16_peak_at_median_sclk_TFLOP/s"], 4)
    return r


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

    # c2 cold: one iteration (L=1) of each of 20 distinct copies of the block
    # (535 MB, twice the MALL: every copy streams from HBM), captured in one
    # graph (qg_loop_range enqueues its kernels into the caller's capture) and
    # timed with HIP events over its replays -- the single-pass rate that the
    # loop's reuse is measured against.
    inp = workloads.block(1, seed=0)
    blk = qg.pack_block(inp.W, 4, D, F)
    copies = []
    for _ in range(20):
        copies.append(qg.Block(D, F, *(qg.PackedWeight(w.bits, w.K, w.N, w.codes.clone(),
                                                      w.scales.clone(), w.zeros.clone())
                                       for w in (blk.qkv, blk.out, blk.up, blk.down))))
    scratch = qg.alloc_loop_scratch(blk, 1)
    h = inp.X.float().to(dev)
    cold = graph_leg(torch, lambda i: qg.qg_loop_range(copies[i], h, 0, 1, scratch), len(copies),
                     replays=10)
    out["c2_int4_block_m1_cold_l1"] = {"ms_per_iteration": round(cold * 1e3, 4),
                                       "GB/s": round(blk.nbytes() / cold / 1e9, 1),
                                       "frac_hbm": round(blk.nbytes() / cold / 1e9 / HBM_PEAK_GBS, 4),
                                       "method": "graph of 20 L=1 calls on distinct copies, "
                                                 "HIP events over 10 replays"}
    # Where the warm loop's bytes come from: L=1 calls alternating between two
    # copies (53.5 MB: MALL-resident, but each copy's per-XCD share has been
    # displaced from the L2 by the other's) against L=1 calls on one copy.
    two = graph_leg(torch, lambda i: qg.qg_loop_range(copies[i % 2], h, 0, 1, scratch), 20,
                    replays=10)
    one = graph_leg(torch, lambda i: qg.qg_loop_range(copies[0], h, 0, 1, scratch), 20, replays=10)
    out["c2_int4_block_m1_l2_residency"] = {
        "us_per_iteration_same_copy": round(one * 1e6, 2),
        "us_per_iteration_two_copies_alternating": round(two * 1e6, 2),
        "method": "graphs of 20 L=1 calls, HIP events over 10 replays: the difference is what the "
                  "L2 saves when the block's per-XCD share stays in it"}
    del copies
    sync()
    # The same single-pass rate for the INT2 block (40 copies, 535 MB: every
    # copy again streams from HBM), beside the INT4 one: the INT2/INT4 time
    # ratio where the weights come from HBM, against the warm loop's.
    blk2 = qg.pack_block(inp.W, 2, D, F)
    copies = []
    for _ in range(40):
        copies.append(qg.Block(D, F, *(qg.PackedWeight(w.bits, w.K, w.N, w.codes.clone(),
                                                      w.scales.clone(), w.zeros.clone())
                                       for w in (blk2.qkv, blk2.out, blk2.up, blk2.down))))
    scratch2 = qg.alloc_loop_scratch(blk2, 1)
    cold2 = graph_leg(torch, lambda i: qg.qg_loop_range(copies[i], h, 0, 1, scratch2), len(copies),
                      replays=5)
    out["c4a_int2_block_m1_cold_l1"] = {"ms_per_iteration": round(cold2 * 1e3, 4),
                                        "GB/s": round(blk2.nbytes() / cold2 / 1e9, 1),
                                        "frac_hbm": round(blk2.nbytes() / cold2 / 1e9 / HBM_PEAK_GBS, 4),
                                        "int2_over_int4_time": round(cold2 / cold, 3),
                                        "method": "graph of 40 L=1 calls on distinct copies, "
                                                  "HIP events over 5 replays"}
    del copies, blk2, scratch2
    sync()

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

    # NEXT-4: chunk-first prefill of M = 2048 rows in chunks of 512
    # (prefill_chunk) through L = 8 iterations with the FP16-h cache written,
    # against the single-shot M = 2048 loop; and the h cache's K and V rebuild
    # (one GEMM of the last iteration's cached x, M = 512, on the K and V rows
    # of the QKV weight).
    inp = workloads.block(2048, seed=0)
    blk = qg.pack_block(inp.W, 4, D, F)
    h = inp.X.float().to(dev)
    hcache = torch.empty((8, 2048, D), dtype=torch.float16, device=dev)
    sc = torch.empty(qg.qg_loop_chunked_scratch_bytes(blk, 2048, 512), dtype=torch.uint8,
                     device=dev)

    def wall(fn, reps):
        fn()
        sync()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        sync()
        return (time.perf_counter() - t0) / reps

    chunked = wall(lambda: qg.qg_loop_range_chunked(blk, h, 0, 8, 512, sc, hcache=hcache), 10)
    single_scratch = qg.alloc_loop_scratch(blk, 2048)
    single = wall(lambda: qg.qg_loop_range(blk, h, 0, 8, single_scratch), 10)
    kv = blk.qkv.rows(D, 3 * D)
    xk = hcache[7, :512]
    Ykv = torch.empty(512, 2 * D, dtype=torch.float16, device=dev)
    rebuild = graph_leg(torch, lambda i: qg.qg_gemm_int4(xk, kv, Y=Ykv), 20, replays=20)
    flops = block_flops(2048) * 8
    out["next4_int4_chunked_prefill_m2048_c512_l8"] = {
        "ms_per_call": round(chunked * 1e3, 4), "TFLOP/s": round(flops / chunked / 1e12, 2),
        "frac_mfma": round(flops / chunked / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
        "single_shot_ms_per_call": round(single * 1e3, 4),
        "single_shot_TFLOP/s": round(flops / single / 1e12, 2),
        "kv_rebuild_m512_us": round(rebuild * 1e6, 2),
        "kv_rebuild_TFLOP/s": round(2.0 * 512 * D * 2 * D / rebuild / 1e12, 2),
        "method": "wall clock over 10 calls after a warm call (chunked, single shot); the K/V "
                  "rebuild GEMM graph-timed"}
    del blk, h, hcache, sc, single_scratch, kv, xk, Ykv
    sync()

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
    # In place, INT2 rows kept at the INT4 row stride (the pages' form, one
    # launch per weight): the INT4 data is restored from a saved copy before
    # each block (outside the timed calls).
    saved = [w.codes.clone() for w in w4s] + [w.scales.clone() for w in w4s] + \
        [w.zeros.clone() for w in w4s]
    t_in = 0.0
    for _ in range(reps):
        for i, w in enumerate(w4s):
            w.codes.copy_(saved[i])
            w.scales.copy_(saved[4 + i])
            w.zeros.copy_(saved[8 + i])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for w in w4s:
            qg.qg_requant_4to2(w, in_place=True)
        torch.cuda.synchronize()
        t_in += time.perf_counter() - t0
    t_in /= reps
    out["next1_requant_int4_to_int2_block_in_place"] = {
        "ms_per_block": round(t_in * 1e3, 4), "form": "INT4 row stride kept, one launch per weight",
        "bytes_moved": moved, "GB/s": round(moved / t_in / 1e9, 1)}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-clocks", action="store_true",
                    help="skip the clock-sampling windows (for kernel-trace runs: their extra "
                         "iterations, with a sysfs reader beside them, would dominate the trace)")
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
    ap.add_argument("--loops-target", action="store_true",
                    help="only run the loop workloads of the per-launch breakdown (for "
                         "rocprofv3 --kernel-trace and --pmc runs)")
    ap.add_argument("--loops-from", nargs="+", metavar="CSV",
                    help="write profiles/loop_kernels.json and .md from a --kernel-trace CSV of "
                         "--loops-target, then any --pmc counter CSVs of it (no GPU)")
    ap.add_argument("--loops-command", default="",
                    help="the command lines that produced the --loops-from CSVs, recorded as is")
    ap.add_argument("--trace-from", metavar="KERNEL_TRACE_CSV",
                    help="write profiles/roofline_trace.json and .md from a rocprofv3 "
                         "--kernel-trace CSV of this script run with --no-cpu --no-extra --no-clocks (no GPU)")
    ap.add_argument("--trace-command", default="",
                    help="the command line that produced the trace, recorded as is")
    args = ap.parse_args()

    if args.traffic_from:
        traffic_from(args.traffic_from[0], args.traffic_from[1], args.traffic_command)
        return
    if args.trace_from:
        trace_from(args.trace_from, args.trace_command)
        return
    if args.loops_from:
        loops_from(args.loops_from[0], args.loops_from[1:], args.loops_command)
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
    if args.loops_target:
        loops_target(qg, torch, workloads)
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
    # clock levels under the same workload (its own untimed window)
    clocks = None if args.no_clocks else sustained_clocks(
        torch, lambda: qg.qg_loop_range(blk, h, 0, L_MAIN, scratch), device_pci(torch))
    log(f"clocks under the decode loop: {clocks}")

    # ---- M=512 chunked prefill (C3): the INT4 block at M=512 rows for L=8;
    # the metric's TFLOP/s leg, and the loop whose kernels the prefill
    # roofline is taken from.
    c3 = c3_leg(qg, torch, workloads, clocks=not args.no_clocks)
    log(f"c3: {c3}")

    # ---- live legs: the decode roofline kernel's shape (the down-projection
    # GEMV, K=8192, N=2048, the same kernel and grid as in the loop) and the
    # M=512 FFN up projection (K=2048, N=8192, the same kernel and tile plan
    # as in the loop), each graph-timed over back-to-back launches with HIP
    # events on the stream that runs them.
    u = torch.empty(1, F, dtype=torch.float16, device=dev).normal_()
    y = torch.empty(1, D, dtype=torch.float16, device=dev)
    avg_s = graph_leg(torch, lambda i: qg.qg_gemm_int4(u, blk.down, Y=y), 200, replays=5)
    live_decode = {"kernel": "k_gemv (down projection, K=8192, N=2048, M=1)",
                   "bytes": blk.down.nbytes(), "us": round(avg_s * 1e6, 3),
                   "GB/s": round(blk.down.nbytes() / avg_s / 1e9, 1),
                   "method": "HIP events around 5 replays of a graph of 200 back-to-back "
                             "launches on cache-warm weights (period per launch)"}
    xp = torch.empty(512, D, dtype=torch.float16, device=dev).normal_()
    yp = torch.empty(512, F, dtype=torch.float16, device=dev)
    avg_p = graph_leg(torch, lambda i: qg.qg_gemm_int4(xp, blk.up, Y=yp), 50, replays=10)
    fl = 2.0 * 512 * D * F
    live_prefill = {"kernel": "ring MFMA GEMM (up projection, M=512, K=2048, N=8192)",
                    "flop": fl, "us": round(avg_p * 1e6, 3),
                    "TFLOP/s": round(fl / avg_p / 1e12, 1),
                    "method": "HIP events around 10 replays of a graph of 50 back-to-back "
                              "launches (period per launch)"}
    del xp, yp
    mem = memory_ceilings(torch)
    log(f"memory ceilings: {mem}")
    rec = trace_record()
    roofline, roofline_prefill = roofline_entries(rec, live_decode, live_prefill, mem)
    # traffic: FETCH_SIZE + WRITE_SIZE per launch of the same kernel, scaled
    # by the calibration copy, from the committed counter records
    tr = traffic_record()
    roofline["traffic"] = None
    if tr is not None and rec is not None and roofline.get("projection") in tr["projections"]:
        roofline["traffic"] = tr["projections"][roofline["projection"]]["hbm_bytes"]
        roofline["traffic_source"] = "profiles/traffic.json"
    lr = loops_record()
    if lr is not None and rec is not None:
        for e in lr["configs"]["c3_int4_block_m512_l8"]["kernels"]:
            d = e.get("derived", {})
            if e["label"] == roofline_prefill.get("projection") and "fetch_MB" in d and "write_MB" in d:
                roofline_prefill["traffic"] = int(round((d["fetch_MB"] + d["write_MB"]) * 1e6))
                roofline_prefill["traffic_source"] = "profiles/loop_kernels.json"
    log(f"roofline: {roofline}")
    log(f"roofline_prefill: {roofline_prefill}")

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
        "roofline_prefill": roofline_prefill,
        "c3_int4_block_m512_l8": c3,
        "memory": mem,
        "step_distribution": step_dist,
        "device": dict(device_info(torch), clocks_during_main_workload=clocks),
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
