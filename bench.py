#!/usr/bin/env python3
"""Benchmark of the HGEMM hot path on one MI355X.

A step is one C = A * Bt^T launch of the library's TN FP16 kernel at
M = N = K = 8192 (FP16 inputs uniform in [-1, 1], FP32 accumulation, FP16
output): the configuration whose throughput is quoted as a fraction of the
MI355X dense FP16 matrix peak.  Inputs are seeded synthetic data, resident
in HBM before the timed region starts.

Before the warmup steps the workload runs back to back for --settle-ms
(300 ms by default): when load starts after idle, the part's power
controller first pulls the engine clock far below the level it settles at,
and recovers over tens of milliseconds (`--clock-trace` measures this); the
settle phase keeps that transient out of the timed region and is reported in
the JSON line.

Prints one JSON line with TFLOPS (2*M*N*K / time), the roofline position of
the kernel (HIP-event timing of every launch on the launch stream, the engine
clock from the kernel's measurement copy and the fraction of the peak at
that clock), the same figures for all five workloads, and the CPU oracle's
throughput on a bounded sample of the headline workload.
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

PEAK_TFLOPS = 2516.6  # MI355X dense FP16/BF16 matrix peak: 256 CU x 4096 FLOP/clk x 2.4 GHz
CU_FLOP_PER_CLK = 256 * 4096  # the same peak per engine clock (the clock-adjusted peak's slope)
HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_hgemm_tn_f16_8192.json")
# the benched kernel's device code (the traffic figures stay valid while it is unchanged;
# its launch configuration, group_m 4 with the XCD remap, is recorded beside them)
KERNEL_SOURCES = ["device.hpp", "common.hpp", "gemm_kernel.hpp"]


def kernel_source_digest() -> str:
    """Digest of the benched kernel's device code, comments and layout left out
    (a comment edit does not change the kernel the counters were taken on)."""
    import re
    h = hashlib.sha256()
    for s in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "dense_half_precision_amd", "csrc", s)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_bytes(kernel_name: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_digest") != kernel_source_digest() or t.get("kernel") != kernel_name:
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(w, A, B, budget_s: float):
    """The CPU oracle on a bounded band of full output rows of the workload."""
    import oracle
    oracle.build(0, force=False)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    band = 16
    rows = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s and rows < w.M:
        r1 = min(w.M, rows + band)
        oracle.hgemm(w.layout, w.dtype, A, B, rows=(rows, r1))
        rows = r1
        band = min(band * 2, 256)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * w.N * w.K
    return {"value": flops / dt / 1e12, "unit": "TFLOPS", "cores": threads, "kind": "oracle",
            "sample": f"full output rows [0,{rows}) of {w.M} ({rows * w.N} of {w.M * w.N} "
                      f"elements, FP64 accumulation) in {dt:.1f} s"}


def oracle_table(only: int = 0) -> int:
    """CPU oracle timings per workload on this host (no GPU involved): full
    output for the three smaller workloads (and the smallest on one thread, in
    a child process), the 4096-element sample check and one band of M/64 full
    rows, extrapolated x64, for the two largest.  One JSON line each."""
    import subprocess
    import numpy as np
    import oracle
    from dense_half_precision_amd import inputs
    oracle.build(0, force=False)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    for w in inputs.WORKLOADS:
        if only and w.index != only:
            continue
        A, B = inputs.operands(w)
        rec = {"oracle_table": w.name, "threads": threads, "cpu_count": os.cpu_count()}
        if w.M * w.N * w.K <= 4096 ** 3:
            t0 = time.perf_counter()
            oracle.hgemm(w.layout, w.dtype, A, B)
            dt = time.perf_counter() - t0
            rec.update(full_s=round(dt, 4), gflops=round(w.flops / dt / 1e9, 2))
        else:
            rows, cols = inputs.stratified_samples(w.M, w.N, inputs.SAMPLE_SEED_BASE + w.index)
            t0 = time.perf_counter()
            oracle.hgemm_sampled(w.layout, w.dtype, A, B, rows, cols)
            rec["sample4096_s"] = round(time.perf_counter() - t0, 4)
            band = w.M // 64
            t0 = time.perf_counter()
            oracle.hgemm(w.layout, w.dtype, A, B, rows=(0, band))
            dt = time.perf_counter() - t0
            rec.update(band_rows=band, band_s=round(dt, 4), full_s_extrapolated=round(64 * dt, 2),
                       gflops=round(w.flops / (64 * dt) / 1e9, 2))
        print(json.dumps(rec), flush=True)
        if w.index == 1 and threads > 1 and not only:
            env = dict(os.environ, OMP_NUM_THREADS="1")
            r = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-table",
                                "--workload", "1"], env=env)
            if r.returncode != 0:
                return r.returncode
    return 0


def micro() -> int:
    """Microbenchmarks behind the design choices (one JSON line each): matrix-
    core issue rate per shape and operand data, LDS read throughput per
    access pattern, L2 and HBM streaming, and the read path of the NN
    operand at GEMM level (workload 3 computed four ways)."""
    import numpy as np
    import torch
    from dense_half_precision_amd import hgemm, inputs
    hgemm.lib()
    lib = hgemm.lib()
    sp = torch.cuda.current_stream().cuda_stream

    def timed(f, n=10, warm=3):
        for _ in range(warm):
            assert f() == hgemm.OK
        torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            assert f() == hgemm.OK
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    def emit(d):
        print(json.dumps(d), flush=True)

    waves, iters = 1024, 4000
    out = torch.empty(waves * 64, device="cuda")
    clk = torch.zeros(2 * waves, dtype=torch.int64, device="cuda")
    for shape in (0, 1):
        for rnd in (0, 1):
            ms = timed(lambda: lib.hgemm_probe_mfma_rate(shape, rnd, waves, iters, out.data_ptr(),
                                                         clk.data_ptr(), sp))
            c = clk.cpu().numpy().reshape(-1, 2)
            mhz = float(np.median(c[:, 0] / c[:, 1]) * 100.0)  # real-time counter: 100 MHz
            flop = waves * iters * 16 * (32768 if shape == 0 else 16384)
            emit({"micro": "mfma_rate", "shape": "32x32x16" if shape == 0 else "16x16x32",
                  "operands": "random" if rnd else "constant", "ms": round(ms, 4),
                  "tflops": round(flop / ms / 1e9, 1), "sclk_mhz": round(mhz),
                  "pct_of_clock_peak": round(100 * flop / ms / 1e9 / (256 * 4096 * mhz / 1e6), 1)})
    names = {0: "lane-contiguous", 1: "baseline 32-row fragments, XOR", 2: "baseline, plain",
             3: "baseline, XOR by row", 4: "production 16-row fragments, XOR",
             5: "production 16-row fragments, plain", 6: "production transposing read, XOR",
             7: "production transposing read, plain", 8: "16-row fragments on 64-byte rows"}
    wg, it = 512, 2000
    lout = torch.empty(wg * 256, device="cuda")
    for pat in range(9):
        ms = timed(lambda: lib.hgemm_probe_lds_read(wg, it, pat, lout.data_ptr(), sp))
        byts = wg * 256 * it * 16 * 16
        emit({"micro": "lds_read", "pattern": pat, "what": names[pat], "ms": round(ms, 4),
              "tb_per_s": round(byts / ms / 1e9, 2)})
    # which 16 lanes the LDS serves together for 16-byte reads: one pattern per
    # candidate grouping, free of bank conflicts only under that grouping
    for basis in LDS_LANE_GROUPINGS:
        offs = torch.tensor(lds_lane_pattern(basis), dtype=torch.int32, device="cuda")
        ms = timed(lambda: lib.hgemm_probe_lds_lanes(wg, it, offs.data_ptr(), lout.data_ptr(), sp))
        emit({"micro": "lds_lanes", "grouping": list(basis), "ms": round(ms, 4),
              "tb_per_s": round(wg * 256 * it * 16 * 16 / ms / 1e9, 2)})
    # L2-to-CU streaming out of an L2-resident 4 MiB window (each workgroup's
    # 64 KiB slides by 1 KiB per iteration), rows contiguous or 16 KiB apart
    # (one K step of a K = 8192 operand panel)
    window = 4 << 20
    buf = torch.empty(window, dtype=torch.uint8, device="cuda")
    for stride in (128, 16384):
        for mode, what in ((0, "registers"), (1, "direct-to-LDS"),
                           (4, "registers, 64-byte halves"), (5, "direct-to-LDS, 64-byte halves")):
            wgs, its = 1024, 256
            ms = timed(lambda: lib.hgemm_probe_l2_read(wgs, its, mode, buf.data_ptr(), window,
                                                       stride, lout.data_ptr(), sp))
            emit({"micro": "l2_stream", "row_stride": stride, "mode": what, "ms": round(ms, 4),
                  "tb_per_s": round(wgs * its * 65536 / ms / 1e9, 2)})
    w = inputs.workload(3)
    A, B = inputs.operands(w)
    dA = torch.from_numpy(A.view(np.int16)).cuda()
    dB = torch.from_numpy(B.view(np.int16)).cuda()
    dBt = torch.from_numpy(np.ascontiguousarray(B.T).view(np.int16)).cuda()
    dC = torch.empty((w.M, w.N), dtype=torch.int16, device="cuda")
    for name, fn, dB_ in (("tn_bf16_256x256x64", hgemm.hgemm_tn_ex, dBt),
                          ("nn_bf16_256x256x64", hgemm.hgemm_nn_ex, dB),
                          ("nn_bf16_256x256x64_plainlds", hgemm.hgemm_nn_ex, dB),
                          ("rs_nn_bf16_256x256x64_xor", hgemm.hgemm_nn_ex, dB)):
        k = hgemm.kernel_index(name)
        ms = timed(lambda: fn(w.M, w.N, w.K, w.dtype, dA.data_ptr(), dB_.data_ptr(),
                              dC.data_ptr(), sp, kernel=k), n=50, warm=10)
        emit({"micro": "nn_read_path", "workload": w.name, "kernel": name,
              "b_operand": "pre-transposed (Bt), 16-byte reads" if name.startswith("tn") else
              ("register transpose" if name.startswith("rs") else "transposing LDS read"),
              "ms": round(ms, 4), "tflops": round(w.flops / ms / 1e9, 1)})
    # wave specialisation (4 loader + 4 MFMA waves, 128 x 256 tile) against the
    # single-role pipeline on the same tile and the production 256 x 256 kernel,
    # and the 256 x 256 tile on eight waves (two per SIMD), both roles in every
    # wave or two groups alternating memory and MFMA phases
    for (M, N, K) in ((8192, 8192, 8192), (8192, 8192, 16384)):
        A = inputs.draw((M, K), "f16", "uniform", 1)
        Bt = inputs.draw((N, K), "f16", "uniform", 2)
        dA = torch.from_numpy(A.view(np.int16)).cuda()
        dB = torch.from_numpy(Bt.view(np.int16)).cuda()
        dC = torch.empty((M, N), dtype=torch.int16, device="cuda")
        for name in ("tn_f16_256x256x64", "tn_f16_256x256x64_w2x4", "tn_f16_256x256x64_pp",
                     "ws_tn_f16_128x256x64", "tn_f16_128x256x64"):
            k = hgemm.kernel_index(name)
            ms = timed(lambda: hgemm.hgemm_tn_ex(M, N, K, "f16", dA.data_ptr(), dB.data_ptr(),
                                                 dC.data_ptr(), sp, kernel=k), n=50, warm=15)
            emit({"micro": "wave_specialisation", "shape": f"{M}x{N}x{K}", "kernel": name,
                  "roles": "4 loader + 4 MFMA waves" if name.startswith("ws_") else
                  ("8 waves, both roles" if name.endswith("_w2x4") else
                   ("8 waves, two groups alternating memory and MFMA phases"
                    if name.endswith("_pp") else "4 waves, both roles")),
                  "ms": round(ms, 4), "tflops": round(2 * M * N * K / ms / 1e9, 1)})
        del dA, dB, dC
    return 0


def mix() -> int:
    """What memory instructions cost the matrix cores of the wave that issues
    them (one JSON line per case): hgemm_probe_mix with 64 MFMAs per
    iteration and 0..16 loads of each kind (1 KiB straight into LDS; 1 KiB
    into registers then written to LDS; 256 bytes straight into LDS), with
    and without 16 LDS fragment reads; cycles per MFMA (16 at full rate) and
    the extra cycles per load over the case without loads."""
    import numpy as np
    import torch
    from dense_half_precision_amd import hgemm
    lib = hgemm.lib()
    sp = torch.cuda.current_stream().cuda_stream
    wgs, iters, window = 256, 2000, 4 << 20
    buf = torch.zeros(window // 2, dtype=torch.int16, device="cuda")
    out = torch.empty(wgs * 256, device="cuda")
    clk = torch.zeros(2 * 4 * wgs, dtype=torch.int64, device="cuda")
    kinds = {0: "1 KiB direct-to-LDS", 1: "1 KiB into registers, then ds_write", 2: "256 B direct-to-LDS"}
    base = {}
    cases = [(nread, kind, nload) for nread in (0, 16) for kind in (0, 1, 2)
             for nload in (0, 2, 4, 8, 16)]
    cases += [(256 + nread, 0, nload) for nread in (0, 16) for nload in (0, 8, 16)]
    for nread, kind, nload in cases:
        if True:
            if True:
                for rep in range(3):  # the first launch warms the window into L2
                    st = lib.hgemm_probe_mix(kind, nload, nread, wgs, iters, buf.data_ptr(), window,
                                             out.data_ptr(), clk.data_ptr(), sp)
                    if st != hgemm.OK:
                        raise hgemm.HgemmError(st, "mix probe")
                torch.cuda.synchronize()
                c = clk.cpu().numpy().reshape(-1, 2).astype(np.float64)
                cyc = float(np.median(c[:, 0])) / (64.0 * iters)
                mhz = float(np.median(c[:, 0] / c[:, 1]) * 100.0)
                if nload == 0:
                    base[nread] = cyc
                line = {"micro": "mfma_load_mix", "load": kinds[kind], "loads_per_64_mfma": nload,
                        "lds_reads_per_64_mfma": nread % 256, "barrier_per_128_mfma": nread >= 256,
                        "cycles_per_mfma": round(cyc, 3),
                        "mfma_busy": round(16.0 / cyc, 4), "sclk_mhz": round(mhz)}
                if nload > 0:
                    line["extra_cycles_per_load"] = round((cyc - base[nread]) * 64.0 / nload, 2)
                print(json.dumps(line), flush=True)
    return 0


def compare() -> int:
    """This library's automatic choice against torch.mm (the vendor library) on
    the five workloads, one JSON line each, measured two ways: one launch at a
    time (an event pair around each launch and a wait for it: launch latency
    included), and back to back (wall clock over many launches, no events: the
    rate a caller that enqueues without waiting sees).  The two libraries
    alternate, round by round, so that clock drift under the power cap falls
    on both alike."""
    import time
    import numpy as np
    import torch
    from dense_half_precision_amd import hgemm, inputs
    lib = hgemm.lib()
    sp = torch.cuda.current_stream().cuda_stream

    def one_at_a_time(f, n):
        for _ in range(n // 4):
            f()
        torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return ts

    def back_to_back(f, n):
        for _ in range(n // 4):
            f()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            f()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n

    for widx in (1, 2, 3, 4, 5):
        w = inputs.workload(widx)
        A, B = inputs.operands(w)
        dA = torch.from_numpy(A.view(np.int16)).cuda()
        dB = torch.from_numpy(B.view(np.int16)).cuda()
        dC = torch.empty((w.M, w.N), dtype=torch.int16, device="cuda")
        cfn = lib.hgemm_tn if w.layout == "tn" else lib.hgemm_nn
        args = (w.M, w.N, w.K, hgemm.F16 if w.dtype == "f16" else hgemm.BF16,
                dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), sp)

        def ours():
            st = cfn(*args)
            if st != hgemm.OK:
                raise hgemm.HgemmError(st, "compare launch")

        tdt = torch.float16 if w.dtype == "f16" else torch.bfloat16
        a, b = dA.view(tdt), dB.view(tdt)
        vendor = (lambda: torch.mm(a, b.t())) if w.layout == "tn" else (lambda: torch.mm(a, b))
        n = 1000 if w.M <= 2048 else 50
        res = {"ours": ([], []), "torch.mm": ([], [])}
        for _ in range(4):
            for name, f in (("ours", ours), ("torch.mm", vendor)):
                res[name][0].extend(one_at_a_time(f, n))
                res[name][1].append(back_to_back(f, n))
        kern = hgemm.kernel_table()[hgemm.auto_kernel(
            hgemm.TN if w.layout == "tn" else hgemm.NN, w.dtype, w.M, w.N, w.K)]["name"]
        line = {"compare": w.name, "kernel": kern}
        for name, (single, b2b) in res.items():
            t1, t2 = float(np.median(single)), float(np.median(b2b))
            line[name] = {"one_at_a_time_us": round(t1 * 1e6, 2),
                          "one_at_a_time_tflops": round(w.flops / t1 / 1e12, 1),
                          "back_to_back_us": round(t2 * 1e6, 2),
                          "back_to_back_tflops": round(w.flops / t2 / 1e12, 1)}
        print(json.dumps(line), flush=True)
        del dA, dB, dC
    return 0


TAIL_SHAPES = [  # (layout, dtype, M, N, K): tiles of 256 x 256 that leave a partial round
    ("tn", "f16", 6144, 6144, 6144), ("nn", "bf16", 6144, 6144, 6144),
    ("tn", "f16", 7168, 7168, 7168), ("tn", "f16", 4352, 4352, 4096),
    ("nn", "bf16", 1536, 1536, 16384), ("tn", "f16", 512, 512, 65536),
    ("tn", "f16", 1024, 8192, 8192)]


def tail() -> int:
    """K split of the tail (one JSON line per shape): the automatic choice
    without a workspace, with one (hgemm_gemm_ws), and torch.mm (the vendor
    library) on the same operands; the three are timed in alternation so that
    clock drift under the power cap falls on all of them alike."""
    import numpy as np
    import torch
    from dense_half_precision_amd import hgemm, inputs
    sp = torch.cuda.current_stream().cuda_stream
    for lay, dt, M, N, K in TAIL_SHAPES:
        opB = hgemm.OP_T if lay == "tn" else hgemm.OP_N
        A = inputs.draw((M, K), dt, "normal", 1)
        B = inputs.draw((N, K) if lay == "tn" else (K, N), dt, "normal", 2)
        dA = torch.from_numpy(A.view(np.int16)).cuda()
        dB = torch.from_numpy(B.view(np.int16)).cuda()
        dC = torch.empty((M, N), dtype=torch.int16, device="cuda")
        ldb = K if lay == "tn" else N
        need = hgemm.gemm_ws_size(hgemm.OP_N, opB, M, N, K, dt)
        ws = torch.empty(max(need, 16) // 4, dtype=torch.float32, device="cuda")
        args = (hgemm.OP_N, opB, M, N, K, dt, 1.0, dA.data_ptr(), K, dB.data_ptr(), ldb, 0.0,
                dC.data_ptr(), N)
        tdt = torch.float16 if dt == "f16" else torch.bfloat16
        a, b = dA.view(tdt), dB.view(tdt)
        variants = {
            "unsplit": lambda: hgemm.hgemm_gemm(*args, sp),
            "split": lambda: hgemm.hgemm_gemm_ws(*args, ws.data_ptr(), need, sp),
            "torch.mm": (lambda: torch.mm(a, b.t())) if lay == "tn" else (lambda: torch.mm(a, b)),
        }
        times = {k: [] for k in variants}
        for _ in range(5):
            f = variants["unsplit"]
            assert f() == hgemm.OK and variants["split"]() == hgemm.OK
        for _ in range(3):
            for name, f in variants.items():
                for _ in range(3):
                    f()
                torch.cuda.synchronize()
                for _ in range(10):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    f()
                    e1.record()
                    e1.synchronize()
                    times[name].append(e0.elapsed_time(e1))
        flop = 2.0 * M * N * K
        ms = {k: float(np.median(v)) for k, v in times.items()}
        tiles = -(-M // 256) * -(-N // 256)
        print(json.dumps({"tail": f"{lay} {dt} {M}x{N}x{K}", "tiles_256": tiles,
                          "tail_tiles": tiles % 256, "workspace_mib": round(need / 2**20, 2),
                          "segments": need // (262144 * (tiles % 256)) if need else 0,
                          **{f"{k}_tflops": round(flop / v / 1e9, 1) for k, v in ms.items()},
                          "split_vs_unsplit": round(ms["unsplit"] / ms["split"], 3),
                          "split_vs_torch": round(ms["torch.mm"] / ms["split"], 3)}), flush=True)
        del dA, dB, dC, ws
    return 0


# TN f16 shapes of the automatic-choice sweep: squares, other K depths,
# skinny and ragged shapes.
SWEEP_SHAPES = ([(s, s, s) for s in (512, 768, 1024, 1536, 2048, 2560, 3072, 3584, 4096, 5120,
                                    6144, 7168, 8192)]
                + [(4096, 4096, 256), (4096, 4096, 1024), (4096, 4096, 16384), (2048, 2048, 8192),
                   (2048, 2048, 32768), (1024, 1024, 16384), (512, 512, 65536)]
                + [(1024, 8192, 8192), (8192, 1024, 8192), (256, 16384, 4096), (16384, 256, 4096),
                   (2048, 16384, 2048), (16384, 2048, 2048), (8192, 8192, 512)]
                + [(1000, 1000, 1000), (3000, 5000, 2000), (4000, 4000, 4000), (6000, 6000, 3000),
                   (8000, 8000, 8000)])
# A second set, for checking the cost model on shapes it was not tuned on:
# other TN sizes and NN bf16.
SWEEP_CHECK = ([("tn", "f16", s, s, s) for s in (2304, 2816, 3328, 3840, 4608)]
               + [("tn", "f16", 5632, 5632, 2816), ("tn", "f16", 7000, 5000, 4000),
                  ("tn", "f16", 12288, 12288, 2048), ("tn", "f16", 1536, 12288, 4096),
                  ("tn", "f16", 2560, 8192, 4096)]
               + [("nn", "bf16", s, s, s) for s in (2048, 2560, 3072, 4096, 6144)]
               + [("nn", "bf16", 1024, 8192, 8192), ("nn", "bf16", 6000, 6000, 3000)])


# A fifth set: A stored transposed (at_tn: At[K][M], Bt[N][K]; at_nn: At[K][M],
# B[K][N]).
SWEEP_AT = ([("at_tn", "f16", s, s, s) for s in (2048, 3072, 4608, 6144, 8192)]
            + [("at_nn", "f16", s, s, s) for s in (2048, 3072, 4608, 6144)]
            + [("at_tn", "f16", 1024, 8192, 8192), ("at_nn", "f16", 1024, 8192, 8192),
               ("at_nn", "bf16", 6000, 6000, 3000), ("at_tn", "bf16", 1536, 12288, 4096)])


def sweep_wide(count: int = 60, seed: int = 20261203):
    """A third set, drawn at random and not used to set any constant: TN f16
    and NN bf16 (two to one), M and N multiples of 64 in [512, 12288], K a
    multiple of 64 in [256, 16384], at most 2 TFLOP a shape."""
    import numpy as np
    g = np.random.Generator(np.random.PCG64(seed))
    out = []
    while len(out) < count:
        M, N = (64 * int(x) for x in g.integers(8, 193, size=2))
        K = 64 * int(g.integers(4, 257))
        if 2.0 * M * N * K > 2.0e12:
            continue
        lay, dt = ("tn", "f16") if len(out) % 3 != 2 else ("nn", "bf16")
        out.append((lay, dt, M, N, K))
    return out


# A fourth set: single rounds of 64 x 64 tiles (512^2 to 1024^2), K from 1024 to 16384,
# where the operands fall out of the L2 at some K and the ring depth decides.
SWEEP_SMALL = [("tn", "f16", m, m, k) for m in (512, 640, 768, 1024)
               for k in (1024, 2048, 3072, 4096, 8192, 16384)]
SWEEP_TILES = ("256x256x64", "192x256x64", "256x192x64", "192x192x64", "256x128x64", "128x128x64_r3",
               "128x128x64", "64x64x64_r4", "64x64x64")  # those the layout has


def sweep(which: str = "tn", wide_seed: int = 20261203) -> int:
    """The automatic choice against every production kernel (and the K split
    of the tail, given a workspace) over one set of shapes (`which`), operands
    uniform in [-1, 1].  Per shape, every candidate runs back to back between one pair
    of events, queued behind a QueueHold launch, in three alternating rounds
    (median).  One JSON line per shape: TFLOPS of each candidate (with a
    workspace, hgemm_gemm_ws runs the K split of the tail where its cost
    model expects a gain), the automatic choice without a workspace, and how
    far it, and the call with a workspace, fall behind the best candidate; a
    summary line at the end.  `which`: "tn" (SWEEP_SHAPES), "nn" (SWEEP_SHAPES as NN
    bf16), "check" (SWEEP_CHECK), "wide" (sweep_wide(seed=wide_seed)), "small"
    (SWEEP_SMALL) or "at" (SWEEP_AT, through hgemm_gemm_ex)."""
    import numpy as np
    import torch
    from dense_half_precision_amd import hgemm
    sp = torch.cuda.current_stream().cuda_stream
    hold = QueueHold()
    regrets, regrets_ws = [], []
    shapes = ([("tn", "f16", M, N, K) for M, N, K in SWEEP_SHAPES] if which == "tn"
              else [("nn", "bf16", M, N, K) for M, N, K in SWEEP_SHAPES] if which == "nn"
              else SWEEP_CHECK if which == "check" else SWEEP_SMALL if which == "small"
              else SWEEP_AT if which == "at" else sweep_wide(seed=wide_seed))
    for lay, dt, M, N, K in shapes:
        g = torch.Generator(device="cuda").manual_seed(M * 131 + N * 17 + K)
        tdt = torch.float16 if dt == "f16" else torch.bfloat16
        a_t, b_t = lay.startswith("at_"), lay.endswith("tn")
        dA = (torch.rand((K, M) if a_t else (M, K), device="cuda", generator=g) * 2 - 1).to(tdt)
        dB = (torch.rand((N, K) if b_t else (K, N), device="cuda", generator=g) * 2 - 1).to(tdt)
        dC = torch.empty((M, N), dtype=tdt, device="cuda")
        opA, lda = (hgemm.OP_T, M) if a_t else (hgemm.OP_N, K)
        opB, ldb = (hgemm.OP_T, K) if b_t else (hgemm.OP_N, N)
        args = (opA, opB, M, N, K, dt, 1.0, dA.data_ptr(), lda, dB.data_ptr(), ldb,
                0.0, dC.data_ptr(), N)
        need = hgemm.gemm_ws_size(opA, opB, M, N, K, dt)
        ws = torch.empty(max(need, 16) // 4, dtype=torch.float32, device="cuda")
        if a_t:
            def run(k):
                return hgemm.hgemm_gemm(*args, sp, kernel=k)
        else:
            fn = hgemm.hgemm_tn_ex if lay == "tn" else hgemm.hgemm_nn_ex

            def run(k):
                return fn(M, N, K, dt, dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), sp, kernel=k)
        names = {k["name"] for k in hgemm.kernel_table()}
        cands = {name: (lambda k=hgemm.kernel_index(name): run(k))
                 for name in (f"{lay}_{dt}_{t}" for t in SWEEP_TILES) if name in names}
        if need > 0:  # hgemm_gemm_ws: the K split of the tail where it estimates it faster
            cands["auto with workspace"] = lambda: hgemm.hgemm_gemm_ws(
                *args, ws.data_ptr(), need, sp)
        code = {"tn": hgemm.TN, "nn": hgemm.NN, "at_tn": hgemm.AT_TN, "at_nn": hgemm.AT_NN}[lay]
        auto = hgemm.kernel_table()[hgemm.auto_kernel(code, dt, M, N, K)]["name"]
        flop = 2.0 * M * N * K
        n = int(min(200, max(5, 20e-3 / (flop / 1.0e15))))  # about 20 ms a run
        times = {k: [] for k in cands}
        for f in cands.values():
            for _ in range(3):
                if f() != hgemm.OK:
                    raise hgemm.HgemmError(hgemm.ERR_INVALID_ARG, "sweep launch")
        torch.cuda.synchronize()
        for _ in range(3):
            for name, f in cands.items():
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                hold.hold(n * 0.03)
                e0.record()
                for _ in range(n):
                    f()
                e1.record()
                torch.cuda.synchronize()
                times[name].append(e0.elapsed_time(e1) / n)
        ms = {k: float(np.median(v)) for k, v in times.items()}
        # without a workspace the candidates are the kernels; with one, also
        # what hgemm_gemm_ws runs
        best = min((k for k in ms if k != "auto with workspace"), key=ms.get)
        r = ms[auto] / ms[best] - 1.0
        regrets.append(r)
        line = {"sweep": f"{lay} {dt} {M}x{N}x{K}", "tflops": {k: round(flop / v / 1e9, 1) for k, v in ms.items()},
                "auto": auto, "best_kernel": best, "auto_behind_best_kernel_pct": round(100 * r, 1)}
        if need > 0:
            best_all = min(ms.values())
            rws = ms["auto with workspace"] / best_all - 1.0
            regrets_ws.append(rws)
            line["with_workspace_behind_best_pct"] = round(100 * rws, 1)
            line["with_workspace_ahead_of_auto_pct"] = round(100 * (ms[auto] / ms["auto with workspace"] - 1), 1)
        print(json.dumps(line), flush=True)
        del dA, dB, dC, ws
        torch.cuda.empty_cache()
    print(json.dumps({"sweep_summary": which, "shapes": len(shapes),
                      "auto_behind_best_kernel_pct_mean": round(100 * float(np.mean(regrets)), 2),
                      "auto_behind_best_kernel_pct_max": round(100 * float(np.max(regrets)), 1),
                      "shapes_within_2pct": int(sum(r <= 0.02 for r in regrets)),
                      "with_workspace_shapes": len(regrets_ws),
                      "with_workspace_within_2pct_of_best": int(sum(r <= 0.02 for r in regrets_ws))}),
          flush=True)
    return 0


class EngineClock:
    """Engine clock a kernel runs at, from its measurement copy (the "_clk"
    twin of the same kernel, which writes the shader clock and the 100 MHz
    real-time clock at the start and end of every workgroup): total shader
    cycles over total real time of all workgroups of `launches` launches.

    The counter buffer is allocated up front; enqueue() adds the launches to
    the stream without waiting, so that they follow the preceding launches
    with no idle gap (a gap of a few milliseconds is enough for the power
    controller to pull the clock down again); mhz() reads the result after
    the caller has synchronised.  Unavailable (None) if the kernel has no
    measurement copy."""

    def __init__(self, w, dA, dB, dC, kname: str, launches: int):
        import torch
        from dense_half_precision_amd import hgemm
        self.k = None
        try:
            self.k = hgemm.kernel_index(kname + "_clk")
        except KeyError:
            return
        info = hgemm.kernel_table()[self.k]
        self.tiles = -(-w.M // info["bm"]) * -(-w.N // info["bn"])
        self.ts = torch.zeros((launches, self.tiles, 4), dtype=torch.int64, device="cuda")
        opB = hgemm.OP_T if w.layout == "tn" else hgemm.OP_N
        ldb = w.K if w.layout == "tn" else w.N
        self.args = (hgemm.OP_N, opB, w.M, w.N, w.K, w.dtype, 1.0, dA.data_ptr(), w.K,
                     dB.data_ptr(), ldb, 0.0, dC.data_ptr(), w.N)
        self.launches = launches

    def enqueue(self):
        import torch
        from dense_half_precision_amd import hgemm
        if self.k is None:
            return
        sp = torch.cuda.current_stream().cuda_stream
        for i in range(self.launches):
            st = hgemm.hgemm_gemm_ws(*self.args, self.ts[i].data_ptr(), self.tiles * 32, sp,
                                     kernel=self.k)
            if st != hgemm.OK:
                raise hgemm.HgemmError(st, "clock measurement launch")

    def mhz(self):
        import numpy as np
        if self.k is None:
            return None
        t = self.ts.cpu().numpy().astype(np.float64)
        cycles = (t[..., 2] - t[..., 0]).sum()
        real = (t[..., 3] - t[..., 1]).sum()
        return float(cycles / real * 100.0) if real > 0 else None


def settle(launch, settle_ms: float):
    """Launch back to back, in batches of up to 10 launches with a wait after
    each batch, until `settle_ms` of wall time have passed.  When load starts
    after idle, the power controller first pulls the engine clock well below
    where it settles (measured: `bench.py --clock-trace`); this keeps that
    transient out of the timed region.  Returns (launches, ms)."""
    import torch
    n, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(10):
            launch()
            n += 1
        torch.cuda.synchronize()
    return n, round((time.perf_counter() - t0) * 1e3, 1)


# Candidate 16-lane groupings of the LDS's 16-byte reads: the cosets of the
# span of these lane-index XOR masks (the groupings under which the measured
# rates of the fixed read patterns all come out right).
LDS_LANE_GROUPINGS = [(1, 2, 8, 20), (2, 5, 9, 17), (2, 8, 20, 37), (2, 12, 20, 37),
                      (1, 2, 12, 20), (2, 8, 20, 33), (2, 5, 8, 17), (2, 12, 20, 33)]


def lds_lane_pattern(basis, seed: int = 0):
    """64 per-lane byte offsets free of bank conflicts if the LDS serves the
    cosets of span(basis) together: coset g (in order of its smallest lane)
    covers the 16 16-byte bank groups of bytes [256g, 256g + 256) once, in a
    seeded random order (which makes the pattern conflict at least two-way
    under each other candidate)."""
    import numpy as np
    span = {0}
    for v in basis:
        span |= {x ^ v for x in span}
    rng = np.random.default_rng(seed)
    offs, seen, g = [0] * 64, set(), 0
    for l0 in range(64):
        if l0 in seen:
            continue
        grp = sorted(l0 ^ v for v in span)
        seen |= set(grp)
        order = rng.permutation(16)
        for i, lane in enumerate(grp):
            offs[lane] = 256 * g + 16 * int(order[i])
        g += 1
    return offs


class QueueHold:
    """One long launch of the matrix-core rate probe (random FP16 operands,
    one wave per SIMD, so the board draws about what a GEMM draws) that keeps
    the GPU busy while the host enqueues a run of short launches behind it.
    Without it, a kernel shorter than the host's launch path (the ctypes call
    and two event records) leaves the GPU idle between an event and its
    kernel, and the event pair measures that gap too."""

    US_PER_ITER = 0.15  # 1024 waves x 16 MFMAs of 16x16x32 per iteration, about 1.8 PFLOP/s

    def __init__(self):
        import torch
        self.out = torch.empty(1024 * 64, device="cuda")
        self.clocks = torch.empty(2 * 1024, dtype=torch.int64, device="cuda")

    def hold(self, ms: float):
        import torch
        from dense_half_precision_amd import hgemm
        iters = max(8, int(ms * 1e3 / self.US_PER_ITER) // 8 * 8)
        st = hgemm.lib().hgemm_probe_mfma_rate(1, 1, 1024, iters, self.out.data_ptr(),
                                               self.clocks.data_ptr(),
                                               torch.cuda.current_stream().cuda_stream)
        if st != hgemm.OK:
            raise hgemm.HgemmError(st, "queue hold")


def time_workload(w, dA, dB, dC, steps: int, warmup: int, settle_ms: float = 0.0):
    """The automatic choice on one workload: settle, the engine clock
    (measurement copy, enqueued with no gap), `warmup` launches, then `steps`
    launches with HIP events on the launch stream around each, then `steps`
    launches back to back between one pair of events.  Both runs are queued
    behind a QueueHold launch, so that the GPU executes them back to back
    whatever the host's launch rate.  Returns (kernel name, per-launch ms,
    back-to-back ms per launch, MHz)."""
    import numpy as np
    import torch
    from dense_half_precision_amd import hgemm
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    fn = hgemm.lib().hgemm_tn if w.layout == "tn" else hgemm.lib().hgemm_nn
    args = (w.M, w.N, w.K, hgemm.F16 if w.dtype == "f16" else hgemm.BF16, dA.data_ptr(),
            dB.data_ptr(), dC.data_ptr(), sp)
    kname = hgemm.kernel_table()[hgemm.auto_kernel(
        hgemm.TN if w.layout == "tn" else hgemm.NN, w.dtype, w.M, w.N, w.K)]["name"]
    clk = EngineClock(w, dA, dB, dC, kname, launches=steps)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    if settle_ms > 0:
        settle(lambda: fn(*args), settle_ms)
    clk.enqueue()
    for _ in range(warmup):
        fn(*args)
    torch.cuda.synchronize()
    hold = QueueHold()
    hold.hold(steps * 0.05)  # 50 us of host time per launch and its two events
    for a, b in ev:
        a.record(stream)
        st = fn(*args)
        b.record(stream)
        if st != hgemm.OK:
            raise hgemm.HgemmError(st, "workload launch")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hold.hold(steps * 0.03)
    e0.record(stream)
    for _ in range(steps):
        fn(*args)
    e1.record(stream)
    torch.cuda.synchronize()
    b2b = e0.elapsed_time(e1) / steps
    return kname, np.array([a.elapsed_time(b) for a, b in ev]), b2b, clk.mhz()


def workload_line(w, kname, per_ms, mhz, b2b_ms=None):
    import numpy as np
    med = float(np.median(per_ms))
    tf = w.flops / (med * 1e-3) / 1e12
    line = {"workload": w.name, "kernel": kname, "launches": int(len(per_ms)),
            "kernel_us_median": round(med * 1e3, 2), "kernel_us_min": round(float(per_ms.min()) * 1e3, 2),
            "tflops": round(tf, 1), "frac": round(tf / PEAK_TFLOPS, 4),
            "sclk_mhz": round(mhz) if mhz else None,
            "clock_adjusted_frac": round(tf / (CU_FLOP_PER_CLK * mhz * 1e-6), 4) if mhz else None}
    if b2b_ms is not None:
        line["back_to_back_us"] = round(b2b_ms * 1e3, 2)
        line["back_to_back_tflops"] = round(w.flops / (b2b_ms * 1e-3) / 1e12, 1)
    return line


def all_workloads(headline_index: int, headline_line: dict, settle_ms: float):
    """Every workload (1..5): kernel-event median over its launches, TFLOPS,
    fraction of the nameplate peak, engine clock and the fraction of the peak
    at that clock.  The headline workload's line is the one already measured."""
    import numpy as np
    import torch
    from dense_half_precision_amd import inputs
    lines = []
    for w in inputs.WORKLOADS:
        if w.index == headline_index:
            lines.append(headline_line)
            continue
        A, B = inputs.operands(w)
        dA = torch.from_numpy(A.view(np.int16)).cuda()
        dB = torch.from_numpy(B.view(np.int16)).cuda()
        dC = torch.empty((w.M, w.N), dtype=torch.int16, device="cuda")
        del A, B
        small = w.flops < 1e11
        kname, per, b2b, mhz = time_workload(w, dA, dB, dC, steps=200 if small else 30,
                                             warmup=50 if small else 10, settle_ms=settle_ms)
        lines.append(workload_line(w, kname, per, mhz, b2b))
        print(f"[bench] {w.name}: {lines[-1]}", file=sys.stderr, flush=True)
        del dA, dB, dC
        torch.cuda.empty_cache()
    return lines


def phases(widx: int, launches: int, settle_ms: float) -> int:
    """Where the main loop's cycles go: after the settle phase, `launches`
    launches of the workload kernel's "_ph" copy, which reads the shader
    clock around each K step's wait for the next step's loads (W) and its
    barrier (B), the rest of the step (R: its MFMAs, 16 cycles each, with
    the fragment reads, loads and address arithmetic among them; 128 MFMAs
    for the 256 x 256 tile, 32 for 128 x 128), then as many of its "_clk"
    copy (per-workgroup shader cycles of the unchanged kernel).  One JSON
    line: mean cycles per step of each phase over all waves, their spread
    over waves, the tile's start up to the first step's wait and its
    epilogue (cycles per tile), and the unchanged kernel's cycles per step
    (tile cycles / K steps, prologue and epilogue included)."""
    import numpy as np
    import torch
    from dense_half_precision_amd import hgemm, inputs
    w = inputs.workload(widx)
    A, B = inputs.operands(w)
    dA = torch.from_numpy(A.view(np.int16)).cuda()
    dB = torch.from_numpy(B.view(np.int16)).cuda()
    dC = torch.empty((w.M, w.N), dtype=torch.int16, device="cuda")
    kname = hgemm.kernel_table()[hgemm.auto_kernel(
        hgemm.TN if w.layout == "tn" else hgemm.NN, w.dtype, w.M, w.N, w.K)]["name"]
    kph = hgemm.kernel_index(kname + "_ph")
    info = hgemm.kernel_table()[kph]
    tiles = -(-w.M // info["bm"]) * -(-w.N // info["bn"])
    opB = hgemm.OP_T if w.layout == "tn" else hgemm.OP_N
    ldb = w.K if w.layout == "tn" else w.N
    sp = torch.cuda.current_stream().cuda_stream
    args = (hgemm.OP_N, opB, w.M, w.N, w.K, w.dtype, 1.0, dA.data_ptr(), w.K, dB.data_ptr(), ldb,
            0.0, dC.data_ptr(), w.N)
    ph = torch.zeros((launches, tiles, 4, 16), dtype=torch.int32, device="cuda")
    clk = EngineClock(w, dA, dB, dC, kname, launches=launches)
    fn = hgemm.lib().hgemm_tn if w.layout == "tn" else hgemm.lib().hgemm_nn
    largs = (w.M, w.N, w.K, hgemm.F16 if w.dtype == "f16" else hgemm.BF16, dA.data_ptr(),
             dB.data_ptr(), dC.data_ptr(), sp)
    settle(lambda: fn(*largs), settle_ms)
    for i in range(launches):
        st = hgemm.hgemm_gemm_ws(*args, ph[i].data_ptr(), tiles * 256, sp, kernel=kph)
        if st != hgemm.OK:
            raise hgemm.HgemmError(st, "phase-clock launch")
    clk.enqueue()
    torch.cuda.synchronize()
    v = ph.cpu().numpy().astype(np.int64).reshape(-1, 16)  # one row per wave
    kt = v[:, 3]
    assert (kt == kt[0]).all() and kt[0] > 1
    KT = int(kt[0])
    mfma_step = (info["bm"] // 32) * (info["bn"] // 32) * 2  # four waves of BM/2 x BN/2
    wait, bar, rest = v[:, 0] / KT, v[:, 1] / KT, v[:, 2] / (KT - 1)
    total = wait + bar + rest
    # the wait after c also waits for c's own result, and the wait after e
    # (one MFMA after it) for e's: one clock read's round trip, less one MFMA
    rt = float(np.median(v[:, 6]))
    t = clk.ts.cpu().numpy().astype(np.float64)
    tile_cyc = (t[..., 2] - t[..., 0]).ravel()
    q = lambda x: [round(float(np.percentile(x, p)), 1) for p in (10, 50, 90)]
    print(json.dumps({"phases": w.name, "kernel": kname, "launches": launches, "k_steps": KT,
                      "cycles_per_step": {"wait": round(float(wait.mean()), 1),
                                          "barrier": round(float(bar.mean()), 1),
                                          "rest": round(float(rest.mean()), 1),
                                          "total": round(float(total.mean()), 1),
                                          "ideal_mfma": mfma_step * 16},
                      "p10_p50_p90_over_waves": {"wait": q(wait), "barrier": q(bar),
                                                 "rest": q(rest), "total": q(total)},
                      "clock_read_round_trip": rt,
                      "corrected_cycles_per_step": {
                          "wait": round(float(wait.mean()) - rt, 1),
                          "barrier": round(float(bar.mean()), 1),
                          "rest": round(float(rest.mean()) - max(rt - 16.0, 0.0), 1),
                          "total": round(float(total.mean()) - rt - max(rt - 16.0, 0.0), 1)},
                      "last_step_after_barrier": round(float(v[:, 5].mean()), 1),
                      "tile_start_to_first_wait": round(float(v[:, 7].mean()), 1),
                      "epilogue": round(float(v[:, 8].mean()), 1),
                      "loop_cycles_per_step": round(float((v[:, 4] / KT).mean()), 1),
                      "unchanged_kernel_tile_cycles_per_step": round(float(tile_cyc.mean() / KT), 1),
                      "sclk_mhz": round(clk.mhz())}), flush=True)
    return 0


def sustain(widx: int, seconds: float) -> int:
    """The workload's automatic kernel back to back for `seconds` (a synchronisation
    every 20 launches), for watching board power and clocks with an outside
    tool; prints the wall-clock start and end (Unix seconds) and the rate."""
    import numpy as np
    import torch
    from dense_half_precision_amd import hgemm, inputs
    w = inputs.workload(widx)
    A, B = inputs.operands(w)
    dA = torch.from_numpy(A.view(np.int16)).cuda()
    dB = torch.from_numpy(B.view(np.int16)).cuda()
    dC = torch.empty((w.M, w.N), dtype=torch.int16, device="cuda")
    fn = hgemm.hgemm_tn if w.layout == "tn" else hgemm.hgemm_nn
    sp = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    t0 = time.time()
    n = 0
    while time.time() - t0 < seconds:
        for _ in range(20):
            st = fn(w.M, w.N, w.K, w.dtype, dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), sp)
            if st != hgemm.OK:
                raise hgemm.HgemmError(st, "sustained launch")
        n += 20
        torch.cuda.synchronize()
    t1 = time.time()
    print(json.dumps({"sustain": w.name, "start_unix_s": round(t0, 3), "end_unix_s": round(t1, 3),
                      "launches": n, "tflops": round(w.flops * n / (t1 - t0) / 1e12, 1)}), flush=True)
    return 0


def clock_trace(widx: int, launches: int, idle_s: float = 2.0) -> int:
    """The engine clock over a run of back-to-back launches that starts after
    `idle_s` of GPU idle time: the measurement copy of the workload's kernel
    ("_clk" twin) records per-workgroup shader and real-time clocks, and each
    window of 10 launches prints its start time, median duration, clock and
    TFLOPS (one JSON line per window).  Shows how long the power controller
    takes to settle after load starts."""
    import numpy as np
    import torch
    from dense_half_precision_amd import hgemm, inputs
    w = inputs.workload(widx)
    A, B = inputs.operands(w)
    dA = torch.from_numpy(A.view(np.int16)).cuda()
    dB = torch.from_numpy(B.view(np.int16)).cuda()
    dC = torch.empty((w.M, w.N), dtype=torch.int16, device="cuda")
    kname = hgemm.kernel_table()[hgemm.auto_kernel(
        hgemm.TN if w.layout == "tn" else hgemm.NN, w.dtype, w.M, w.N, w.K)]["name"]
    k = hgemm.kernel_index(kname + "_clk")
    info = hgemm.kernel_table()[k]
    tiles = -(-w.M // info["bm"]) * -(-w.N // info["bn"])
    ts = torch.zeros((launches, tiles, 4), dtype=torch.int64, device="cuda")
    opB = hgemm.OP_T if w.layout == "tn" else hgemm.OP_N
    ldb = w.K if w.layout == "tn" else w.N
    sp = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    time.sleep(idle_s)
    for i in range(launches):
        st = hgemm.hgemm_gemm_ws(hgemm.OP_N, opB, w.M, w.N, w.K, w.dtype, 1.0, dA.data_ptr(), w.K,
                                 dB.data_ptr(), ldb, 0.0, dC.data_ptr(), w.N,
                                 ts[i].data_ptr(), tiles * 32, sp, kernel=k)
        if st != hgemm.OK:
            raise hgemm.HgemmError(st, "clock trace launch")
    torch.cuda.synchronize()
    t = ts.cpu().numpy().astype(np.float64)
    r_first = t[..., 1].min()
    win = 10
    for j in range(0, launches, win):
        seg = t[j:j + win]
        dur = (seg[..., 3].max(axis=1) - seg[..., 1].min(axis=1)) / 100.0  # us
        mhz = [((x[:, 2] - x[:, 0]).sum() / (x[:, 3] - x[:, 1]).sum() * 100.0) for x in seg]
        print(json.dumps({"clock_trace": w.name, "kernel": kname, "launches": [j, j + len(seg) - 1],
                          "start_ms": round((seg[..., 1].min() - r_first) / 1e5, 3),
                          "dur_us_median": round(float(np.median(dur)), 2),
                          "sclk_mhz": round(float(np.median(mhz))),
                          "tflops": round(w.flops / float(np.median(dur)) / 1e6, 1)}), flush=True)
    # the second half of the launches, per XCD (workgroup b is dispatched to XCD b mod 8):
    # engine clock, median shader cycles per workgroup, and the sum of workgroup times over
    # 256 CUs x the launch time (how much of the launch the CUs spend inside a tile)
    late = t[launches // 2:]
    xcd = np.arange(tiles) % 8
    cyc = late[..., 2] - late[..., 0]
    real = late[..., 3] - late[..., 1]
    span = late[..., 3].max(axis=1) - late[..., 1].min(axis=1)
    print(json.dumps({"clock_trace_xcd": w.name, "launches": [launches // 2, launches - 1],
                      "sclk_mhz_per_xcd": [round(float(cyc[:, xcd == x].sum() / real[:, xcd == x].sum()
                                                        * 100.0)) for x in range(8)],
                      "kcycles_per_workgroup_per_xcd": [round(float(np.median(cyc[:, xcd == x])) / 1e3, 1)
                                                        for x in range(8)],
                      "workgroup_time_over_cu_time": round(float(np.median(real.sum(axis=1) /
                                                                           (256.0 * span))), 4)}),
          flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=4, help="workload index 1..5 (default 4)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU oracle sample budget (0 disables the cpu_baseline leg)")
    ap.add_argument("--kernel", type=int, default=-1, help="kernel table index (-1 = automatic)")
    ap.add_argument("--group-m", type=int, default=0)
    ap.add_argument("--xcd-remap", type=int, default=-1)
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of the GEMM, run a plain device copy of this many MiB "
                         "(reference point for scaling FETCH_SIZE/WRITE_SIZE counters)")
    ap.add_argument("--micro", action="store_true",
                    help="run the microbenchmarks behind the design choices and exit")
    ap.add_argument("--mix", action="store_true",
                    help="matrix-core rate with loads and LDS reads mixed in (hgemm_probe_mix)")
    ap.add_argument("--tail", action="store_true",
                    help="K split of the tail vs the unsplit choice and torch.mm, per shape")
    ap.add_argument("--vendor", action="store_true",
                    help="run the workload through torch.mm (the vendor library) instead")
    ap.add_argument("--compare", action="store_true",
                    help="automatic choice vs torch.mm on every workload, one launch at a "
                         "time and back to back")
    ap.add_argument("--oracle-table", action="store_true",
                    help="time the CPU oracle on every workload (host only) and exit")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="before the warmup steps, launch the workload back to back for this "
                         "long, so that the engine clock has left the power controller's "
                         "start-of-load dip (0: no settling)")
    ap.add_argument("--clock-trace", type=int, default=0, metavar="LAUNCHES",
                    help="print the engine clock over this many back-to-back launches of the "
                         "workload's kernel after 2 s idle, and exit")
    ap.add_argument("--sustain", type=float, default=0.0, metavar="SECONDS",
                    help="run the workload back to back for this many seconds (for watching "
                         "board power and clocks with an outside tool), print the rate, and exit")
    ap.add_argument("--sweep", choices=("tn", "nn", "check", "wide", "small", "at"), default=None,
                    help="the automatic choice against every production kernel over a grid of "
                         "TN f16 shapes ('tn'), the same as NN bf16 ('nn'), a second set with "
                         "NN bf16 ('check'), A stored transposed ('at'), a seeded "
                         "random third set ('wide') or single rounds of 64 x 64 tiles ('small'), "
                         "and exit")
    ap.add_argument("--wide-seed", type=int, default=20261203,
                    help="seed of the random shapes of --sweep wide")
    ap.add_argument("--phases", type=int, default=0, metavar="LAUNCHES",
                    help="after the settle phase, time the main loop's phases (wait, barrier, "
                         "rest) with the workload kernel's '_ph' copy over this many launches, "
                         "and exit")
    ap.add_argument("--no-workloads", action="store_true",
                    help="leave out the per-workload list (all five workloads timed after "
                         "the headline run)")
    args = ap.parse_args()
    if args.oracle_table:
        return oracle_table(args.workload if "--workload" in sys.argv else 0)
    if args.tail:
        if args.gpus != 1:
            print("bench.py: one GPU only", file=sys.stderr)
            return 2
        return tail()
    if args.clock_trace > 0:
        if args.gpus != 1:
            print("bench.py: one GPU only", file=sys.stderr)
            return 2
        return clock_trace(args.workload, args.clock_trace)
    if args.sustain > 0:
        if args.gpus != 1:
            print("bench.py: one GPU only", file=sys.stderr)
            return 2
        return sustain(args.workload, args.sustain)
    if args.sweep:
        if args.gpus != 1:
            print("bench.py: one GPU only", file=sys.stderr)
            return 2
        return sweep(args.sweep, args.wide_seed)
    if args.phases > 0:
        if args.gpus != 1:
            print("bench.py: one GPU only", file=sys.stderr)
            return 2
        return phases(args.workload, args.phases, args.settle_ms)
    if args.mix:
        if args.gpus != 1:
            print("bench.py: one GPU only", file=sys.stderr)
            return 2
        return mix()
    if args.micro:
        if args.gpus != 1:
            print("bench.py: one GPU only", file=sys.stderr)
            return 2
        return micro()
    if args.compare:
        if args.gpus != 1:
            print("bench.py: one GPU only", file=sys.stderr)
            return 2
        return compare()

    if args.gpus != 1:
        print(f"bench.py: this HGEMM runs on one GPU; --gpus {args.gpus} is not supported "
              f"(an M or N split across GPUs would need no exchange, but it is not "
              f"implemented)", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from dense_half_precision_amd import hgemm, inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 3
    hgemm.lib()  # fail loudly if the HIP library is not built

    if args.copy_mib > 0:
        n = args.copy_mib * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": args.warmup + args.steps}), flush=True)
        return 0

    w = inputs.workload(args.workload)
    A, B = inputs.operands(w)
    dev = torch.device("cuda:0")
    dA = torch.from_numpy(A.view(np.int16)).to(dev)
    dB = torch.from_numpy(B.view(np.int16)).to(dev)
    dC = torch.empty((w.M, w.N), dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    if args.vendor:
        # the same product through torch.mm (the vendor library), for comparison
        # and for counter runs on it; not a result of this library
        tdt = torch.float16 if w.dtype == "f16" else torch.bfloat16
        a, b = dA.view(tdt), dB.view(tdt)
        mm = (lambda: torch.mm(a, b.t())) if w.layout == "tn" else (lambda: torch.mm(a, b))
        for _ in range(args.warmup):
            mm()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            mm()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / args.steps * 1e3
        print(json.dumps({"vendor": "torch.mm", "workload": w.name, "steps": args.steps,
                          "ms_per_step": round(ms, 5), "tflops": round(w.flops / ms / 1e9, 2)}),
              flush=True)
        return 0
    fn = hgemm.hgemm_tn_ex if w.layout == "tn" else hgemm.hgemm_nn_ex
    kern = args.kernel if args.kernel >= 0 else hgemm.auto_kernel(
        hgemm.TN if w.layout == "tn" else hgemm.NN, w.dtype, w.M, w.N, w.K)
    kname = hgemm.kernel_table()[kern]["name"]

    def launch():
        st = fn(w.M, w.N, w.K, w.dtype, dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), sp,
                kernel=kern, group_m=args.group_m, xcd_remap=args.xcd_remap)
        if st != hgemm.OK:
            raise hgemm.HgemmError(st, "bench launch")

    print(f"[bench] {w.describe()}; kernel {kname}; warmup {args.warmup}, steps {args.steps}",
          file=sys.stderr, flush=True)
    # engine clock: the kernel's measurement copy, enqueued between the settle
    # phase and the warmup steps with no gap (outside the timed region)
    clk = EngineClock(w, dA, dB, dC, kname, launches=max(args.steps, 10))
    settled = settle(launch, args.settle_ms) if args.settle_ms > 0 else (0, 0.0)
    print(f"[bench] clock settle: {settled[0]} launches in {settled[1]} ms", file=sys.stderr,
          flush=True)
    clk.enqueue()
    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    mhz = clk.mhz()

    # timed region: events on the launch stream around every launch
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        launch()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])  # ms
    ms_step = wall * 1e3 / args.steps
    value = w.flops / (ms_step * 1e-3) / 1e12
    k_avg = float(per.mean())
    achieved = w.flops / (k_avg * 1e-3) / 1e12
    print(f"[bench] kernel ms: mean {k_avg:.4f} median {np.median(per):.4f} min {per.min():.4f} "
          f"max {per.max():.4f}; wall ms/step {ms_step:.4f}", file=sys.stderr, flush=True)

    print(f"[bench] engine clock {mhz:.0f} MHz" if mhz else "[bench] engine clock n/a",
          file=sys.stderr, flush=True)
    tb = traffic_bytes(kname)
    out = {
        "metric": "HGEMM TFLOPS and % of MI355X dense FP16/BF16 MFMA peak at 4096³/8192³",
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "layout": w.layout, "M": w.M, "N": w.N, "K": w.K,
                   "inputs": w.describe(), "kernel": kname, "accumulate": "fp32",
                   "pct_of_peak": round(100.0 * value / PEAK_TFLOPS, 2),
                   "clock_settle": {"launches": settled[0], "ms": settled[1],
                                    "note": "back-to-back launches before the warmup steps, "
                                            "outside the timed region"}},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4),
                     "traffic": tb,
                     "kernel_ms": {"mean": round(k_avg, 5), "median": round(float(np.median(per)), 5),
                                   "min": round(float(per.min()), 5), "max": round(float(per.max()), 5)},
                     "algorithmic_flops_per_launch": w.flops,
                     "algorithmic_bytes_per_launch": w.algorithmic_bytes,
                     "sclk_mhz": round(mhz) if mhz else None,
                     "clock_adjusted_peak": round(CU_FLOP_PER_CLK * mhz * 1e-6, 1) if mhz else None,
                     "clock_adjusted_frac": (round(achieved / (CU_FLOP_PER_CLK * mhz * 1e-6), 4)
                                             if mhz else None)},
    }
    if not args.no_workloads:
        out["workloads"] = all_workloads(w.index, workload_line(w, kname, per, mhz),
                                         args.settle_ms)
    if args.cpu_seconds > 0:
        print(f"[bench] cpu_baseline: oracle for ~{args.cpu_seconds:.0f} s", file=sys.stderr,
              flush=True)
        out["cpu_baseline"] = cpu_baseline(w, A, B, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
