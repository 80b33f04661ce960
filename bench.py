#!/usr/bin/env python3
"""Benchmark of the MI355X dense GEMM (one JSON line on stdout).

A step is one call of the library's GEMM on the workload's operands, already
resident in HBM: D = A @ B.T in FP16 at M = N = K = 4096 by default ("TIRx
GEMM on Blackwell", "The short version").  ``--workload`` picks another of the
seeded synthetic workloads in ``dense_gemm_08_amd/inputs.py``.

Reported:
* value: TFLOP/s = 2*M*N*K*steps / (wall time of the timed region);
* roofline: the GEMM kernel against the dense FP16/BF16 (or FP8) MFMA peak,
  with its average duration from HIP events recorded on the launch stream
  around the timed calls; HBM-side bytes per call from profiles/traffic.json
  (rocprofv3 counters recorded for this kernel source, else null); and the
  10th/50th/90th percentiles of up to 200 further calls each bracketed by
  its own pair of events (isolated calls: see launch_note);
* cpu_baseline: the CPU oracle's full product (FP64, test infrastructure)
  timed on a bounded block of rows of the same workload on this host's
  cores, with the CPU model.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "e4m3": 5000.0}  # MI355X dense MFMA, published

# The pages' own measured figure for a workload, where one exists: the
# 4096^3 FP16 A.B^T product of their final kernel (two consumers sharing the
# staged B tile) on one NVIDIA B200 ("TIRx GEMM on Blackwell", V9).  Other
# hardware: `vs_baseline` is context, not a target.
PAGE_TFLOPS = {"square_nt": (1263.9, "pages' V9 kernel on one NVIDIA B200 (other hardware; context)")}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="square_nt",
                    help="a workload of dense_gemm_08_amd/inputs.py: WORKLOADS (FP16/BF16), "
                         "SHARD_WORKLOADS (one GPU's share of the large A @ B product split "
                         "over 2, 4 or 8 GPUs) or MX_WORKLOADS (FP8 block-scaled)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=150.0,
                    help="before the warm-up steps, run untimed calls back to back for this many "
                         "milliseconds: under this load the chip's power management takes tens "
                         "of milliseconds to settle its clocks, and the calls in that window run "
                         "up to 30%% slower than in the steady state (0: no settling)")
    ap.add_argument("--workspace", action="store_true",
                    help="call the workspace-passing entry point (dense_gemm_ex / "
                         "gemm_nt_e4m3_mx_ex) with a workspace allocated once, before the "
                         "timed region, instead of the plain entry point (which takes its "
                         "workspace, where the call needs one, from the stream-ordered allocator "
                         "on every call); with --sweep or --small-m-sweep, time that form "
                         "beside the plain entry point")
    ap.add_argument("--split-k", type=int, default=0,
                    help="with --workspace (FP16/BF16 workloads): the plan override "
                         "dense_gemm_options.split_k (0: the library's choice, 1: no split, "
                         "n: n parts)")
    ap.add_argument("--tile-n", type=int, default=0,
                    help="with --workspace (FP16/BF16 workloads): the plan override "
                         "dense_gemm_options.tile_n (0: the library's choice, 128 or 256)")
    ap.add_argument("--ld-pad", type=int, default=0,
                    help="extra elements on every leading dimension (lda, ldb, ldd)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of the GEMM, time a plain device copy of this many MiB "
                         "(the known-size reference for scaling the FETCH_SIZE/WRITE_SIZE "
                         "counters of a rocprofv3 --pmc run)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM bytes per launch measured with rocprofv3 counters")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of one workload, time D = A @ B.T (FP16) at M = 8192 over a grid "
                         "of N and K (one JSON line per shape, torch.mm timed beside it)")
    ap.add_argument("--shapes", default="",
                    help="with --sweep: a comma-separated list of MxNxK shapes to time instead "
                         "of the grid (e.g. 4096x4096x4096,8192x16384x16384)")
    ap.add_argument("--small-m-sweep", action="store_true",
                    help="instead of one workload, time D = A @ B.T (FP16) at small M (1 to 512) "
                         "against N, K of 4096 to 16384, torch.mm timed beside it (shapes outside "
                         "the pages' workloads: where the 256-row tile computes mostly padding)")
    ap.add_argument("--small-m-sweep-nn", action="store_true",
                    help="the same for D = A @ B (BF16, B row-major K x N) at M of 1 to 128, "
                         "where the small-output kernel and the tiled one divide the shapes")
    ap.add_argument("--small-m-sweep-mx", action="store_true",
                    help="the same for the FP8 block-scaled D = A @ B.T at M of 1 to 128, "
                         "torch._scaled_mm timed beside it")
    ap.add_argument("--seed", type=int, default=8192)
    ap.add_argument("--ladder", action="store_true",
                    help="instead of one workload, time each optimisation-step kernel "
                         "(gemm_nt_f16_ladder levels 1-9) on the 4096^3 FP16 workload "
                         "(one JSON line per level)")
    ap.add_argument("--ladder-levels", default="1,2,3,4,5,6,7,8,9",
                    help="with --ladder: the levels to time, comma-separated")
    ap.add_argument("--ladder-seconds", type=float, default=0.0,
                    help="with --ladder: time each level over this many seconds of back-to-back "
                         "calls (after the clock settling) instead of --steps / 5 calls")
    ap.add_argument("--wave-fill", action="store_true",
                    help="instead of one workload, time D = A @ B.T (FP16) at M = 256 t, N = K = "
                         "4096 for t = 8 ... 16 (128 to 256 tiles of 256 x 256 on the chip's "
                         "256 CUs, one tile each, no split), each for --fill-seconds after the "
                         "clock settling: how the call time follows the number of busy CUs")
    ap.add_argument("--fill-seconds", type=float, default=4.0,
                    help="with --wave-fill: seconds of back-to-back calls timed per shape")
    ap.add_argument("--mx-sweep", action="store_true",
                    help="instead of one workload, time the FP8 block-scaled product at M = 8192 "
                         "over the sweep grid (one JSON line per shape, torch._scaled_mm with "
                         "the same block scales and with per-tensor scales timed beside it)")
    return ap.parse_args()


SWEEP_GRID = [1024, 2048, 4096, 8192, 16384]


def sweep_shapes(k_extra: int = 40):
    """M = 8192 with N and K over powers of two from 1024 to 16384, plus
    ragged neighbours: N + 128 (a half-filled last tile column) at K = 4096
    and K + k_extra (a partial last K step; 32 for the block-scaled product,
    whose K is a multiple of its 32-value scale blocks) at N = 4096."""
    shapes = [(8192, n, k) for n in SWEEP_GRID for k in SWEEP_GRID]
    shapes += [(8192, n + 128, 4096) for n in SWEEP_GRID]
    shapes += [(8192, 4096, k + k_extra) for k in SWEEP_GRID]
    return shapes


LADDER = {
    1: "V3: 128x128 tiles, one workgroup each, thread copies, no overlap",
    2: "V4: + LDS-DMA loads (the copy engine)",
    3: "V5: + two LDS stages (loads overlap compute)",
    4: "V6: + persistent grouped XCD-aware grid",
    5: "V8/V9: + 256x256 tiles (staged tiles shared by two waves each)",
    6: "library kernel: + fine-grained schedule",
    7: "V7: level 4 + a producer wave issuing every load (warp specialization)",
    8: "level 5 with 32x32x16 MFMAs instead of 16x16x32 (MFMA shape comparison)",
    9: "level 5 with eight 128x64 waves (two per SIMD) instead of four 128x128",
}


def run_ladder(args):
    """Each optimisation-step kernel on the 4096^3 FP16 A @ B.T workload
    (operands resident in HBM): clock settling and warm-up, then HIP events
    around back-to-back calls on the launch stream."""
    import torch
    from dense_gemm_08_amd import binding, inputs
    lib = binding.load_library()
    w = inputs.WORKLOADS["square_nt"]
    A, B = inputs.make_operands(w)
    dev = torch.device("cuda:0")
    Ad = torch.from_numpy(A.view(np.int16)).to(dev)
    Bd = torch.from_numpy(B.view(np.int16)).to(dev)
    Dd = torch.empty((w.M, w.N), dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream()
    levels = [int(x) for x in args.ladder_levels.split(",") if x]
    for level in levels:
        what = LADDER[level]

        def step():
            st = lib.gemm_nt_f16_ladder(level, w.M, w.N, w.K, Ad.data_ptr(), w.K, Bd.data_ptr(),
                                        w.K, Dd.data_ptr(), w.N, stream.cuda_stream)
            if st != 0:
                raise binding.DenseGemmError(st, "gemm_nt_f16_ladder")
        t_end = time.perf_counter() + args.settle_ms * 1e-3
        while time.perf_counter() < t_end:
            for _ in range(8):
                step()
            torch.cuda.synchronize()
        for _ in range(max(3, args.warmup // 10)):
            step()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        steps = max(5, args.steps // 5)
        e0.record(stream)
        if args.ladder_seconds > 0:
            steps = 0
            t_end = time.perf_counter() + args.ladder_seconds
            while time.perf_counter() < t_end:
                for _ in range(20):
                    step()
                steps += 20
                torch.cuda.synchronize()
        else:
            for _ in range(steps):
                step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        print(json.dumps({"mode": "ladder", "level": level, "what": what, "M": w.M, "N": w.N,
                          "K": w.K, "steps": steps, "kernel_ms": round(ms, 5),
                          "tflops": round(w.flops / ms / 1e9, 1)}), flush=True)


SMALL_M = [(m, n, k) for m in (1, 16, 64, 128, 256, 512)
           for n, k in ((4096, 4096), (8192, 8192), (16384, 4096))]
SMALL_M_NN = [(m, n, k) for m in (1, 16, 64, 128)
              for n, k in ((128, 4096), (1024, 1024), (1024, 4096), (4096, 4096), (8192, 8192),
                           (16384, 4096))]


def run_sweep(args, shapes=None, layout="nt"):
    """Per shape: N(0,1)/8 operands (FP16 for D = A @ B.T, BF16 for D = A @ B)
    from torch's seeded device generator (timing only; tests check these
    shapes' paths against the oracle), warm-up, then HIP events around about
    50 ms of back-to-back calls on the launch stream, torch.mm's beside them.
    Each line names the kernel the library's plan runs (small-output or
    tiled)."""
    import ctypes
    import torch
    from dense_gemm_08_amd import binding
    lib = binding.load_library()
    fmt = "f16" if layout == "nt" else "bf16"
    dtype = torch.half if layout == "nt" else torch.bfloat16
    entry = lib.gemm_nt_f16 if layout == "nt" else lib.gemm_nn_bf16
    plan = (ctypes.c_int64 * 10)()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    stream = torch.cuda.current_stream()

    def timed(fn, steps, warm):
        for _ in range(warm):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    for M, N, K in (shapes or sweep_shapes()):
        A = (torch.randn(M, K, device=dev, generator=gen) * 0.125).to(dtype)
        B = (torch.randn(*((N, K) if layout == "nt" else (K, N)), device=dev, generator=gen)
             * 0.125).to(dtype)
        ldb = K if layout == "nt" else N
        D = torch.empty(M, N, dtype=dtype, device=dev)
        Dt = torch.empty(M, N, dtype=dtype, device=dev)
        flops = 2.0 * M * N * K
        steps = max(5, min(200, int(0.05 / (flops / 1.2e15))))
        if lib.dense_gemm_plan(0 if layout == "nt" else 1, M, N, K, cus, plan) != 0:
            raise RuntimeError("no plan for %d x %d x %d" % (M, N, K))

        def ours():
            st = entry(M, N, K, A.data_ptr(), K, B.data_ptr(), ldb, D.data_ptr(), N,
                       stream.cuda_stream)
            if st != 0:
                raise binding.DenseGemmError(st, "gemm_%s_%s" % (layout, fmt))

        def ref():
            torch.mm(A, B.t() if layout == "nt" else B, out=Dt)

        ms = timed(ours, steps, max(3, steps // 4))
        ms_ref = timed(ref, steps, max(3, steps // 4))
        nbytes = 2.0 * (M * K + N * K + M * N)  # A, B and D once
        line = {"mode": "sweep", "layout": layout, "dtype": fmt, "M": M, "N": N, "K": K,
                "kernel": "small" if plan[7] == 512 else "tiled",
                "tile": [int(plan[0]), int(plan[1])], "splits": int(plan[8]),
                "steps": steps,
                "kernel_ms": round(ms, 5), "tflops": round(flops / ms / 1e9, 1),
                "alg_tb_s": round(nbytes / ms / 1e9, 3),
                "torch_mm_ms": round(ms_ref, 5),
                "torch_mm_tflops": round(flops / ms_ref / 1e9, 1),
                "torch_mm_alg_tb_s": round(nbytes / ms_ref / 1e9, 3)}
        if args.workspace:
            # the same product through dense_gemm_ex, its workspace allocated
            # once (no stream-ordered allocation per call)
            need = binding.workspace_size(layout, fmt, M, N, K, A.data_ptr(), K, B.data_ptr(),
                                          ldb)
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

            def ours_ws():
                st = lib.dense_gemm_ex(binding.OPS[(layout, fmt)], M, N, K, A.data_ptr(), K,
                                       B.data_ptr(), ldb, D.data_ptr(), N, None, ws.data_ptr(),
                                       need, stream.cuda_stream)
                if st != 0:
                    raise binding.DenseGemmError(st, "dense_gemm_ex")
            ms_ws = timed(ours_ws, steps, max(3, steps // 4))
            line.update({"workspace_bytes": need, "ex_ms": round(ms_ws, 5),
                         "ex_alg_tb_s": round(nbytes / ms_ws / 1e9, 3)})
            del ws
        print(json.dumps(line), flush=True)
        del A, B, D, Dt


WAVE_FILL = [8, 10, 12, 14, 15, 16]


def run_wave_fill(args):
    """Products with 128 ... 256 tiles of 256 x 256 (one per CU at most) and
    the same K, through dense_gemm_ex with the tile width and the split fixed
    (256 wide, no split), so that only the number of busy CUs changes.  Per
    shape: the clock settling, then HIP events around --fill-seconds of
    back-to-back calls.  Under the board's power limit, a call time that
    falls in proportion to the tiles means the idle CUs' power goes to the
    busy ones; a flat one, that the idle CUs are lost."""
    import ctypes
    import torch
    from dense_gemm_08_amd import binding
    lib = binding.load_library()
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    stream = torch.cuda.current_stream()
    opts = binding.Options(1, 256)
    N = K = 4096
    B = (torch.randn(N, K, device=dev, generator=gen) * 0.125).half()
    A_all = (torch.randn(256 * max(WAVE_FILL), K, device=dev, generator=gen) * 0.125).half()
    D = torch.empty(256 * max(WAVE_FILL), N, dtype=torch.half, device=dev)
    rows = []
    for t in WAVE_FILL:
        M = 256 * t
        need = binding.workspace_size("nt", "f16", M, N, K, A_all.data_ptr(), K, B.data_ptr(), K,
                                      opts)
        if need:
            raise RuntimeError("the wave-fill shapes need no workspace, got %d bytes" % need)

        def step():
            st = lib.dense_gemm_ex(binding.OPS[("nt", "f16")], M, N, K, A_all.data_ptr(), K,
                                   B.data_ptr(), K, D.data_ptr(), N, ctypes.byref(opts),
                                   None, 0, stream.cuda_stream)
            if st != 0:
                raise binding.DenseGemmError(st, "dense_gemm_ex")
        t_end = time.perf_counter() + args.settle_ms * 1e-3
        while time.perf_counter() < t_end:
            for _ in range(8):
                step()
            torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        steps = 0
        e0.record(stream)
        t_end = time.perf_counter() + args.fill_seconds
        while time.perf_counter() < t_end:
            for _ in range(20):
                step()
            steps += 20
            torch.cuda.synchronize()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        rows.append((t, ms))
        flops = 2.0 * M * N * K
        print(json.dumps({"mode": "wave_fill", "M": M, "N": N, "K": K, "tiles": 16 * t,
                          "steps": steps, "kernel_ms": round(ms, 5),
                          "tflops": round(flops / ms / 1e9, 1)}), flush=True)
    full = dict(rows).get(16)
    if full:
        for t, ms in rows:
            print(json.dumps({"mode": "wave_fill_ratio", "tiles": 16 * t,
                              "time_over_full": round(ms / full, 4),
                              "tiles_over_full": round(t / 16, 4)}), flush=True)


def _event_timer(stream):
    import torch

    def timed(fn, steps, warm):
        for _ in range(warm):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps
    return timed


SMALL_M_MX = [(m, n, k) for m in (1, 16, 64, 128)
              for n, k in ((1024, 1024), (1024, 4096), (4096, 4096), (4096, 8192),
                           (8192, 8192), (16384, 4096))]


def run_mx_sweep(args, shapes=None):
    """The FP8 block-scaled product over the M = 8192 sweep shapes (or the
    given ones): random finite E4M3 codes and E8M0 scales from torch's seeded
    device generator (timing only; tests check the product against the
    oracle), HIP events around about 50 ms of back-to-back calls.  Beside it,
    torch._scaled_mm with the same 1 x 32 block scales and, where it runs,
    with one scale per tensor (the library products of this PyTorch build).
    Each line names the kernel the library's plan runs (small-output or
    tiled) and its K parts."""
    import ctypes
    import torch
    from dense_gemm_08_amd import binding
    lib = binding.load_library()
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    stream = torch.cuda.current_stream()
    timed = _event_timer(stream)
    plan = (ctypes.c_int64 * 10)()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for M, N, K in (shapes or sweep_shapes(k_extra=32)):
        A = torch.randint(0, 255, (M, K), device=dev, generator=gen, dtype=torch.uint8)
        B = torch.randint(0, 255, (N, K), device=dev, generator=gen, dtype=torch.uint8)
        A[(A & 0x7F) == 0x7F] = 0
        B[(B & 0x7F) == 0x7F] = 0
        SA = torch.randint(120, 134, (M, K // 32), device=dev, generator=gen, dtype=torch.uint8)
        SB = torch.randint(120, 134, (N, K // 32), device=dev, generator=gen, dtype=torch.uint8)
        D = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        flops = 2.0 * M * N * K
        steps = max(5, min(200, int(0.05 / (flops / 2.4e15))))

        def ours():
            st = lib.gemm_nt_e4m3_mx(M, N, K, A.data_ptr(), K, SA.data_ptr(), K // 32,
                                     B.data_ptr(), K, SB.data_ptr(), K // 32, D.data_ptr(), N,
                                     stream.cuda_stream)
            if st != 0:
                raise binding.DenseGemmError(st, "gemm_nt_e4m3_mx")

        if lib.gemm_nt_e4m3_mx_plan(M, N, K, cus, plan) != 0:
            raise RuntimeError("no plan for %d x %d x %d" % (M, N, K))
        nbytes = M * K + N * K + (M + N) * (K // 32) + 2.0 * M * N  # A, B, scales, D once
        rec = {"mode": "mx_sweep", "M": M, "N": N, "K": K, "steps": steps,
               "kernel": "small" if plan[7] == 512 else "tiled", "tile": [int(plan[0]), int(plan[1])],
               "splits": int(plan[8])}
        ms = timed(ours, steps, max(3, steps // 4))
        rec.update(kernel_ms=round(ms, 5), tflops=round(flops / ms / 1e9, 1),
                   alg_tb_s=round(nbytes / ms / 1e9, 3))
        if args.workspace:
            # the same product through gemm_nt_e4m3_mx_ex, its workspace
            # allocated once (no stream-ordered allocation per call)
            need = binding.mx_workspace_size(M, N, K)
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

            def ours_ws():
                st = lib.gemm_nt_e4m3_mx_ex(M, N, K, A.data_ptr(), K, SA.data_ptr(), K // 32,
                                            B.data_ptr(), K, SB.data_ptr(), K // 32, D.data_ptr(),
                                            N, ws.data_ptr(), need, stream.cuda_stream)
                if st != 0:
                    raise binding.DenseGemmError(st, "gemm_nt_e4m3_mx_ex")
            ms_ws = timed(ours_ws, steps, max(3, steps // 4))
            rec.update(workspace_bytes=need, ex_ms=round(ms_ws, 5),
                       ex_alg_tb_s=round(nbytes / ms_ws / 1e9, 3))
            del ws
        a8, b8 = A.view(torch.float8_e4m3fn), B.view(torch.float8_e4m3fn)
        refs = {
            "scaled_mm_mx": lambda: torch._scaled_mm(
                a8, b8.t(), scale_a=SA.view(torch.float8_e8m0fnu),
                scale_b=SB.view(torch.float8_e8m0fnu), out_dtype=torch.bfloat16),
            "scaled_mm_tensor": lambda: torch._scaled_mm(
                a8, b8.t(), scale_a=torch.ones((), device=dev),
                scale_b=torch.ones((), device=dev), out_dtype=torch.bfloat16),
        }
        for name, fn in refs.items():
            try:
                ms_ref = timed(fn, steps, max(3, steps // 4))
                rec[name + "_ms"] = round(ms_ref, 5)
                rec[name + "_tflops"] = round(flops / ms_ref / 1e9, 1)
            except (RuntimeError, TypeError, AttributeError) as ex:
                rec[name + "_tflops"] = None
                rec[name + "_error"] = str(ex).splitlines()[0][:120]
        print(json.dumps(rec), flush=True)
        del A, B, SA, SB, D


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_threads() -> int:
    return int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))


def _time_rows(run, M: int, target_s: float):
    """Time ``run(n)`` (the oracle on the first n rows) on a block of rows
    grown from 16 until one run takes at least half of target_s (or covers
    all M rows); returns the rows and seconds of that last run."""
    n = min(M, 16)
    while True:
        t0 = time.perf_counter()
        run(n)
        dt = time.perf_counter() - t0
        if dt >= 0.5 * target_s or n >= M:
            return n, dt
        n = int(min(M, max(2 * n, n * target_s / max(dt, 1e-6))))


def cpu_baseline_mx(w, A, SA, B, SB, target_s: float):
    """Time the oracle's block-scaled full product on a block of rows."""
    import oracle
    N, K = w.N, w.K
    nrows, dt = _time_rows(lambda n: oracle.gemm_mx(A[:n], SA[:n], B, SB), w.M, target_s)
    return {"value": 2.0 * nrows * N * K / dt / 1e12, "unit": "TFLOP/s", "cores": _cpu_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "the first %d rows of D (%d x %d outputs, K=%d) by oracle.gemm_mx: FP64 sums "
                      "of decoded E4M3 times E8M0 scales, %.1f s" % (nrows, nrows, N, K, dt)}


def cpu_baseline(w, A, B, target_s: float):
    """Time the oracle's full product on a block of rows (all N columns)."""
    import oracle
    K, N = w.K, w.N
    nrows, dt = _time_rows(lambda n: oracle.gemm(w.layout, w.fmt, A[:n], B, M=n, N=N, K=K),
                           w.M, target_s)
    flops = 2.0 * nrows * N * K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _cpu_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "the first %d rows of D (%d x %d outputs, K=%d) by oracle.gemm: FP64 "
                      "accumulation, %.1f s" % (nrows, nrows, N, K, dt)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this GEMM has no multi-GPU path "
              "(run with --gpus 1; one GPU's share of the large A @ B product split over "
              "2, 4 or 8 GPUs runs as --workload large_nn_rows<g> or large_nn_cols<g>)",
              file=sys.stderr)
        sys.exit(2)

    if (args.split_k or args.tile_n) and not args.workspace:
        raise SystemExit("--split-k and --tile-n are options of dense_gemm_ex: add --workspace")

    from dense_gemm_08_amd import inputs
    known = set(inputs.WORKLOADS) | set(inputs.SHARD_WORKLOADS) | set(inputs.MX_WORKLOADS)
    if args.workload not in known:
        raise SystemExit("unknown workload %r (one of: %s)" % (args.workload,
                                                               ", ".join(sorted(known))))
    try:
        shapes = [tuple(int(v) for v in x.split("x")) for x in args.shapes.split(",") if x]
    except ValueError:
        shapes = [()]
    if any(len(t) != 3 or min(t) < 1 for t in shapes):
        raise SystemExit("--shapes takes MxNxK triples of positive sizes")

    import torch
    from dense_gemm_08_amd import binding

    if args.sweep:
        run_sweep(args, shapes or None)
        return
    if args.small_m_sweep:
        run_sweep(args, SMALL_M)
        return
    if args.small_m_sweep_nn:
        run_sweep(args, SMALL_M_NN, layout="nn")
        return
    if args.ladder:
        run_ladder(args)
        return
    if args.mx_sweep:
        run_mx_sweep(args)
        return
    if args.small_m_sweep_mx:
        run_mx_sweep(args, SMALL_M_MX)
        return
    if args.wave_fill:
        run_wave_fill(args)
        return

    if args.copy_mib:
        n = args.copy_mib << 20
        src = torch.ones(n // 2, dtype=torch.int16, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"mode": "copy", "bytes_read": n, "bytes_written": n,
                          "GB_per_s": 2 * n / dt / 1e9}), flush=True)
        return

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    lib = binding.load_library()
    pad = args.ld_pad
    if args.workload in inputs.MX_WORKLOADS:
        w = inputs.MX_WORKLOADS[args.workload]
        if pad % 16:
            raise SystemExit("--ld-pad must be a multiple of 16 for the FP8 workloads")
        A, SA, B, SB = inputs.mx_operands(w.M, w.N, w.K, w.seed, kind=w.kind)
        nb = w.K // 32
        lda = ldb = w.K + pad
        ldd = w.N + pad
        Ad = torch.zeros((w.M, lda), dtype=torch.uint8, device=dev)
        Ad[:, :w.K] = torch.from_numpy(A).to(dev)
        Bd = torch.zeros((w.N, ldb), dtype=torch.uint8, device=dev)
        Bd[:, :w.K] = torch.from_numpy(B).to(dev)
        SAd = torch.from_numpy(SA).to(dev)
        SBd = torch.from_numpy(SB).to(dev)
        Dd = torch.empty((w.M, ldd), dtype=torch.int16, device=dev)
        fmt, src = "e4m3", "gemm_mx_kernel.h"
        if args.workspace:
            import ctypes
            need = ctypes.c_size_t()
            assert lib.gemm_nt_e4m3_mx_workspace_size(w.M, w.N, w.K, 0,
                                                      ctypes.byref(need)) == 0
            ws = torch.empty(max(need.value, 1), dtype=torch.uint8, device=dev)

            def step():
                st = lib.gemm_nt_e4m3_mx_ex(w.M, w.N, w.K, Ad.data_ptr(), lda, SAd.data_ptr(), nb,
                                            Bd.data_ptr(), ldb, SBd.data_ptr(), nb, Dd.data_ptr(),
                                            ldd, ws.data_ptr(), need.value, sh)
                if st != 0:
                    raise binding.DenseGemmError(st, "gemm_nt_e4m3_mx_ex")
        else:
            def step():
                st = lib.gemm_nt_e4m3_mx(w.M, w.N, w.K, Ad.data_ptr(), lda, SAd.data_ptr(), nb,
                                         Bd.data_ptr(), ldb, SBd.data_ptr(), nb, Dd.data_ptr(),
                                         ldd, sh)
                if st != 0:
                    raise binding.DenseGemmError(st, "gemm_nt_e4m3_mx")
        config = {"workload": w.name, "layout": "nt", "M": w.M, "N": w.N, "K": w.K,
                  "lda": lda, "ldb": ldb, "ldd": ldd, "elements": "e4m3",
                  "scales": "e8m0 per 32 K values of a row", "out": "bf16",
                  "recipe": w.kind, "seed": w.seed}
    else:
        w = {**inputs.WORKLOADS, **inputs.SHARD_WORKLOADS}[args.workload]
        entry = getattr(lib, {("nt", "f16"): "gemm_nt_f16", ("nn", "bf16"): "gemm_nn_bf16",
                              ("nt", "bf16"): "gemm_nt_bf16", ("nn", "f16"): "gemm_nn_f16"}
                        [(w.layout, w.fmt)])
        A, B = inputs.make_operands(w)
        lda = w.K + pad
        ldb = (w.K if w.layout == "nt" else w.N) + pad
        ldd = w.N + pad
        Ad = torch.zeros((A.shape[0], lda), dtype=torch.int16, device=dev)
        Ad[:, :A.shape[1]] = torch.from_numpy(A.view(np.int16)).to(dev)
        Bd = torch.zeros((B.shape[0], ldb), dtype=torch.int16, device=dev)
        Bd[:, :B.shape[1]] = torch.from_numpy(B.view(np.int16)).to(dev)
        Dd = torch.empty((w.M, ldd), dtype=torch.int16, device=dev)
        fmt, src = w.fmt, "gemm_kernel.h"
        if args.workspace:
            import ctypes
            opts = binding.Options(args.split_k, args.tile_n)
            need = binding.workspace_size(w.layout, w.fmt, w.M, w.N, w.K, Ad.data_ptr(), lda,
                                          Bd.data_ptr(), ldb, opts)
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
            op = binding.OPS[(w.layout, w.fmt)]

            def step():
                st = lib.dense_gemm_ex(op, w.M, w.N, w.K, Ad.data_ptr(), lda, Bd.data_ptr(), ldb,
                                       Dd.data_ptr(), ldd, ctypes.byref(opts), ws.data_ptr(),
                                       need, sh)
                if st != 0:
                    raise binding.DenseGemmError(st, "dense_gemm_ex")
        else:
            def step():
                st = entry(w.M, w.N, w.K, Ad.data_ptr(), lda, Bd.data_ptr(), ldb, Dd.data_ptr(),
                           ldd, sh)
                if st != 0:
                    raise binding.DenseGemmError(st, "gemm")
        config = {"workload": w.name, "layout": w.layout, "M": w.M, "N": w.N, "K": w.K,
                  "lda": lda, "ldb": ldb, "ldd": ldd, "dist": w.dist, "seed": w.seed}
        if w.name in inputs.SHARD_WORKLOADS:
            g = int(w.name[-1])
            config["share_of"] = {"workload": "large_nn", "gpus": g,
                                  "split": "M" if "_rows" in w.name else "N"}
        if args.split_k or args.tile_n:
            config["options"] = {"split_k": args.split_k, "tile_n": args.tile_n}
    config["entry"] = ("dense_gemm_ex" if src == "gemm_kernel.h" else "gemm_nt_e4m3_mx_ex") \
        if args.workspace else ("gemm_nt_e4m3_mx" if src == "gemm_mx_kernel.h" else entry.__name__)

    # untimed: let the clocks settle under this load, then the warm-up steps
    settle_calls = 0
    t_end = time.perf_counter() + args.settle_ms * 1e-3
    while time.perf_counter() < t_end:
        for _ in range(8):
            step()
        settle_calls += 8
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = ev0.elapsed_time(ev1) / args.steps

    # per-launch spread (after the timed region, so it does not perturb it):
    # an event pair around each of up to 200 more back-to-back calls
    n_pl = min(args.steps, 200)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_pl)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    per_launch = sorted(a.elapsed_time(b) for a, b in evs)
    pct = lambda q: per_launch[min(n_pl - 1, int(q * n_pl))]  # noqa: E731

    flops = float(w.flops)
    value = flops * args.steps / wall / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[fmt]

    traffic = None
    try:
        with open(args.traffic_json) as f:
            tj = json.load(f)
        rec = tj.get(w.name)
        if rec and rec.get("kernel_source_sha") == source_sha(src):
            traffic = rec["bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        traffic = None

    out = {
        "metric": "TFLOP/s and % of dense FP16 MFMA peak, D=A\u00b7B\u1d40 FP16 at M=N=K=4096"
                  if w.name == "square_nt" else "TFLOP/s, %s" % w.name,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / PAGE_TFLOPS[w.name][0], 4) if w.name in PAGE_TFLOPS else None,
        "dtype": fmt,
        "data": "synthetic",
        "config": config,
        "settle": {"ms": args.settle_ms, "calls": settle_calls,
                   "note": "untimed calls before the warm-up steps, for the clocks to reach "
                           "their steady state under this load"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic,
                     "traffic_source": "profiles/traffic.json: rocprofv3 --pmc FETCH_SIZE and "
                                       "WRITE_SIZE of this workload, recorded for kernel source "
                                       "%s" % source_sha(src) if traffic is not None else
                                       "none recorded for this kernel source",
                     "kernel_ms": kern_ms,
                     "launch_ms_p10": pct(0.1), "launch_ms_p50": pct(0.5),
                     "launch_ms_p90": pct(0.9), "launch_samples": n_pl,
                     "launch_note": "calls timed one by one, each between its own pair of HIP "
                                    "events recorded on the launch stream: the pair's own cost "
                                    "is in every sample; kernel_ms (back-to-back calls) is what "
                                    "achieved is computed from"},
    }
    if w.name in PAGE_TFLOPS:
        out["vs_baseline_basis"] = {"value": PAGE_TFLOPS[w.name][0], "unit": "TFLOP/s",
                                    "what": PAGE_TFLOPS[w.name][1]}
    if not args.no_cpu_baseline:
        if fmt == "e4m3":
            out["cpu_baseline"] = cpu_baseline_mx(w, A, SA, B, SB, args.cpu_seconds)
        else:
            out["cpu_baseline"] = cpu_baseline(w, A, B, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def source_sha(name: str = "gemm_kernel.h") -> str:
    """sha256 prefix of a kernel source (gemm_kernel.h with
    gemm_small_kernel.h, or gemm_mx_kernel.h with gemm_mx_small_kernel.h),
    the headers it shares (the
    split-K reduction's included) and the launch planning (plan.cpp,
    plan.h), with comments and blank space removed: the traffic figures
    recorded for it stay valid across comment edits and other host-side
    changes, not across changes of the kernels or of which kernels a call
    runs."""
    import hashlib
    import re
    h = hashlib.sha256()
    # (plan.cpp and plan.h decide the kernel, the tile shapes and splits,
    # i.e. which kernels run; FP16/BF16 products may run the small-output
    # kernel)
    files = [name, "cdna_ops.h", "tile_sched.h", "tile_config.h", "split_reduce.h", "plan.cpp",
             "plan.h"]
    if name == "gemm_kernel.h":
        files.append("gemm_small_kernel.h")
    elif name == "gemm_mx_kernel.h":
        files.append("gemm_mx_small_kernel.h")
    for f in files:
        with open(os.path.join(ROOT, "dense_gemm_08_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(re.sub(r"\s+", " ", text).encode())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
