"""Benchmark of the block-scaled FP8 linear on one MI355X.

Workload: the Llama-3-8B-shaped FP8 linears -- (K, N) in {(4096, 4096),
(4096, 6144), (4096, 28672), (14336, 4096)} x M in {1, 16, 128, 2048, 8192}
(20 runs), bf16 activations N(0, 1) with 0.1% outlier channels x50, weights
N(0, 0.02), 1x128 dynamic act groups, 128x128 weight blocks, fp32 scales.

One step = one FP8 linear forward for every run: dynamic activation
quantization (fp8_quant_act) followed by the block-scaled GEMM
(fp8_block_gemm).  Weights are quantized once before timing (load-time step)
and two quantized copies are alternated step by step so that decode-sized
runs read their weights from HBM, not from the 256 MB Infinity Cache.

Printed: one JSON line on stdout (value = GEMM TFLOP/s including the act
quantization, over the whole step), with the roofline of the dominant kernel
(the large-M GEMM, timed with HIP events on the launch stream inside the
timed region) and the CPU oracle's rate on a bounded sample.  Per-run
details go to stderr and into the JSON ``detail`` field.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "block-scaled FP8 GEMM TFLOP/s (incl. act quant) and % of FP8 MFMA/HBM roofline"
SHAPES = [(4096, 4096), (4096, 6144), (4096, 28672), (14336, 4096)]   # (K, N)
MS = [1, 16, 128, 2048, 8192]
LARGE_M = 256            # runs with M above this use the LDS MFMA kernel
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algo_bytes(M, N, K, sb=4):
    """Bytes the linear must move: act quant (read bf16 X, write codes and
    scales) plus GEMM (read codes and scales of X and W, write bf16 Y)."""
    G = -(-K // 128)
    NB = -(-N // 128)
    quant = 2 * M * K + M * K + sb * M * G
    gemm = M * K + N * K + sb * M * G + sb * NB * G + 2 * M * N
    return quant, gemm


def cpu_baseline(budget_s=12.0):
    """The oracle (numpy, fp64 accumulation) on a bounded sample: 256 tokens
    against the first 2048 output features of each of the four shapes, act
    quantization + block GEMM, repeated until the time budget is used."""
    import numpy as np
    from block_scaled_precision_fp8_amd import synth
    from oracle import quant as Q, gemm as G
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = os.cpu_count() or 1
    Ms, Ns = 256, 2048
    cases = []
    for i, (K, N) in enumerate(SHAPES):
        x = synth.llama_acts(Ms, K, seed=100 + i)
        w = synth.normal_bf16((Ns, K), 0.02, "llama", "w", index=i, seed=100)
        wq, ws = Q.quant_weight(w)            # load-time step, not timed
        cases.append((x, wq, ws, 2.0 * Ms * Ns * K))
    flops = 0.0
    t0 = time.perf_counter()
    reps = 0
    while True:
        for x, wq, ws, f in cases:
            xq, xs = Q.quant_act(x)
            G.block_gemm(xq, xs, wq, ws)
            flops += f
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(min(cores, blas_threads)),
            "kind": "oracle",
            "sample": f"act quant + block GEMM, M={Ms} x first {Ns} outputs of each of the 4 "
                      f"Llama-3-8B (K,N) shapes, fp32 scales, {reps} passes in {dt:.1f} s; "
                      f"host cpus={os.cpu_count()}, affinity={cores}, blas threads={blas_threads}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the path; multi-GPU runs are not "
              "part of this library (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from block_scaled_precision_fp8_amd import lib as L, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L.load()

    # ---- weights: quantized once (load-time), two copies per shape
    weights = {}
    for i, (K, N) in enumerate(SHAPES):
        copies = []
        for c in range(2):
            wb = synth.device_normal_bf16((N, K), 0.02, "llama", "w", index=10 * i + c)
            wq = torch.empty((N, K), dtype=torch.uint8, device=dev)
            ws = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
            L.fp8_quant_weight(wb, wq, ws)
            del wb
            copies.append((wq, ws))
        weights[(K, N)] = copies
    # ---- activations and outputs per run
    runs = []
    for i, (K, N) in enumerate(SHAPES):
        for M in MS:
            x = synth.device_llama_acts(M, K, index=100 * i + M)
            xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
            xs = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            need = L.workspace_size(L.OP_BLOCK_GEMM, M, N, K)
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
            runs.append(dict(M=M, K=K, N=N, x=x, xq=xq, xs=xs, y=y, ws=ws))
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step(s, evs=None):
        for j, r in enumerate(runs):
            wq, wsc = weights[(r["K"], r["N"])][s & 1]
            if evs is not None:
                evs[j][0].record(stream)
            L.fp8_quant_act(r["x"], r["xq"], r["xs"], stream=sp)
            if evs is not None:
                evs[j][1].record(stream)
            L.fp8_block_gemm(r["xq"], r["xs"], wq, wsc, r["y"], workspace=r["ws"], stream=sp)
            if evs is not None:
                evs[j][2].record(stream)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()

    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in runs]
           for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(args.steps):
        step(s, evs[s])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps

    flops_step = sum(2.0 * r["M"] * r["N"] * r["K"] for r in runs)
    value = flops_step / (ms_per_step * 1e-3) / 1e12

    # ---- per-run and per-kernel times (HIP events on the launch stream)
    detail = []
    big_flops = big_ms = 0.0
    for j, r in enumerate(runs):
        q = np.array([evs[s][j][0].elapsed_time(evs[s][j][1]) for s in range(args.steps)])
        g = np.array([evs[s][j][1].elapsed_time(evs[s][j][2]) for s in range(args.steps)])
        M, N, K = r["M"], r["N"], r["K"]
        fl = 2.0 * M * N * K
        qb, gb = algo_bytes(M, N, K)
        qm, gm = float(np.mean(q)), float(np.mean(g))
        d = dict(M=M, K=K, N=N, quant_us=round(qm * 1e3, 2), gemm_us=round(gm * 1e3, 2),
                 linear_tflops=round(fl / ((qm + gm) * 1e-3) / 1e12, 2),
                 gemm_tflops=round(fl / (gm * 1e-3) / 1e12, 2),
                 quant_gbs=round(qb / (qm * 1e-3) / 1e9, 1),
                 gemm_gbs=round(gb / (gm * 1e-3) / 1e9, 1),
                 linear_gbs=round((qb + gb) / ((qm + gm) * 1e-3) / 1e9, 1))
        d["frac_fp8_peak"] = round(d["gemm_tflops"] / PEAK_FP8_TFLOPS, 4)
        d["frac_hbm_gemm"] = round(d["gemm_gbs"] / PEAK_HBM_GBS, 4)
        detail.append(d)
        if M > LARGE_M:
            big_flops += fl * args.steps
            big_ms += float(np.sum(g))
        log(f"M={M:5d} K={K:5d} N={N:5d}  quant {qm*1e3:8.1f} us ({d['quant_gbs']:7.1f} GB/s)"
            f"  gemm {gm*1e3:8.1f} us ({d['gemm_tflops']:7.1f} TF/s, {d['gemm_gbs']:7.1f} GB/s)"
            f"  linear {d['linear_tflops']:7.1f} TF/s")

    achieved = big_flops / (big_ms * 1e-3) / 1e12
    n_big = sum(1 for r in runs if r["M"] > LARGE_M)
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                "traffic": None,
                "kernel": "gemm_lds_kernel (fp32 scales), the large-M block-scaled GEMM",
                "launches_per_step": n_big,
                "avg_launch_us": round(big_ms / (args.steps * n_big) * 1e3, 2)}

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline()

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": "Llama-3-8B-shaped FP8 linears: (K,N) in {(4096,4096),"
                               "(4096,6144),(4096,28672),(14336,4096)} x M in "
                               "{1,16,128,2048,8192}; 1x128 act groups, 128x128 weight "
                               "blocks, fp32 scales, bf16 out",
                   "runs_per_step": len(runs), "flops_per_step": flops_step},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "detail": detail,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
