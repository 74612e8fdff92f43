"""Benchmark of the block-scaled FP8 / NVFP4-style linear path on one MI355X.

Headline workload (``value``): the Llama-3-8B-shaped FP8 linears -- (K, N) in
{(4096, 4096), (4096, 6144), (4096, 28672), (14336, 4096)} x M in
{1, 16, 128, 2048, 8192} (20 runs), bf16 activations N(0, 1) with 0.1%
outlier channels x50, weights N(0, 0.02), 1x128 dynamic act groups, 128x128
weight blocks, fp32 scales.  One step = one FP8 linear forward for every run:
dynamic activation quantization (fp8_quant_act) then the block-scaled GEMM
(fp8_block_gemm).  Weights are quantized once before timing (load-time step)
into four copies per shape, rotated so that consecutive runs of one shape
never share a copy: decode-sized runs read their weights from HBM rather
than from the 256 MB Infinity Cache.
value = GEMM flops of the step / step time (TFLOP/s, act quant included).
Inside the timed steps HIP events bracket only the 256 x 256-tile GEMM
launches (the roofline below); the per-run breakdown in ``detail`` comes
from a second pass of the same steps after the timed region, so its events
do not add to the step time.
Decode-sized runs (M <= 16) whose activation quantization the library fuses
into the GEMM launch are one fp8_linear call; the others are fp8_quant_act
then fp8_block_gemm, the two launches fp8_linear makes for them.

The other rows of the path are timed in the same run and reported in
``detail`` (not in ``value``): DeepSeek-V3-shaped linears with UE8M0 scales,
the MoE expert MLP (256 experts, Zipf-routed top-8: gate/up grouped GEMM,
the same with the fused SiLU-mul requant, the down GEMM on its output, and
the gate/up GEMM with MXFP4 expert weights), the
NVFP4-style MLP (fp4_quant + fp4_group_gemm) with its FP8 attention
projection, the FP8 activation x MXFP4 weight linear at DeepSeek-V3 expert
shapes, FP8 linears with (32, 32) weight blocks, and weight quantization.

``roofline`` is for the dominant kernel, the large-M GEMM with 256 x 256 tiles
(gemm_lds_kernel, every run the library sends to it, split-K ones included
with their whole 2MNK; bsfp8_gemm_kernel says which): algorithmic flops over
its launches / its summed duration from HIP events
recorded on the launch stream inside the timed region.  ``traffic`` comes
from the committed rocprofv3 PMC summary when that summary was taken on the
current kernel source, else null.  ``launch_us`` gives the median, p10 and
p90 of the dominant kernel's timed launches, ``ms_per_step_stats`` those of
the timed steps.  ``roofline_decode`` is the HBM roofline of the decode-sized
runs (M <= 16, act quant included): their algorithmic bytes over the time of
one pass over them, launched back to back with events only at the pass
boundaries (a decode step's launch pattern; events between launches would
add their own gaps); median, p10, p90 over ``steps`` passes.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--suites ...]
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "block-scaled FP8 GEMM TFLOP/s (incl. act quant) and % of FP8 MFMA/HBM roofline"
LLAMA_SHAPES = [(4096, 4096), (4096, 6144), (4096, 28672), (14336, 4096)]   # (K, N)
LLAMA_MS = [1, 16, 128, 2048, 8192]
DEEPSEEK_SHAPES = [(7168, 1536), (1536, 24576), (7168, 18432), (18432, 7168)]
DEEPSEEK_MS = [1, 64, 4096]
WEIGHT_COPIES = 4         # weight sets rotated through the linear runs
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense FP8 MFMA
PEAK_F16_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_lds_kernel_llama_traffic.txt")
# the large-M GEMM's code: its kernel source and the device helpers it includes
GEMM_SOURCES = [os.path.join(ROOT, "block_scaled_precision_fp8_amd", "csrc", f)
                for f in ("gemm_fp8.hip", "bsfp8_internal.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash():
    h = hashlib.sha256()
    for path in GEMM_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """bytes per launch of the large-M GEMM from the committed PMC summary,
    if it was measured on the current kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ": " in line and not line.lstrip().startswith("#"):
                k, v = line.rsplit(": ", 1)     # keys may hold a colon themselves
                kv[k.strip()] = v.strip()
    if kv.get("gemm sources sha256[:16]") != source_hash():
        return None
    try:
        return float(kv["hbm bytes per launch (scaled)"])
    except (KeyError, ValueError):
        return None


def copies_for(nbytes):
    """weight copies to rotate so that the rotation spans 2x the 256 MB cache"""
    return max(2, -(-(512 << 20) // nbytes))


def act_bytes(M, K, sb):
    G = -(-K // 128)
    return 2 * M * K + M * K + sb * M * G


def gemm_bytes(M, N, K, sb):
    G = -(-K // 128)
    NB = -(-N // 128)
    return M * K + N * K + sb * M * G + sb * NB * G + 2 * M * N


class Timer:
    """HIP events on the launch stream around every call in the timed loop."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        self.ev = {}

    def mark(self, key):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self.ev.setdefault(key, []).append(e)

    def all_ms(self, a, b):
        """ms between marks a and b, one per occurrence"""
        return [x.elapsed_time(y) for x, y in zip(self.ev[a], self.ev[b])]

    def ms(self, a, b):
        """mean ms between marks a and b (matched by occurrence)"""
        v = self.all_ms(a, b)
        return sum(v) / len(v)


def pstats(v, scale=1.0, nd=2):
    """median, p10 and p90 of a list of durations (times `scale`)"""
    a = np.sort(np.asarray(v, dtype=np.float64)) * scale
    return {"median": round(float(np.median(a)), nd), "p10": round(float(np.percentile(a, 10)), nd),
            "p90": round(float(np.percentile(a, 90)), nd), "n": int(len(a))}


def run_linears(torch, L, synth, shapes, ms, fmt, workload, steps, warmup, dev, sp):
    """act quant + block GEMM over a set of (K, N) x M runs; returns per-run
    details, the step time, the step's flops and the large-M GEMM totals."""
    sdt = torch.float32 if fmt == 0 else torch.uint8
    weights = {}
    for i, (K, N) in enumerate(shapes):
        copies = []
        for c in range(WEIGHT_COPIES):
            sigma = 0.02 if workload == "llama" else 0.01
            wb = synth.device_normal_bf16((N, K), sigma, workload, "w", index=10 * i + c)
            wq = torch.empty((N, K), dtype=torch.uint8, device=dev)
            ws = torch.empty((N // 128, K // 128), dtype=sdt, device=dev)
            L.fp8_quant_weight(wb, wq, ws, scale_fmt=fmt)
            del wb
            copies.append((wq, ws))
        weights[(K, N)] = copies
    runs = []
    for i, (K, N) in enumerate(shapes):
        for M in ms:
            if workload == "llama":
                x = synth.device_llama_acts(M, K, index=100 * i + M)
            else:
                x = synth.device_deepseek_acts(M, K, index=100 * i + M)
            need = L.workspace_size(L.OP_BLOCK_GEMM, M, N, K)
            # decode-sized runs whose quantization fp8_linear fuses into the
            # GEMM launch go through fp8_linear (one launch)
            fused = (L.gemm_kernel(M, N, K)[0] == L.GEMM_DECODE
                     and L.workspace_size(L.OP_LINEAR, M, N, K) == 0)
            big = (not fused) and L.gemm_kernel(M, N, K)[0] == L.GEMM_TILE_256x256
            runs.append(dict(M=M, K=K, N=N, x=x, fused=fused, big=big,
                             xq=torch.empty((M, K), dtype=torch.uint8, device=dev),
                             xs=torch.empty((M, K // 128), dtype=sdt, device=dev),
                             y=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                             ws=torch.empty(max(need, 16), dtype=torch.uint8, device=dev)))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step(s, tm=None, big_only=False, only=None):
        """one pass over every run (or the runs whose indices `only` lists);
        tm marks around every launch, or with big_only around the
        256 x 256-tile GEMM launches only"""
        for j, r in enumerate(runs):
            if only is not None and j not in only:
                continue
            # consecutive runs of one shape read different copies, so no run
            # finds its weights in the 256 MB last-level cache
            wq, wsc = weights[(r["K"], r["N"])][(s + j) % WEIGHT_COPIES]
            every = tm is not None and not big_only
            if every:
                tm.mark(("q", j))
            if r["fused"]:
                L.fp8_linear(r["x"], wq, wsc, r["y"], scale_fmt=fmt, stream=sp)
                if every:
                    tm.mark(("g", j))
                    tm.mark(("e", j))
                continue
            L.fp8_quant_act(r["x"], r["xq"], r["xs"], scale_fmt=fmt, stream=sp)
            mark = tm is not None and (every or r["big"])
            if mark:
                tm.mark(("g", j))
            L.fp8_block_gemm(r["xq"], r["xs"], wq, wsc, r["y"], scale_fmt=fmt,
                             workspace=r["ws"], stream=sp)
            if mark:
                tm.mark(("e", j))

    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    # timed region: events only around the dominant kernel's launches (the
    # roofline); the per-run breakdown comes from a second, untimed pass
    tb = Timer(torch, stream)
    # one event per step boundary: the step time's median / p10 / p90 besides
    # the whole-run mean
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    bounds[0].record(stream)
    for s in range(steps):
        step(s, tb, big_only=True)
        bounds[s + 1].record(stream)
    torch.cuda.synchronize()
    ms_step = bounds[0].elapsed_time(bounds[-1]) / steps
    step_ms = [bounds[i].elapsed_time(bounds[i + 1]) for i in range(steps)]
    tm = Timer(torch, stream)
    for s in range(steps):
        step(s, tm)
    torch.cuda.synchronize()
    # the decode-sized runs (M <= 16) back to back, events at pass boundaries
    dec_idx = {j for j, r in enumerate(runs) if r["M"] <= 16}
    dec_pass_ms = []
    if dec_idx:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for s in range(steps):
            step(s, only=dec_idx)
            ev[s + 1].record(stream)
        torch.cuda.synchronize()
        dec_pass_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    sb = 4 if fmt == 0 else 1
    detail, big_flops, big_ms, n_big, flops = [], 0.0, 0.0, 0, 0.0
    dec_bytes, dec_ms = 0.0, 0.0
    big_launch_us = []          # every timed launch of the 256 x 256 tile
    for j, r in enumerate(runs):
        M, N, K = r["M"], r["N"], r["K"]
        qm, gm = tm.ms(("q", j), ("g", j)), tm.ms(("g", j), ("e", j))
        fl = 2.0 * M * N * K
        flops += fl
        if r["fused"]:
            # one launch: bf16 activations in, weights + scales, bf16 out
            lm = qm
            lb = 2 * M * K + gemm_bytes(M, N, K, sb) - M * K - sb * M * (-(-K // 128))
            d = dict(M=M, K=K, N=N, fused_quant=True, linear_us=round(lm * 1e3, 2),
                     linear_tflops=round(fl / (lm * 1e-3) / 1e12, 2),
                     linear_gbs=round(lb / (lm * 1e-3) / 1e9, 1),
                     frac_hbm=round(lb / (lm * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))
            dec_bytes += lb
            dec_ms += lm
            log(f"[{workload}] M={M:5d} K={K:5d} N={N:5d} fused linear {lm*1e3:8.1f} us "
                f"({d['linear_gbs']:7.1f} GB/s, {d['linear_tflops']:7.1f} TF/s)")
            detail.append(d)
            continue
        qb, gb = act_bytes(M, K, sb), gemm_bytes(M, N, K, sb)
        d = dict(M=M, K=K, N=N, quant_us=round(qm * 1e3, 2), gemm_us=round(gm * 1e3, 2),
                 linear_tflops=round(fl / ((qm + gm) * 1e-3) / 1e12, 2),
                 gemm_tflops=round(fl / (gm * 1e-3) / 1e12, 2),
                 frac_fp8_peak=round(fl / (gm * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                 quant_gbs=round(qb / (qm * 1e-3) / 1e9, 1),
                 gemm_gbs=round(gb / (gm * 1e-3) / 1e9, 1),
                 frac_hbm_gemm=round(gb / (gm * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))
        if M <= 16:
            dec_bytes += qb + gb
            dec_ms += qm + gm
        detail.append(d)
        if r["big"]:
            big_flops += fl
            big_ms += tb.ms(("g", j), ("e", j))
            n_big += 1
            big_launch_us += [v * 1e3 for v in tb.all_ms(("g", j), ("e", j))]
        log(f"[{workload}] M={M:5d} K={K:5d} N={N:5d} quant {qm*1e3:8.1f} us "
            f"({d['quant_gbs']:7.1f} GB/s)  gemm {gm*1e3:8.1f} us ({d['gemm_tflops']:7.1f} TF/s, "
            f"{d['gemm_gbs']:7.1f} GB/s)  linear {d['linear_tflops']:7.1f} TF/s")
    decode = None
    if dec_pass_ms:
        # all M <= 16 runs' bytes (act quant included) over one back-to-back
        # pass over them (median over the passes; p10 / p90 besides); the sum
        # of the per-launch event times is kept for comparison
        med = float(np.median(dec_pass_ms))
        decode = dict(runs="M <= 16", bytes=dec_bytes, us=round(med * 1e3, 1),
                      us_per_step=pstats(dec_pass_ms, 1e3, 1),
                      us_launch_events=round(dec_ms * 1e3, 1),
                      gbs=round(dec_bytes / (med * 1e-3) / 1e9, 1),
                      frac_hbm=round(dec_bytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))
    for r in runs:
        r.clear()
    weights.clear()
    torch.cuda.empty_cache()
    return dict(detail=detail, ms_step=ms_step, step_ms=step_ms, flops=flops,
                big_flops=big_flops, big_ms=big_ms, n_big=n_big, decode=decode,
                big_launch_us=big_launch_us)


def run_moe(torch, L, synth, steps, warmup, dev, sp):
    """MoE expert MLP (256 experts, hidden 7168, intermediate 2048, 4096
    tokens routed top-8 by Zipf popularity): the gate/up grouped GEMM
    (7168 -> 2 x 2048) alone and with the fused SiLU-mul + 1x128 requant
    epilogue, and the down grouped GEMM (2048 -> 7168) on that epilogue's
    FP8 output; ``ffn_us`` is act quant + fused gate/up + down."""
    E, H, I, TOK, TOPK = 256, 7168, 2048, 4096, 8
    tok, off = synth.moe_routing(TOK, E, TOPK)
    T = len(tok)
    seg = torch.from_numpy(off).to(dev)
    x = synth.device_normal_bf16((TOK, H), 1.0, "moe", "x")[torch.from_numpy(tok).to(dev)]
    counts = (off[1:] - off[:-1])
    nb = int((counts > 0).sum())
    W = {}
    for name, N, K in (("gate_up", 2 * I, H), ("down", H, I)):
        wq = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
        ws = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device=dev)
        for e in range(E):
            wb = synth.device_normal_bf16((N, K), 0.02, "moe", "w" if name == "gate_up" else "w2", e)
            L.fp8_quant_weight(wb, wq[e], ws[e])
            del wb
        W[name] = (wq, ws)
    # the gate/up experts again as MXFP4 (E2M1 in 1 x 32 groups, E8M0 scales)
    wq4 = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=dev)
    ws4 = torch.empty((E, 2 * I, H // 32), dtype=torch.uint8, device=dev)
    for e in range(E):
        wb = synth.device_normal_bf16((2 * I, H), 0.02, "moe", "w", e)
        L.mxfp4_quant_weight(wb, wq4[e], ws4[e])
        del wb
    xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
    xs = torch.empty((T, H // 128), dtype=torch.float32, device=dev)
    y1 = torch.empty((T, 2 * I), dtype=torch.bfloat16, device=dev)
    hq = torch.empty((T, I), dtype=torch.uint8, device=dev)
    hs = torch.empty((T, I // 128), dtype=torch.float32, device=dev)
    y2 = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step(tm=None):
        mark = tm.mark if tm else (lambda k: None)
        mark("q")
        L.fp8_quant_act(x, xq, xs, stream=sp)
        mark("g")
        L.fp8_grouped_gemm(xq, xs, W["gate_up"][0], W["gate_up"][1], seg, y1, stream=sp)
        mark("f")
        L.fp8_grouped_gemm_silu_mul_quant(xq, xs, W["gate_up"][0], W["gate_up"][1], seg, hq, hs,
                                          stream=sp)
        mark("d")
        L.fp8_grouped_gemm(hq, hs, W["down"][0], W["down"][1], seg, y2, stream=sp)
        mark("e")
        L.fp8_fp4_grouped_gemm(xq, xs, wq4, ws4, seg, y1, stream=sp)
        mark("w4")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    tm = Timer(torch, stream)
    for _ in range(steps):
        step(tm)
    torch.cuda.synchronize()
    qm, gm, fm, dm = tm.ms("q", "g"), tm.ms("g", "f"), tm.ms("f", "d"), tm.ms("d", "e")
    w4m = tm.ms("e", "w4")

    def row(ms, N, K, out_bytes):
        fl = 2.0 * T * N * K
        gb = nb * (N * K + 4 * (N // 128) * (K // 128)) + T * (K + 4 * (K // 128)) + out_bytes
        return dict(T=T, N=N, K=K, experts=E, nonempty=nb, us=round(ms * 1e3, 1),
                    tflops=round(fl / (ms * 1e-3) / 1e12, 1),
                    gbs=round(gb / (ms * 1e-3) / 1e9, 1),
                    frac_hbm=round(gb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))
    res = {"act_quant_us": round(qm * 1e3, 1),
           "gate_up": row(gm, 2 * I, H, 2 * T * 2 * I),
           "gate_up_silu_mul_quant": row(fm, 2 * I, H, T * I + 4 * T * (I // 128)),
           "down": row(dm, H, I, 2 * T * H),
           "gate_up_mxfp4": dict(row(w4m, 2 * I, H, 2 * T * 2 * I),
                                 gbs=round((nb * 2 * I * (H // 2 + H // 32) + T * (H + 4 * (H // 128))
                                            + 2 * T * 2 * I) / (w4m * 1e-3) / 1e9, 1)),
           "ffn_us": round((qm + fm + dm) * 1e3, 1)}
    g4 = res["gate_up_mxfp4"]
    g4["frac_hbm"] = round(g4["gbs"] / PEAK_HBM_GBS, 4)
    log(f"[moe] T={T}: act quant {qm*1e3:.1f} us, gate/up {gm*1e3:.1f} us, fused gate/up + "
        f"silu-mul quant {fm*1e3:.1f} us, down {dm*1e3:.1f} us, ffn {res['ffn_us']} us, "
        f"gate/up with MXFP4 experts {w4m*1e3:.1f} us ({g4['gbs']} GB/s)")
    del W, xq, xs, y1, hq, hs, y2, wq4, ws4
    torch.cuda.empty_cache()
    res["rows_per_expert"] = dict(max=int(counts.max()), median=float(np.median(counts)),
                                  min=int(counts.min()))
    return res


def run_nvfp4(torch, L, synth, steps, warmup, dev, sp):
    """NVFP4-style MLP (gate/up 12288 -> 28672, down 28672 -> 12288; fp4_quant
    of the activations + fp4_group_gemm) and the FP8 attention projection
    (12288 x 12288, 1x128 / 128x128, fp32 scales) at M in {1, 32, 4096}."""
    HID, INTER = 12288, 28672
    out = []
    mats = {}
    for name, N, K in (("gate_up", INTER, HID), ("down", HID, INTER)):
        copies = []
        for c in range(copies_for(N * (K // 2 + K // 16))):
            wb = synth.device_normal_bf16((N, K), 0.015, "nvfp4", "w", index=N + c)
            q = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
            s = torch.empty((N, K // 16), dtype=torch.uint8, device=dev)
            t = torch.empty((1,), dtype=torch.float32, device=dev)
            L.fp4_quant(wb, q, s, t)
            del wb
            copies.append((q, s, t))
        mats[name] = (N, K, copies)
    attn = []
    for c in range(copies_for(HID * HID)):
        wb = synth.device_normal_bf16((HID, HID), 0.015, "nvfp4", "w", index=7 + c)
        wq = torch.empty((HID, HID), dtype=torch.uint8, device=dev)
        ws = torch.empty((HID // 128, HID // 128), dtype=torch.float32, device=dev)
        L.fp8_quant_weight(wb, wq, ws)
        del wb
        attn.append((wq, ws))
    stream = torch.cuda.current_stream()
    for M in (1, 32, 4096):
        for name in ("gate_up", "down", "attn_fp8"):
            if name == "attn_fp8":
                N, K = HID, HID
            else:
                N, K, copies = mats[name]
            x = synth.device_normal_bf16((M, K), 1.0, "nvfp4", "x", index=M)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            if name == "attn_fp8":
                need = L.workspace_size(L.OP_LINEAR, M, N, K)
                wsp = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

                def call(s, tm=None):
                    if tm:
                        tm.mark("a")
                    wq, wsc = attn[s % len(attn)]
                    L.fp8_linear(x, wq, wsc, y, workspace=wsp, stream=sp)
                    if tm:
                        tm.mark("b")
                        tm.mark("c")
            else:
                qx = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
                sx = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
                tx = torch.empty((1,), dtype=torch.float32, device=dev)
                wqs = torch.empty(L.workspace_size(L.OP_FP4_QUANT, M, 0, K), dtype=torch.uint8,
                                  device=dev)
                need = L.workspace_size(L.OP_FP4_GEMM, M, N, K)
                wsg = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

                def call(s, tm=None):
                    q, sc, t = copies[s % len(copies)]
                    if tm:
                        tm.mark("a")
                    L.fp4_quant(x, qx, sx, tx, workspace=wqs, stream=sp)
                    if tm:
                        tm.mark("b")
                    L.fp4_group_gemm(qx, sx, tx, q, sc, t, y, workspace=wsg, stream=sp)
                    if tm:
                        tm.mark("c")
            for s in range(warmup):
                call(s)
            torch.cuda.synchronize()
            tm = Timer(torch, stream)
            for s in range(steps):
                call(s, tm)
            torch.cuda.synchronize()
            qm, gm = tm.ms("a", "b"), tm.ms("b", "c")
            fl = 2.0 * M * N * K
            if name == "attn_fp8":
                tot = qm
                byt = act_bytes(M, K, 4) + gemm_bytes(M, N, K, 4)
                d = dict(M=M, K=K, N=N, kind="fp8_linear", us=round(tot * 1e3, 2),
                         tflops=round(fl / (tot * 1e-3) / 1e12, 2),
                         gbs=round(byt / (tot * 1e-3) / 1e9, 1))
            else:
                wb = N * (K // 2 + K // 16)
                gb = wb + M * (K // 2 + K // 16) + 2 * M * N
                d = dict(M=M, K=K, N=N, kind=f"fp4_{name}", quant_us=round(qm * 1e3, 2),
                         gemm_us=round(gm * 1e3, 2),
                         gemm_tflops=round(fl / (gm * 1e-3) / 1e12, 2),
                         frac_f16_peak=round(fl / (gm * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
                         gemm_gbs=round(gb / (gm * 1e-3) / 1e9, 1),
                         frac_hbm=round(gb / (gm * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))
            out.append(d)
            log(f"[nvfp4] {d}")
    return out


def run_mxfp4(torch, L, synth, steps, warmup, dev, sp):
    """FP8 activations (1x128 groups, UE8M0 scales) x MXFP4 weights (E2M1 in
    1x32 groups with UE8M0 scales) at the DeepSeek-V3 expert-sized shapes
    (7168 -> 18432, 18432 -> 7168), M in {1, 64, 4096}: act quant then
    fp8_fp4_gemm.  Weight copies rotate over more than twice the 256 MB cache
    so decode reads HBM."""
    out = []
    stream = torch.cuda.current_stream()
    for K, N in ((7168, 18432), (18432, 7168)):
        copies = []
        for c in range(copies_for(N * (K // 2 + K // 32))):
            wb = synth.device_normal_bf16((N, K), 0.01, "deepseek", "w", index=N + 17 * c)
            q = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
            s = torch.empty((N, K // 32), dtype=torch.uint8, device=dev)
            L.mxfp4_quant_weight(wb, q, s, stream=sp)
            del wb
            copies.append((q, s))
        for M in (1, 64, 4096):
            x = synth.device_deepseek_acts(M, K, index=M)
            xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
            xs = torch.empty((M, K // 128), dtype=torch.uint8, device=dev)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            need = L.workspace_size(L.OP_FP8_FP4_GEMM, M, N, K)
            wsp = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

            def call(i, tm=None):
                q, sc = copies[i % len(copies)]
                if tm:
                    tm.mark("a")
                L.fp8_quant_act(x, xq, xs, scale_fmt=L.SCALE_UE8M0, stream=sp)
                if tm:
                    tm.mark("b")
                L.fp8_fp4_gemm(xq, xs, q, sc, y, scale_fmt=L.SCALE_UE8M0, workspace=wsp,
                               stream=sp)
                if tm:
                    tm.mark("c")
            for i in range(warmup):
                call(i)
            torch.cuda.synchronize()
            tm = Timer(torch, stream)
            for i in range(steps):
                call(i, tm)
            torch.cuda.synchronize()
            qm, gm = tm.ms("a", "b"), tm.ms("b", "c")
            fl = 2.0 * M * N * K
            gb = N * (K // 2 + K // 32) + M * (K + K // 128) + 2 * M * N
            d = dict(M=M, K=K, N=N, quant_us=round(qm * 1e3, 2), gemm_us=round(gm * 1e3, 2),
                     tflops_incl_quant=round(fl / ((qm + gm) * 1e-3) / 1e12, 1),
                     gemm_tflops=round(fl / (gm * 1e-3) / 1e12, 1),
                     frac_fp8_peak=round(fl / (gm * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                     gemm_gbs=round(gb / (gm * 1e-3) / 1e9, 1),
                     frac_hbm=round(gb / (gm * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))
            out.append(d)
            log(f"[mxfp4] {d}")
            del x, xq, xs, y, wsp
        del copies
        torch.cuda.empty_cache()
    return out


def run_block32(torch, L, synth, steps, warmup, dev, sp, fmt=0):
    """FP8 linears with (32, 32) weight blocks and 1x32 act groups (fp32
    scales, or UE8M0 with fmt=1) at Llama-3-8B o_proj / gate+up shapes:
    fp8_linear, act quant included."""
    out = []
    stream = torch.cuda.current_stream()
    sdt = torch.uint8 if fmt else torch.float32
    for M, K, N in ((16, 4096, 4096), (2048, 4096, 4096), (8192, 4096, 28672)):
        wb = synth.device_normal_bf16((N, K), 0.02, "llama", "w", index=N + 32)
        copies = []
        for c in range(copies_for(N * K)):
            wq = torch.empty((N, K), dtype=torch.uint8, device=dev)
            ws = torch.empty((N // 32, K // 32), dtype=sdt, device=dev)
            L.fp8_quant_weight(wb, wq, ws, block_n=32, block_k=32, scale_fmt=fmt, stream=sp)
            copies.append((wq, ws))
        del wb
        x = synth.device_llama_acts(M, K, index=M)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        wsp = torch.empty(L.workspace_size(L.OP_LINEAR_B32, M, N, K), dtype=torch.uint8,
                          device=dev)

        def call(i):
            wq, ws = copies[i % len(copies)]
            L.fp8_linear(x, wq, ws, y, block_n=32, block_k=32, scale_fmt=fmt, workspace=wsp,
                         stream=sp)
        for i in range(warmup):
            call(i)
        torch.cuda.synchronize()
        tm = Timer(torch, stream)
        for i in range(steps):
            tm.mark("a")
            call(i)
            tm.mark("b")
        torch.cuda.synchronize()
        ms = tm.ms("a", "b")
        fl = 2.0 * M * N * K
        sb = 1 if fmt else 4                                      # bytes per scale
        sa, sw = sb * M * (K // 32), sb * (N // 32) * (K // 32)
        byt = (3 * M * K + sa) + (M * K + sa + N * K + sw + 2 * M * N)   # quant + GEMM
        d = dict(M=M, K=K, N=N, linear_us=round(ms * 1e3, 2),
                 tflops=round(fl / (ms * 1e-3) / 1e12, 1),
                 frac_fp8_peak=round(fl / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                 gbs=round(byt / (ms * 1e-3) / 1e9, 1))
        out.append(d)
        log(f"[block32 fmt={fmt}] {d}")
        del copies, x, y, wsp
        torch.cuda.empty_cache()
    return out


def run_wquant(torch, L, synth, steps, warmup, dev, sp):
    """Weight quantization (load-time step) of the 28672 x 4096 weight."""
    N, K = 28672, 4096
    wb = synth.device_normal_bf16((N, K), 0.02, "llama", "w", index=99)
    wq = torch.empty((N, K), dtype=torch.uint8, device=dev)
    ws = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        L.fp8_quant_weight(wb, wq, ws, stream=sp)
    torch.cuda.synchronize()
    tm = Timer(torch, stream)
    for _ in range(steps):
        tm.mark("a")
        L.fp8_quant_weight(wb, wq, ws, stream=sp)
        tm.mark("b")
    torch.cuda.synchronize()
    m = tm.ms("a", "b")
    byt = 3 * N * K + 4 * (N // 128) * (K // 128)
    return dict(N=N, K=K, us=round(m * 1e3, 1), gbs=round(byt / (m * 1e-3) / 1e9, 1),
                frac_hbm=round(byt / (m * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))


def cpu_baseline(budget_s=12.0):
    """The oracle (numpy, fp64 accumulation) on a bounded sample: 256 tokens
    against the first 2048 output features of each of the four Llama shapes,
    act quantization + block GEMM, repeated until the time budget is used."""
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
    for i, (K, N) in enumerate(LLAMA_SHAPES):
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
    ap.add_argument("--suites", default="deepseek,moe,nvfp4,mxfp4,block32,wquant",
                    help="extra rows timed for `detail` (comma list, or 'none')")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size "
                         "kernel for calibrating rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the path; multi-GPU runs are not "
              "part of this library (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_scaled_precision_fp8_amd import lib as L, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L.load()
    sp = torch.cuda.current_stream().cuda_stream
    if args.copy_calib_mib:
        n = args.copy_calib_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    r = run_linears(torch, L, synth, LLAMA_SHAPES, LLAMA_MS, 0, "llama", args.steps,
                    args.warmup, dev, sp)
    value = r["flops"] / (r["ms_step"] * 1e-3) / 1e12
    achieved = r["big_flops"] / (r["big_ms"] * 1e-3) / 1e12
    traffic = read_traffic()
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                "traffic": traffic,
                "kernel": "gemm_lds_kernel<0,4,2,64,128,false,false,false,false,false,false> (fp32 scales, 256x256 "
                          "tiles), large-M block-scaled GEMM",
                "launches_per_step": r["n_big"],
                "avg_launch_us": round(r["big_ms"] / r["n_big"] * 1e3, 2),
                "launch_us": pstats(r["big_launch_us"]),
                "algorithmic_gflop_per_launch": round(r["big_flops"] / r["n_big"] / 1e9, 2)}
    dec = r["decode"]
    roofline_decode = None
    if dec:
        roofline_decode = {
            "bound": "hbm", "achieved": dec["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": dec["frac_hbm"], "traffic": None,
            "kernel": "gemm_decode_kernel / gemm_decode_pers_kernel (M <= 16; act quant "
                      "included, fused where fp8_linear fuses it)",
            "runs": "the 8 Llama-3-8B linears with M in {1, 16}",
            "algorithmic_bytes_per_step": dec["bytes"], "us_per_step": dec["us_per_step"]}
    detail = {"llama": r["detail"], "llama_decode_hbm": r["decode"]}
    suites = [] if args.suites == "none" else args.suites.split(",")
    if "deepseek" in suites:
        d = run_linears(torch, L, synth, DEEPSEEK_SHAPES, DEEPSEEK_MS, 1, "deepseek",
                        max(5, args.steps // 2), 2, dev, sp)
        detail["deepseek_ue8m0"] = d["detail"]
        detail["deepseek_decode_hbm"] = d["decode"]
        detail["deepseek_ue8m0_tile256_tflops"] = round(d["big_flops"] / (d["big_ms"] * 1e-3)
                                                        / 1e12, 1)
    if "moe" in suites:
        detail["moe"] = run_moe(torch, L, synth, max(5, args.steps // 2), 2, dev, sp)
    if "nvfp4" in suites:
        detail["nvfp4_mlp_fp8_attn"] = run_nvfp4(torch, L, synth, max(5, args.steps // 2), 2,
                                                 dev, sp)
    if "mxfp4" in suites:
        detail["fp8_x_mxfp4_ue8m0"] = run_mxfp4(torch, L, synth, max(5, args.steps // 2), 2,
                                                dev, sp)
    if "block32" in suites:
        detail["block32_fp32_scales"] = run_block32(torch, L, synth, max(5, args.steps // 2), 2,
                                                    dev, sp)
        detail["block32_ue8m0"] = run_block32(torch, L, synth, max(5, args.steps // 2), 2, dev,
                                              sp, fmt=1)
    if "wquant" in suites:
        detail["weight_quant"] = run_wquant(torch, L, synth, 10, 2, dev, sp)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline()

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": "Llama-3-8B-shaped FP8 linears: (K,N) in {(4096,4096),"
                               "(4096,6144),(4096,28672),(14336,4096)} x M in "
                               "{1,16,128,2048,8192}; 1x128 act groups, 128x128 weight "
                               "blocks, fp32 scales, bf16 out",
                   "runs_per_step": 20, "flops_per_step": r["flops"]},
        "ms_per_step_stats": pstats(r["step_ms"], 1.0, 4),
        "roofline": roofline,
        "roofline_decode": roofline_decode,
        "cpu_baseline": cpu,
        "detail": detail,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
