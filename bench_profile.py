"""Summarise rocprofv3 counter runs of bench.py into profiles/.

    python bench_profile.py traffic --fetch F.csv --write W.csv --copy-mib N \\
        --cmd "..." --out profiles/gemm_lds_kernel_llama_traffic.txt
    python bench_profile.py stats --stats S.csv --cmd "..." --out profiles/X.txt

`traffic`: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the large-M GEMM
launches, each scaled by true bytes / counter reading of the plain copy
kernel of N MiB that `bench.py --copy-calib-mib N` runs first; records the
sha256 of the GEMM sources (gemm_fp8.hip and the bsfp8_internal.h device
helpers) so bench.py only uses it for the same kernel.
`stats`: the kernel table of a --kernel-trace --stats run.
`mfma`: MFMA busy share and counted flops of the large-M GEMM from a
--pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_F8 run
(--kernel, --mops, --peak and --title select another kernel, other MOPS
counters -- summed -- and their peak, e.g. the FP8 x MXFP4 tile with
SQ_INSTS_VALU_MFMA_MOPS_F8,SQ_INSTS_VALU_MFMA_MOPS_F6F4).
`decode`: HBM bytes per decode-GEMM dispatch (gemm_decode_kernel and
gemm_decode_pers_kernel) over its duration, from the FETCH_SIZE run (scaled
by the same copy calibration).
`l1`: what bounds the operand loads of the large-M GEMM, from two --pmc
runs (a third, TCC_HIT_sum TCC_MISS_sum, adds the L2 hit rate): texture-data stalls on L1, L1 pending and tag-conflict stalls, address
stalls, and the L1-to-L2 request count and average latency, with the
concurrency they imply (Little's law).
`summary`: the text form of one bench.py JSON line.
`keep`: copy a counter CSV keeping only the rows of kernels whose names
contain one of the ';'-separated --kernels substrings (a whole-bench counter
run writes tens of MB).
`bound`: for the kernels named by --kernels (label=substring pairs), per
launch shape (grid), the share of each hardware limit the launches reach,
from five counter runs of one command: HBM traffic (FETCH_SIZE, WRITE_SIZE,
scaled by the copy kernel's readings) against 8 TB/s, MFMA busy cycles
(SQ_VALU_MFMA_BUSY_CYCLES) and VALU issue (SQ_INSTS_VALU, 4 cycles per wave
instruction) against the SIMD cycles, texture address and data unit busy
cycles (TA_TA_BUSY_sum, TD_TD_BUSY_sum) against the CU cycles, and the L2
hit rate; the largest share names the bounding counter.
`trace`: from a --kernel-trace run of the default bench command and that
run's JSON line, the dominant kernel's average over the timed steps, the
roofline fraction it implies, and the gaps between kernels in that window.
"""

import argparse
import json
import csv
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
# the large-M GEMM's code: its kernel source and the device helpers it includes
GEMM_SOURCES = [os.path.join(ROOT, "block_scaled_precision_fp8_amd", "csrc", f)
                for f in ("gemm_fp8.hip", "bsfp8_internal.h")]
# the dense fp32-scale 256x256 tile (grouped, W4, SiLU-mul off), whatever follows
GEMM_KERNEL = "gemm_lds_kernel<0, 4, 2, 64, 128, false, false, false,"


def per_kernel(path, counter):
    vals = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return vals


def pick(vals, needle):
    out = []
    for k, v in vals.items():
        if needle in k:
            out += v
    return out


def traffic(a):
    fetch = per_kernel(a.fetch, "FETCH_SIZE")
    write = per_kernel(a.write, "WRITE_SIZE")
    copy_kib = a.copy_mib * 1024.0
    cf = max(pick(fetch, "copy"), default=None)
    cw = max(pick(write, "copy"), default=None)
    if not cf or not cw:
        sys.exit("no copy kernel found in the counter files")
    sf, sw = copy_kib / cf, copy_kib / cw
    gf, gw = pick(fetch, GEMM_KERNEL), pick(write, GEMM_KERNEL)
    if not gf or not gw:
        sys.exit("no large-M GEMM launches found")
    fkib, wkib = sum(gf) / len(gf), sum(gw) / len(gw)
    tot = (fkib * sf + wkib * sw) * 1024.0
    hs = hashlib.sha256()
    for path in GEMM_SOURCES:
        with open(path, "rb") as f:
            hs.update(f.read())
    h = hs.hexdigest()[:16]
    lines = [
        "# HBM traffic of the large-M block-scaled GEMM (fp32 scales), Llama-3-8B linears",
        f"# commands: {a.cmd}",
        f"kernel: {GEMM_KERNEL}",
        f"gemm sources sha256[:16]: {h}",
        f"launches averaged: {len(gf)}",
        f"copy kernel: {a.copy_mib} MiB read + {a.copy_mib} MiB written; "
        f"FETCH_SIZE {cf:.0f} KiB, WRITE_SIZE {cw:.0f} KiB",
        f"scale factors (true / counter): fetch {sf:.4f}, write {sw:.4f}",
        f"FETCH_SIZE per launch (KiB, raw): {fkib:.0f}",
        f"WRITE_SIZE per launch (KiB, raw): {wkib:.0f}",
        f"hbm bytes per launch (scaled): {tot:.0f}",
    ]
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def dispatches(path):
    """Dispatch_Id -> {name, grid, ns, counter values} from a counter CSV"""
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = out.setdefault(r["Dispatch_Id"], {
                "name": r["Kernel_Name"], "grid": int(r["Grid_Size"]),
                "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def mfma(a):
    """MFMA busy share of SIMD cycles and counted MFMA flops of one kernel"""
    simds, xcds = 256 * 4, 8
    rows = [d for d in dispatches(a.pmc).values() if a.kernel in d["name"]]
    if not rows:
        sys.exit(f"no dispatches of {a.kernel} found")
    mops = a.mops.split(",")
    # the CSV sums GRBM_GUI_ACTIVE over the 8 XCDs: one XCD's count is the
    # kernel's active cycles (dividing by the dispatch time gives the clock)
    cyc = [d["GRBM_GUI_ACTIVE"] / xcds for d in rows]
    util = [d["SQ_VALU_MFMA_BUSY_CYCLES"] / (c * simds) for d, c in zip(rows, cyc)]
    ghz = [c / d["ns"] for d, c in zip(rows, cyc)]
    tf = [sum(d.get(c, 0.0) for c in mops) * 512 / d["ns"] / 1e3 for d in rows]
    per = {c: sum(d.get(c, 0.0) for d in rows) for c in mops}
    lines = [
        f"# MFMA utilisation of {a.title}",
        f"# command: {a.cmd}",
        f"kernel: {a.kernel}",
        f"dispatches: {len(rows)}",
        "MFMA busy / (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs), mean over dispatches: "
        f"{100 * sum(util) / len(util):.1f}% (min {100 * min(util):.1f}%, max {100 * max(util):.1f}%)",
        f"clock implied by GRBM_GUI_ACTIVE per XCD / dispatch time: {sum(ghz) / len(ghz):.2f} GHz",
        f"flops counted ({' + '.join(mops)}) x 512 / dispatch time, mean: "
        f"{sum(tf) / len(tf):.0f} TFLOP/s (dense peak {a.peak:.0f})",
    ]
    if len(mops) > 1:
        tot = sum(per.values()) or 1.0
        lines.append("share of the counted MOPS: " +
                     ", ".join(f"{c} {100 * v / tot:.1f}%" for c, v in per.items()))
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def decode(a):
    """HBM bytes fetched per decode-kernel dispatch over its duration"""
    ds = dispatches(a.fetch)
    copy = [d for d in ds.values() if "copy" in d["name"]]
    if not copy:
        sys.exit("no copy kernel found")
    sf = a.copy_mib * 1024.0 / max(d["FETCH_SIZE"] for d in copy)
    groups = {}
    for d in ds.values():
        if "gemm_decode_" not in d["name"]:   # gemm_decode_kernel, gemm_decode_pers_kernel
            continue
        mb = d["FETCH_SIZE"] * sf * 1024 / 1e6
        key = (d["name"].split("(")[0].replace("void bsfp8::detail::", ""), d["grid"] // 1024,
               round(mb))
        groups.setdefault(key, []).append((mb, d["ns"]))
    lines = [f"# HBM reads of the decode GEMM (M <= 16) per dispatch, {a.title}",
             f"# command: {a.cmd}",
             f"FETCH_SIZE scale (true / counter, {a.copy_mib} MiB copy): {sf:.4f}",
             "# kernel | workgroups (N/16) | dispatches | MB fetched | us | GB/s"]
    for (name, wg, _), v in sorted(groups.items(), key=lambda t: (t[0][1], t[0][2])):
        mb = sum(x for x, _ in v) / len(v)
        us = sum(t for _, t in v) / len(v) / 1e3
        lines.append(f"{name} | {wg} | {len(v)} | {mb:.1f} | {us:.1f} | {mb * 1e3 / us:.0f}")
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def l1(a):
    """L1-miss concurrency bound of the large-M GEMM's LDS-DMA operand loads"""
    cus = 256
    rows = {}
    for path in (a.pmc1, a.pmc2):
        for k, d in dispatches(path).items():
            if GEMM_KERNEL in d["name"]:
                rows.setdefault(path, []).append(d)
    r1, r2 = rows.get(a.pmc1), rows.get(a.pmc2)
    if not r1 or not r2:
        sys.exit("no large-M GEMM dispatches found")

    def mean_per_cu_cycle(rs, key):
        return sum(d[key] / (d["GRBM_GUI_ACTIVE"] / 8 * cus) for d in rs) / len(rs)

    req = sum(d["TCP_TCC_READ_REQ_sum"] for d in r2)
    lat = sum(d["TCP_TCC_READ_REQ_LATENCY_sum"] for d in r2) / req
    waves = sum(d["TA_BUFFER_READ_LDS_WAVEFRONTS_sum"] for d in r2)
    cyc = sum(d["GRBM_GUI_ACTIVE"] / 8 for d in r2)
    # bytes the DMA moves: 64 lanes x 16 bytes per LDS-load wavefront
    bpc = waves * 1024.0 / (cyc * cus)
    rpc = req / (cyc * cus)                      # L1-to-L2 read requests per CU cycle
    lines = [
        "# What bounds the operand loads of the large-M block-scaled GEMM (fp32 scales), Llama-3-8B linears",
        f"# commands: {a.cmd}",
        f"kernel: {GEMM_KERNEL}",
        f"dispatches: {len(r1)} (stall pass), {len(r2)} (request pass)",
        "fractions of CU cycles (counter sum / (GRBM_GUI_ACTIVE per XCD x 256 CUs)):",
        f"  TD busy {mean_per_cu_cycle(r2, 'TD_TD_BUSY_sum'):.3f}, of which stalled on L1 data "
        f"(TD_TC_STALL) {mean_per_cu_cycle(r1, 'TD_TC_STALL_sum'):.3f}",
        f"  L1 pending stall {mean_per_cu_cycle(r1, 'TCP_PENDING_STALL_CYCLES_sum'):.3f}, "
        f"L1 read tag-conflict stall {mean_per_cu_cycle(r1, 'TCP_READ_TAGCONFLICT_STALL_CYCLES_sum'):.3f}",
        f"  TA address stalled by L1 {mean_per_cu_cycle(r1, 'TA_ADDR_STALLED_BY_TC_CYCLES_sum'):.3f}",
        f"LDS-DMA wavefronts: {waves:.0f}; L1-to-L2 read requests per wavefront: {req / waves:.1f}",
        f"average L1-to-L2 read latency: {lat:.0f} cycles",
        f"operand bytes through L1 per CU cycle: {bpc:.1f} (DMA bytes per L2 request: "
        f"{waves * 1024.0 / req:.0f})",
        f"L2 read requests in flight per CU (Little's law: requests per CU cycle x latency): "
        f"{rpc * lat:.0f}",
        f"bytes per CU cycle the 256x256 tile needs at the full FP8 MFMA rate "
        f"(4 SIMDs x 2048 flop/cycle / 256 flop/byte): 32.0",
    ]
    if a.pmc3:
        # L2 hits and misses of the same launches (reads and the epilogue's
        # writes): the misses are the requests whose operand lines no other
        # concurrent tile has brought into this XCD's L2 yet
        r3 = [d for d in dispatches(a.pmc3).values() if GEMM_KERNEL in d["name"]]
        hit = sum(d["TCC_HIT_sum"] for d in r3)
        miss = sum(d["TCC_MISS_sum"] for d in r3)
        lines.append(f"L2 hit rate (TCC_HIT / (TCC_HIT + TCC_MISS)) over {len(r3)} launches: "
                     f"{100 * hit / max(hit + miss, 1.0):.1f}%")
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def stats(a):
    rows = list(csv.DictReader(open(a.stats)))
    lines = [f"# rocprofv3 kernel statistics; command: {a.cmd}",
             "# name | calls | total ns | average ns | percent"]
    for r in rows[: a.top]:
        name = r.get("Name", "")
        if len(name) > 110:
            name = name[:107] + "..."
        lines.append(f"{name} | {r.get('Calls')} | {r.get('TotalDurationNs')} | "
                     f"{r.get('AverageNs')} | {r.get('Percentage')}")
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def trace(a):
    """kernel-trace run of bench.py: the dominant kernel's average duration
    over the timed steps of the Llama step (its launches in order: warm-up
    steps, timed steps, the untimed detail pass), the roofline fraction it
    implies, the bench line of the same run, and the gaps between kernels
    inside the timed window"""
    rows = list(csv.DictReader(open(a.trace)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    with open(a.json) as f:
        d = json.loads(f.read().strip().splitlines()[-1])
    rl = d["roofline"]
    per = int(rl["launches_per_step"])
    idx = [i for i, r in enumerate(rows) if a.kernel in r["Kernel_Name"]]
    lo, hi = a.warmup * per, (a.warmup + a.steps) * per
    timed = idx[lo:hi]
    dur = [(int(rows[i]["End_Timestamp"]) - int(rows[i]["Start_Timestamp"])) / 1e3 for i in timed]
    avg = sum(dur) / len(dur)
    gflop = float(rl["algorithmic_gflop_per_launch"])
    t0, t1 = int(rows[timed[0]]["Start_Timestamp"]), int(rows[timed[-1]]["End_Timestamp"])
    win = [r for r in rows if int(r["Start_Timestamp"]) >= t0 and int(r["End_Timestamp"]) <= t1]
    busy = sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in win) / 1e3
    span = (t1 - t0) / 1e3
    lines = [
        f"# dominant kernel over the timed steps, from one kernel-trace run of bench.py; command: {a.cmd}",
        f"kernel: {a.kernel}",
        f"dispatches in the run: {len(idx)}; timed-step dispatches: {len(dur)} "
        f"(occurrences {lo}..{hi - 1}: {a.warmup} warm-up steps x {per} come first)",
        f"average duration over the timed steps (us): {avg:.2f}",
        f"algorithmic GFLOP per launch: {gflop}",
        f"achieved TFLOP/s: {gflop / avg * 1e3:.1f}; fraction of the 5000 TFLOP/s dense FP8 peak: "
        f"{gflop / avg * 1e3 / 5000.0:.4f}",
        f"the same run's bench line: value {d['value']} TFLOP/s, ms_per_step {d['ms_per_step']}, "
        f"roofline achieved {rl['achieved']} frac {rl['frac']} (HIP events: avg_launch_us "
        f"{rl['avg_launch_us']})",
        f"timed window: {span:.1f} us, {len(win)} kernels, {busy:.1f} us busy, "
        f"{span - busy:.1f} us between kernels ({(span - busy) / len(win):.2f} us per kernel)",
    ]
    # where one timed step's time goes, by kernel (name cut at the argument list)
    by = {}
    for r in win:
        name = r["Kernel_Name"].split("(")[0]
        t = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        n, tot = by.get(name, (0, 0.0))
        by[name] = (n + 1, tot + t)
    lines.append(f"# per timed step ({a.steps} steps): kernel | launches | us | share of the step span")
    for name, (n, tot) in sorted(by.items(), key=lambda kv: -kv[1][1]):
        lines.append(f"{name} | {n / a.steps:.1f} | {tot / a.steps:.1f} | {tot / span:.3f}")
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summary(a):
    """one bench.py JSON line -> the text summary kept under profiles/"""
    with open(a.json) as f:
        d = json.loads(f.read().strip().splitlines()[-1])
    lines = [f"# bench.py (all suites) on one MI355X; command: {a.cmd}",
             f"value ({d['config']['workload'][:60]}...): {d['value']} {d['unit']}, "
             f"ms_per_step {d['ms_per_step']}",
             "roofline: " + json.dumps(d["roofline"]),
             "cpu_baseline: " + json.dumps(d["cpu_baseline"]),
             "# per-run details"]
    for key, val in d["detail"].items():
        if isinstance(val, list):
            lines += [f"{key}: " + json.dumps(r) for r in val]
        else:
            lines.append(f"{key}: " + json.dumps(val))
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")


def keep(a):
    """the rows of the selected kernels of one counter CSV"""
    needles = a.kernels.split(";")
    with open(a.src) as f, open(a.dst, "w", newline="") as g:
        r = csv.DictReader(f)
        w = csv.DictWriter(g, fieldnames=r.fieldnames)
        w.writeheader()
        for row in r:
            if any(n in row["Kernel_Name"] for n in needles):
                w.writerow(row)


def bound(a):
    """which hardware limit each selected kernel's launches come closest to"""
    simds, cus, xcds = 1024, 256, 8
    runs = {k: dispatches(getattr(a, k)) for k in ("fetch", "write", "sq", "l2", "tx")}
    scale = {}
    for k, ctr in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        copy = [d[ctr] for d in runs[k].values() if "copy" in d["name"]]
        if not copy:
            sys.exit(f"no copy kernel in the {ctr} run")
        scale[k] = a.copy_mib * 1024.0 / max(copy)
    sel = [kv.split("=", 1) for kv in a.kernels.split(";")]
    mops = a.mops.split(",")

    def groups(rs):
        g = {}
        for d in rs.values():
            for label, needle in sel:
                if needle in d["name"]:
                    g.setdefault((label, d["grid"]), []).append(d)
        return g

    G = {k: groups(v) for k, v in runs.items()}
    lines = [f"# What bounds {a.title}", f"# commands: {a.cmd}",
             f"FETCH_SIZE / WRITE_SIZE scale (true / counter, {a.copy_mib} MiB copy): "
             f"{scale['fetch']:.4f} / {scale['write']:.4f}",
             "# kernel | grid | launches | us | HBM read MB | HBM write MB | HBM share of 8 TB/s | "
             "MFMA busy | MFMA TF/s | VALU issue share | TA busy | TD busy | L2 hit | nearest limit"]
    for key in sorted(G["fetch"], key=lambda t: (t[0], t[1])):
        def mean(run, f):
            rs = G[run].get(key, [])
            return sum(f(d) for d in rs) / len(rs) if rs else float("nan")
        us = mean("fetch", lambda d: d["ns"]) / 1e3
        rd = mean("fetch", lambda d: d["FETCH_SIZE"] * scale["fetch"] * 1024 / 1e6)
        wr = mean("write", lambda d: d["WRITE_SIZE"] * scale["write"] * 1024 / 1e6)
        hbm = (rd + wr) * 1e6 / (us * 1e-6) / 8e12
        cyc = lambda d: d["GRBM_GUI_ACTIVE"] / xcds
        mf = mean("sq", lambda d: d["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc(d) * simds))
        tf = mean("sq", lambda d: sum(d.get(c, 0.0) for c in mops) * 512 / d["ns"] / 1e3)
        va = mean("sq", lambda d: d["SQ_INSTS_VALU"] * 4 / (cyc(d) * simds))
        ta = mean("tx", lambda d: d["TA_TA_BUSY_sum"] / (cyc(d) * cus))
        td = mean("tx", lambda d: d["TD_TD_BUSY_sum"] / (cyc(d) * cus))
        hit = mean("l2", lambda d: d["TCC_HIT_sum"] / max(d["TCC_HIT_sum"] + d["TCC_MISS_sum"], 1.0))
        lim = max((("HBM (FETCH_SIZE + WRITE_SIZE)", hbm), ("MFMA (SQ_VALU_MFMA_BUSY_CYCLES)", mf),
                   ("VALU (SQ_INSTS_VALU)", va), ("TA (TA_TA_BUSY_sum)", ta),
                   ("TD (TD_TD_BUSY_sum)", td)), key=lambda t: t[1])
        n = len(G["fetch"][key])
        lines.append(f"{key[0]} | {key[1]} | {n} | {us:.1f} | {rd:.1f} | {wr:.1f} | {hbm:.3f} | "
                     f"{mf:.3f} | {tf:.0f} | {va:.3f} | {ta:.3f} | {td:.3f} | {100 * hit:.1f}% | "
                     f"{lim[0]} {lim[1]:.3f}")
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--out", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--stats", required=True)
    s.add_argument("--cmd", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--top", type=int, default=12)
    m = sub.add_parser("mfma")
    m.add_argument("--pmc", required=True)
    m.add_argument("--cmd", required=True)
    m.add_argument("--out", required=True)
    m.add_argument("--kernel", default=GEMM_KERNEL)
    m.add_argument("--mops", default="SQ_INSTS_VALU_MFMA_MOPS_F8")
    m.add_argument("--peak", type=float, default=5000.0)
    m.add_argument("--title", default="the large-M block-scaled GEMM (fp32 scales), Llama-3-8B linears")
    d = sub.add_parser("decode")
    d.add_argument("--fetch", required=True)
    d.add_argument("--copy-mib", type=int, required=True)
    d.add_argument("--cmd", required=True)
    d.add_argument("--out", required=True)
    d.add_argument("--title", default="Llama-3-8B linears")
    l = sub.add_parser("l1")
    l.add_argument("--pmc1", required=True)
    l.add_argument("--pmc2", required=True)
    l.add_argument("--pmc3", default=None, help="optional TCC_HIT_sum TCC_MISS_sum run")
    l.add_argument("--cmd", required=True)
    l.add_argument("--out", required=True)
    tr = sub.add_parser("trace")
    tr.add_argument("--trace", required=True)
    tr.add_argument("--json", required=True)
    tr.add_argument("--cmd", required=True)
    tr.add_argument("--out", required=True)
    tr.add_argument("--kernel", default=GEMM_KERNEL)
    tr.add_argument("--warmup", type=int, default=5)
    tr.add_argument("--steps", type=int, default=20)
    kp = sub.add_parser("keep")
    kp.add_argument("--src", required=True)
    kp.add_argument("--dst", required=True)
    kp.add_argument("--kernels", required=True)
    bd = sub.add_parser("bound")
    for k in ("fetch", "write", "sq", "l2", "tx"):
        bd.add_argument("--" + k, required=True)
    bd.add_argument("--copy-mib", type=int, required=True)
    bd.add_argument("--kernels", required=True, help="label=substring;label=substring...")
    bd.add_argument("--mops", default="SQ_INSTS_VALU_MFMA_MOPS_F8")
    bd.add_argument("--title", required=True)
    bd.add_argument("--cmd", required=True)
    bd.add_argument("--out", required=True)
    b = sub.add_parser("summary")
    b.add_argument("--json", required=True)
    b.add_argument("--cmd", required=True)
    b.add_argument("--out", required=True)
    a = ap.parse_args()
    {"traffic": traffic, "stats": stats, "summary": summary, "mfma": mfma,
     "decode": decode, "l1": l1, "trace": trace, "bound": bound, "keep": keep}[a.what](a)


if __name__ == "__main__":
    main()
