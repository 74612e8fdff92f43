"""Summarise rocprofv3 counter runs of bench.py into profiles/.

    python bench_profile.py traffic --fetch F.csv --write W.csv --copy-mib N \\
        --cmd "..." --out profiles/gemm_lds_kernel_llama_traffic.txt
    python bench_profile.py stats --stats S.csv --cmd "..." --out profiles/X.txt

`traffic`: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the large-M GEMM
launches, each scaled by true bytes / counter reading of the plain copy
kernel of N MiB that `bench.py --copy-calib-mib N` runs first; records the
sha256 of the GEMM source so bench.py only uses it for the same kernel.
`stats`: the kernel table of a --kernel-trace --stats run.
`summary`: the text form of one bench.py JSON line.
"""

import argparse
import json
import csv
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
GEMM_SOURCE = os.path.join(ROOT, "block_scaled_precision_fp8_amd", "csrc", "gemm_fp8.hip")
GEMM_KERNEL = "gemm_lds_kernel<0, 4, 2, 64, 128, false, false, false>"


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
    with open(GEMM_SOURCE, "rb") as f:
        h = hashlib.sha256(f.read()).hexdigest()[:16]
    lines = [
        "# HBM traffic of the large-M block-scaled GEMM (fp32 scales), Llama-3-8B linears",
        f"# commands: {a.cmd}",
        f"kernel: {GEMM_KERNEL}",
        f"gemm_fp8.hip sha256[:16]: {h}",
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
    b = sub.add_parser("summary")
    b.add_argument("--json", required=True)
    b.add_argument("--cmd", required=True)
    b.add_argument("--out", required=True)
    a = ap.parse_args()
    {"traffic": traffic, "stats": stats, "summary": summary}[a.what](a)


if __name__ == "__main__":
    main()
