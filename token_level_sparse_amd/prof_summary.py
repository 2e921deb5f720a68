"""Text summaries of rocprofv3 output for the profiles/ folder, and the
lookup bench.py uses to report measured HBM traffic.

    # per-kernel durations from a `rocprofv3 --kernel-trace --stats
    # --output-format csv` run
    python -m token_level_sparse_amd.prof_summary stats KERNEL_STATS_CSV --cmd "..."

    # HBM bytes per launch from two `rocprofv3 --pmc` runs of the same command
    # (FETCH_SIZE, then WRITE_SIZE), each scaled by what the same counter reads
    # for a plain copy of known size (hbm_copy_probe.py)
    python -m token_level_sparse_amd.prof_summary traffic FETCH_CSV WRITE_CSV \\
        COPY_FETCH_CSV COPY_WRITE_CSV --copy-mib 1024 --cmd "..." --kernel score_kernel

    # L2 (TCC) hit rate per kernel from one `rocprofv3 --pmc TCC_HIT_sum
    # TCC_MISS_sum` run
    python -m token_level_sparse_amd.prof_summary l2 PMC_CSV --cmd "..."

The traffic summary records a hash of the kernel sources it was measured
with; read_traffic returns nothing once those sources have changed, so a
stale measurement is never reported for a changed kernel.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# sources of the fused score + chunk-select kernel (the dominant launch)
SCORE_KERNEL_SOURCES = ("csrc/score.hip", "csrc/select.hpp", "csrc/common.hpp")


def kernel_source_hash(sources=SCORE_KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(_HERE, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def _short(name: str) -> str:
    name = name.replace("jssa::(anonymous namespace)::", "")
    name = name[5:] if name.startswith("void ") else name
    name = name.split("(")[0] if "(" in name else name
    return name.replace(" ", "")


def stats_text(path: str, cmd: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["# rocprofv3 --kernel-trace --stats: per-kernel durations", f"# command: {cmd}", "",
           f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'share%':>7s}"]
    for r in rows:
        out.append(f"{_short(r['Name'])[:60]:60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                   f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):7.2f}")
    return "\n".join(out) + "\n"


def _per_kernel(path: str, counter: str):
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            agg[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in agg.items()}


def traffic_text(fetch_csv, write_csv, cfetch_csv, cwrite_csv, copy_mib, cmd, copy_cmd, kernel) -> str:
    copy_bytes = copy_mib << 20
    cf = _per_kernel(cfetch_csv, "FETCH_SIZE")
    cw = _per_kernel(cwrite_csv, "WRITE_SIZE")
    copy_name = max(cf, key=cf.get)                       # the copy is the largest reader
    f_scale = copy_bytes / (cf[copy_name] * 1024)
    w_scale = copy_bytes / (cw[copy_name] * 1024)
    fk = _per_kernel(fetch_csv, "FETCH_SIZE")
    wk = _per_kernel(write_csv, "WRITE_SIZE")
    out = ["# HBM bytes per launch from rocprofv3 --pmc (FETCH_SIZE and WRITE_SIZE in separate runs)",
           f"# command: {cmd}",
           f"# calibration command: {copy_cmd}",
           f"# calibration: a {copy_mib} MiB copy ({copy_name}) reads {cf[copy_name]:.1f} KiB FETCH_SIZE and "
           f"{cw[copy_name]:.1f} KiB WRITE_SIZE per launch",
           f"fetch_scale: {f_scale:.4f}",
           f"write_scale: {w_scale:.4f}",
           f"source_sha256: {kernel_source_hash()}",
           f"kernel: {kernel}", "",
           f"{'kernel':40s} {'fetch_KiB':>12s} {'write_KiB':>12s} {'fetch_bytes':>14s} {'write_bytes':>14s}"]
    for name in sorted(set(fk) | set(wk)):
        f, w = fk.get(name, 0.0), wk.get(name, 0.0)
        out.append(f"{name[:40]:40s} {f:12.1f} {w:12.1f} {f * 1024 * f_scale:14.0f} {w * 1024 * w_scale:14.0f}")
    return "\n".join(out) + "\n"


def l2_text(path: str, cmd: str) -> str:
    hit = _per_kernel(path, "TCC_HIT_sum")
    miss = _per_kernel(path, "TCC_MISS_sum")
    out = ["# L2 (TCC) requests per launch from rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum",
           f"# command: {cmd}", "",
           f"{'kernel':60s} {'hits':>12s} {'misses':>12s} {'hit_rate':>9s}"]
    for name in sorted(set(hit) | set(miss), key=lambda n: -(hit.get(n, 0.0) + miss.get(n, 0.0))):
        h, m = hit.get(name, 0.0), miss.get(name, 0.0)
        rate = h / (h + m) if h + m > 0 else float("nan")
        out.append(f"{name[:60]:60s} {h:12.0f} {m:12.0f} {rate:9.3f}")
    return "\n".join(out) + "\n"


def read_traffic(path: str, kernel: str):
    """HBM bytes per launch of `kernel` (fetch + write) from a traffic summary,
    or None when the file is missing or the kernel sources changed since."""
    if not os.path.exists(path):
        return None
    meta, table = {}, {}
    for line in open(path):
        line = line.rstrip("\n")
        if not line or line.startswith("#"):
            continue
        if ": " in line and not line.startswith(" "):
            k, v = line.split(": ", 1)
            meta[k] = v
            continue
        parts = line.split()
        if len(parts) == 5 and parts[0] != "kernel":
            table[parts[0]] = (float(parts[3]), float(parts[4]))
    if meta.get("source_sha256") != kernel_source_hash() or kernel not in table:
        return None
    fetch, write = table[kernel]
    return {"fetch_bytes": int(fetch), "write_bytes": int(write), "bytes": int(fetch + write)}


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("copy_fetch_csv")
    t.add_argument("copy_write_csv")
    t.add_argument("--copy-mib", type=int, default=1024)
    t.add_argument("--cmd", required=True)
    t.add_argument("--copy-cmd", required=True)
    t.add_argument("--kernel", required=True)
    l2 = sub.add_parser("l2")
    l2.add_argument("csv")
    l2.add_argument("--cmd", required=True)
    a = ap.parse_args()
    if a.what == "stats":
        print(stats_text(a.csv, a.cmd), end="")
    elif a.what == "l2":
        print(l2_text(a.csv, a.cmd), end="")
    else:
        print(traffic_text(a.fetch_csv, a.write_csv, a.copy_fetch_csv, a.copy_write_csv, a.copy_mib, a.cmd,
                           a.copy_cmd, a.kernel), end="")


if __name__ == "__main__":
    main()
