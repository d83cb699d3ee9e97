"""Summaries of rocprofv3 CSV output for this library's kernels.

  python -m bit_quantized_expert_router_amd.profsum stats DIR
      per-kernel dispatch count and average / min / max duration from the
      `*kernel_stats.csv` that `rocprofv3 --kernel-trace --stats
      --output-format csv -d DIR` writes.

  python -m bit_quantized_expert_router_amd.profsum counters DIR [--match NAME]
      per-kernel averages of every counter of a `rocprofv3 --pmc` run, with
      the shader clock and the MFMA-busy and VALU-issue shares of the SIMD
      cycles when GRBM_GUI_ACTIVE, SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU and
      SQ_INSTS_MFMA were collected.

  python -m bit_quantized_expert_router_amd.profsum traffic FETCH_DIR WRITE_DIR
          --kernel NAME --calib-bytes N [--sources FILE ...]
      HBM bytes per dispatch of kernel NAME from two `rocprofv3 --pmc`
      passes (FETCH_SIZE, then WRITE_SIZE; both counters are in KiB per
      dispatch).  Each counter is scaled by the factor that makes it read N
      bytes on the largest device-to-device copy kernel of the same run (a
      plain copy of N bytes reads N and writes N).  With --sources, the
      sha256 of those files (comments and blank lines removed) is printed so
      that a reader can tell whether the kernel has changed since the
      counters were taken.

  python -m bit_quantized_expert_router_amd.profsum segments DIR --kernel NAME
          --split N1,N2,... [--labels L1,L2,...]
      the dispatches of kernel NAME from `*kernel_trace.csv`, in start-time
      order, cut into consecutive runs of N1, N2, ... dispatches (the phases
      of a program whose dispatch counts are known), with the count and the
      average / min / max duration of each run.

Reads CSV only; runs nothing.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import statistics
import sys

COPY_KERNEL = "copyBuffer"


def _short(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "").replace("moeq2::", "")
    return n.split("(")[0].replace("void ", "").strip()


def _one(pattern: str, root: str) -> str:
    found = sorted(glob.glob(os.path.join(root, "**", pattern), recursive=True))
    if not found:
        sys.exit(f"profsum: no {pattern} under {root}")
    return found[0]


def stats(root: str, match: str = "moeq2") -> list[dict]:
    rows = list(csv.DictReader(open(_one("*kernel_stats.csv", root))))
    out = []
    for r in rows:
        if match not in r["Name"] and COPY_KERNEL not in r["Name"]:
            continue
        out.append({"kernel": _short(r["Name"]), "calls": int(r["Calls"]),
                    "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                    "max_us": float(r["MaxNs"]) / 1e3,
                    "total_ms": float(r["TotalDurationNs"]) / 1e6})
    return out


def segments(root: str, kernel: str, split: list[int]) -> list[dict]:
    """Durations (us) of kernel's dispatches in start order, cut into
    consecutive runs of the given sizes."""
    rows = [r for r in csv.DictReader(open(_one("*kernel_trace.csv", root)))
            if _short(r["Kernel_Name"]).split("<")[0] == kernel]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    if sum(split) != len(rows):
        sys.exit(f"profsum: {kernel} has {len(rows)} dispatches, the split covers {sum(split)}")
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    out, i = [], 0
    for n in split:
        part = dur[i:i + n]
        i += n
        out.append({"calls": n, "avg_us": statistics.mean(part) if part else float("nan"),
                    "min_us": min(part) if part else float("nan"), "max_us": max(part) if part else float("nan")})
    return out


def counter_per_dispatch(root: str, counter: str) -> dict[str, list[float]]:
    """kernel -> [counter value of each dispatch] (values summed over the
    per-XCD / per-instance rows of one dispatch)."""
    per = {}
    for f in sorted(glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True)):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            did = next((r[c] for c in ("Dispatch_Id", "Dispatch-Id", "Correlation_Id") if c in r), "")
            key = (_short(r.get("Kernel_Name", r.get("Kernel-Name", ""))), did)
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out: dict[str, list[float]] = {}
    for (k, _), v in per.items():
        out.setdefault(k, []).append(v)
    return out


def counters(root: str, match: str = "prefill", xcds: int = 8, simds: int = 1024) -> list[dict]:
    """Per kernel (name containing `match`, split by grid size): dispatches,
    average duration from the trace timestamps, the average of every counter
    per dispatch, and, with GRBM_GUI_ACTIVE among them (summed over the
    `xcds` XCD instances), the shader clock and the share of SIMD cycles with
    the MFMA unit busy (SQ_VALU_MFMA_BUSY_CYCLES) and with non-MFMA VALU
    instructions issuing (4 cycles each for a wave of 64 on a 16-lane SIMD)."""
    per: dict = {}
    dur: dict = {}
    for f in sorted(glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True)):
        for r in csv.DictReader(open(f)):
            name = _short(r.get("Kernel_Name", ""))
            if match not in name:
                continue
            key = (name, int(r.get("Grid_Size", 0) or 0))
            did = r.get("Dispatch_Id", "")
            per.setdefault(key, {}).setdefault(r["Counter_Name"], {})
            per[key][r["Counter_Name"]][did] = per[key][r["Counter_Name"]].get(did, 0.0) + float(r["Counter_Value"])
            dur.setdefault(key, {})[did] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    out = []
    for key in sorted(per):
        avg = {c: statistics.mean(v.values()) for c, v in per[key].items()}
        row = {"kernel": key[0], "grid": key[1], "dispatches": len(dur[key]),
               "avg_us": statistics.mean(dur[key].values()) / 1e3, "counters": avg}
        if "GRBM_GUI_ACTIVE" in avg:
            cyc = avg["GRBM_GUI_ACTIVE"] / xcds
            row["clock_GHz"] = cyc / (row["avg_us"] * 1e3)
            if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
                row["mfma_busy_pct"] = 100.0 * avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * simds)
            if "SQ_INSTS_VALU" in avg and "SQ_INSTS_MFMA" in avg:
                row["valu_issue_pct"] = 100.0 * 4 * (avg["SQ_INSTS_VALU"] - avg["SQ_INSTS_MFMA"]) / (cyc * simds)
        out.append(row)
    return out


def strip_comments(text: str) -> str:
    """C/C++ source without its comments and blank lines, and with trailing
    spaces removed: what the compiler sees, up to layout.  String and
    character literals are kept as they are (a `//` inside one is code)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c and text[j] != "\n":
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    lines = (l.rstrip() for l in "".join(out).splitlines())
    return "\n".join(l for l in lines if l) + "\n"


def code_sha256(paths) -> str:
    """sha256 over the listed sources with comments and blank lines removed,
    so that a change of comments alone does not mark counters as stale."""
    h = hashlib.sha256()
    for p in paths:
        h.update(strip_comments(open(p, encoding="utf-8").read()).encode())
    return h.hexdigest()


def main(argv=None):
    ap = argparse.ArgumentParser(prog="profsum")
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--match", default="prefill")
    g = sub.add_parser("segments")
    g.add_argument("dir")
    g.add_argument("--kernel", required=True)
    g.add_argument("--split", required=True)
    g.add_argument("--labels", default="")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--kernel", required=True)
    t.add_argument("--calib-bytes", type=int, required=True)
    t.add_argument("--sources", nargs="*", default=[])
    a = ap.parse_args(argv)

    if a.cmd == "counters":
        for r in counters(a.dir, a.match):
            derived = "".join(f"  {k} {r[k]:.2f}" for k in ("clock_GHz", "mfma_busy_pct", "valu_issue_pct") if k in r)
            print(f"{r['kernel']}  grid {r['grid']}  dispatches {r['dispatches']}  avg_us {r['avg_us']:.2f}{derived}")
            for cn, v in sorted(r["counters"].items()):
                print(f"    {cn}: {v:.6g}")
        return

    if a.cmd == "segments":
        split = [int(v) for v in a.split.split(",")]
        labels = a.labels.split(",") if a.labels else [f"part{i}" for i in range(len(split))]
        print(f"{a.kernel}")
        print(f"{'segment':<24} {'calls':>7} {'avg_us':>9} {'min_us':>9} {'max_us':>9}")
        for lab, r in zip(labels, segments(a.dir, a.kernel, split)):
            print(f"{lab[:24]:<24} {r['calls']:>7} {r['avg_us']:>9.2f} {r['min_us']:>9.2f} {r['max_us']:>9.2f}")
        return

    if a.cmd == "stats":
        print(f"{'kernel':<40} {'calls':>7} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'total_ms':>10}")
        for r in stats(a.dir):
            print(f"{r['kernel'][:40]:<40} {r['calls']:>7} {r['avg_us']:>9.2f} {r['min_us']:>9.2f} "
                  f"{r['max_us']:>9.2f} {r['total_ms']:>10.3f}")
        return

    res = {}
    for label, root, counter in (("fetch", a.fetch_dir, "FETCH_SIZE"),
                                 ("write", a.write_dir, "WRITE_SIZE")):
        per = counter_per_dispatch(root, counter)
        copies = [v for k, vs in per.items() if COPY_KERNEL in k for v in vs]
        if not copies:
            sys.exit(f"profsum: no {COPY_KERNEL} dispatch with {counter} in {root}")
        calib_kib = max(copies)
        factor = a.calib_bytes / (calib_kib * 1024.0)
        vals = [v for k, vs in per.items() if k.split("<")[0] == a.kernel for v in vs]
        if not vals:
            sys.exit(f"profsum: kernel {a.kernel} has no {counter} rows in {root}")
        kib = statistics.mean(vals)
        res[label] = (counter, calib_kib, factor, len(vals), kib, kib * 1024.0 * factor)
    print(f"kernel: {a.kernel}")
    for label, (counter, calib_kib, factor, n, kib, b) in res.items():
        print(f"{label}_counter: {counter}")
        print(f"{label}_copy_KiB: {calib_kib:.1f}")
        print(f"{label}_scale: {factor:.5f}")
        print(f"{label}_dispatches: {n}")
        print(f"{label}_KiB_per_dispatch: {kib:.1f}")
        print(f"{label}_bytes_per_launch: {b:.0f}")
    print(f"traffic_bytes_per_launch: {res['fetch'][5] + res['write'][5]:.0f}")
    if a.sources:
        print(f"sources: {' '.join(a.sources)}")
        print(f"source_sha256: {code_sha256(a.sources)}")


if __name__ == "__main__":
    main()
