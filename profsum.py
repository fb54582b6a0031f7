"""Summaries of rocprofv3 CSV output (kernel statistics and counter means).

    python profsum.py stats DIR [N]
        top N kernels of DIR/**/*_kernel_stats.csv by total time
    python profsum.py pmc DIR REGEX
        per-dispatch mean of every counter in DIR/**/*_counter_collection.csv
        over the kernels whose name matches REGEX
    python profsum.py trace DIR REGEX
        dispatch count and mean / median duration from DIR/**/*_kernel_trace.csv
    python profsum.py grids DIR REGEX
        the pmc means (counter CSVs) or trace durations (trace CSVs) of the
        matching kernels, one line per kernel name and grid size
"""
import collections
import csv
import glob
import os
import re
import statistics
import sys


def _files(d, suffix):
    return sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))


def stats(d, n=25):
    rows = []
    for f in _files(d, "_kernel_stats.csv"):
        rows += list(csv.DictReader(open(f)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    print("| kernel | calls | total ms | avg us | % |")
    print("|---|---|---|---|---|")
    for r in rows[:n]:
        name = r["Name"]
        name = name if len(name) < 90 else name[:87] + "..."
        print("| `%s` | %s | %.2f | %.2f | %.2f |" % (
            name, r["Calls"], float(r["TotalDurationNs"]) / 1e6, float(r["AverageNs"]) / 1e3,
            float(r["Percentage"])))


def pmc(d, regex):
    rx = re.compile(regex)
    agg = collections.defaultdict(float)
    disp = collections.defaultdict(set)
    for f in _files(d, "_counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            if not rx.search(r["Kernel_Name"]):
                continue
            agg[r["Counter_Name"]] += float(r["Counter_Value"])
            disp[r["Counter_Name"]].add(r["Dispatch_Id"])
    for c in sorted(agg):
        print("%s: %d dispatches, mean %.6g per dispatch" % (c, len(disp[c]), agg[c] / len(disp[c])))


def trace(d, regex):
    rx = re.compile(regex)
    durs = []
    for f in _files(d, "_kernel_trace.csv"):
        for r in csv.DictReader(open(f)):
            if rx.search(r["Kernel_Name"]):
                durs.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if durs:
        print("%d dispatches, mean %.2f us, median %.2f us" % (len(durs), statistics.mean(durs),
                                                              statistics.median(durs)))


def _grid(r):
    if "Grid_Size" in r:
        return int(r["Grid_Size"])
    return int(r.get("Grid_Size_X", 0)) * int(r.get("Grid_Size_Y", 1) or 1) * int(
        r.get("Grid_Size_Z", 1) or 1)


def grids(d, regex):
    rx = re.compile(regex)
    agg = collections.defaultdict(float)
    disp = collections.defaultdict(set)
    for f in _files(d, "_counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            if rx.search(r["Kernel_Name"]):
                key = (r["Kernel_Name"][:70], _grid(r), r["Counter_Name"])
                agg[key] += float(r["Counter_Value"])
                disp[key].add(r["Dispatch_Id"])
    for k in sorted(agg):
        print("%s grid %d %s: %d dispatches, mean %.6g" % (k[0], k[1], k[2], len(disp[k]),
                                                           agg[k] / len(disp[k])))
    durs = collections.defaultdict(list)
    for f in _files(d, "_kernel_trace.csv"):
        for r in csv.DictReader(open(f)):
            if rx.search(r["Kernel_Name"]):
                durs[(r["Kernel_Name"][:70], _grid(r))].append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    for k in sorted(durs):
        v = durs[k]
        print("%s grid %d: %d dispatches, mean %.2f us, median %.2f us" % (
            k[0], k[1], len(v), statistics.mean(v), statistics.median(v)))


if __name__ == "__main__":
    cmd, d = sys.argv[1], sys.argv[2]
    if cmd == "stats":
        stats(d, int(sys.argv[3]) if len(sys.argv) > 3 else 25)
    elif cmd == "pmc":
        pmc(d, sys.argv[3])
    elif cmd == "grids":
        grids(d, sys.argv[3])
    else:
        trace(d, sys.argv[3])
