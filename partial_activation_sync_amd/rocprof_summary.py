"""Turns rocprofv3 CSV output into the short summaries kept with the benchmark.

    python -m partial_activation_sync_amd.rocprof_summary stats <dir> <title> <command>
    python -m partial_activation_sync_amd.rocprof_summary traffic <fetch_dir> <write_dir>
           <copy_fetch_dir> <copy_write_dir> <copy_bytes> <kernel_regex> <key> <source_file>

``stats`` prints a markdown table of per-kernel call counts and durations from the
``*_kernel_stats.csv`` of a ``--kernel-trace --stats`` run.  ``traffic`` reads the
``*_counter_collection.csv`` of four ``--pmc`` runs (FETCH_SIZE and WRITE_SIZE, in KiB
per dispatch, for the kernel and for a plain copy of known size), scales each counter
by the copy's known bytes / its reading, and merges the per-launch HBM bytes of the
kernel into profiles/traffic.json under ``key``, with the SHA-256 of the kernel source
the counters were taken on.
"""
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _one(pattern):
    hits = glob.glob(pattern, recursive=True)
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def stats(d, title, command):
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*kernel_stats.csv")))))
    out = [f"# {title}", "", f"Command: `{command}`", "",
           "| kernel | calls | average (us) | min (us) | max (us) | share |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        short = re.sub(r"\(.*", "", name.replace("caat::(anonymous namespace)::", ""))
        out.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{float(r['Percentage']):.1f}% |")
    return "\n".join(out) + "\n"


def _counter(d, name, kernel_regex):
    vals = []
    for r in csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))):
        if r["Counter_Name"] == name and re.search(kernel_regex, r["Kernel_Name"]):
            vals.append(float(r["Counter_Value"]) * 1024.0)   # KiB -> bytes
    if not vals:
        raise ValueError(f"no {name} rows for {kernel_regex} in {d}")
    return statistics.median(vals), len(vals)


def traffic(fetch_dir, write_dir, cfetch_dir, cwrite_dir, copy_bytes, kernel_regex, key, src):
    copy_bytes = float(copy_bytes)
    cf, _ = _counter(cfetch_dir, "FETCH_SIZE", "copy|Copy|elementwise")
    cw, _ = _counter(cwrite_dir, "WRITE_SIZE", "copy|Copy|elementwise")
    kf, nf = _counter(fetch_dir, "FETCH_SIZE", kernel_regex)
    kw, nw = _counter(write_dir, "WRITE_SIZE", kernel_regex)
    sf, sw = copy_bytes / cf, copy_bytes / cw
    rec = {
        "fetch_bytes": kf * sf, "write_bytes": kw * sw,
        "bytes_per_launch": kf * sf + kw * sw,
        "fetch_scale": sf, "write_scale": sw,
        "dispatches": [nf, nw], "kernel_regex": kernel_regex,
        "source_sha256": hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest(),
        "source": src,
    }
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data[key] = rec
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    return rec


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        print(stats(sys.argv[2], sys.argv[3], sys.argv[4]), end="")
    elif sys.argv[1] == "traffic":
        print(json.dumps(traffic(*sys.argv[2:10]), indent=1))
    else:
        raise SystemExit(__doc__)
