"""Turns rocprofv3 CSV output into the short summaries kept with the benchmark.

    python -m partial_activation_sync_amd.rocprof_summary stats <dir> <title> <command>
    python -m partial_activation_sync_amd.rocprof_summary traffic <fetch_dir> <write_dir>
           <copy_fetch_dir> <copy_write_dir> <copy_bytes> <select> <key> <source_file>

``stats`` prints a markdown table of per-kernel call counts and durations from the
``*_kernel_stats.csv`` of a ``--kernel-trace --stats`` run.  ``traffic`` reads the
``*_counter_collection.csv`` of four ``--pmc`` runs (FETCH_SIZE and WRITE_SIZE, in KiB
per dispatch, for the kernel and for a plain copy of known size), takes the median over
the dispatches ``select`` names (a kernel-name regex, or a sequence of them with the
index of the launch wanted; see ``_select``), scales each counter
by the copy's known bytes / its reading, and merges the per-launch HBM bytes of the
kernel into profiles/traffic.json under ``key``, with the SHA-256 of the code the counters
were taken on (the kernel source and its local headers, comments and whitespace left
out, so that a comment edit keeps the record valid).
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


_TOKENS = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|\s+|[^\s"\'/]+|.',
                     re.S)


def _code(path):
    text = open(path, encoding="utf-8").read()
    out = []
    for m in _TOKENS.finditer(text):
        t = m.group(0)
        out.append(" " if t.startswith("//") or t.startswith("/*") or t.isspace() else t)
    return re.sub(r" +", " ", "".join(out)).strip()


def code_sha256(path):
    """SHA-256 of a C/C++/HIP source and the local headers it includes (``#include "..."``,
    followed recursively), with comments dropped and each run of whitespace made one
    space: it changes when the code does, not when only a comment does."""
    seen, order, todo = set(), [], [os.path.abspath(path)]
    while todo:
        f = todo.pop(0)
        if f in seen:
            continue
        seen.add(f)
        code = _code(f)
        order.append(code)
        for inc in re.findall(r'# ?include "([^"]+)"', code):
            for g in (os.path.join(os.path.dirname(f), inc), os.path.join(ROOT, "include", inc)):
                if os.path.exists(g):
                    todo.append(os.path.abspath(g))
                    break
    return hashlib.sha256("\n".join(order).encode()).hexdigest()


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


def _select(rows, select):
    """The dispatches that ``select`` names, in dispatch order.  ``select`` is a kernel-name
    regex (every matching dispatch), or ``re_0;re_1;...;re_m@i``: each run of m + 1
    consecutive dispatches whose names match re_0 .. re_m in turn gives its i-th one (a
    launch picked out by its neighbours, where one kernel serves several steps)."""
    pats, _, idx = select.partition("@")
    pats = [re.compile(x) for x in pats.split(";")]
    idx = int(idx or 0)
    if not 0 <= idx < len(pats):
        raise ValueError(f"index {idx} outside the sequence {select}")
    rows = sorted(rows, key=lambda r: int(r["Dispatch_Id"]))
    out, j = [], 0
    while j + len(pats) <= len(rows):
        if all(p.search(rows[j + k]["Kernel_Name"]) for k, p in enumerate(pats)):
            out.append(rows[j + idx])
            j += len(pats)
        else:
            j += 1
    return out


def _counter(d, name, select):
    rows = [r for r in csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv"))))
            if r["Counter_Name"] == name]
    vals = [float(r["Counter_Value"]) * 1024.0 for r in _select(rows, select)]   # KiB -> bytes
    if not vals:
        raise ValueError(f"no {name} rows for {select} in {d}")
    return statistics.median(vals), len(vals)


def traffic(fetch_dir, write_dir, cfetch_dir, cwrite_dir, copy_bytes, select, key, src):
    copy_bytes = float(copy_bytes)
    cf, _ = _counter(cfetch_dir, "FETCH_SIZE", "copy|Copy|elementwise")
    cw, _ = _counter(cwrite_dir, "WRITE_SIZE", "copy|Copy|elementwise")
    kf, nf = _counter(fetch_dir, "FETCH_SIZE", select)
    kw, nw = _counter(write_dir, "WRITE_SIZE", select)
    sf, sw = copy_bytes / cf, copy_bytes / cw
    rec = {
        "fetch_bytes": kf * sf, "write_bytes": kw * sw,
        "bytes_per_launch": kf * sf + kw * sw,
        "fetch_scale": sf, "write_scale": sw,
        "dispatches": [nf, nw], "kernel_regex": select,
        "code_sha256": code_sha256(os.path.join(ROOT, src)),
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
