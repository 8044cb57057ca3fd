"""Turns rocprofv3 CSV output into the short summaries kept with the benchmark.

    python -m partial_activation_sync_amd.rocprof_summary stats <dir> <title> <command>
    python -m partial_activation_sync_amd.rocprof_summary traffic <fetch_dir> <write_dir>
           <copy_fetch_dir> <copy_write_dir> <copy_bytes> <select> <key> <source_file>

    python -m partial_activation_sync_amd.rocprof_summary mfma <dir> <title> <command>
           [<name regex>=<label> ...]

``mfma`` reads the ``*_counter_collection.csv`` of a run with ``--pmc
SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE``
and prints, per dispatch of each MFMA kernel, its duration, bf16 MFMA FLOPs (MOPS x
512), the achieved rate, the clock (GRBM_GUI_ACTIVE per XCD over the duration) and the
MFMA utilisation (busy cycles summed over the SIMDs / (GUI_ACTIVE per XCD x SIMDs), the
MfmaUtil expression rocprofv3 lists), medians over the dispatches with the same launch
position in the step.

    python -m partial_activation_sync_amd.rocprof_summary steps <dir> [<label> ...]

``steps`` reads the ``*_kernel_trace.csv`` of a ``--kernel-trace`` run and prints the mean,
median and minimum duration of each launch position of the repeating step (the library's
kernels only; the labels name the positions in order), and the mean gap between launches.

    python -m partial_activation_sync_amd.rocprof_summary coverage <dir> <library>

``coverage`` compares the kernels a shared library holds (the ``*.kd`` kernel-descriptor
symbols of its code object) with those a ``--kernel-trace --stats`` run launched (its
``*_kernel_stats.csv``), and lists the ones never launched.

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
    """SHA-256 of a C/C++/HIP source (or a list of them) and the local headers it includes
    (``#include "..."``, followed recursively), with comments dropped and each run of
    whitespace made one space: it changes when the code does, not when only a comment
    does."""
    paths = list(path) if isinstance(path, (list, tuple)) else [path]
    seen, order, todo = set(), [], [os.path.abspath(p) for p in paths]
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
        "code_sha256": code_sha256([os.path.join(ROOT, f) for f in src.split("+")]),
        "source": src,
    }
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data[key] = rec
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    return rec


def _period(names):
    """Length and count of the step that repeats from the first launch on: the shortest p
    whose pattern holds for at least three steps (or the whole run), and how many whole
    steps follow it from the start (a run may end with other kernels, e.g. timing of a
    different pass)."""
    for p in range(1, len(names) + 1):
        span = min(len(names), 3 * p)
        if all(names[i] == names[i % p] for i in range(span)):
            n = 0
            while (n + 1) * p <= len(names) and names[n * p:(n + 1) * p] == names[:p]:
                n += 1
            return p, n
    return len(names), 1


def _short(name):
    return re.sub(r"\(.*", "", name.replace("caat::(anonymous namespace)::", ""))


def steps(d, labels=()):
    rows = [r for r in csv.DictReader(open(_one(os.path.join(d, "**", "*kernel_trace.csv"))))
            if "caat" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    names = [_short(r["Kernel_Name"]) for r in rows]
    per, n = _period(names)
    out = ["| # | step | kernel | launches | mean (us) | median (us) | min (us) |",
           "|---|---|---|---|---|---|---|"]
    total = 0.0
    for i in range(per):
        ds = [(int(rows[k * per + i]["End_Timestamp"]) - int(rows[k * per + i]["Start_Timestamp"])) / 1e3
              for k in range(n)]
        total += statistics.mean(ds)
        lab = labels[i] if i < len(labels) else ""
        out.append(f"| {i} | {lab} | `{names[i]}` | {n} | {statistics.mean(ds):.1f} | "
                   f"{statistics.median(ds):.1f} | {min(ds):.1f} |")
    gaps = [(int(rows[k + 1]["Start_Timestamp"]) - int(rows[k]["End_Timestamp"])) / 1e3
            for k in range(n * per - 1) if (k + 1) % per]
    out.append(f"| | sum | | | {total:.1f} | | |")
    out.append("")
    out.append(f"Mean gap between consecutive launches of a step: {statistics.mean(gaps):.2f} us "
               f"(median {statistics.median(gaps):.2f}).")
    return "\n".join(out) + "\n"


def mfma(d, title, command, labels=(), simds=1024, xcds=8):
    """Per MFMA dispatch (in launch order within a repeating step): duration, FLOPs from
    SQ_INSTS_VALU_MFMA_MOPS_BF16, clock and MFMA utilisation; medians by position."""
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))))
    by = {}
    for r in rows:
        e = by.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"],
                                                  "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        e[r["Counter_Name"]] = float(r["Counter_Value"])
    # The library's kernels only (torch's fills and copies set up the inputs).
    disp = [by[k] for k in sorted(by) if "caat" in by[k]["name"]]
    # The step repeats: find its period from the kernel-name sequence.
    names = [_short(e["name"]) for e in disp]
    period, nsteps = _period(names)
    disp = disp[:period * nsteps]
    lab = [(re.compile(k), v) for k, v in labels]
    out = [f"# {title}", "", f"Command: `{command}`", "",
           "| # | kernel | step | dispatches | duration (us) | MFMA TFLOP | TFLOP/s | of 2.5 PF "
           "| clock (GHz) | MFMA busy at that clock |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    for i in range(period):
        grp = disp[i::period]
        if not any(e.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0) > 0 for e in grp):
            continue
        us = statistics.median(e["ns"] for e in grp) / 1e3
        fl = statistics.median(e["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for e in grp) * 512
        gui = statistics.median(e["GRBM_GUI_ACTIVE"] for e in grp) / xcds
        busy = statistics.median(e["SQ_VALU_MFMA_BUSY_CYCLES"] for e in grp)
        step = next((v for k, v in lab if k.search(f"{i}:{names[i]}")), "")
        out.append(f"| {i} | `{names[i]}` | {step} | {len(grp)} | {us:.1f} | {fl / 1e12:.4f} | "
                   f"{fl / us / 1e6:.0f} | {fl / us / 1e6 / 2500:.3f} | {gui / us / 1e3:.2f} | "
                   f"{busy / (gui * simds):.3f} |")
    return "\n".join(out) + "\n"


def _demangle(names):
    import subprocess
    r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True)
    out = r.stdout.split("\n") if r.returncode == 0 else list(names)
    return [o.split("(")[0].replace("(anonymous namespace)::", "").strip() for o in out[:len(names)]]


def coverage(trace_dir, library):
    """Markdown summary: kernels held by ``library`` against kernels launched in the trace."""
    data = open(library, "rb").read()
    held = sorted({m.decode()[:-3] for m in re.findall(rb"_Z[0-9A-Za-z_]+\.kd(?=\x00)", data)})
    path = glob.glob(os.path.join(trace_dir, "**", "*_kernel_stats.csv"), recursive=True)[0]
    launched = set(_demangle([r["Name"] for r in csv.DictReader(open(path))]))
    held_names = _demangle(held)
    never = sorted(n for n in held_names if n not in launched)
    out = [f"Kernels in `{os.path.basename(library)}`: {len(held_names)}; launched by the traced "
           f"run: {len(held_names) - len(never)}; never launched: {len(never)}."]
    out += [f"- `{n}`" for n in never]
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        print(stats(sys.argv[2], sys.argv[3], sys.argv[4]), end="")
    elif sys.argv[1] == "steps":
        print(steps(sys.argv[2], sys.argv[3:]), end="")
    elif sys.argv[1] == "mfma":
        print(mfma(sys.argv[2], sys.argv[3], sys.argv[4],
                   [tuple(a.split("=", 1)) for a in sys.argv[5:]]), end="")
    elif sys.argv[1] == "coverage":
        print(coverage(sys.argv[2], sys.argv[3]), end="")
    elif sys.argv[1] == "traffic":
        print(json.dumps(traffic(*sys.argv[2:10]), indent=1))
    else:
        raise SystemExit(__doc__)
