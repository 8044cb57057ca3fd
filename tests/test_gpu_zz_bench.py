"""bench.py's output line: the fields, types and internal consistency of the JSON object
it prints (a short run of each pass), and its refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=600):
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                       capture_output=True, text=True, timeout=timeout)
    return r


def _line(r):
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert lines, r.stderr[-2000:]
    return json.loads(lines[-1])


def _check_common(d, steps, warmup):
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["higher_is_better"] is True and d["scaling"] in ("weak", "strong")
    assert d["vs_baseline"] is None
    assert isinstance(d["config"].get("workload"), str)
    roof = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    assert roof["bound"] in ("hbm", "mfma", "alu")
    assert roof["unit"] == ("GB/s" if roof["bound"] == "hbm" else "TFLOP/s")
    assert roof["peak"] == (8000.0 if roof["bound"] == "hbm" else 2500.0)
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert roof["traffic"] is None or roof["traffic"] > 0


@pytest.mark.gpu
def test_bench_forward_default_line():
    d = _line(_bench("--steps", "2", "--warmup", "1", "--cpu-budget", "1"))
    _check_common(d, 2, 1)
    assert d["unit"] == "tokens/s" and d["dtype"] == "bf16"
    assert d["config"]["workload"] == "7b-prefill-pair-bf16"
    base = d["cpu_baseline"]
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in base, k
    assert base["kind"] == "oracle" and base["value"] > 0 and base["cores"] >= 1
    for k in ("sublayers", "exchange_derived", "per_gpu_share", "step_ms_stats"):
        assert d.get(k) is not None, k
    st = d["step_ms_stats"]
    assert st["min"] <= st["median"] <= st["max"] and st["min"] <= st["mean"] <= st["max"]
    assert d["exchange_derived"]["reduction"] == pytest.approx(1 - d["config"]["n_s"] / d["config"]["h"],
                                                               abs=1e-4)


@pytest.mark.gpu
@pytest.mark.parametrize("pass_", ["backward", "block"])
def test_bench_other_passes_line(pass_):
    d = _line(_bench("--pass", pass_, "--workload", "130m-pair-bf16", "--steps", "2",
                     "--warmup", "1", "--cpu-budget", "0"))
    _check_common(d, 2, 1)
    assert d["config"]["workload"] == "130m-pair-bf16"


def test_bench_refuses_more_than_one_gpu():
    r = _bench("--gpus", "2", timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr


def test_code_sha_ignores_comments_only(tmp_path):
    """The stored HBM-traffic record stays valid across comment edits of the kernel source
    and lapses when its code changes."""
    from partial_activation_sync_amd.rocprof_summary import code_sha256
    base = 'int f(int a) {\n  // sum\n  return a + 1; /* one */\n}\nconst char *s = "// kept";\n'
    variants = {
        "same": base,
        "comment": base.replace("// sum", "// the sum of a and one").replace("/* one */", ""),
        "blank": base.replace("\n  return", "\n\n      return"),
        "code": base.replace("a + 1", "a + 2"),
        "string": base.replace('"// kept"', '"// gone"'),
    }
    sha = {}
    for k, text in variants.items():
        f = tmp_path / f"{k}.hip"
        f.write_text(text)
        sha[k] = code_sha256(str(f))
    assert sha["same"] == sha["comment"] == sha["blank"]
    assert sha["code"] != sha["same"] and sha["string"] != sha["same"]
    # A local header the source includes is part of its code.
    (tmp_path / "h.h").write_text("#define ONE 1 // one\n")
    (tmp_path / "m.hip").write_text('#include "h.h"\nint g() { return ONE; }\n')
    before = code_sha256(str(tmp_path / "m.hip"))
    (tmp_path / "h.h").write_text("#define ONE 1 /* still one */\n")
    assert code_sha256(str(tmp_path / "m.hip")) == before
    (tmp_path / "h.h").write_text("#define ONE 2\n")
    assert code_sha256(str(tmp_path / "m.hip")) != before
