"""Benchmark: tokens/s of the CAAT partial-sync sublayer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--T T] [--p P]
                    [--pass forward|backward] [--graph]

A step is one pass of the whole path over one batch: for a pair workload the
attention out-projection sublayer (row-parallel GEMM K2, then the fused partial
channel-reduce + residual + norm K3) followed by the MLP sublayer (K1 column-parallel
GEMM + activation, K2, K3), all P ranks emulated on the one GPU.  Inputs are resident
in HBM before the timed region starts.  Each kernel is enqueued through its own C
entry point with an event between consecutive kernels on the stream the library
launches on, which yields the step time and every kernel's average duration from the
same timed steps.

With --pass block a step is one full transformer block of a pair workload: the QKV
projection, the causal attention core and both sublayers (caat_block_forward, which
records the caller's events after each of its steps).

With --pass backward a step is the backward of the whole path instead (the MLP
sublayer's backward, then the out-projection sublayer's), through caat_backward; the
library records the caller's events after each of its steps, so every kernel's
average duration again comes from the timed steps.

Prints ONE JSON line on stdout (details on stderr).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/sec per CAAT sublayer fwd (1 GPU, P emulated); % MFMA or HBM roofline"
METRIC_BWD = "tokens/sec per CAAT sublayer bwd (1 GPU, P emulated); % MFMA or HBM roofline"
METRIC_BLOCK = "tokens/sec per CAAT block fwd (1 GPU, P emulated); % MFMA or HBM roofline"
PEAK = {"mfma": 2500.0, "hbm": 8000.0}   # MI355X: bf16 dense TFLOP/s, HBM3E GB/s
DEFAULT_WORKLOAD = "7b-prefill-pair-bf16"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_work(w, T, name, store_resid, n_s, fused, direct=False):
    """Algorithmic FLOPs and HBM bytes of one step of the path ("attn.K2", "mlp.K1", ...),
    or of one of the two row-parallel launches of the fused path ("mlp.K2.shared",
    "mlp.K2.private").  fused: the library sums the shared channels inside the row GEMM
    (caat_forward_fused) and K3 reads S [T][n_s] once plus every rank's private columns.
    direct (caat_forward_private_in_epilogue, with store_resid): the row GEMM reads the
    residual and writes out_resid's private columns (fused: from n_s; per-rank: from n_s
    rounded up to 8), and K3 reads those rows back in place of the partials and the
    residual and writes out_resid's other columns only."""
    P, h, fs = w.P, w.h, w.f_s
    b = 2 if w.dtype == "bf16" else 4
    F1 = 2 * fs if w.act == "swiglu" else fs
    E = P * T * h
    direct = direct and store_resid
    if name == "mlp.K1":
        return 2.0 * P * T * h * F1, b * (P * T * h + P * F1 * h + P * T * fs)
    first = n_s if fused else (n_s + 7) // 8 * 8      # first column of the direct rows
    priv = P * T * (h - n_s)
    if direct and not fused:
        # partials for columns below `first`, then read residual + write out_resid above
        part = P * T * first + 2 * P * T * (h - first)
    else:
        part = (priv + T * n_s if fused else E) + (priv if direct else 0)
    k = fs if name.startswith("mlp") else h // P
    if name.endswith("K2"):
        return 2.0 * P * T * k * h, b * (P * T * k + P * h * k + part)
    if name.endswith("K2.shared"):
        return 2.0 * P * T * k * n_s, b * (P * T * k + P * n_s * k + T * n_s)
    if name.endswith("K2.private"):
        return (2.0 * P * T * k * (h - n_s),
                b * (P * T * k + P * (h - n_s) * k + priv * (2 if direct else 1)))
    if name.endswith("K3"):
        if direct and fused:   # S, the residual (shared), r (private) in; out, out_resid (shared) out
            return 0.0, b * (T * n_s + E + E + P * T * n_s + 2 * h)
        if direct:             # partials + residual below `first`, r above; out, out_resid below
            return 0.0, b * (P * T * first + E + E + P * T * first + 2 * h)
        return 0.0, b * (part + E + E + (E if store_resid else 0) + 2 * h)
    raise KeyError(name)


def kernel_work_bwd(w, T, sub, step):
    """Algorithmic FLOPs and HBM bytes of one backward step of one sublayer (the steps
    of caat_backward: BWD_STEPS)."""
    P, h = w.P, w.h
    b = 2 if w.dtype == "bf16" else 4
    E = P * T * h
    Tp = (T + 7) // 8 * 8
    if sub == "attn":
        k2, F1, fs = h // P, 0, 0
    else:
        fs = w.f_s
        k2, F1 = fs, (2 * fs if w.act == "swiglu" else fs)
    if step == "norm":       # read r, dout, dres; write dZt, dresid
        return 0.0, b * 5 * E
    if step == "W2T":
        return 0.0, b * 2 * P * h * k2
    if step == "dY":
        return 2.0 * P * T * h * k2, b * (P * k2 * h + E + P * T * k2)
    if step == "a":
        return 2.0 * P * T * h * F1, b * (P * F1 * h + E + P * T * F1)
    if step == "act":
        return 0.0, b * 2 * (P * T * F1 + P * T * fs)
    if step == "W1T":
        return 0.0, b * 2 * P * F1 * h
    if step == "dx":
        return 2.0 * P * T * F1 * h, b * (P * h * F1 + P * T * F1 + E)
    if step == "daT_xT":
        return 0.0, b * 2 * (P * T * F1 + E)
    if step == "dW1":
        return 2.0 * P * F1 * h * Tp, b * (P * h * Tp + P * F1 * Tp + P * F1 * h)
    if step == "YT_dZtT":
        return 0.0, b * 2 * (P * T * k2 + E)
    if step == "dW2":
        return 2.0 * P * h * k2 * Tp, b * (P * k2 * Tp + P * h * Tp + P * h * k2)
    raise KeyError(step)




def traffic_key(workload, T, kernel_name):
    return f"{workload}:T={T}:{kernel_name}"


def kernel_source(name, T, dtype):
    """The source files of the kernel a step launches (fp32 GEMMs: the FMA kernel; bf16
    GEMMs at T <= 64 tokens: the weight-streaming decode kernels, whose source also
    holds the rule that hands some of them to the MFMA tile kernel, and that kernel)."""
    csrc = os.path.join(ROOT, "partial_activation_sync_amd", "csrc")
    if name.endswith("K3"):
        return [os.path.join(csrc, "psync_norm.hip")]
    if dtype != "bf16":
        return [os.path.join(csrc, "gemm_f32.hip")]
    if T <= 64:
        return [os.path.join(csrc, "gemm_decode.hip"), os.path.join(csrc, "gemm_bf16.hip")]
    return [os.path.join(csrc, "gemm_bf16.hip")]


def traffic_for(kernel_file, key):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    measurement, if it was taken on the kernel source as it is now (else None)."""
    from partial_activation_sync_amd.rocprof_summary import code_sha256
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(key)
    except (ValueError, OSError):
        return None
    if not rec or rec.get("code_sha256") != code_sha256(kernel_file):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, inputs, p, budget_s):
    """The oracle (fp64 C, OpenMP) on a bounded sample of token rows of the same workload."""
    import oracle
    import torch
    from partial_activation_sync_amd import synth
    from tests.oracle_ref import reference

    T = inputs["ctx"].shape[1] if "ctx" in inputs else inputs["x"].shape[1]
    probe = synth.sample_rows(T, min(T, 8))
    t0 = time.perf_counter()
    reference(w, inputs, rows=probe, p=p)
    per_row = (time.perf_counter() - t0) / len(probe)
    n = int(max(8, min(T, budget_s / max(per_row, 1e-9))))
    # Each call also pays a fixed set-up cost (widening the inputs to fp64), so the
    # probe overestimates the cost of a row: grow the sample once if it fell short.
    for _ in range(2):
        rows = synth.sample_rows(T, n)
        t0 = time.perf_counter()
        ref = reference(w, inputs, rows=rows, p=p)
        dt = time.perf_counter() - t0
        if dt >= 0.6 * budget_s or n >= T:
            break
        n = int(min(T, n * budget_s / max(dt, 1e-9)))
    # A batch the oracle finishes well inside the budget (every row already sampled: the
    # decode batches) is timed over repeated calls, so the sample is still ~budget_s.
    reps = 1
    if dt < 0.6 * budget_s:
        reps = max(1, int(budget_s / max(dt, 1e-9)))
        t0 = time.perf_counter()
        for _ in range(reps):
            reference(w, inputs, rows=rows, p=p)
        dt = time.perf_counter() - t0
    del torch
    what = f"{len(rows)} of {T} token rows" + (f", {reps} calls" if reps > 1 else "")
    base = {"value": reps * len(rows) / dt, "unit": "tokens/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"{what} of {w.name} (all {w.P} ranks, every sublayer), fp64, {dt:.1f} s; "
                      f"rows are independent, so tokens/s = rows / s"}
    return base, rows, ref


def cpu_baseline_backward(w, inputs, p, budget_s):
    """The oracle backward (fp64 C, OpenMP) of the whole path on a bounded sample of token
    rows: the oracle forward of the out-projection gives the MLP's input, then the MLP
    backward, then the out-projection backward fed with the MLP's input gradients."""
    import oracle
    import numpy as np
    from partial_activation_sync_amd import synth
    from tests.oracle_ref import ACT, NORM

    T = inputs["ctx"].shape[1] if "ctx" in inputs else inputs["x"].shape[1]
    n_s = oracle.shared_channels(w.h, p)
    norm = NORM[w.norm]
    gamma, beta = inputs["gamma"].float(), inputs["beta"].float()
    W1, W2 = inputs["W1"].float(), inputs["W2"].float()
    dt = inputs["W1"].dtype

    def one(rows):
        n = len(rows)
        dout = synth.normal((w.P, T, w.h), synth.DOUT, dtype=dt)[:, rows].float()
        dres = synth.normal((w.P, T, w.h), synth.DRES, dtype=dt)[:, rows].float()
        t0 = time.perf_counter()
        if "ctx" in inputs:
            ctx, x0 = inputs["ctx"][:, rows].float(), inputs["x0"][:, rows].float()
            Wo = inputs["Wo"].float()
            a_out, a_res = oracle.sublayer(ctx, None, Wo, gamma, beta=beta, resid=x0,
                                           act=oracle.NONE, norm=norm, n_s=n_s, eps=w.eps)
            g = oracle.sublayer_backward(a_out, W1, W2, gamma, dout, act=ACT[w.act], norm=norm,
                                         n_s=n_s, resid=a_res, dres=dres, eps=w.eps)
            oracle.sublayer_backward(ctx, None, Wo, gamma, g["dx"], act=oracle.NONE, norm=norm,
                                     n_s=n_s, resid=x0, dres=g["dresid"], eps=w.eps)
        else:
            oracle.sublayer_backward(inputs["x"][:, rows].float(), W1, W2, gamma, dout,
                                     act=ACT[w.act], norm=norm, n_s=n_s, dres=dres, eps=w.eps)
        return time.perf_counter() - t0

    n = 8
    dt_s = one(synth.sample_rows(T, n))
    for _ in range(3):
        if dt_s >= 0.6 * budget_s or n >= T:
            break
        n = int(min(T, max(n + 1, n * budget_s / max(dt_s, 1e-9))))
        rows = synth.sample_rows(T, n)
        dt_s = one(rows)
    return {"value": n / dt_s, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"backward of {n} of {T} token rows of {w.name} (all {w.P} ranks, every "
                      f"sublayer; weight gradients over the sampled rows), fp64, {dt_s:.1f} s"}


def bench_backward(args, w, T, p):
    import torch
    import partial_activation_sync_amd as caat
    from partial_activation_sync_amd import runner

    log(f"[bench] backward {w.name} T={T} p={p} P={w.P} h={w.h} ffn={w.ffn} act={w.act} "
        f"norm={w.norm}")
    inputs = runner.make_inputs(w, T=T)
    run = runner.Run(w, inputs, p=p, store_resid=True, weight_copies=1)
    stored = args.preact == "stored"
    F1 = 2 * w.f_s if w.act == "swiglu" else w.f_s
    # bf16 weight-gradient GEMMs contract over tokens from the token-major operands
    # (no transposes) when every width is a multiple of 8, as the library decides.
    tn = w.dtype == "bf16" and all(n % 8 == 0 for n in (w.h, w.f_s, F1, w.h // w.P))
    br = runner.BackwardRun(run, store_preact=stored)
    torch.cuda.synchronize()
    subs = ["mlp"] + (["attn"] if run.attn is not None else [])
    steps = caat.BWD_STEPS
    K = args.steps

    def events(n):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in ev:             # torch creates the HIP event on its first record
            e.record()
        return ev

    start = events(K)
    ev = {sub: [events(len(steps)) for _ in range(K)] for sub in subs}
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        br.step()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for s in range(K):
        start[s].record()
        br.step(events_mlp=[e.cuda_event for e in ev["mlp"][s]],
                events_attn=[e.cuda_event for e in ev["attn"][s]] if "attn" in subs else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    last = ev[subs[-1]]
    span_ms = start[0].elapsed_time(last[K - 1][-1]) / K
    kern_ms = {}
    for s in range(K):
        prev = start[s]
        for sub in subs:
            for i, name in enumerate(steps):
                key = f"{sub}.{name}"
                kern_ms[key] = kern_ms.get(key, 0.0) + prev.elapsed_time(ev[sub][s][i]) / K
                prev = ev[sub][s][i]
    log(f"[bench] {K} backward steps: {span_ms:.4f} ms/step, wall {wall / K * 1e3:.3f} ms/step")
    detail = {}
    for key, ms in kern_ms.items():
        sub, name = key.split(".")
        flops, nbytes = kernel_work_bwd(w, T, sub, name)
        if sub == "attn" and name in ("a", "act", "W1T", "dx", "daT_xT", "dW1"):
            continue          # no first GEMM in the out-projection
        if name == "a" and stored:
            continue          # the pre-activation comes from the training forward
        if name in ("daT_xT", "YT_dZtT") and tn:
            continue          # bf16 weight gradients read the token-major operands
        d = {"ms": round(ms, 4), "share": round(ms / span_ms, 3)}
        if flops:
            d["TFLOP/s"] = round(flops / ms / 1e9, 1)
            d["mfma_frac"] = round(flops / ms / 1e9 / PEAK["mfma"], 3)
        d["GB/s"] = round(nbytes / ms / 1e6, 1)
        d["hbm_frac"] = round(nbytes / ms / 1e6 / PEAK["hbm"], 3)
        detail[key] = d
        log(f"[bench]   {key:16s} {ms:8.4f} ms  {d}")
    dom = max(detail, key=lambda k: detail[k]["ms"])
    sub, name = dom.split(".")
    flops, nbytes = kernel_work_bwd(w, T, sub, name)
    ridge = PEAK["mfma"] * 1e12 / (PEAK["hbm"] * 1e9)
    ms = kern_ms[dom]
    if flops and flops / nbytes >= ridge:
        achieved = flops / ms / 1e9
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK["mfma"],
                "unit": "TFLOP/s", "frac": round(achieved / PEAK["mfma"], 4)}
    else:
        achieved = nbytes / ms / 1e6
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK["hbm"],
                "unit": "GB/s", "frac": round(achieved / PEAK["hbm"], 4)}
    roof["kernel"] = dom
    roof["algorithmic_per_launch"] = flops if flops else nbytes
    csrc = os.path.join(ROOT, "partial_activation_sync_amd", "csrc")
    if not flops:
        src = [os.path.join(csrc, "backward.hip")]
    elif tn and name in ("dW1", "dW2"):
        src = [os.path.join(csrc, "gemm_tn.hip")]
    else:
        src = kernel_source("K2", T, w.dtype)
    roof["traffic"] = traffic_for(src, traffic_key(w.name + ":bwd", T, dom))
    # What the stored pre-activation costs the forward: a training forward (K1's epilogue
    # also writes x W1^T) against the plain one, same inputs, same stream.
    fwd_ms = {}
    for name, pre in (("plain", None), ("train", br.preact)):
        if name == "train" and pre is None:
            continue
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(2):
            run.step(preact=pre)
        e0.record()
        for _ in range(5):
            run.step(preact=pre)
        e1.record()
        torch.cuda.synchronize()
        fwd_ms[name] = round(e0.elapsed_time(e1) / 5, 4)
    log(f"[bench] forward per step: {fwd_ms} (train: also stores the pre-activation)")
    base = None
    if args.cpu_budget > 0:
        log("[bench] timing the oracle backward on host cores ...")
        base = cpu_baseline_backward(w, inputs, p, args.cpu_budget)
        log(f"[bench] cpu baseline: {base}")
    line = {
        "metric": METRIC_BWD, "value": round(T / (span_ms / 1e3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(span_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic: seeded N(0,1) activations and upstream gradients, N(0,0.02^2) weights",
        "config": {"workload": w.name, "pass": "backward", "P": w.P, "h": w.h, "ffn": w.ffn,
                   "T": T, "p": p, "n_s": run.mlp.n_s, "act": w.act, "norm": w.norm,
                   "sublayers": list(w.sublayers), "parallelism": f"tp{w.P} emulated on 1 GPU",
                   "preact": args.preact},
        "roofline": roof,
        "cpu_baseline": base,
        "kernels": detail,
        "forward_ms": fwd_ms,
    }
    print(json.dumps(line), flush=True)


def kernel_work_block(w, T, step):
    """Algorithmic FLOPs and HBM bytes of one step of the full block (BLOCK_STEPS)."""
    P, h = w.P, w.h
    hp = h // P
    nh = w.heads // P
    d = hp // nh
    S = w.seq
    b = 2
    if step == "qkv":
        return 2.0 * P * T * h * 3 * hp, b * (P * T * h + P * 3 * hp * h + P * T * 3 * hp)
    if step == "vT":
        return 0.0, b * 2 * P * T * hp
    if step == "attn":
        pairs = (T // S) * S * (S + 1) // 2          # causal (query, key) pairs per head
        return 4.0 * P * nh * d * pairs, b * (P * T * 3 * hp + P * T * hp)
    raise KeyError(step)


def bench_block(args, w, T, p):
    import torch
    import partial_activation_sync_amd as caat
    from partial_activation_sync_amd import synth

    if not (w.heads and w.seq) or T % w.seq:
        print(f"--pass block needs a pair workload with heads and a sequence length dividing T "
              f"({w.name}: heads={w.heads}, seq={w.seq}, T={T})", flush=True)
        sys.exit(2)
    P, h, S = w.P, w.h, w.seq
    nh, hp = w.heads // P, h // P
    log(f"[bench] block {w.name} T={T} S={S} P={P} h={h} heads/rank={nh} ffn={w.ffn} p={p}")
    bf = torch.bfloat16
    F1 = 2 * w.f_s if w.act == "swiglu" else w.f_s
    n = lambda shape, tid, **kw: synth.normal(shape, tid, dtype=bf, **kw).cuda()
    x, r = n((P, T, h), synth.X), n((P, T, h), synth.X0)
    Wqkv, Wo = n((P, 3 * hp, h), synth.WQKV, std=0.02), n((P, h, hp), synth.WO, std=0.02)
    W1, W2 = n((P, F1, h), synth.W1, std=0.02), n((P, h, w.f_s), synth.W2, std=0.02)
    g, beta = torch.ones(h, dtype=bf, device="cuda"), torch.zeros(h, dtype=bf, device="cuda")
    out, out_r = torch.empty_like(x), torch.empty_like(x)
    blk = caat.Block(h, w.ffn, P, p, nh, norm=w.norm, act=w.act, eps=w.eps)
    steps = caat.BLOCK_STEPS
    K = args.steps

    def events(k):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(k)]
        for e in ev:
            e.record()
        return ev

    start = events(K)
    ev = [events(len(steps)) for _ in range(K)]
    torch.cuda.synchronize()
    step = lambda evs=None: blk.forward(T, S, x, r, Wqkv, Wo, W1, W2, g, g, out, out_r,
                                        beta_attn=beta, beta_mlp=beta, events=evs)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for s in range(K):
        start[s].record()
        step([e.cuda_event for e in ev[s]])
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    span_ms = start[0].elapsed_time(ev[K - 1][-1]) / K
    ms = {name: sum((start[s] if i == 0 else ev[s][i - 1]).elapsed_time(ev[s][i])
                    for s in range(K)) / K for i, name in enumerate(steps)}
    log(f"[bench] {K} block steps: {span_ms:.4f} ms/step, wall {wall / K * 1e3:.3f} ms/step")
    detail = {}
    for name, t in ms.items():
        d = {"ms": round(t, 4), "share": round(t / span_ms, 3)}
        if name in ("qkv", "vT", "attn"):
            flops, nbytes = kernel_work_block(w, T, name)
            if flops:
                d["TFLOP/s"] = round(flops / t / 1e9, 1)
                d["mfma_frac"] = round(flops / t / 1e9 / PEAK["mfma"], 3)
            d["GB/s"] = round(nbytes / t / 1e6, 1)
            d["hbm_frac"] = round(nbytes / t / 1e6 / PEAK["hbm"], 3)
        detail[name] = d
        log(f"[bench]   {name:14s} {t:8.4f} ms  {d}")
    # The sublayer steps hold several kernels each (their rooflines are the forward
    # pass's); the roofline here is the dominant single-kernel step of the block.
    dom = max(("qkv", "attn"), key=lambda k: ms[k])
    flops, nbytes = kernel_work_block(w, T, dom)
    achieved = flops / ms[dom] / 1e9
    src = ([os.path.join(ROOT, "partial_activation_sync_amd", "csrc", "attention.hip")]
           if dom == "attn" else kernel_source("K2", T, w.dtype))
    roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK["mfma"],
            "unit": "TFLOP/s", "frac": round(achieved / PEAK["mfma"], 4), "kernel": dom,
            "algorithmic_per_launch": flops,
            "traffic": traffic_for(src, traffic_key(w.name + ":block", T, dom))}
    line = {
        "metric": METRIC_BLOCK, "value": round(T / (span_ms / 1e3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(span_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) activations, N(0,0.02^2) weights",
        "config": {"workload": w.name, "pass": "block", "P": P, "h": h, "ffn": w.ffn, "T": T,
                   "seq": S, "heads": w.heads, "p": p, "act": w.act, "norm": w.norm,
                   "parallelism": f"tp{P} emulated on 1 GPU"},
        "roofline": roof,
        "cpu_baseline": None,
        "kernels": detail,
    }
    print(json.dumps(line), flush=True)


COPY_BYTES = 512 << 20


def _events(n):
    """n timing events, each recorded once so that torch creates its HIP event."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in ev:
        e.record()
    return ev


def timed_steps(run, K, warmup, rotate=1):
    """K steps of Run.step through caat_forward_timed: the library records an event after
    each of its steps (FWD_STEPS) on the stream it launches on.  Returns the per-step
    wall span (ms, from the first step's start to the last step's end, / K), the sorted
    per-step durations, and {sublayer: {step: mean ms}} over the K steps."""
    import torch
    import partial_activation_sync_amd as caat

    subs = (["attn"] if run.attn is not None else []) + ["mlp"]
    n = len(caat.FWD_STEPS)
    for i in range(warmup):
        run.step(copy=i % rotate)
    torch.cuda.synchronize()
    start = _events(K)
    ev = [{sub: _events(n) for sub in subs} for _ in range(K)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for k in range(K):
        start[k].record()
        raw = {sub: [e.cuda_event for e in ev[k][sub]] for sub in subs}
        run.step(events_attn=raw.get("attn"), events_mlp=raw["mlp"], copy=k % rotate)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    last = ev[K - 1][subs[-1]][n - 1]
    span = start[0].elapsed_time(last) / K
    per_step = sorted(start[k].elapsed_time(ev[k][subs[-1]][n - 1]) for k in range(K))
    ms = {sub: {name: 0.0 for name in caat.FWD_STEPS} for sub in subs}
    for k in range(K):
        prev = start[k]
        for sub in subs:
            for i, name in enumerate(caat.FWD_STEPS):
                ms[sub][name] += prev.elapsed_time(ev[k][sub][i]) / K
                prev = ev[k][sub][i]
    return span, per_step, ms, wall / K


def launch_names(sub, fused, n_s, h):
    """{FWD_STEPS name: reported kernel name} for the steps of a sublayer that launch a
    kernel (the out-projection has no K1; the fused path splits K2 into two launches,
    the shared one absent at n_s = 0 and the private one at n_s = h)."""
    out = {}
    if sub == "mlp":
        out["K1"] = "mlp.K1"
    if fused:
        if n_s > 0:
            out["K2"] = f"{sub}.K2.shared"
        if n_s < h:
            out["K2_private"] = f"{sub}.K2.private"
    else:
        out["K2"] = f"{sub}.K2"
    out["K3"] = f"{sub}.K3"
    return out


def per_gpu_share(w, T, p, steps, warmup):
    """One rank's shard at its real shape (P_launch = 1): the kernels one GPU of a P-GPU
    deployment would run for its share of the path (the collective itself aside).  The
    MLP shard is a P = 1 sublayer with ffn / P channels; the out-projection's per-rank
    GEMM (h / P -> h) is the row-parallel GEMM of a P = 1 sublayer with ffn = h / P, whose
    first GEMM is not counted.  K3 runs on the rank's own rows, with the shared channels
    taken from its own GEMM where a deployment would take them from the exchange."""
    import dataclasses
    from partial_activation_sync_amd import runner
    from partial_activation_sync_amd import workloads as W

    shard = dataclasses.replace(w, name=w.name + "-shard", P=1, ffn=w.f_s,
                                sublayers=(W.MLP,), replicated_x=False)
    runs = [("mlp", runner.Run(shard, runner.make_inputs(shard, T=T), p=p, store_resid=True))]
    if W.ATTN_OUT in w.sublayers:
        proj = dataclasses.replace(shard, ffn=w.h // w.P, act="gelu")
        runs.insert(0, ("attn", runner.Run(proj, runner.make_inputs(proj, T=T), p=p,
                                           store_resid=True)))
    ms = {}
    for sub, run in runs:
        _, _, st, _ = timed_steps(run, steps, warmup)
        st = st["mlp"]
        if sub == "attn":
            ms["attn.K2"] = st["K2"] + st["K2_private"]
            ms["attn.K3"] = st["K3"]
        else:
            ms["mlp.K1"] = st["K1"]
            ms["mlp.K2"] = st["K2"] + st["K2_private"]
            ms["mlp.K3"] = st["K3"]
    return {k: round(v, 4) for k, v in ms.items()}, sum(ms.values())


def source_sha():
    """The git commit when the tree is a checkout, else None; and a SHA-256 over the
    library's sources, its header and this script, which identifies the code either way."""
    import hashlib
    import subprocess
    try:
        head = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                              text=True, timeout=10).stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        head = None
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "partial_activation_sync_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc))
    files += [os.path.join(ROOT, "include", "caat.h"), os.path.abspath(__file__)]
    for f in files:
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return head, h.hexdigest()


def calibrate_copy():
    """A plain device-to-device copy of COPY_BYTES, five times: under rocprofv3 --pmc
    its FETCH_SIZE / WRITE_SIZE per dispatch give the counters' scale factor."""
    import torch
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "dispatches": 5}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--T", type=int, default=None)
    ap.add_argument("--p", type=float, default=None)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline (0: skip)")
    ap.add_argument("--rotate", type=int, default=None,
                    help="weight copies to cycle through (default: 3 when the weights of a "
                         "step fit in the 256 MB Infinity Cache twice over, else 1)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step as a captured HIP graph (one graph per weight "
                         "copy, replayed); value and ms_per_step then come from the replays")
    ap.add_argument("--preact", choices=("stored", "recompute"), default="stored",
                    help="backward: read the pre-activation a training forward stored, or "
                         "recompute it with a GEMM")
    ap.add_argument("--pass", dest="pass_", choices=("forward", "backward", "block"), default="forward",
                    help="time the forward (default) or the backward of the path")
    ap.add_argument("--mlp-only", action="store_true",
                    help="pair workloads: time the MLP sublayer alone (input and residual "
                         "x ~ N(0,1) per rank, same shapes)")
    ap.add_argument("--no-share", action="store_true",
                    help="skip the one-rank (P_launch = 1) timing")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a device copy of known size (HBM counter calibration)")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy()
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only: every tensor-parallel rank is emulated on a "
              f"single device (asked for --gpus {args.gpus}, WORLD_SIZE {world}).", flush=True)
        sys.exit(2)

    import torch
    from partial_activation_sync_amd import runner
    from partial_activation_sync_amd import workloads as W

    w = W.ALL[args.workload]
    if args.mlp_only:
        w = W.with_(w, name=w.name + ":mlp-only", sublayers=(W.MLP,))
    T = args.T or w.T
    p = w.p if args.p is None else args.p
    torch.cuda.set_device(0)
    if args.pass_ == "backward":
        return bench_backward(args, w, T, p)
    if args.pass_ == "block":
        return bench_block(args, w, T, p)
    import partial_activation_sync_amd as caat

    log(f"[bench] {w.name} T={T} p={p} P={w.P} h={w.h} ffn={w.ffn} act={w.act} norm={w.norm}")
    t0 = time.perf_counter()
    inputs = runner.make_inputs(w, T=T)
    wbytes = sum(v.numel() * v.element_size() for k, v in inputs.items() if k in ("W1", "W2", "Wo"))
    rotate = args.rotate or (3 if T <= 64 else 1)
    run = runner.Run(w, inputs, p=p, store_resid=True, weight_copies=rotate)
    torch.cuda.synchronize()
    log(f"[bench] inputs resident in HBM ({time.perf_counter() - t0:.1f} s); "
        f"weights {wbytes / 1e6:.1f} MB x {rotate} copies")
    n_s = run.mlp.n_s
    subs = (["attn"] if run.attn is not None else []) + ["mlp"]
    # The path the library takes for each sublayer (the fused row-parallel GEMM or not),
    # asked of it.
    handles = {"attn": run.attn, "mlp": run.mlp}
    fused = {sub: caat.caat_forward_fused(handles[sub].handle, T) for sub in subs}
    direct = {sub: caat.caat_forward_private_in_epilogue(handles[sub].handle, T) for sub in subs}

    K = args.steps
    span_ms, per_step, step_ms, wall = timed_steps(run, K, args.warmup, rotate)
    step_mean = sum(per_step) / K
    step_stats = {"mean": round(step_mean, 4),
                  "median": round(per_step[K // 2] if K % 2 else
                                  (per_step[K // 2 - 1] + per_step[K // 2]) / 2, 4),
                  "min": round(per_step[0], 4), "max": round(per_step[-1], 4)}
    # Per launch (the fused K2 is two launches), and per step of the method (K2 whole).
    launch_ms, kern_ms = {}, {}
    for sub in subs:
        for step, name in launch_names(sub, fused[sub], n_s, w.h).items():
            launch_ms[name] = step_ms[sub][step]
        if sub == "mlp":
            kern_ms["mlp.K1"] = step_ms[sub]["K1"]
        kern_ms[f"{sub}.K2"] = step_ms[sub]["K2"] + step_ms[sub]["K2_private"]
        kern_ms[f"{sub}.K3"] = step_ms[sub]["K3"]
    ms_per_step = span_ms
    eager_ms = span_ms

    if args.graph:
        # The library only enqueues kernels on the caller's stream (no allocation, no
        # host synchronisation), so one step is captured as it runs eagerly.
        graphs = []
        for c in range(rotate):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run.step(copy=c)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % rotate].replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for k in range(K):
            graphs[k % rotate].replay()
        e1.record()
        torch.cuda.synchronize()
        ms_per_step = e0.elapsed_time(e1) / K
        log(f"[bench] {K} graph replays: {ms_per_step:.4f} ms/step (eager {eager_ms:.4f})")
    value = T / (ms_per_step / 1e3)
    log(f"[bench] {K} steps: {eager_ms:.4f} ms/step (events), wall {wall * 1e3:.3f} ms/step")

    work = lambda name: kernel_work(w, T, name, store_resid=True, n_s=n_s,
                                    fused=fused[name.split(".")[0]],
                                    direct=direct[name.split(".")[0]])

    def describe(name, ms):
        flops, nbytes = work(name)
        d = {"ms": round(ms, 4), "share": round(ms / step_mean, 3)}
        if flops:
            d["TFLOP/s"] = round(flops / ms / 1e9, 1)
            d["mfma_frac"] = round(flops / ms / 1e9 / PEAK["mfma"], 3)
        d["GB/s"] = round(nbytes / ms / 1e6, 1)
        d["hbm_frac"] = round(nbytes / ms / 1e6 / PEAK["hbm"], 3)
        return d

    detail = {name: describe(name, ms) for name, ms in kern_ms.items()}
    for name, ms in launch_ms.items():
        if name not in detail:
            detail[name] = describe(name, ms)
    for name, d in detail.items():
        log(f"[bench]   {name:16s} {d['ms']:8.4f} ms  {d}")

    # The roofline object is the dominant single launch's.
    dom = max(launch_ms, key=launch_ms.get)
    flops, nbytes = work(dom)
    src = kernel_source(dom, T, w.dtype)
    ridge = PEAK["mfma"] * 1e12 / (PEAK["hbm"] * 1e9)   # FLOP per byte where the roofs meet
    if flops and flops / nbytes >= ridge:
        achieved = flops / launch_ms[dom] / 1e9
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK["mfma"],
                "unit": "TFLOP/s", "frac": round(achieved / PEAK["mfma"], 4)}
    else:
        achieved = nbytes / launch_ms[dom] / 1e6
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK["hbm"],
                "unit": "GB/s", "frac": round(achieved / PEAK["hbm"], 4)}
    roof["kernel"] = dom
    roof["algorithmic_per_launch"] = flops if flops else nbytes
    roof["traffic"] = traffic_for(src, traffic_key(w.name, T, dom))

    # Per sublayer: sum of the launches' roofline times (each at the larger of its FLOP
    # time at the MFMA peak and its byte time at the HBM peak) over the measured time.
    sublayers = {}
    for name, ms in launch_ms.items():
        flops, nbytes = work(name)
        roof_ms = max(flops / (PEAK["mfma"] * 1e12), nbytes / (PEAK["hbm"] * 1e9)) * 1e3
        e = sublayers.setdefault("attn_out" if name.startswith("attn") else "mlp",
                                 {"ms": 0.0, "roof_ms": 0.0})
        e["ms"] += ms
        e["roof_ms"] += roof_ms
    for e in sublayers.values():
        e["frac"] = round(e["roof_ms"] / e["ms"], 4)
        e["ms"] = round(e["ms"], 4)
        e["roof_ms"] = round(e["roof_ms"], 4)
    log(f"[bench] sublayer roofline fractions: {sublayers}")

    # Derived, not measured: what a P-GPU deployment would exchange per rank and sublayer
    # for the shared block (reduce-scatter + all-gather, 2 T n_s b), against a full
    # all-reduce of all h channels.
    b = 2 if w.dtype == "bf16" else 4
    exchange = {"per_rank_per_sublayer_bytes": 2 * T * n_s * b,
                "full_sync_bytes": 2 * T * w.h * b,
                "reduction": round(1.0 - n_s / w.h, 4)}

    share = None
    if w.P > 1 and T > 64 and not args.no_share:
        share_ms, share_step = per_gpu_share(w, T, p, K, args.warmup)
        share = {"kernels_ms": share_ms, "step_ms": round(share_step, 4),
                 "emulated_step_ms_per_rank": round(ms_per_step / w.P, 4)}
        log(f"[bench] one rank's shard (P_launch = 1): {share}")

    base, parity = None, None
    if args.cpu_budget > 0:
        log("[bench] timing the oracle on host cores ...")
        base, rows, ref = cpu_baseline(w, inputs, p, args.cpu_budget)
        log(f"[bench] cpu baseline: {base}")
        # The timed run's own outputs (the last step read weight copy (K - 1) % rotate;
        # every copy holds the same values) on the oracle's sampled rows.
        from tests.oracle_ref import TOL, compare
        errs = compare(w, run.outputs(), ref, rows=rows)
        parity = {"rows": len(rows), "tol": TOL[w.dtype],
                  "max_abs_err_over_max_abs": {k: float(f"{v:.3e}") for k, v in errs.items()},
                  "ok": all(v <= TOL[w.dtype] for v in errs.values())}
        log(f"[bench] parity of the timed outputs against the oracle: {parity}")

    head, code_sha = source_sha()
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic: seeded N(0,1) activations, N(0,0.02^2) weights",
        "config": {"workload": w.name, "P": w.P, "h": w.h, "ffn": w.ffn, "T": T, "p": p,
                   "weight_copies": rotate, "hip_graph": bool(args.graph),
                   "n_s": n_s, "fused_row_gemm": fused, "private_rows_in_gemm": direct,
                   "act": w.act, "norm": w.norm,
                   "sublayers": list(w.sublayers),
                   "parallelism": f"tp{w.P} emulated on 1 GPU"},
        "roofline": roof,
        "cpu_baseline": base,
        "parity": parity,
        "kernels": detail,
        "step_ms_stats": step_stats,
        "sublayers": sublayers,
        "exchange_derived": exchange,
        "per_gpu_share": share,
        "git_sha": head,
        "code_sha256": code_sha,
        "entry_point": "caat_forward_timed (= caat_forward_ex with step events)",
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
