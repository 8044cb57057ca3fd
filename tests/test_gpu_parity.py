"""GPU parity: libcaat (HIP, gfx950) against the fp64 oracle on the same seeded inputs.

Bar (per output tensor): max |gpu - oracle| / max |oracle| <= 1e-4 for fp32 storage,
<= 2e-2 for bf16 storage.  The channel mask is checked bit-exactly on integer-coded
partials.  Full-size workloads are compared on sampled token rows (token rows never
interact, so a row's oracle value does not depend on the others).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import partial_activation_sync_amd as caat
from partial_activation_sync_amd import runner, synth, workloads as W
from tests.oracle_ref import TOL, compare, reference

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _run_and_compare(w, T=None, p=None, s_priv=1.0, norm_params="unit", rows=None):
    _say(f"[case] {w.name} T={T or w.T} p={p if p is not None else w.p} s={s_priv} "
         f"norm_params={norm_params} rows={'all' if rows is None else len(rows)}")
    inputs = runner.make_inputs(w, T=T, norm_params=norm_params)
    run = runner.Run(w, inputs, p=p, s_priv=s_priv)
    run.step()
    torch.cuda.synchronize()
    ref = reference(w, inputs, rows=rows, p=p, s_priv=s_priv)
    errs = compare(w, run.outputs(), ref, rows=rows)
    _say("   errors:", {k: f"{v:.2e}" for k, v in errs.items()})
    assert {"out", "out_resid"} <= set(errs), errs
    for k, e in errs.items():
        assert e <= TOL[w.dtype], (k, e)
    return run, inputs


# ---------------------------------------------------------------------------
# Workloads at sizes the oracle finishes in seconds: several tiles + a ragged tail
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("s_priv", [1.0, math.sqrt(2.0)])
@pytest.mark.parametrize("norm_params", ["unit", "random"])
def test_tiny_mlp_fp32_full(s_priv, norm_params):
    _run_and_compare(W.TINY_MLP_F32, s_priv=s_priv, norm_params=norm_params)


def test_tiny_mlp_fp32_ragged():
    _run_and_compare(W.TINY_MLP_F32, T=77, norm_params="random")


@pytest.mark.parametrize("T", [1, 300])
def test_130m_pair_ragged(T):
    _run_and_compare(W.PAIR_130M_BF16, T=T, norm_params="random")


@pytest.mark.parametrize("p", W.SWEEP_P_1P1B)
def test_1p1b_mlp_ragged(p):
    _run_and_compare(W.MLP_1P1B_BF16, T=300, p=p, norm_params="random")


def test_7b_prefill_ragged():
    _run_and_compare(W.PREFILL_7B_BF16, T=131, norm_params="random")


@pytest.mark.parametrize("T", W.DECODE_T)
def test_7b_decode_full(T):
    _run_and_compare(W.DECODE_7B_BF16, T=T)


# Decode batch sizes between the benchmarked ones: each weight-streaming launch shape
# (one or two weight blocks per wave, 1 to 4 token blocks, ragged last block).
@pytest.mark.parametrize("T", [9, 16, 17, 40])
def test_7b_decode_launch_shapes(T):
    _run_and_compare(W.DECODE_7B_BF16, T=T, norm_params="random")


# ---------------------------------------------------------------------------
# Full sizes, in the launch configuration the benchmark times: sampled rows
# ---------------------------------------------------------------------------
def test_130m_pair_full_size_sampled():
    w = W.PAIR_130M_BF16
    _run_and_compare(w, rows=synth.sample_rows(w.T, 64))


@pytest.mark.parametrize("p", W.SWEEP_P_1P1B)
def test_1p1b_mlp_full_size_sampled(p):
    w = W.MLP_1P1B_BF16
    _run_and_compare(w, p=p, rows=synth.sample_rows(w.T, 64))


def test_7b_prefill_full_size_sampled():
    w = W.PREFILL_7B_BF16
    _run_and_compare(w, rows=synth.sample_rows(w.T, 64))


def test_7b_prefill_ragged_large_tiles():
    """T = 7992: the 256 x 256 tiles (8 waves, epilogue through LDS) with a last token
    tile of 56 rows; the sampled rows include the last token."""
    T = 7992
    _run_and_compare(W.PREFILL_7B_BF16, T=T, norm_params="random", rows=synth.sample_rows(T, 64))


# ---------------------------------------------------------------------------
# Steps on their own
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("wname,T", [("tiny-mlp-fp32", 128), ("1.1b-mlp-bf16", 200),
                                     ("130m-pair-bf16", 100)])
def test_partials_match_oracle(wname, T):
    """K1 + K2 alone: the per-rank partials Zt before any reduction."""
    w = W.ALL[wname]
    _say(f"[case] partials {wname} T={T}")
    inputs = runner.make_inputs(w, T=T)
    d = {k: v.cuda() for k, v in inputs.items()}
    s = caat.Sublayer(w.h, w.ffn, w.P, w.p, norm=w.norm, act=w.act, dtype=w.dtype)
    dt = runner.torch_dtype(w)
    x = d["x"] if "x" in d else synth.normal((w.P, T, w.h), synth.X, dtype=dt).cuda()
    Y = torch.empty((w.P, T, w.f_s), dtype=dt, device="cuda")
    Z = torch.empty((w.P, T, w.h), dtype=dt, device="cuda")
    caat.caat_column_gemm_act(s.handle, T, x, d["W1"], Y)
    caat.caat_row_gemm(s.handle, T, Y, d["W2"], Z)
    torch.cuda.synchronize()
    act = {"gelu": oracle.GELU, "gelu_tanh": oracle.GELU_TANH, "swiglu": oracle.SWIGLU}[w.act]
    _, _, zt = oracle.sublayer(x.cpu(), inputs["W1"], inputs["W2"], inputs["gamma"], act=act,
                               norm=oracle.RMSNORM, n_s=0, want_partials=True)
    err = (Z.double().cpu().numpy() - zt).__abs__().max() / abs(zt).max()
    _say(f"   partials error {err:.2e}")
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("act", ["gelu", "gelu_tanh", "swiglu"])
@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
def test_activation_and_norm_variants(act, norm):
    w = W.with_(W.MLP_1P1B_BF16, act=act, norm=norm, P=4, h=512, ffn=4 * 264, T=260, p=0.3)
    _run_and_compare(w, norm_params="random", s_priv=2.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("P,h,ffn,T", [(1, 8, 8, 1), (16, 128, 16 * 8, 5), (3, 264, 3 * 40, 67),
                                       (5, 200, 5 * 48, 129)])
def test_edge_shapes(dtype, P, h, ffn, T):
    for act in ("gelu", "swiglu"):
        w = W.with_(W.TINY_MLP_F32, dtype=dtype, P=P, h=h, ffn=ffn, T=T, p=0.37, act=act,
                    norm="layernorm", replicated_x=False)
        _run_and_compare(w, norm_params="random")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_out_projection_edge_shapes(dtype):
    w = W.with_(W.PAIR_130M_BF16, dtype=dtype, P=2, h=272, ffn=2 * 136, T=45, p=0.61)
    _run_and_compare(w, norm_params="random")


# ---------------------------------------------------------------------------
# The channel mask, bit-exact; cross-rank identity at p = 1; determinism
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("P", [1, 2, 4, 8])
@pytest.mark.parametrize("h", [256, 4096])
def test_mask_bit_exact(dtype, P, h):
    """Integer-coded partials Zt_m = 2^m, resid = 0: out_resid = 2^P - 1 on shared
    channels and 2^m * s_priv on private ones, exactly (representable in bf16)."""
    T = 3
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for n_s in sorted({0, 1, 63, 64, 65, 179, h - 1, h}):
        p = n_s / h
        s = caat.Sublayer(h, 8 * P, P, p, norm="rmsnorm", act="gelu", dtype=dtype, s_priv=2.0)
        assert s.n_s == n_s
        Z = torch.stack([torch.full((T, h), 2.0 ** m, dtype=dt) for m in range(P)]).cuda()
        resid = torch.zeros((P, T, h), dtype=dt, device="cuda")
        gamma = torch.ones(h, dtype=dt, device="cuda")
        out = torch.empty_like(resid)
        out_resid = torch.empty_like(resid)
        caat.caat_partial_sync_norm(s.handle, T, Z, resid, gamma, None, out, out_resid)
        torch.cuda.synchronize()
        want = torch.empty((P, T, h), dtype=torch.float64)
        for m in range(P):
            want[m, :, :n_s] = 2.0 ** P - 1
            want[m, :, n_s:] = 2.0 ** m * 2.0
        assert torch.equal(out_resid.double().cpu(), want), (P, h, n_s)


def test_p1_ranks_bitwise_identical():
    w = W.with_(W.MLP_1P1B_BF16, T=96, replicated_x=True, p=1.0)
    inputs = runner.make_inputs(w, norm_params="random")
    run = runner.Run(w, inputs)
    run.step()
    torch.cuda.synchronize()
    for m in range(1, w.P):
        assert torch.equal(run.out[m], run.out[0])
        assert torch.equal(run.out_resid[m], run.out_resid[0])


def test_p_below_1_ranks_differ_only_in_private_channels():
    w = W.with_(W.MLP_1P1B_BF16, T=32, replicated_x=True, p=0.25)
    run = runner.Run(w, runner.make_inputs(w))
    run.step()
    torch.cuda.synchronize()
    n_s = run.mlp.n_s
    r = run.out_resid
    for m in range(1, w.P):
        assert torch.equal(r[m, :, :n_s], r[0, :, :n_s])
        assert not torch.equal(r[m, :, n_s:], r[0, :, n_s:])


def test_run_to_run_deterministic():
    w = W.with_(W.PREFILL_7B_BF16, T=520)
    run = runner.Run(w, runner.make_inputs(w, norm_params="random"))
    run.step()
    first = {k: v.clone() for k, v in run.outputs().items()}
    for _ in range(3):
        run.step()
    torch.cuda.synchronize()
    for k, v in run.outputs().items():
        assert torch.equal(v, first[k]), k


def test_forward_plain_entry_point():
    """caat_forward (residual = input, no out_resid) against the oracle."""
    w = W.with_(W.MLP_1P1B_BF16, T=70)
    inputs = runner.make_inputs(w)
    d = {k: v.cuda() for k, v in inputs.items()}
    s = caat.Sublayer(w.h, w.ffn, w.P, w.p, norm=w.norm, act=w.act, dtype=w.dtype)
    s.workspace(w.T)
    out = torch.empty_like(d["x"])
    caat.caat_forward(s.handle, w.T, d["x"], d["W1"], d["W2"], d["gamma"], out)
    torch.cuda.synchronize()
    ref = reference(w, inputs)
    errs = compare(w, {"out": out}, ref)
    assert errs["out"] <= TOL[w.dtype]


# ---------------------------------------------------------------------------
# The fused path: shared channels reduced inside the row-parallel GEMM
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("wname,T,p", [("tiny-mlp-fp32", 77, 0.5), ("1.1b-mlp-bf16", 200, 0.25),
                                       ("1.1b-mlp-bf16", 33, 1.0), ("1.1b-mlp-bf16", 40, 0.0),
                                       ("130m-pair-bf16", 300, 0.5), ("7b-decode-pair-bf16", 8, 0.5)])
def test_row_gemm_reduce_matches_oracle(wname, T, p):
    """S [T][n_s] = sum over ranks of the shared partial columns, and the private
    columns of every rank's partials, against the oracle's per-rank partials."""
    w = W.ALL[wname]
    _say(f"[case] row_gemm_reduce {wname} T={T} p={p}")
    inputs = runner.make_inputs(w, T=T)
    d = {k: v.cuda() for k, v in inputs.items()}
    dt = runner.torch_dtype(w)
    act_name = "none" if "ctx" in d else w.act
    s = caat.Sublayer(w.h, w.ffn, w.P, p, norm=w.norm, act=act_name, dtype=w.dtype)
    n_s = s.n_s
    if act_name == "none":
        inp, W2 = d["ctx"], d["Wo"]
    else:
        Y = torch.empty((w.P, T, w.f_s), dtype=dt, device="cuda")
        caat.caat_column_gemm_act(s.handle, T, d["x"], d["W1"], Y)
        inp, W2 = Y, d["W2"]
    S = torch.full((T, max(n_s, 8)), float("nan"), dtype=dt, device="cuda")
    Z = torch.full((w.P, T, w.h), float("nan"), dtype=dt, device="cuda")
    caat.caat_row_gemm_reduce(s.handle, T, inp, W2, S if n_s else None, Z if n_s < w.h else None)
    torch.cuda.synchronize()
    if act_name == "none":
        _, _, zt = oracle.sublayer(inputs["ctx"], None, inputs["Wo"], inputs["gamma"],
                                   resid=inputs["x0"], act=oracle.NONE, norm=oracle.RMSNORM,
                                   n_s=0, want_partials=True)
    else:
        act = {"gelu": oracle.GELU, "gelu_tanh": oracle.GELU_TANH, "swiglu": oracle.SWIGLU}[w.act]
        _, _, zt = oracle.sublayer(inputs["x"], inputs["W1"], inputs["W2"], inputs["gamma"],
                                   act=act, norm=oracle.RMSNORM, n_s=0, want_partials=True)
    if n_s:
        ref = zt[:, :, :n_s].sum(0)
        err = np.abs(S[:, :n_s].double().cpu().numpy() - ref).max() / np.abs(ref).max()
        _say(f"   S error {err:.2e}")
        assert err <= TOL[w.dtype]
    if n_s < w.h:
        ref = zt[:, :, n_s:]
        err = np.abs(Z[:, :, n_s:].double().cpu().numpy() - ref).max() / np.abs(ref).max()
        _say(f"   private partials error {err:.2e}")
        assert err <= TOL[w.dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("P,h,T", [(8, 4096, 1), (8, 8192, 3), (16, 4096, 5), (16, 8192, 2),
                                   (4, 16384, 2), (3, 4096, 64), (2, 264, 7)])
def test_partial_sync_norm_small_batch(dtype, P, h, T):
    """K3 for T <= 64 (one workgroup per token and rank) on every rank-count and row-width
    dispatch: all of a thread's loads first for P <= 8 (one or two chunks per thread) and
    for P <= 16 (one chunk), one rank at a time otherwise."""
    _partial_sync_norm_case(dtype, P, h, T)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_partial_sync_norm_streaming(dtype):
    """K3 for T > 64 (one workgroup per token) on partials of every rank, at a size whose
    launch moves more than 256 MB (nontemporal row loads and stores), ragged T."""
    _partial_sync_norm_case(dtype, 8, 4096, 1100)


def _partial_sync_norm_case(dtype, P, h, T):
    """caat_partial_sync_norm with LayerNorm, beta and a private scale, against the
    oracle's reduce + norm."""
    _say(f"[case] partial_sync_norm {dtype} P={P} h={h} T={T}")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    s = caat.Sublayer(h, 8 * P, P, 0.37, norm="layernorm", act="gelu", dtype=dtype, s_priv=1.5)
    Z = synth.normal((P, T, h), synth.PARTIALS, dtype=dt)
    R = synth.normal((P, T, h), synth.RESID, dtype=dt)
    gamma = synth.normal((h,), synth.GAMMA, std=0.1, mean=1.0, dtype=dt)
    beta = synth.normal((h,), synth.BETA, std=0.1, dtype=dt)
    out = torch.empty((P, T, h), dtype=dt, device="cuda")
    out_resid = torch.empty_like(out)
    caat.caat_partial_sync_norm(s.handle, T, Z.cuda(), R.cuda(), gamma.cuda(), beta.cuda(),
                                out, out_resid)
    torch.cuda.synchronize()
    ref_out, ref_res = oracle.partial_sync_norm(Z, R, gamma, beta=beta, norm=oracle.LAYERNORM,
                                                n_s=s.n_s, s_priv=1.5)
    from tests.oracle_ref import rel_err
    e1, e2 = rel_err(out, ref_out), rel_err(out_resid, ref_res)
    _say(f"   errors out {e1:.2e} out_resid {e2:.2e}")
    assert e1 <= TOL[dtype] and e2 <= TOL[dtype], (e1, e2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("P,h,T,p", [(8, 4096, 5, 0.5), (4, 768, 33, 0.25), (2, 256, 64, 1.0),
                                     (3, 264, 7, 0.0), (8, 4096, 1100, 0.5), (4, 2048, 300, 0.25)])
def test_sync_norm_matches_oracle(dtype, P, h, T, p):
    """K3 on a given S and private partials equals the oracle's reduce + norm on partials
    whose shared columns hold S on rank 0 and zeros on the other ranks.  T = 1100 at P = 8,
    h = 4096 moves more than 256 MB per launch and takes the nontemporal row loads and
    stores; T = 300 at P = 4, h = 2048 takes the ordinary ones."""
    _say(f"[case] sync_norm {dtype} P={P} h={h} T={T} p={p}")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    s = caat.Sublayer(h, 8 * P, P, p, norm="layernorm", act="gelu", dtype=dtype, s_priv=1.5)
    n_s = s.n_s
    Sv = synth.normal((T, max(n_s, 8)), synth.PARTIALS, std=2.0, dtype=dt)
    Z = synth.normal((P, T, h), synth.PARTIALS + 100, dtype=dt)
    R = synth.normal((P, T, h), synth.RESID, dtype=dt)
    gamma = synth.normal((h,), synth.GAMMA, std=0.1, mean=1.0, dtype=dt)
    beta = synth.normal((h,), synth.BETA, std=0.1, dtype=dt)
    out = torch.empty((P, T, h), dtype=dt, device="cuda")
    out_resid = torch.empty_like(out)
    caat.caat_sync_norm(s.handle, T, Sv.cuda() if n_s else None, Z.cuda() if n_s < h else None,
                        R.cuda(), gamma.cuda(), beta.cuda(), out, out_resid)
    torch.cuda.synchronize()
    zo = Z.float().clone()
    zo[:, :, :n_s] = 0
    zo[0, :, :n_s] = Sv[:, :n_s].float()
    ref_out, ref_res = oracle.partial_sync_norm(zo, R, gamma, beta=beta, norm=oracle.LAYERNORM,
                                                n_s=n_s, s_priv=1.5)
    tol = TOL[dtype]
    from tests.oracle_ref import rel_err
    e1, e2 = rel_err(out, ref_out), rel_err(out_resid, ref_res)
    _say(f"   errors out {e1:.2e} out_resid {e2:.2e}")
    assert e1 <= tol and e2 <= tol


def test_forward_p0_and_p1_fused():
    for p in (0.0, 1.0):
        w = W.with_(W.PREFILL_7B_BF16, T=70, p=p)
        _run_and_compare(w, norm_params="random")


def test_graph_replay_matches_eager():
    """One decode step captured as a HIP graph: every replay (with eager work between
    replays) reproduces the eager outputs bitwise."""
    w = W.with_(W.DECODE_7B_BF16, T=8)
    run = runner.Run(w, runner.make_inputs(w, norm_params="random"))
    steps = list(run.attn_steps()) + list(run.mlp_steps())
    for k in steps:
        k()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in run.outputs().items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in steps:
            k()
    for rep in range(3):
        for v in run.outputs().values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in run.outputs().items():
            assert torch.equal(v, eager[k]), (rep, k)
