"""GPU parity of the sublayer backward: libcaat (HIP, gfx950) against the fp64 oracle.

"Tensor-Parallelism with Partially Synchronized Activations", §4 "Forward-backward
mismatch" (Eq. 10-13) and App. B (Eq. 26-30): the norm derivative per rank, then the
reduce over ranks of the shared channels, the norm parameters' gradients summed over
ranks, then the two GEMMs and the activation.  The GPU runs its own forward first
(the backward reads the forward's out_resid); the oracle recomputes everything from
the same seeded inputs in fp64.  Bar per gradient tensor: max |gpu - oracle| /
max |oracle| <= 1e-4 (fp32 storage), <= 2e-2 (bf16 storage).  The mask of the
backward reduce is checked bit-exactly on integer-coded gradients.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import partial_activation_sync_amd as caat
from partial_activation_sync_amd import synth
from tests.oracle_ref import ACT, NORM, TOL, rel_err

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _inputs(P, T, h, ffn, act, dtype, resid_given, dres_given, seed=synth.BASE_SEED):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    none = act == "none"
    fs = 0 if none else ffn // P
    kin = h // P if none else h
    F1 = 2 * fs if act == "swiglu" else fs
    k2 = kin if none else fs
    d = {
        "x": synth.normal((P, T, kin), synth.CTX if none else synth.X, dtype=dt, seed=seed),
        "W1": None if none else synth.normal((P, F1, h), synth.W1, std=0.02, dtype=dt, seed=seed),
        "W2": synth.normal((P, h, k2), synth.WO if none else synth.W2, std=0.02, dtype=dt,
                           seed=seed),
        "gamma": synth.normal((h,), synth.GAMMA, std=0.1, mean=1.0, dtype=dt, seed=seed),
        "beta": synth.normal((h,), synth.BETA, std=0.1, dtype=dt, seed=seed),
        "resid": synth.normal((P, T, h), synth.X0, dtype=dt, seed=seed) if resid_given else None,
        "dout": synth.normal((P, T, h), synth.DOUT, dtype=dt, seed=seed),
        "dres": synth.normal((P, T, h), synth.DRES, dtype=dt, seed=seed) if dres_given else None,
    }
    return d


def _run(P, T, h, ffn, act, norm, p, dtype, s_priv=1.0, resid_given=True, dres_given=True):
    _say(f"[case] backward P={P} T={T} h={h} ffn={ffn} act={act} norm={norm} p={p} "
         f"{dtype} s={s_priv:.3f} resid={resid_given} dres={dres_given}")
    d = _inputs(P, T, h, ffn, act, dtype, resid_given, dres_given)
    dev = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    sub = caat.Sublayer(h, ffn, P, p, norm=norm, act=act, dtype=dtype, eps=1e-5, s_priv=s_priv)
    dt = sub.torch_dtype
    out = torch.empty((P, T, h), dtype=dt, device="cuda")
    out_resid = torch.empty_like(out)
    sub.forward(dev["x"], dev["W1"], dev["W2"], dev["gamma"], out, resid=dev["resid"],
                beta=dev["beta"], out_resid=out_resid)
    g = {
        "dx": torch.full_like(dev["x"], float("nan")),
        "dresid": torch.full((P, T, h), float("nan"), dtype=dt, device="cuda") if resid_given else None,
        "dW1": torch.full_like(dev["W1"], float("nan")) if act != "none" else None,
        "dW2": torch.full_like(dev["W2"], float("nan")),
        "dgamma": torch.full((h,), float("nan"), dtype=torch.float32, device="cuda"),
        "dbeta": torch.full((h,), float("nan"), dtype=torch.float32, device="cuda"),
    }
    sub.backward(dev["x"], dev["W1"], dev["W2"], dev["gamma"], out_resid, dev["dout"], g["dx"],
                 g["dW2"], g["dgamma"], dW1=g["dW1"], dres=dev["dres"], dresid=g["dresid"],
                 dbeta=g["dbeta"])
    torch.cuda.synchronize()
    ref = oracle.sublayer_backward(
        d["x"], d["W1"], d["W2"], d["gamma"], d["dout"],
        act=oracle.NONE if act == "none" else ACT[act], norm=NORM[norm],
        n_s=sub.n_s, resid=d["resid"], dres=d["dres"], s_priv=s_priv, eps=1e-5)
    errs = {}
    for k, v in g.items():
        if v is None:
            continue
        assert torch.isfinite(v.float()).all(), f"{k} has non-finite values"
        if k == "dbeta" and norm == "rmsnorm":
            assert torch.all(v == 0), "dbeta must be zero for RMSNorm"
            continue
        errs[k] = rel_err(v, ref[k])
    _say("   errors:", {k: f"{e:.2e}" for k, e in errs.items()})
    for k, e in errs.items():
        assert e <= TOL[dtype], (k, e)
    return errs


def test_backward_tiny_fp32():
    _run(2, 77, 256, 1024, "gelu", "layernorm", 0.5, "f32")


@pytest.mark.parametrize("act,norm,p,s_priv", [
    ("swiglu", "rmsnorm", 0.3, 2.0),        # n_s = 153: boundary inside a chunk
    ("gelu", "layernorm", 0.5, 1.0),
    ("gelu_tanh", "layernorm", 1.0, 1.0),
    ("swiglu", "layernorm", 0.0, 2.0),
])
def test_backward_mlp_bf16(act, norm, p, s_priv):
    _run(4, 130, 512, 4 * 264, act, norm, p, "bf16", s_priv=s_priv)


def test_backward_mlp_residual_is_input():
    """resid = x: the residual gradient is added into din (dresid not given)."""
    _run(4, 96, 512, 4 * 264, "swiglu", "rmsnorm", 0.5, "bf16", resid_given=False,
         dres_given=False)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_out_projection(dtype):
    _run(4, 100, 512, 0, "none", "layernorm", 0.37, dtype, s_priv=2.0)


def test_backward_single_rank_and_small_batch():
    _run(1, 9, 256, 512, "gelu", "rmsnorm", 0.5, "bf16")
    _run(8, 3, 256, 8 * 64, "swiglu", "layernorm", 0.25, "bf16")


@pytest.mark.parametrize("h", [8192, 16384])
@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_wide_rows(h, norm, dtype):
    """Rows of 8192 and 16384 channels: the norm derivative with two and four chunks per
    thread (fewer ranks per register group)."""
    _run(2, 20, h, 2 * 64, "gelu", norm, 0.5, dtype)


def test_backward_fp32_swiglu_residual_is_input():
    """fp32 SwiGLU backward (its activation derivative) with resid = x, so the residual
    gradient is added into din."""
    _run(2, 40, 256, 2 * 96, "swiglu", "rmsnorm", 0.4, "f32", resid_given=False,
         dres_given=False)


def test_backward_7b_dims():
    """The 7B shapes (h = 4096, SwiGLU ffn = 11008, P = 8) at a short batch."""
    _run(8, 72, 4096, 11008, "swiglu", "rmsnorm", 0.5, "bf16")


@pytest.mark.parametrize("n_s_p", [0.0, 1.0 / 256, 63 / 256, 0.25, 65 / 256, 179 / 256,
                                   255 / 256, 1.0])
def test_backward_reduce_mask_bit_exact(n_s_p):
    """Integer-coded gradients: dout = 0, dres_m = 2^m.  Then g_m = 2^m exactly, the
    shared channels of every rank's dZt are 2^P - 1 and the private ones s_priv 2^m."""
    P, T, h = 3, 5, 256
    sub = caat.Sublayer(h, 8 * P, P, n_s_p, norm="layernorm", act="gelu", dtype="f32",
                        s_priv=2.0)
    n_s = sub.n_s
    dres = torch.stack([torch.full((T, h), float(2 ** m)) for m in range(P)]).cuda()
    r = synth.normal((P, T, h), synth.RESID).cuda()
    dout = torch.zeros((P, T, h), device="cuda")
    gamma = torch.ones(h, device="cuda")
    dz = torch.full((P, T, h), float("nan"), device="cuda")
    dres_out = torch.full_like(dz, float("nan"))
    dg = torch.full((h,), float("nan"), device="cuda")
    db = torch.full((h,), float("nan"), device="cuda")
    ws = torch.empty(caat.caat_backward_workspace_bytes(sub.handle, T), dtype=torch.uint8,
                     device="cuda")
    caat.caat_partial_sync_norm_backward(sub.handle, T, r, dout, dres, gamma, dz, dres_out, dg,
                                         db, ws)
    torch.cuda.synchronize()
    want = torch.empty((P, T, h))
    for m in range(P):
        want[m, :, :n_s] = float(2 ** P - 1)
        want[m, :, n_s:] = 2.0 * 2 ** m
    assert torch.equal(dz.cpu(), want)
    assert torch.equal(dres_out.cpu(), dres.cpu())
    assert torch.equal(dg.cpu(), torch.zeros(h)) and torch.equal(db.cpu(), torch.zeros(h))


def test_backward_deterministic():
    a = _run(4, 130, 512, 4 * 264, "swiglu", "rmsnorm", 0.5, "bf16")
    b = _run(4, 130, 512, 4 * 264, "swiglu", "rmsnorm", 0.5, "bf16")
    assert a == b


def test_backward_pair_chain_matches_oracle():
    """The pair's backward as the benchmark runs it: the MLP sublayer's backward, then
    the out-projection's backward fed with the MLP's input and residual gradients."""
    from partial_activation_sync_amd import runner, workloads as W
    w, T = W.PAIR_130M_BF16, 96
    _say(f"[case] pair backward chain {w.name} T={T}")
    inputs = runner.make_inputs(w, T=T, norm_params="random")
    run = runner.Run(w, inputs)
    br = runner.BackwardRun(run)
    br.step()
    torch.cuda.synchronize()
    n_s = oracle.shared_channels(w.h, w.p)
    norm = NORM[w.norm]
    f = lambda t: t.float()
    gamma, beta = f(inputs["gamma"]), f(inputs["beta"])
    a_out, a_res = oracle.sublayer(f(inputs["ctx"]), None, f(inputs["Wo"]), gamma, beta=beta,
                                   resid=f(inputs["x0"]), act=oracle.NONE, norm=norm, n_s=n_s,
                                   eps=w.eps)
    gm = oracle.sublayer_backward(a_out, f(inputs["W1"]), f(inputs["W2"]), gamma, f(br.dout),
                                  act=ACT[w.act], norm=norm, n_s=n_s, resid=a_res,
                                  dres=f(br.dres), eps=w.eps)
    ga = oracle.sublayer_backward(f(inputs["ctx"]), None, f(inputs["Wo"]), gamma, gm["dx"],
                                  act=oracle.NONE, norm=norm, n_s=n_s, resid=f(inputs["x0"]),
                                  dres=gm["dresid"], eps=w.eps)
    names = {"din": "dx", "dresid": "dresid", "dW1": "dW1", "dW2": "dW2", "dgamma": "dgamma",
             "dbeta": "dbeta"}
    errs = {f"mlp.{k}": rel_err(v, gm[names[k]]) for k, v in br.mlp_g.items() if v is not None}
    errs.update({f"attn.{k}": rel_err(v, ga[names[k]]) for k, v in br.attn_g.items()})
    _say("   errors:", {k: f"{e:.2e}" for k, e in errs.items()})
    for k, e in errs.items():
        assert e <= TOL["bf16"], (k, e)


@pytest.mark.parametrize("act,dtype,T,h,ffn", [("swiglu", "bf16", 192, 256, 768),
                                               ("gelu", "bf16", 130, 256, 768),
                                               ("swiglu", "bf16", 24, 256, 768),
                                               ("gelu_tanh", "f32", 40, 256, 768),
                                               ("swiglu", "bf16", 57, 1024, 4 * 1400)])
def test_stored_preactivation(act, dtype, T, h, ffn):
    """caat_forward_train: the same out / out_resid as caat_forward_ex bit for bit, the
    pre-activation x W1^T against the oracle's linear layer, and a backward fed with it
    bit-identical to the backward that recomputes it (T = 24: the weight-streaming
    kernels, which fill the pre-activation with a separate GEMM; T = 57 at h = 1024: the
    64-token MFMA tiles, whose per-tile K order also calls for that separate GEMM)."""
    P = 4
    _say(f"[case] stored pre-activation act={act} {dtype} T={T}")
    d = _inputs(P, T, h, ffn, act, dtype, resid_given=True, dres_given=True)
    dev = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    sub = caat.Sublayer(h, ffn, P, 0.5, norm="rmsnorm", act=act, dtype=dtype, eps=1e-5)
    dt = sub.torch_dtype
    F1 = dev["W1"].shape[1]
    outs = {}
    for train in (False, True):
        out = torch.empty((P, T, h), dtype=dt, device="cuda")
        out_resid = torch.empty_like(out)
        pre = torch.full((P, T, F1), float("nan"), dtype=dt, device="cuda") if train else None
        sub.forward(dev["x"], dev["W1"], dev["W2"], dev["gamma"], out, resid=dev["resid"],
                    beta=dev["beta"], out_resid=out_resid, preact=pre)
        outs[train] = (out, out_resid, pre)
    torch.cuda.synchronize()
    assert torch.equal(outs[True][0], outs[False][0])
    assert torch.equal(outs[True][1], outs[False][1])
    pre = outs[True][2]
    ref = oracle.linear(d["x"].float(), d["W1"].float())
    err = rel_err(pre, ref)
    _say(f"   pre-activation error {err:.2e}")
    assert err <= TOL[dtype]
    grads = {}
    for stored in (False, True):
        g = {
            "dx": torch.empty_like(dev["x"]),
            "dresid": torch.empty((P, T, h), dtype=dt, device="cuda"),
            "dW1": torch.empty_like(dev["W1"]),
            "dW2": torch.empty_like(dev["W2"]),
            "dgamma": torch.empty((h,), dtype=torch.float32, device="cuda"),
        }
        sub.backward(dev["x"], dev["W1"], dev["W2"], dev["gamma"], outs[False][1], dev["dout"],
                     g["dx"], g["dW2"], g["dgamma"], dW1=g["dW1"], dres=dev["dres"],
                     dresid=g["dresid"], preact=pre if stored else None)
        grads[stored] = g
    torch.cuda.synchronize()
    for k in grads[False]:
        assert torch.equal(grads[True][k], grads[False][k]), k


def test_stored_preactivation_large_tiles():
    """7B dims, T = 1024: K1 runs on the 256 x 256 tiles (8 waves), whose epilogue writes
    the gate and up pre-activations through the LDS image.  The training forward's outputs
    equal the plain forward's bit for bit, the pre-activation matches an fp32 matmul of the
    same bf16 inputs, and the backward fed with it equals the recomputing one bit for bit."""
    P, T, h, ffn = 8, 1024, 4096, 11008
    _say(f"[case] stored pre-activation, large tiles P={P} T={T} h={h} ffn={ffn}")
    d = _inputs(P, T, h, ffn, "swiglu", "bf16", resid_given=True, dres_given=True)
    dev = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    sub = caat.Sublayer(h, ffn, P, 0.5, norm="rmsnorm", act="swiglu", dtype="bf16", eps=1e-5)
    F1 = dev["W1"].shape[1]
    res = {}
    for train in (False, True):
        out = torch.empty((P, T, h), dtype=torch.bfloat16, device="cuda")
        out_resid = torch.empty_like(out)
        pre = torch.empty((P, T, F1), dtype=torch.bfloat16, device="cuda") if train else None
        sub.forward(dev["x"], dev["W1"], dev["W2"], dev["gamma"], out, resid=dev["resid"],
                    out_resid=out_resid, preact=pre)
        res[train] = (out, out_resid, pre)
    torch.cuda.synchronize()
    assert torch.equal(res[True][0], res[False][0])
    assert torch.equal(res[True][1], res[False][1])
    pre = res[True][2]
    ref = torch.matmul(dev["x"].float(), dev["W1"].float().transpose(1, 2).contiguous())
    err = float((pre.float() - ref).abs().max() / ref.abs().max())
    _say(f"   pre-activation error vs fp32 matmul {err:.2e}")
    assert err <= TOL["bf16"]
    grads = {}
    for stored in (False, True):
        g = {"dx": torch.empty_like(dev["x"]), "dresid": torch.empty((P, T, h), dtype=torch.bfloat16, device="cuda"),
             "dW1": torch.empty_like(dev["W1"]), "dW2": torch.empty_like(dev["W2"]),
             "dgamma": torch.empty((h,), dtype=torch.float32, device="cuda")}
        sub.backward(dev["x"], dev["W1"], dev["W2"], dev["gamma"], res[False][1], dev["dout"],
                     g["dx"], g["dW2"], g["dgamma"], dW1=g["dW1"], dres=dev["dres"],
                     dresid=g["dresid"], preact=pre if stored else None)
        grads[stored] = g
    torch.cuda.synchronize()
    for k in grads[False]:
        assert torch.equal(grads[True][k], grads[False][k]), k
