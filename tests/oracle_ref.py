"""Oracle chain for a workload and the parity metric (test infrastructure).

Runs the fp64 oracle over the same CPU inputs the GPU run gets, for all token rows or
a sample of them (token rows never interact), chaining the out-projection sublayer
into the MLP sublayer exactly as the GPU path does.
"""
import numpy as np
import torch

import oracle
from partial_activation_sync_amd.workloads import ATTN_OUT

ACT = {"gelu": oracle.GELU, "gelu_tanh": oracle.GELU_TANH, "swiglu": oracle.SWIGLU}
NORM = {"layernorm": oracle.LAYERNORM, "rmsnorm": oracle.RMSNORM}

# Parity bar: max |gpu - oracle| / max |oracle| per output tensor.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def reference(w, inputs, rows=None, p=None, s_priv=1.0):
    p = w.p if p is None else p
    n_s = oracle.shared_channels(w.h, p)
    norm = NORM[w.norm]

    def sel(t):
        t = t.float()
        return t[:, rows] if rows is not None else t

    gamma, beta = inputs["gamma"].float(), inputs["beta"].float()
    res = {}
    if ATTN_OUT in w.sublayers:
        a_out, a_res = oracle.sublayer(sel(inputs["ctx"]), None, inputs["Wo"].float(), gamma,
                                       beta=beta, resid=sel(inputs["x0"]), act=oracle.NONE,
                                       norm=norm, n_s=n_s, s_priv=s_priv, eps=w.eps)
        res["attn_out"], res["attn_out_resid"] = a_out, a_res
        mlp_in, mlp_resid = a_out, a_res
    else:
        mlp_in, mlp_resid = sel(inputs["x"]), None
    out, out_res = oracle.sublayer(mlp_in, inputs["W1"].float(), inputs["W2"].float(), gamma,
                                   beta=beta, resid=mlp_resid, act=ACT[w.act], norm=norm,
                                   n_s=n_s, s_priv=s_priv, eps=w.eps)
    res["out"], res["out_resid"] = out, out_res
    return res


def rel_err(gpu, ref):
    g = gpu.detach().float().cpu().numpy().astype(np.float64) if isinstance(gpu, torch.Tensor) else gpu
    r = np.asarray(ref, np.float64)
    denom = np.abs(r).max()
    return float(np.abs(g - r).max() / (denom if denom > 0 else 1.0))


def compare(w, gpu_outputs, ref, rows=None):
    """{name: relative error} over the outputs both sides have."""
    errs = {}
    for k, r in ref.items():
        if k not in gpu_outputs or gpu_outputs[k] is None:
            continue
        g = gpu_outputs[k]
        if rows is not None:
            g = g[:, rows.to(g.device)]
        errs[k] = rel_err(g, r)
    return errs
