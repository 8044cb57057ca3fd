"""Runs a workload (see ``workloads``) through libcaat on the GPU.

Inputs come from ``synth`` (seeded, CPU) and are copied to the device once; a step
then only enqueues the library's kernels.  No arithmetic of the method happens here.

Input recipe (tensor ids from ``synth``):
  MLP-only workloads: x ~ N(0,1) [P][T][h] (one draw copied to every rank when the
    workload says so), W1 ~ N(0, 0.02^2) [P][F1][h], W2 ~ N(0, 0.02^2) [P][h][f_s];
    the residual is x itself.
  Pair workloads: H ~ N(0,1) [P][T][h/P] (per-rank head outputs), x0 ~ N(0,1)
    [P][T][h] (the residual entering the attention sublayer), Wo ~ N(0, 0.02^2)
    [P][h][h/P]; then the MLP takes the attention output as input and the
    attention's residual output as residual.
  gamma = 1, beta = 0 ("unit"), or gamma ~ 1 + N(0, 0.1^2), beta ~ N(0, 0.1^2) ("random").
"""
import torch

from . import synth
from .workloads import ATTN_OUT, MLP, Workload
from . import Sublayer

WEIGHT_STD = 0.02


def torch_dtype(w: Workload):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def make_inputs(w: Workload, T=None, norm_params="unit", seed=synth.BASE_SEED):
    """CPU tensors for one workload (weights do not depend on T)."""
    T = w.T if T is None else T
    P, h, fs = w.P, w.h, w.f_s
    dt = torch_dtype(w)
    F1 = 2 * fs if w.act == "swiglu" else fs
    d = {}
    if ATTN_OUT in w.sublayers:
        d["ctx"] = synth.normal((P, T, h // P), synth.CTX, dtype=dt, seed=seed)
        d["x0"] = synth.normal((P, T, h), synth.X0, dtype=dt, seed=seed)
        d["Wo"] = synth.normal((P, h, h // P), synth.WO, std=WEIGHT_STD, dtype=dt, seed=seed)
    else:
        if w.replicated_x:
            d["x"] = synth.replicated((T, h), P, synth.X, dtype=dt, seed=seed)
        else:
            d["x"] = synth.normal((P, T, h), synth.X, dtype=dt, seed=seed)
    d["W1"] = synth.normal((P, F1, h), synth.W1, std=WEIGHT_STD, dtype=dt, seed=seed)
    d["W2"] = synth.normal((P, h, fs), synth.W2, std=WEIGHT_STD, dtype=dt, seed=seed)
    if norm_params == "unit":
        d["gamma"] = torch.ones(h, dtype=dt)
        d["beta"] = torch.zeros(h, dtype=dt)
    else:
        d["gamma"] = synth.normal((h,), synth.GAMMA, std=0.1, mean=1.0, dtype=dt, seed=seed)
        d["beta"] = synth.normal((h,), synth.BETA, std=0.1, dtype=dt, seed=seed)
    return d


class Run:
    """Device-resident inputs, outputs and handles for one workload at one T."""

    def __init__(self, w: Workload, inputs: dict, p=None, s_priv=1.0, device="cuda",
                 store_resid=True, weight_copies=1):
        self.w = w
        self.p = w.p if p is None else p
        self.dev = {k: v.to(device) for k, v in inputs.items()}
        # Extra copies of the weights, so that a benchmark can rotate through more bytes
        # than the 256 MB Infinity Cache holds (weight-streaming shapes).
        self.weight_sets = [{k: self.dev[k] for k in ("W1", "W2", "Wo") if k in self.dev}]
        for _ in range(1, weight_copies):
            self.weight_sets.append({k: v.clone() for k, v in self.weight_sets[0].items()})
        P, h = w.P, w.h
        self.T = T = (self.dev["ctx"] if "ctx" in self.dev else self.dev["x"]).shape[1]
        dt = torch_dtype(w)
        self.attn = None
        if ATTN_OUT in w.sublayers:
            self.attn = Sublayer(h, 0, P, self.p, norm=w.norm, act="none", dtype=w.dtype,
                                 eps=w.eps, s_priv=s_priv)
            self.attn.workspace(T, device)
            self.attn_out = torch.empty((P, T, h), dtype=dt, device=device)
            self.attn_out_resid = torch.empty((P, T, h), dtype=dt, device=device)
        self.mlp = Sublayer(h, w.ffn, P, self.p, norm=w.norm, act=w.act, dtype=w.dtype,
                            eps=w.eps, s_priv=s_priv)
        self.mlp.workspace(T, device)
        self.out = torch.empty((P, T, h), dtype=dt, device=device)
        self.out_resid = torch.empty((P, T, h), dtype=dt, device=device) if store_resid else None

    def step(self, stream=None, preact=None, events_attn=None, events_mlp=None, copy=0):
        """One forward of the whole path (out-projection sublayer, then the MLP), through
        caat_forward_ex, or caat_forward_timed when events are given (raw hipEvent_t
        handles recorded after each of the library's FWD_STEPS of that sublayer).
        preact: a [P][T][F1] tensor that receives the MLP's pre-activation (a training
        forward).  copy: which weight copy to read (see weight_copies)."""
        d = dict(self.dev, **self.weight_sets[copy])
        if self.attn is not None:
            self.attn.forward(d["ctx"], None, d["Wo"], d["gamma"], self.attn_out, resid=d["x0"],
                              beta=d["beta"], out_resid=self.attn_out_resid, stream=stream,
                              events=events_attn)
            mlp_in, mlp_resid = self.attn_out, self.attn_out_resid
        else:
            mlp_in, mlp_resid = d["x"], d["x"]
        self.mlp.forward(mlp_in, d["W1"], d["W2"], d["gamma"], self.out, resid=mlp_resid,
                         beta=d["beta"], out_resid=self.out_resid, stream=stream, preact=preact,
                         events=events_mlp)

    def outputs(self):
        o = {"out": self.out}
        if self.out_resid is not None:
            o["out_resid"] = self.out_resid
        if self.attn is not None:
            o["attn_out"] = self.attn_out
            o["attn_out_resid"] = self.attn_out_resid
        return o


class BackwardRun:
    """The backward of the whole path after one forward: the MLP sublayer's backward
    (upstream gradients dout, dres drawn from ``synth``), then, for pair workloads, the
    out-projection sublayer's backward fed with the gradients of the MLP's input and
    residual (the chain rule through the pair).  A step only enqueues library calls."""

    def __init__(self, run: Run, seed=synth.BASE_SEED, store_preact=True):
        """store_preact: the forward is a training forward that stores the MLP's
        pre-activation, which the backward then reads instead of recomputing."""
        self.run = run
        w = run.w
        P, T, h = w.P, run.T, w.h
        dt = torch_dtype(w)
        dev = run.out.device
        if run.out_resid is None:
            raise ValueError("the backward needs the forward's out_resid")
        F1 = 2 * w.f_s if w.act == "swiglu" else w.f_s
        self.preact = torch.empty((P, T, F1), dtype=dt, device=dev) if store_preact else None
        run.step(preact=self.preact)
        self.dout = synth.normal((P, T, h), synth.DOUT, dtype=dt, seed=seed).to(dev)
        self.dres = synth.normal((P, T, h), synth.DRES, dtype=dt, seed=seed).to(dev)
        e = lambda shape, dtype=dt: torch.empty(shape, dtype=dtype, device=dev)
        F1 = 2 * w.f_s if w.act == "swiglu" else w.f_s
        pair = run.attn is not None
        self.mlp_g = {"din": e((P, T, h)), "dresid": e((P, T, h)) if pair else None,
                      "dW1": e((P, F1, h)), "dW2": e((P, h, w.f_s)),
                      "dgamma": e((h,), torch.float32), "dbeta": e((h,), torch.float32)}
        self.attn_g = None
        if pair:
            self.attn_g = {"din": e((P, T, h // P)), "dresid": e((P, T, h)),
                           "dW2": e((P, h, h // P)), "dgamma": e((h,), torch.float32),
                           "dbeta": e((h,), torch.float32)}

    def step(self, events_mlp=None, events_attn=None):
        run, d, g = self.run, self.run.dev, self.mlp_g
        mlp_in = run.attn_out if run.attn is not None else d["x"]
        run.mlp.backward(mlp_in, d["W1"], d["W2"], d["gamma"], run.out_resid, self.dout, g["din"],
                         g["dW2"], g["dgamma"], dW1=g["dW1"], dres=self.dres, dresid=g["dresid"],
                         dbeta=g["dbeta"], events=events_mlp, preact=self.preact)
        if run.attn is not None:
            a = self.attn_g
            run.attn.backward(d["ctx"], None, d["Wo"], d["gamma"], run.attn_out_resid, g["din"],
                              a["din"], a["dW2"], a["dgamma"], dres=g["dresid"],
                              dresid=a["dresid"], dbeta=a["dbeta"], events=events_attn)
