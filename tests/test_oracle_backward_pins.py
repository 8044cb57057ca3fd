"""Pins for the backward oracle: what the mathematics fixes, independent of the oracle.

Source: "Tensor-Parallelism with Partially Synchronized Activations".
  - §4 "Forward-backward mismatch" (Eq. 9-13) and App. B (Eq. 25-30): the backward of
    the sublayer is the gradient of the forward.  Here that is checked directly:
    central finite differences of the (separately pinned) forward oracle, over every
    entry of every input on tiny shapes.  A wrong placement of the reduce (before the
    norm derivative instead of after it), a dropped residual term, a missing private
    scale or a wrong activation derivative all fail it.
  - p = 1 is the unsharded layer (§3, Eq. 5 / Eq. 21): torch fp64 autograd on the
    assembled full matrices gives the same gradients.
  - p = 0 is P independent layers (§1): torch fp64 autograd per rank.
Everything here runs on the CPU.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(777)


def _rand(*shape, std=1.0):
    return (RNG.standard_normal(shape) * std).astype(np.float32)


def _case(P, T, h, ffn, act, resid_given, dres_given):
    if act == oracle.NONE:
        kin, F1, k2 = h // P, 0, h // P
    else:
        fs = ffn // P
        kin, F1, k2 = h, (2 * fs if act == oracle.SWIGLU else fs), fs
    d = {
        "x": _rand(P, T, kin),
        "W1": _rand(P, F1, h, std=0.3) if act != oracle.NONE else None,
        "W2": _rand(P, h, k2, std=0.3),
        "gamma": (1.0 + _rand(h, std=0.2)).astype(np.float32),
        "beta": _rand(h, std=0.2),
        "resid": _rand(P, T, h) if resid_given else None,
        "dout": _rand(P, T, h),
        "dres": _rand(P, T, h) if dres_given else None,
    }
    return d


def _loss(d, **kw):
    out, out_resid = oracle.sublayer(d["x"], d["W1"], d["W2"], d["gamma"], beta=d["beta"],
                                     resid=d["resid"], **kw)
    L = float(np.sum(out * d["dout"].astype(np.float64)))
    if d["dres"] is not None:
        L += float(np.sum(out_resid * d["dres"].astype(np.float64)))
    return L


FD_CASES = [
    # act, norm, P, h, ffn, p, s_priv, resid given, dres given
    (oracle.GELU, oracle.LAYERNORM, 3, 16, 24, 0.5, 1.0, True, True),
    (oracle.GELU_TANH, oracle.RMSNORM, 3, 16, 24, 0.3, math.sqrt(3), False, False),
    (oracle.SWIGLU, oracle.RMSNORM, 2, 16, 16, 1.0, 1.0, True, True),
    (oracle.SWIGLU, oracle.LAYERNORM, 3, 16, 24, 0.0, math.sqrt(3), False, True),
    (oracle.NONE, oracle.LAYERNORM, 3, 12, 0, 0.5, 1.0, True, True),
    (oracle.NONE, oracle.RMSNORM, 4, 16, 0, 0.25, 2.0, True, False),
    (oracle.GELU, oracle.LAYERNORM, 1, 16, 8, 0.5, 1.0, True, True),
]


@pytest.mark.parametrize("act,norm,P,h,ffn,p,s_priv,resid_given,dres_given", FD_CASES)
def test_backward_matches_finite_differences(act, norm, P, h, ffn, p, s_priv, resid_given,
                                             dres_given):
    T = 3
    d = _case(P, T, h, ffn, act, resid_given, dres_given)
    n_s = oracle.shared_channels(h, p)
    kw = dict(act=act, norm=norm, n_s=n_s, s_priv=s_priv, eps=1e-5)
    g = oracle.sublayer_backward(d["x"], d["W1"], d["W2"], d["gamma"], d["dout"],
                                 resid=d["resid"], dres=d["dres"], **kw)
    targets = [("x", "dx"), ("W2", "dW2"), ("gamma", "dgamma"), ("beta", "dbeta")]
    if act != oracle.NONE:
        targets.append(("W1", "dW1"))
    if resid_given:
        targets.append(("resid", "dresid"))
    for name, gname in targets:
        v = d[name]
        fd = np.empty(v.shape, np.float64)
        step = np.float32(2.0 ** -9)
        for i in np.ndindex(v.shape):
            orig = v[i]
            v[i] = orig + step
            hi, lp = np.float64(v[i]), _loss(d, **kw)
            v[i] = orig - step
            lo, lm = np.float64(v[i]), _loss(d, **kw)
            v[i] = orig
            fd[i] = (lp - lm) / (hi - lo)
        want = g[gname]
        if name == "beta" and norm == oracle.RMSNORM:
            assert np.all(want == 0.0)
        scale = max(np.max(np.abs(fd)), 1e-3)
        err = np.max(np.abs(want - fd)) / scale
        assert err < 2e-4, f"{gname}: max rel err {err:.2e} vs finite differences"


def _act_t(act, a, fs):
    if act == oracle.GELU:
        return F.gelu(a)
    if act == oracle.GELU_TANH:
        return F.gelu(a, approximate="tanh")
    if act == oracle.SWIGLU:
        return F.silu(a[..., :fs]) * a[..., fs:]
    raise ValueError(act)


def _norm_t(r, gamma, beta, norm, eps):
    if norm == oracle.LAYERNORM:
        return F.layer_norm(r, (r.shape[-1],), gamma, beta, eps)
    return F.rms_norm(r, (r.shape[-1],), gamma, eps)


@pytest.mark.parametrize("act,norm", [(oracle.GELU, oracle.LAYERNORM),
                                      (oracle.SWIGLU, oracle.RMSNORM),
                                      (oracle.NONE, oracle.LAYERNORM)])
def test_backward_p1_equals_unsharded_autograd(act, norm):
    """p = 1: gradients of the sharded layer equal those of the unsharded layer (torch
    fp64 autograd on the full matrices), with the replicated input's gradient summed
    over ranks."""
    P, T, h = 4, 5, 32
    ffn = 48
    d = _case(P, T, h, ffn, act, resid_given=True, dres_given=True)
    d["resid"] = np.broadcast_to(d["resid"][0], d["resid"].shape).copy()
    if act != oracle.NONE:
        d["x"] = np.broadcast_to(d["x"][0], d["x"].shape).copy()
    g = oracle.sublayer_backward(d["x"], d["W1"], d["W2"], d["gamma"], d["dout"],
                                 resid=d["resid"], dres=d["dres"], act=act, norm=norm,
                                 n_s=h, s_priv=1.0, eps=1e-5)
    t64 = lambda a: torch.tensor(np.asarray(a, np.float64))
    W2 = t64(d["W2"])
    B = torch.cat([W2[m].T for m in range(P)], 0).requires_grad_()       # [P k2][h]
    gamma, beta = t64(d["gamma"]).requires_grad_(), t64(d["beta"]).requires_grad_()
    R = t64(d["resid"][0]).requires_grad_()
    if act == oracle.NONE:
        H = torch.cat([t64(d["x"][m]) for m in range(P)], 1).requires_grad_()  # [T][h]
        z = H @ B
    else:
        fs = ffn // P
        W1 = t64(d["W1"])
        x = t64(d["x"][0]).requires_grad_()
        if act == oracle.SWIGLU:
            Ag = torch.cat([W1[m][:fs].T for m in range(P)], 1)
            Au = torch.cat([W1[m][fs:].T for m in range(P)], 1)
            A = torch.cat([Ag, Au], 1).requires_grad_()
            a = x @ A
            y = F.silu(a[:, :ffn]) * a[:, ffn:]
        else:
            A = torch.cat([W1[m].T for m in range(P)], 1).requires_grad_()
            y = _act_t(act, x @ A, fs)
        z = y @ B
    r = R + z
    out = _norm_t(r, gamma, beta, norm, 1e-5)
    L = ((out * t64(d["dout"]).sum(0)).sum() + (r * t64(d["dres"]).sum(0)).sum())
    L.backward()

    def close(a, b):
        a, b = np.asarray(a), np.asarray(b)
        assert np.max(np.abs(a - b)) <= 1e-9 * max(1.0, np.max(np.abs(b)))

    close(g["dgamma"], gamma.grad)
    if norm == oracle.LAYERNORM:
        close(g["dbeta"], beta.grad)
    else:
        assert np.all(g["dbeta"] == 0.0)
    close(g["dresid"].sum(0), R.grad)
    Bg = B.grad.numpy()
    k2 = d["W2"].shape[2]
    for m in range(P):
        close(g["dW2"][m], Bg[m * k2:(m + 1) * k2].T)
    if act == oracle.NONE:
        for m in range(P):
            close(g["dx"][m], H.grad.numpy()[:, m * k2:(m + 1) * k2])
    else:
        close(g["dx"].sum(0), x.grad)
        fs = ffn // P
        Agr = A.grad.numpy()
        for m in range(P):
            if act == oracle.SWIGLU:
                close(g["dW1"][m][:fs], Agr[:, m * fs:(m + 1) * fs].T)
                close(g["dW1"][m][fs:], Agr[:, ffn + m * fs:ffn + (m + 1) * fs].T)
            else:
                close(g["dW1"][m], Agr[:, m * fs:(m + 1) * fs].T)


@pytest.mark.parametrize("act,norm,resid_given", [(oracle.GELU_TANH, oracle.RMSNORM, False),
                                                  (oracle.SWIGLU, oracle.LAYERNORM, True)])
def test_backward_p0_equals_independent_layers(act, norm, resid_given):
    """p = 0: every rank is an independent layer whose output is scaled by s_priv."""
    P, T, h, ffn, s = 3, 4, 24, 36, 1.7
    d = _case(P, T, h, ffn, act, resid_given, dres_given=True)
    g = oracle.sublayer_backward(d["x"], d["W1"], d["W2"], d["gamma"], d["dout"],
                                 resid=d["resid"], dres=d["dres"], act=act, norm=norm,
                                 n_s=0, s_priv=s, eps=1e-5)
    t64 = lambda a: torch.tensor(np.asarray(a, np.float64))
    fs = ffn // P
    dg = np.zeros(h)
    for m in range(P):
        x = t64(d["x"][m]).requires_grad_()
        W1 = t64(d["W1"][m]).requires_grad_()
        W2 = t64(d["W2"][m]).requires_grad_()
        gamma, beta = t64(d["gamma"]).requires_grad_(), t64(d["beta"]).requires_grad_()
        R = t64(d["resid"][m]).requires_grad_() if resid_given else x
        r = R + s * (_act_t(act, x @ W1.T, fs) @ W2.T)
        out = _norm_t(r, gamma, beta, norm, 1e-5)
        L = (out * t64(d["dout"][m])).sum() + (r * t64(d["dres"][m])).sum()
        L.backward()
        for a, b in ((g["dx"][m], x.grad), (g["dW1"][m], W1.grad), (g["dW2"][m], W2.grad)):
            assert np.max(np.abs(a - b.numpy())) <= 1e-9 * max(1.0, float(b.abs().max()))
        if resid_given:
            assert np.max(np.abs(g["dresid"][m] - R.grad.numpy())) <= 1e-9 * float(R.grad.abs().max())
        dg += gamma.grad.numpy()
    assert np.max(np.abs(g["dgamma"] - dg)) <= 1e-9 * max(1.0, np.max(np.abs(dg)))
