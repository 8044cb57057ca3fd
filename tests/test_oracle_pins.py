"""Pins for the oracle: what the page and the mathematics fix, independent of the oracle.

Source: "Tensor-Parallelism with Partially Synchronized Activations".
  - p = 1 turns the partial channel-reduce into a full all-reduce (§3), and the
    sharded MLP then equals the unsharded one by distributivity (§3.1, Eq. 1 vs
    Eq. 5; App. A.2, Eq. 20 vs Eq. 21).
  - p = 0 makes every rank an independent layer (§1, the "ensemble" extreme).
  - The P = 2 block form of the MLP (§3.1, Eq. 7-8) and of the attention output
    projection (App. A.1, Eq. 19).
  - Residual + normalization after the reduce (§4, Eq. 9), LayerNorm / RMSNorm.
  - Private channel scaling restores equal variance (§4, Eq. 14-15).
Everything here runs on the CPU.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy import special, stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


def _rand(*shape, std=1.0):
    return (RNG.standard_normal(shape) * std).astype(np.float32)


def _act_np(act, a_gate, a_up=None):
    """Activations written with library routines (scipy / torch), not the oracle's formula."""
    if act == oracle.GELU:
        return a_gate * stats.norm.cdf(a_gate)          # x * Phi(x)
    if act == oracle.GELU_TANH:
        return F.gelu(torch.from_numpy(a_gate), approximate="tanh").numpy()
    if act == oracle.SWIGLU:
        return a_gate * special.expit(a_gate) * a_up    # silu(g) * u
    raise ValueError(act)


def _norm_torch(r, gamma, beta, norm, eps):
    t = torch.from_numpy(np.asarray(r, np.float64))
    g = torch.from_numpy(np.asarray(gamma, np.float64))
    if norm == oracle.LAYERNORM:
        b = torch.from_numpy(np.asarray(beta, np.float64)) if beta is not None else None
        return F.layer_norm(t, (t.shape[-1],), g, b, eps).numpy()
    return F.rms_norm(t, (t.shape[-1],), g, eps).numpy()


def _mlp_case(P, T, h, ffn, act, replicated):
    fs = ffn // P
    F1 = 2 * fs if act == oracle.SWIGLU else fs
    if replicated:
        x = np.broadcast_to(_rand(T, h), (P, T, h)).copy()
    else:
        x = _rand(P, T, h)
    W1 = _rand(P, F1, h, std=0.2)
    W2 = _rand(P, h, fs, std=0.2)
    gamma = (1 + _rand(h, std=0.1)).astype(np.float32)
    beta = _rand(h, std=0.1)
    return x, W1, W2, gamma, beta


# ---------------------------------------------------------------------------
# n_s: which channels are shared (§3; App. A.2, Eq. 22: l < floor(h p))
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("h,p,expect", [
    (4096, 0.5, 2048), (2048, 0.25, 512), (2048, 1.0, 2048), (768, 0.5, 384),
    (256, 0.5, 128), (100, 0.29, 29), (10, 0.25, 2), (7, 0.5, 3), (4096, 0.0, 0),
    (4096, 0.703125, 2880), (4096, 1.0 / 3.0, 1365), (1, 0.999, 0), (3, 2.0 / 3.0, 2),
])
def test_shared_channel_count(h, p, expect):
    assert oracle.shared_channels(h, p) == expect


# ---------------------------------------------------------------------------
# The nonlinearity against textbook values and library routines
# ---------------------------------------------------------------------------
def test_activation_values():
    # GeLU(x) = x * Phi(x); Phi(1) = 0.8413447460685429 (standard normal table).
    assert oracle.activation(oracle.GELU, 1.0) == pytest.approx(0.8413447460685429, rel=1e-15)
    assert oracle.activation(oracle.GELU, -1.0) == pytest.approx(-0.15865525393145707, rel=1e-14)
    assert oracle.activation(oracle.GELU, 0.0) == 0.0
    assert oracle.activation(oracle.GELU, 40.0) == 40.0
    # silu(1) = 1 / (1 + e^-1) = 0.7310585786300049
    assert oracle.activation(oracle.SWIGLU, 1.0, 1.0) == pytest.approx(0.7310585786300049, rel=1e-15)
    assert oracle.activation(oracle.SWIGLU, 2.0, -3.0) == pytest.approx(-3.0 * 2.0 * special.expit(2.0), rel=1e-15)
    assert oracle.activation(oracle.NONE, -2.5) == -2.5
    xs = np.linspace(-6, 6, 97)
    for a in xs:
        assert oracle.activation(oracle.GELU, a) == pytest.approx(a * stats.norm.cdf(a), rel=1e-12, abs=1e-300)
        want_tanh = F.gelu(torch.tensor(a, dtype=torch.float64), approximate="tanh").item()
        assert oracle.activation(oracle.GELU_TANH, a) == pytest.approx(want_tanh, rel=1e-12, abs=1e-300)
        # torch's fp64 gelu uses 1 + erf(.), which cancels for a << 0: absolute check only.
        want_exact = F.gelu(torch.tensor(a, dtype=torch.float64)).item()
        assert oracle.activation(oracle.GELU, a) == pytest.approx(want_exact, rel=1e-12, abs=1e-15)


# ---------------------------------------------------------------------------
# p = 1: the full all-reduce; the sharded layer equals the unsharded one
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("act", [oracle.GELU, oracle.GELU_TANH, oracle.SWIGLU])
@pytest.mark.parametrize("norm", [oracle.LAYERNORM, oracle.RMSNORM])
def test_p1_equals_unsharded_mlp(act, norm):
    P, T, h, ffn = 4, 6, 32, 64
    x, W1, W2, gamma, beta = _mlp_case(P, T, h, ffn, act, replicated=True)
    fs = ffn // P
    X = x[0].astype(np.float64)
    # Assemble the unsharded A (h x ffn) and B (ffn x h): A = [A_1 ... A_P] by
    # columns (Eq. 2), B = [B_1; ...; B_P] by rows (Eq. 4).
    if act == oracle.SWIGLU:
        Ag = np.concatenate([W1[m, :fs, :].T for m in range(P)], axis=1).astype(np.float64)
        Au = np.concatenate([W1[m, fs:, :].T for m in range(P)], axis=1).astype(np.float64)
        Y = _act_np(act, X @ Ag, X @ Au)
    else:
        A = np.concatenate([W1[m].T for m in range(P)], axis=1).astype(np.float64)
        Y = _act_np(act, X @ A)
    B = np.concatenate([W2[m].T for m in range(P)], axis=0).astype(np.float64)
    Z = Y @ B                                        # Eq. 1: Z = sigma(X A) B
    r = Z + X                                        # Eq. 9 with R = the input
    want = _norm_torch(r, gamma, beta, norm, 1e-5)
    n_s = oracle.shared_channels(h, 1.0)
    out, out_resid = oracle.sublayer(x, W1, W2, gamma, beta=beta, act=act, norm=norm, n_s=n_s)
    for m in range(P):
        np.testing.assert_allclose(out_resid[m], r, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(out[m], want, rtol=1e-10, atol=1e-10)


def test_p1_equals_unsharded_attention_out_projection():
    # App. A.1 Eq. 17 / App. A.2 Eq. 23: Z = [H_1 ... H_P] O.
    P, T, h = 4, 5, 32
    H = _rand(P, T, h // P)
    O = _rand(h, h, std=0.2)                          # O: h x h, rows split by rank
    W2 = np.stack([O[m * (h // P):(m + 1) * (h // P), :].T for m in range(P)]).copy()
    resid = _rand(P, T, h)
    gamma = np.ones(h, np.float32)
    Y = np.concatenate([H[m] for m in range(P)], axis=1).astype(np.float64)
    Z = Y @ O.astype(np.float64)
    out, out_resid = oracle.sublayer(H, None, W2, gamma, resid=resid, act=oracle.NONE,
                                     norm=oracle.RMSNORM, n_s=h)
    for m in range(P):
        np.testing.assert_allclose(out_resid[m], Z + resid[m], rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(out[m], _norm_torch(Z + resid[m], gamma, None, oracle.RMSNORM, 1e-5),
                                   rtol=1e-10, atol=1e-10)


# ---------------------------------------------------------------------------
# p = 0: P independent layers (no channel is reduced)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("act", [oracle.GELU, oracle.SWIGLU])
def test_p0_equals_independent_layers(act):
    P, T, h, ffn = 3, 5, 24, 48
    x, W1, W2, gamma, beta = _mlp_case(P, T, h, ffn, act, replicated=False)
    fs = ffn // P
    out, out_resid = oracle.sublayer(x, W1, W2, gamma, beta=beta, act=act,
                                     norm=oracle.LAYERNORM, n_s=0)
    for m in range(P):
        X = x[m].astype(np.float64)
        if act == oracle.SWIGLU:
            Y = _act_np(act, X @ W1[m, :fs].T.astype(np.float64), X @ W1[m, fs:].T.astype(np.float64))
        else:
            Y = _act_np(act, X @ W1[m].T.astype(np.float64))
        r = Y @ W2[m].T.astype(np.float64) + X
        np.testing.assert_allclose(out_resid[m], r, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(out[m], _norm_torch(r, gamma, beta, oracle.LAYERNORM, 1e-5),
                                   rtol=1e-10, atol=1e-10)


def test_single_rank_ignores_p():
    P, T, h, ffn = 1, 4, 16, 32
    x, W1, W2, gamma, beta = _mlp_case(P, T, h, ffn, oracle.GELU, replicated=False)
    ref = oracle.sublayer(x, W1, W2, gamma, act=oracle.GELU, norm=oracle.RMSNORM, n_s=0)
    for n_s in (1, 7, 16):
        got = oracle.sublayer(x, W1, W2, gamma, act=oracle.GELU, norm=oracle.RMSNORM, n_s=n_s)
        np.testing.assert_array_equal(got[0], ref[0])


# ---------------------------------------------------------------------------
# P = 2 block form, literally as printed: Eq. 7-8 (MLP) and Eq. 19 (attention)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n_s", [0, 5, 8, 13, 16])
def test_two_rank_block_form_mlp(n_s):
    P, T, h, ffn = 2, 4, 16, 24
    act = oracle.GELU
    x, W1, W2, gamma, beta = _mlp_case(P, T, h, ffn, act, replicated=False)
    X1, X2 = x[0].astype(np.float64), x[1].astype(np.float64)
    A1, A2 = W1[0].T.astype(np.float64), W1[1].T.astype(np.float64)
    Y1, Y2 = _act_np(act, X1 @ A1), _act_np(act, X2 @ A2)           # Eq. 6
    Bdev1, Bdev2 = W2[0].T.astype(np.float64), W2[1].T.astype(np.float64)
    B11, B21 = Bdev1[:, :n_s], Bdev1[:, n_s:]                       # Eq. 7: device 1 rows
    B12, B22 = Bdev2[:, :n_s], Bdev2[:, n_s:]                       #        device 2 rows
    shared = Y1 @ B11 + Y2 @ B12
    Z1 = np.concatenate([shared, Y1 @ B21], axis=1)                 # Eq. 8
    Z2 = np.concatenate([shared, Y2 @ B22], axis=1)
    _, out_resid = oracle.sublayer(x, W1, W2, gamma, act=act, norm=oracle.LAYERNORM, n_s=n_s)
    np.testing.assert_allclose(out_resid[0], Z1 + X1, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(out_resid[1], Z2 + X2, rtol=1e-11, atol=1e-11)


def test_worked_example_eq19():
    with open(os.path.join(GOLDEN, "eq19_worked_example.json")) as f:
        g = json.load(f)
    H = np.array(g["H"], np.float32)                 # [P=2][T=1][h/P=2]
    O = np.array(g["O"], np.float32)                 # [h][h]
    W2 = np.stack([O[0:2, :].T, O[2:4, :].T]).copy()  # rank m holds rows of O, stored [h][h/P]
    R = np.array(g["R"], np.float32)
    gamma = np.array(g["gamma"], np.float32)
    beta = np.array(g["beta"], np.float32)
    for case in g["cases"]:
        n_s = oracle.shared_channels(4, case["p"])
        assert n_s == case["n_s"]
        norm = oracle.LAYERNORM if case["norm"] == "layernorm" else oracle.RMSNORM
        out, out_resid = oracle.sublayer(H, None, W2, gamma, beta=beta, resid=R, act=oracle.NONE,
                                         norm=norm, n_s=n_s, eps=case["eps"])
        np.testing.assert_array_equal(out_resid, np.array(case["out_resid"], np.float64))
        np.testing.assert_allclose(out, np.array(case["out"]), rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------------------
# The reduce + residual + norm step on its own
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("P", [1, 2, 3, 8])
@pytest.mark.parametrize("n_s_case", ["zero", "one", "63", "64", "65", "179", "h-1", "h"])
def test_mask_integer_coded(P, n_s_case):
    T, h = 3, 256
    named = {"zero": 0, "one": 1, "h-1": h - 1, "h": h}
    n_s = named[n_s_case] if n_s_case in named else int(n_s_case)
    s_priv = math.sqrt(P)
    partials = np.stack([np.full((T, h), 2.0 ** m, np.float32) for m in range(P)])
    resid = np.zeros((P, T, h), np.float32)
    gamma = np.ones(h, np.float32)
    _, out_resid = oracle.partial_sync_norm(partials, resid, gamma, norm=oracle.RMSNORM,
                                            n_s=n_s, s_priv=s_priv)
    for m in range(P):
        np.testing.assert_array_equal(out_resid[m, :, :n_s], 2.0 ** P - 1)
        np.testing.assert_allclose(out_resid[m, :, n_s:], 2.0 ** m * s_priv, rtol=1e-15)


def test_private_scaling_is_linear_in_partials():
    P, T, h, ffn = 4, 3, 32, 64
    x, W1, W2, gamma, beta = _mlp_case(P, T, h, ffn, oracle.SWIGLU, replicated=False)
    n_s = 12
    for s in (1.0, 2.0, math.sqrt(P)):
        _, out_resid, zt = oracle.sublayer(x, W1, W2, gamma, act=oracle.SWIGLU, norm=oracle.RMSNORM,
                                           n_s=n_s, s_priv=s, want_partials=True)
        np.testing.assert_allclose(out_resid[:, :, n_s:], x[:, :, n_s:] + s * zt[:, :, n_s:],
                                   rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(out_resid[:, :, :n_s], x[:, :, :n_s] + zt[:, :, :n_s].sum(0),
                                   rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("norm", [oracle.LAYERNORM, oracle.RMSNORM])
def test_norm_closed_forms(norm):
    P, T, h = 2, 16, 64
    partials = _rand(P, T, h) * 3 + 1
    resid = _rand(P, T, h)
    gamma = np.ones(h, np.float32)
    eps = 1e-5
    out, out_resid = oracle.partial_sync_norm(partials, resid, gamma, norm=norm, n_s=20, eps=eps)
    if norm == oracle.LAYERNORM:
        v = out_resid.var(axis=-1)
        np.testing.assert_allclose(out.mean(axis=-1), 0.0, atol=1e-13)
        np.testing.assert_allclose(out.var(axis=-1), v / (v + eps), rtol=1e-12)
    else:
        ms = (out_resid ** 2).mean(axis=-1)
        np.testing.assert_allclose((out ** 2).mean(axis=-1), ms / (ms + eps), rtol=1e-12)


@pytest.mark.parametrize("norm", [oracle.LAYERNORM, oracle.RMSNORM])
def test_norm_matches_library(norm):
    P, T, h = 3, 8, 48
    partials = _rand(P, T, h)
    resid = _rand(P, T, h)
    gamma = (1 + _rand(h, std=0.2)).astype(np.float32)
    beta = _rand(h, std=0.2)
    out, out_resid = oracle.partial_sync_norm(partials, resid, gamma, beta=beta, norm=norm, n_s=10)
    want = _norm_torch(out_resid, gamma, beta if norm == oracle.LAYERNORM else None, norm, 1e-5)
    np.testing.assert_allclose(out, want, rtol=1e-11, atol=1e-12)


def test_variance_ratio_eq14_15():
    """Shared channels carry ~P times the variance of private ones; sqrt(P) scaling equalizes."""
    P, T, h, ffn = 4, 256, 128, 256
    x = _rand(P, T, h)
    W1 = _rand(P, ffn // P, h, std=0.1)
    W2 = _rand(P, h, ffn // P, std=0.1)
    gamma = np.ones(h, np.float32)
    resid = np.zeros((P, T, h), np.float32)
    n_s = 64
    for s, expect in ((1.0, P), (math.sqrt(P), 1.0)):
        _, out_resid = oracle.sublayer(x, W1, W2, gamma, resid=resid, act=oracle.GELU,
                                       norm=oracle.RMSNORM, n_s=n_s, s_priv=s)
        ratio = out_resid[:, :, :n_s].var() / out_resid[:, :, n_s:].var()
        assert ratio == pytest.approx(expect, rel=0.15)


def test_bruteforce_tiny():
    """Nested Python loops over lists (no numpy, no C) on a tiny case."""
    P, T, h, ffn, n_s, eps = 2, 2, 6, 8, 3, 1e-5
    fs = ffn // P
    x, W1, W2, gamma, beta = _mlp_case(P, T, h, ffn, oracle.SWIGLU, replicated=False)
    X, A, B, G, Bt = x.tolist(), W1.tolist(), W2.tolist(), gamma.tolist(), beta.tolist()
    zt = [[[0.0] * h for _ in range(T)] for _ in range(P)]
    for m in range(P):
        for t in range(T):
            y = []
            for k in range(fs):
                g = sum(X[m][t][j] * A[m][k][j] for j in range(h))
                u = sum(X[m][t][j] * A[m][fs + k][j] for j in range(h))
                y.append(g / (1 + math.exp(-g)) * u)
            for l in range(h):
                zt[m][t][l] = sum(y[k] * B[m][l][k] for k in range(fs))
    out, out_resid = oracle.sublayer(x, W1, W2, gamma, beta=beta, act=oracle.SWIGLU,
                                     norm=oracle.LAYERNORM, n_s=n_s, eps=eps)
    for m in range(P):
        for t in range(T):
            r = [X[m][t][l] + (sum(zt[q][t][l] for q in range(P)) if l < n_s else zt[m][t][l])
                 for l in range(h)]
            mu = sum(r) / h
            var = sum((v - mu) ** 2 for v in r) / h
            for l in range(h):
                assert out_resid[m][t][l] == pytest.approx(r[l], rel=1e-12, abs=1e-12)
                o = (r[l] - mu) / math.sqrt(var + eps) * G[l] + Bt[l]
                assert out[m][t][l] == pytest.approx(o, rel=1e-10, abs=1e-10)


def test_rejects_bad_arguments():
    x = _rand(2, 3, 8)
    W2 = _rand(2, 8, 4)
    with pytest.raises(ValueError):
        oracle.sublayer(x, _rand(2, 4, 8), W2, np.ones(8, np.float32), act=oracle.GELU,
                        norm=oracle.LAYERNORM, n_s=9)
    with pytest.raises(ValueError):
        oracle.partial_sync_norm(_rand(2, 3, 8), _rand(2, 3, 8), np.ones(8, np.float32), norm=7, n_s=2)
