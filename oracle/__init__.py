"""Oracle for the CAAT partial-sync sublayer forward and backward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library and its
Python binding never import it, and the two share no code.

The arithmetic lives in ``caat_oracle.c`` (plain C, fp64, OpenMP over rank and
token rows); this module only converts arrays and calls it.  Source of the method:
"Tensor-Parallelism with Partially Synchronized Activations", App. A.2 Eq. 22 and 24,
§3.2 (logical devices), §4 Eq. 9 and "Private channel scaling"; the backward follows
§4 "Forward-backward mismatch" (Eq. 10-13) and App. B (Eq. 26-30).

Parity status: every function here is pinned by ``tests/test_oracle_pins.py`` and
``tests/test_oracle_backward_pins.py`` against closed forms, library routines on
special cases, the page's P = 2 block form (Eq. 8 / Eq. 19), a hand-derived worked
example, brute force on tiny shapes and (backward) central finite differences of
the forward.
The bf16 roundings of the GPU path (intermediate activations, partials, outputs)
are not modelled: the page fixes none of them, and the tolerance absorbs them.
"""
import ctypes
import os

import numpy as np

from . import build as _build

GELU, GELU_TANH, SWIGLU, NONE = 0, 1, 2, 3
LAYERNORM, RMSNORM = 0, 1

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        fp = ctypes.POINTER(ctypes.c_float)
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_shared_channels.argtypes = [ctypes.c_int, ctypes.c_double]
        lib.oracle_shared_channels.restype = ctypes.c_int
        lib.oracle_activation.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double]
        lib.oracle_activation.restype = ctypes.c_double
        lib.oracle_sublayer.argtypes = (
            [ctypes.c_int] * 7 + [ctypes.c_double, ctypes.c_double]
            + [fp] * 6 + [dp] * 3)
        lib.oracle_sublayer.restype = ctypes.c_int
        lib.oracle_partial_sync_norm.argtypes = (
            [ctypes.c_int] * 5 + [ctypes.c_double, ctypes.c_double]
            + [fp] * 4 + [dp] * 2)
        lib.oracle_partial_sync_norm.restype = ctypes.c_int
        lib.oracle_sublayer_backward.argtypes = (
            [ctypes.c_int] * 7 + [ctypes.c_double, ctypes.c_double]
            + [fp] * 7 + [dp] * 6)
        lib.oracle_sublayer_backward.restype = ctypes.c_int
        lib.oracle_linear.argtypes = [ctypes.c_int] * 4 + [fp] * 2 + [dp]
        lib.oracle_linear.restype = ctypes.c_int
        lib.oracle_attention.argtypes = [ctypes.c_int] * 5 + [fp] + [dp]
        lib.oracle_attention.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor: widen exactly to float32 on the CPU
        a = a.detach().to("cpu").float().numpy()
    return np.ascontiguousarray(a, dtype=np.float32)


def _fptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_float)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _dptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def threads() -> int:
    """OpenMP threads the oracle runs on."""
    return _load().oracle_threads()


def shared_channels(h: int, p: float) -> int:
    """n_s = floor(h p) (App. A.2, Eq. 22), near-integers counted as integers."""
    return _load().oracle_shared_channels(int(h), float(p))


def activation(act: int, g: float, u: float = 0.0) -> float:
    """The nonlinearity sigma of Eq. 20-22 on one value (SwiGLU: silu(g) * u)."""
    return _load().oracle_activation(int(act), float(g), float(u))


def sublayer(x, W1, W2, gamma, *, act, norm, n_s, ffn=0, beta=None, resid=None,
             s_priv=1.0, eps=1e-5, want_partials=False):
    """Forward of one CAAT sublayer for every rank, in fp64.

    x [P][T][kin]; W1 [P][F1][h] (ignored for act=NONE); W2 [P][h][k2];
    gamma, beta [h]; resid [P][T][h] or None (= x).  Returns (out, out_resid) or
    (out, out_resid, partials), float64 arrays of shape [P][T][h].
    """
    x = _f32(x)
    W2 = _f32(W2)
    P, T, kin = x.shape
    h = W2.shape[1]
    if act == NONE:
        W1 = None
        ffn = 0
    else:
        W1 = _f32(W1)
        fs = W2.shape[2]
        ffn = fs * P
    gamma = _f32(gamma)
    beta = _f32(beta)
    resid = _f32(resid)
    out = np.empty((P, T, h), np.float64)
    out_resid = np.empty((P, T, h), np.float64)
    zt = np.empty((P, T, h), np.float64) if want_partials else None
    rc = _load().oracle_sublayer(P, T, h, ffn, act, norm, n_s, float(s_priv), float(eps),
                                 _fptr(x), _fptr(resid), _fptr(W1), _fptr(W2),
                                 _fptr(gamma), _fptr(beta),
                                 _dptr(zt), _dptr(out), _dptr(out_resid))
    if rc != 0:
        raise ValueError("oracle_sublayer rejected its arguments")
    if want_partials:
        return out, out_resid, zt
    return out, out_resid


def partial_sync_norm(partials, resid, gamma, *, norm, n_s, beta=None, s_priv=1.0, eps=1e-5):
    """Partial channel-reduce + residual + norm on given partials [P][T][h], fp64."""
    partials = _f32(partials)
    resid = _f32(resid)
    gamma = _f32(gamma)
    beta = _f32(beta)
    P, T, h = partials.shape
    out = np.empty((P, T, h), np.float64)
    out_resid = np.empty((P, T, h), np.float64)
    rc = _load().oracle_partial_sync_norm(P, T, h, norm, n_s, float(s_priv), float(eps),
                                          _fptr(partials), _fptr(resid), _fptr(gamma),
                                          _fptr(beta), _dptr(out), _dptr(out_resid))
    if rc != 0:
        raise ValueError("oracle_partial_sync_norm rejected its arguments")
    return out, out_resid


def sublayer_backward(x, W1, W2, gamma, dout, *, act, norm, n_s, resid=None, dres=None,
                      s_priv=1.0, eps=1e-5):
    """Backward of one CAAT sublayer for every rank, in fp64 (§4, App. B).

    Forward inputs as for ``sublayer``; dout [P][T][h] is the gradient of the loss
    w.r.t. out and dres [P][T][h] (None: zero) w.r.t. out_resid.  Returns a dict of
    float64 arrays: dx [P][T][kin] (with resid=None the residual gradient is included),
    dresid [P][T][h], dW1 [P][F1][h] (None for act=NONE), dW2 [P][h][k2], dgamma [h],
    dbeta [h] (zero for RMSNorm).
    """
    x = _f32(x)
    W2 = _f32(W2)
    P, T, kin = x.shape
    h, k2 = W2.shape[1], W2.shape[2]
    if act == NONE:
        W1 = None
        ffn, F1 = 0, 0
    else:
        W1 = _f32(W1)
        ffn = k2 * P
        F1 = W1.shape[1]
    gamma, resid, dout, dres = _f32(gamma), _f32(resid), _f32(dout), _f32(dres)
    res = {
        "dx": np.empty((P, T, kin), np.float64),
        "dresid": np.empty((P, T, h), np.float64),
        "dW1": np.empty((P, F1, h), np.float64) if act != NONE else None,
        "dW2": np.empty((P, h, k2), np.float64),
        "dgamma": np.empty((h,), np.float64),
        "dbeta": np.empty((h,), np.float64),
    }
    rc = _load().oracle_sublayer_backward(
        P, T, h, ffn, act, norm, n_s, float(s_priv), float(eps),
        _fptr(x), _fptr(resid), _fptr(W1), _fptr(W2), _fptr(gamma), _fptr(dout), _fptr(dres),
        _dptr(res["dx"]), _dptr(res["dresid"]), _dptr(res["dW1"]), _dptr(res["dW2"]),
        _dptr(res["dgamma"]), _dptr(res["dbeta"]))
    if rc != 0:
        raise ValueError("oracle_sublayer_backward rejected its arguments")
    return res


def linear(x, W):
    """Per-rank linear layer, fp64: out[m][t][n] = sum_k x[m][t][k] W[m][n][k]."""
    x, W = _f32(x), _f32(W)
    P, T, K = x.shape
    N = W.shape[1]
    out = np.empty((P, T, N), np.float64)
    if _load().oracle_linear(P, T, K, N, _fptr(x), _fptr(W), _dptr(out)) != 0:
        raise ValueError("oracle_linear rejected its arguments")
    return out


def attention(qkv, *, S, nh, d):
    """Causal self-attention of every head of every rank (App. A, Eq. 16 / 18 / 24), fp64.

    qkv [P][T][3 nh d] (Q, K, V of the rank's heads); T = nseq * S tokens, causal within
    each sequence of S.  Returns H [P][T][nh d]."""
    qkv = _f32(qkv)
    P, T, _ = qkv.shape
    H = np.empty((P, T, nh * d), np.float64)
    if _load().oracle_attention(P, T, S, nh, d, _fptr(qkv), _dptr(H)) != 0:
        raise ValueError("oracle_attention rejected its arguments")
    return H


def block_forward(h_in, r_in, Wqkv, Wo, W1, W2, gamma_a, gamma_m, *, S, nh, d, act, norm, n_s,
                  beta_a=None, beta_m=None, s_priv=1.0, eps=1e-5):
    """One transformer block with partially synchronized activations, every rank on one
    device (§3.2): per rank, QKV projection of the block input h_in, causal attention,
    then the out-projection sublayer (residual r_in) and the MLP sublayer (Eq. 22 / 24,
    Eq. 9).  Returns (out, out_resid) of the MLP sublayer: the next block's (h_in, r_in)."""
    qkv = linear(h_in, Wqkv)
    H = attention(qkv, S=S, nh=nh, d=d)
    a_out, a_res = sublayer(H, None, Wo, gamma_a, act=NONE, norm=norm, n_s=n_s, beta=beta_a,
                            resid=r_in, s_priv=s_priv, eps=eps)
    return sublayer(a_out, W1, W2, gamma_m, act=act, norm=norm, n_s=n_s, beta=beta_m,
                    resid=a_res, s_priv=s_priv, eps=eps)
