"""Pins for the oracle's full-block pieces: the QKV projection, the causal attention core
and the block chain (App. A, Eq. 16-18, 24; §3.2 logical devices; §4 Eq. 9).

  - linear: numpy fp64 matmul (library routine).
  - attention: torch fp64 scaled_dot_product_attention with a causal mask (library
    routine), per sequence; exact special cases: the first token of a sequence returns
    its own value row; zero keys give uniform weights, so each output is the running
    mean of the values; sequences do not see each other.
  - block: at p = 1 with a replicated input the sharded block equals the unsharded
    transformer block (all heads, full out-projection, full MLP) computed with torch
    fp64 (§3: p = 1 is the all-reduce).
Everything here runs on the CPU.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(4242)


def _rand(*shape, std=1.0):
    return (RNG.standard_normal(shape) * std).astype(np.float32)


def test_linear_matches_matmul():
    x, W = _rand(3, 7, 24), _rand(3, 10, 24)
    want = np.einsum("mtk,mnk->mtn", x.astype(np.float64), W.astype(np.float64))
    assert np.max(np.abs(oracle.linear(x, W) - want)) <= 1e-12 * np.max(np.abs(want))


def _sdpa(qkv, S, nh, d):
    """torch fp64 causal attention per sequence, same layout as the oracle."""
    P, T, _ = qkv.shape
    t = torch.tensor(qkv, dtype=torch.float64)
    out = torch.empty((P, T, nh * d), dtype=torch.float64)
    for s0 in range(0, T, S):
        blk = t[:, s0:s0 + S]                                     # [P][S][3 nh d]
        q, k, v = (blk[..., i * nh * d:(i + 1) * nh * d].reshape(P, S, nh, d).transpose(1, 2)
                   for i in range(3))
        o = F.scaled_dot_product_attention(q.contiguous(), k.contiguous(), v.contiguous(),
                                           is_causal=True)
        out[:, s0:s0 + S] = o.transpose(1, 2).reshape(P, S, nh * d)
    return out.numpy()


@pytest.mark.parametrize("P,S,nseq,nh,d", [(2, 9, 2, 3, 8), (1, 33, 1, 1, 16), (3, 5, 3, 2, 4)])
def test_attention_matches_torch_sdpa(P, S, nseq, nh, d):
    qkv = _rand(P, S * nseq, 3 * nh * d)
    got = oracle.attention(qkv, S=S, nh=nh, d=d)
    want = _sdpa(qkv, S, nh, d)
    assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


def test_attention_exact_cases():
    P, S, nseq, nh, d = 2, 6, 2, 2, 4
    qkv = _rand(P, S * nseq, 3 * nh * d)
    H = oracle.attention(qkv, S=S, nh=nh, d=d)
    v = qkv[..., 2 * nh * d:].astype(np.float64)
    for s0 in range(0, S * nseq, S):            # first token: only itself to attend to
        assert np.array_equal(H[:, s0], v[:, s0])
    z = qkv.copy()
    z[..., nh * d:2 * nh * d] = 0.0             # zero keys: uniform weights
    Hz = oracle.attention(z, S=S, nh=nh, d=d)
    vz = z[..., 2 * nh * d:].astype(np.float64)
    for s0 in range(0, S * nseq, S):
        run = np.cumsum(vz[:, s0:s0 + S], axis=1) / np.arange(1, S + 1)[None, :, None]
        assert np.max(np.abs(Hz[:, s0:s0 + S] - run)) <= 1e-12
    w = qkv.copy()
    w[:, :S, nh * d:] += 5.0                   # change sequence 0's keys and values
    Hw = oracle.attention(w, S=S, nh=nh, d=d)
    assert np.array_equal(Hw[:, S:], H[:, S:])  # sequence 1 is untouched


@pytest.mark.parametrize("act,norm", [(oracle.SWIGLU, oracle.RMSNORM), (oracle.GELU, oracle.LAYERNORM)])
def test_block_p1_equals_unsharded_block(act, norm):
    P, nh, d, S, nseq = 2, 2, 8, 7, 2
    h = P * nh * d
    T = S * nseq
    ffn = 2 * 24
    fs = ffn // P
    F1 = 2 * fs if act == oracle.SWIGLU else fs
    x = np.broadcast_to(_rand(T, h), (P, T, h)).copy()
    r = np.broadcast_to(_rand(T, h), (P, T, h)).copy()
    Wqkv, Wo = _rand(P, 3 * nh * d, h, std=0.3), _rand(P, h, nh * d, std=0.3)
    W1, W2 = _rand(P, F1, h, std=0.3), _rand(P, h, fs, std=0.3)
    ga, gm = (1 + _rand(h, std=0.1)).astype(np.float32), (1 + _rand(h, std=0.1)).astype(np.float32)
    ba, bm = _rand(h, std=0.1), _rand(h, std=0.1)
    out, res = oracle.block_forward(x, r, Wqkv, Wo, W1, W2, ga, gm, S=S, nh=nh, d=d, act=act,
                                    norm=norm, n_s=h, beta_a=ba, beta_m=bm)
    t64 = lambda a: torch.tensor(np.asarray(a, np.float64))
    X, R = t64(x[0]), t64(r[0])
    # unsharded weights: head columns of every rank side by side
    q = torch.cat([X @ t64(Wqkv[m][:nh * d]).T for m in range(P)], 1)
    k = torch.cat([X @ t64(Wqkv[m][nh * d:2 * nh * d]).T for m in range(P)], 1)
    v = torch.cat([X @ t64(Wqkv[m][2 * nh * d:]).T for m in range(P)], 1)
    qkv_full = torch.cat([q, k, v], 1)[None].numpy().astype(np.float32)
    Hf = torch.tensor(_sdpa(qkv_full, S, P * nh, d)[0])
    O = torch.cat([t64(Wo[m]).T for m in range(P)], 0)               # [h][h]
    norm_t = (lambda z, g, b: F.layer_norm(z, (h,), t64(g), t64(b), 1e-5)) if norm == oracle.LAYERNORM \
        else (lambda z, g, b: F.rms_norm(z, (h,), t64(g), 1e-5))
    ra = R + Hf @ O
    a = norm_t(ra, ga, ba)
    if act == oracle.SWIGLU:
        G = torch.cat([t64(W1[m][:fs]).T for m in range(P)], 1)
        U = torch.cat([t64(W1[m][fs:]).T for m in range(P)], 1)
        y = F.silu(a @ G) * (a @ U)
    else:
        A = torch.cat([t64(W1[m]).T for m in range(P)], 1)
        y = F.gelu(a @ A)
    B = torch.cat([t64(W2[m]).T for m in range(P)], 0)
    rm = ra + y @ B
    om = norm_t(rm, gm, bm)
    for m in range(P):
        # the attention output passes through float32 between the oracle's sublayers
        assert np.max(np.abs(res[m] - rm.numpy())) <= 1e-5 * np.max(np.abs(rm.numpy()))
        assert np.max(np.abs(out[m] - om.numpy())) <= 1e-5 * np.max(np.abs(om.numpy()))
