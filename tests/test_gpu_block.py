"""GPU parity of the full block with logical devices: the attention core and the chained
block (QKV projection, attention, out-projection sublayer, MLP sublayer) against the
fp64 oracle on the same seeded inputs.

"Tensor-Parallelism with Partially Synchronized Activations", App. A.1 Eq. 16 / 18,
App. A.2 Eq. 22 / 24, §3.2 (logical devices), §4 Eq. 9.  Bar per output tensor:
max |gpu - oracle| / max |oracle| <= 2e-2 (bf16 storage).
"""
import numpy as np
import pytest
import torch

import oracle
import partial_activation_sync_amd as caat
from partial_activation_sync_amd import synth
from tests.oracle_ref import ACT, NORM, TOL, rel_err

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("P,S,nseq,nh,d", [
    (2, 200, 2, 3, 64),     # ragged query block (72) and key block (8)
    (4, 136, 2, 2, 64),
    (1, 8, 3, 1, 128),      # sequences shorter than a key block
    (8, 256, 1, 4, 128),
    (8, 1024, 2, 4, 128),   # the 7B head layout, two sequences
    (3, 4096, 1, 1, 128),   # a long sequence
])
def test_attention_matches_oracle(P, S, nseq, nh, d):
    T = S * nseq
    _say(f"[case] attention P={P} S={S} nseq={nseq} nh={nh} d={d}")
    qkv = synth.normal((P, T, 3 * nh * d), synth.QKV, dtype=BF16)
    H = torch.full((P, T, nh * d), float("nan"), dtype=BF16, device="cuda")
    ws = torch.empty(caat.caat_attention_workspace_bytes(P, T, nh, d), dtype=torch.uint8,
                     device="cuda")
    caat.caat_attention(P, T, S, nh, d, qkv.cuda(), H, ws)
    torch.cuda.synchronize()
    ref = oracle.attention(qkv.float(), S=S, nh=nh, d=d)
    err = rel_err(H, ref)
    _say(f"   error {err:.2e}")
    assert torch.isfinite(H.float()).all()
    assert err <= TOL["bf16"]


def test_attention_first_token_returns_its_value_row():
    """A sequence's first token attends only to itself: H = v exactly (bf16 in, bf16 out)."""
    P, S, nseq, nh, d = 2, 64, 3, 2, 128
    T = S * nseq
    qkv = synth.normal((P, T, 3 * nh * d), synth.QKV, dtype=BF16).cuda()
    H = torch.empty((P, T, nh * d), dtype=BF16, device="cuda")
    ws = torch.empty(caat.caat_attention_workspace_bytes(P, T, nh, d), dtype=torch.uint8,
                     device="cuda")
    caat.caat_attention(P, T, S, nh, d, qkv, H, ws)
    torch.cuda.synchronize()
    for s0 in range(0, T, S):
        assert torch.equal(H[:, s0], qkv[:, s0, 2 * nh * d:])


def _block_weights(P, h, ffn, nh, act, layer):
    hp = h // P
    fs = ffn // P
    F1 = 2 * fs if act == "swiglu" else fs
    seed = synth.BASE_SEED + 1000 * layer
    n = lambda shape, tid, **kw: synth.normal(shape, tid, dtype=BF16, seed=seed, **kw)
    return {
        "Wqkv": n((P, 3 * hp, h), synth.WQKV, std=0.02),
        "Wo": n((P, h, hp), synth.WO, std=0.02),
        "W1": n((P, F1, h), synth.W1, std=0.02),
        "W2": n((P, h, fs), synth.W2, std=0.02),
        "ga": n((h,), synth.GAMMA, std=0.1, mean=1.0),
        "gm": n((h,), synth.GAMMA + 100, std=0.1, mean=1.0),
        "ba": n((h,), synth.BETA, std=0.1),
        "bm": n((h,), synth.BETA + 100, std=0.1),
    }


def _run_blocks(P, h, ffn, nh, S, nseq, act, norm, p, layers):
    T = S * nseq
    _say(f"[case] block P={P} h={h} ffn={ffn} nh={nh} S={S} nseq={nseq} {act} {norm} p={p} "
         f"layers={layers}")
    blk = caat.Block(h, ffn, P, p, nh, norm=norm, act=act)
    x = synth.normal((P, T, h), synth.X, dtype=BF16)
    r = synth.normal((P, T, h), synth.X0, dtype=BF16)
    xg, rg = x.cuda(), r.cuda()
    ref_x, ref_r = x.float().numpy(), r.float().numpy()
    d = h // P // nh
    n_s = oracle.shared_channels(h, p)
    errs = []
    for layer in range(layers):
        w = _block_weights(P, h, ffn, nh, act, layer)
        wg = {k: v.cuda() for k, v in w.items()}
        out = torch.empty((P, T, h), dtype=BF16, device="cuda")
        out_r = torch.empty_like(out)
        blk.forward(T, S, xg, rg, wg["Wqkv"], wg["Wo"], wg["W1"], wg["W2"], wg["ga"], wg["gm"],
                    out, out_r, beta_attn=wg["ba"], beta_mlp=wg["bm"])
        torch.cuda.synchronize()
        f = lambda t: t.float().numpy()
        ref_x, ref_r = oracle.block_forward(
            ref_x, ref_r, f(w["Wqkv"]), f(w["Wo"]), f(w["W1"]), f(w["W2"]), f(w["ga"]),
            f(w["gm"]), S=S, nh=nh, d=d, act=ACT[act], norm=NORM[norm], n_s=n_s,
            beta_a=f(w["ba"]), beta_m=f(w["bm"]))
        e = (rel_err(out, ref_x), rel_err(out_r, ref_r))
        _say(f"   layer {layer}: out {e[0]:.2e} out_resid {e[1]:.2e}")
        errs.append(e)
        xg, rg = out, out_r
    for e in errs:
        assert max(e) <= TOL["bf16"], errs
    return xg, rg


def test_block_two_layers_diverging_ranks():
    """Two chained blocks at p = 0.5: the ranks' inputs differ after the first block."""
    out, _ = _run_blocks(4, 512, 4 * 264, 2, 136, 2, "swiglu", "rmsnorm", 0.5, layers=2)
    assert not torch.equal(out[0], out[1])


def test_block_gelu_layernorm():
    _run_blocks(4, 768, 3072, 3, 128, 2, "gelu", "layernorm", 0.5, layers=1)


def test_block_7b_dims():
    _run_blocks(8, 4096, 11008, 4, 64, 2, "swiglu", "rmsnorm", 0.5, layers=1)
