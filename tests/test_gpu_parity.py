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
# (one or two weight blocks per wave, 1 to 4 token blocks, ragged last block), and the
# 64-token MFMA tiles that take over the plain long contractions past 8 tokens (K2:
# T = 9, 16), the SwiGLU GEMM past 16 (T = 17, 33, 40) and every GEMM past 48 (T = 49,
# 56: the out-projection too); ragged tiles throughout.
@pytest.mark.parametrize("T", [5, 8, 9, 16, 17, 33, 40, 49, 56])
def test_7b_decode_launch_shapes(T):
    _run_and_compare(W.DECODE_7B_BF16, T=T, norm_params="random")


def test_decode_mfma_tiles_more_than_cus():
    """Wider layers than 7B at T = 56: 272 SwiGLU tiles of 64 tokens in K1 and 320 in K2,
    more than the 256 CUs, so both take the two-stage form of the 64-token tiles."""
    w = W.with_(W.DECODE_7B_BF16, h=5120, ffn=8 * 2176, heads=40)
    _run_and_compare(w, T=56, norm_params="random")


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
@pytest.mark.parametrize("P,h,ffn,T", [(1, 8, 8, 1), (16, 128, 16 * 8, 5), (16, 256, 16 * 16, 100),
                                       (3, 264, 3 * 40, 67),
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


@pytest.mark.parametrize("P,h,ffn,T,act", [(2, 200, 2 * 136, 45, "gelu"),
                                            (4, 264, 4 * 264, 300, "swiglu"),
                                            (4, 264, 4 * 264, 300, "gelu"),
                                            (8, 520, 8 * 520, 300, "gelu_tanh"),
                                            (8, 520, 8 * 520, 300, "gelu"),
                                            (8, 520, 8 * 520, 300, "swiglu")])
def test_f32_gemm_tile_sizes(P, h, ffn, T, act):
    """The fp32 GEMM's three tile shapes through the whole sublayer: 16 x 16 (fewer than 256
    tiles of 32 x 32), 32 x 32 and 64 x 64 (at least 256 tiles of that size), with the
    activation epilogues, each with a ragged token tile and a contraction that is not a
    multiple of the 16-wide K step."""
    f_s = ffn // P
    tiles = lambda tb, n: P * -(-n // tb) * -(-T // tb)
    want = {0: 16, 1: 32, 2: 64}[[(2, 200), (4, 264), (8, 520)].index((P, h))]
    got = [64 if tiles(64, n) >= 256 else 32 if tiles(32, n) >= 256 else 16 for n in (f_s, h)]
    assert got == [want, want], got
    w = W.with_(W.TINY_MLP_F32, P=P, h=h, ffn=ffn, T=T, p=0.41, act=act, norm="rmsnorm",
                replicated_x=False)
    _run_and_compare(w, norm_params="random", s_priv=math.sqrt(P))


def test_per_rank_private_rows_on_small_tiles():
    """The per-rank row GEMM writing the private chunks into out_resid (P T h >= 2^25, n_s
    not a multiple of 8) on a shape where the 128 x 128 tiles finish first: 784 tiles of
    256 x 256 take 4 rounds, 2716 of 128 x 128 six half-efficiency ones (P = 4, h = 12320,
    T = 769, a 64-wide FFN shard), against the oracle on sampled rows."""
    T, h, p = 769, 12320, 0.301
    w = W.with_(W.PAIR_130M_BF16, sublayers=("mlp",), P=4, h=h, ffn=4 * 64, T=T, p=p,
                act="gelu", norm="rmsnorm", replicated_x=False)
    hd = caat.Sublayer(h, 4 * 64, 4, p, act="gelu", dtype="bf16")
    assert hd.n_s % 8 != 0 and not caat.caat_forward_fused(hd.handle, T)
    assert caat.caat_forward_private_in_epilogue(hd.handle, T)
    _run_and_compare(w, norm_params="random", rows=synth.sample_rows(T, 48))


@pytest.mark.parametrize("act", ["gelu", "gelu_tanh"])
def test_gelu_mlp_large_tiles(act):
    """A GeLU MLP large enough for the 256 x 256 tiles (K1 with the erf or tanh GeLU
    epilogue; 512 tiles of 256 x 256 over K = 1024), against the oracle on sampled rows."""
    T = 4096
    w = W.with_(W.PAIR_130M_BF16, sublayers=("mlp",), P=8, h=1024, ffn=8 * 1024, T=T, p=0.45,
                act=act, norm="layernorm", replicated_x=False)
    _run_and_compare(w, norm_params="random", rows=synth.sample_rows(T, 48))


@pytest.mark.parametrize("act", ["gelu", "gelu_tanh"])
@pytest.mark.parametrize("T", [5, 12, 24, 40])
def test_gelu_decode_short_contraction(act, T):
    """GeLU MLPs at decode batch sizes with a contraction under 1024 (the 130M widths): the
    weight-streaming kernel up to 48 tokens, with one, two and three 16-token blocks."""
    _run_and_compare(W.with_(W.PAIR_130M_BF16, sublayers=("mlp",), T=T, act=act),
                     norm_params="random")


@pytest.mark.parametrize("act", ["gelu", "gelu_tanh"])
@pytest.mark.parametrize("P,ffn,T", [(4, 4 * 512, 1), (4, 4 * 512, 8), (4, 4 * 512, 12),
                                     (4, 4 * 512, 40), (4, 4 * 512, 64), (8, 8 * 4224, 33)])
def test_gelu_decode_batches(act, P, ffn, T):
    """GeLU MLPs at decode batch sizes with h >= 1024: the weight-streaming kernel with the
    contraction split over four waves (T <= 8) and the 64-token MFMA tiles with the GeLU
    epilogue past that, in their four-stage (few tiles) and two-stage (more tiles than CUs)
    forms."""
    w = W.with_(W.PAIR_130M_BF16, sublayers=("mlp",), P=P, h=1024, ffn=ffn, T=T, p=0.5,
                act=act, norm="rmsnorm", replicated_x=False)
    _run_and_compare(w, norm_params="random")


@pytest.mark.parametrize("act,dtype,P,h,fs,T,p", [
    ("swiglu", "bf16", 4, 1024, 256, 8192, 0.5),     # fused, private rows from the GEMM epilogue
    ("swiglu", "bf16", 4, 1024, 256, 8192, 0.501),   # per-rank, private chunks from the epilogue
    ("gelu", "bf16", 4, 1024, 256, 300, 0.37),       # per-rank, stored partials
    ("none", "bf16", 8, 4096, 0, 5, 0.5),            # decode: per-rank K3 (one token, one rank)
    ("gelu", "f32", 16, 1024, 64, 100, 0.3),         # fp32, multi-pass K3
])
def test_residual_updated_in_place(act, dtype, P, h, fs, T, p):
    """out_resid may be the resid buffer itself (the residual stream updated in place): each
    element of r is read and then written by the same thread, in K3 and in the row GEMM's
    residual epilogue alike, so the outputs are bitwise those of separate buffers."""
    _say(f"[case] in-place residual {act} {dtype} P={P} h={h} T={T} p={p}")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kin = h // P if act == "none" else h
    F1 = 2 * fs if act == "swiglu" else fs
    x = synth.normal((P, T, kin), synth.X, dtype=dt).cuda()
    W1 = None if act == "none" else (synth.normal((P, F1, h), synth.W1, std=0.02, dtype=dt).cuda())
    W2 = synth.normal((P, h, fs if act != "none" else kin), synth.W2, std=0.02, dtype=dt).cuda()
    R = synth.normal((P, T, h), synth.X0, dtype=dt).cuda()
    gamma = synth.normal((h,), synth.GAMMA, std=0.1, mean=1.0, dtype=dt).cuda()
    s = caat.Sublayer(h, P * fs, P, p, norm="rmsnorm", act=act, dtype=dtype, s_priv=1.5)
    out1 = torch.empty_like(R)
    res1 = torch.empty_like(R)
    s.forward(x, W1, W2, gamma, out1, resid=R, out_resid=res1)
    R2 = R.clone()
    out2 = torch.empty_like(R)
    s.forward(x, W1, W2, gamma, out2, resid=R2, out_resid=R2)
    R3 = R.clone()
    res3 = torch.empty_like(R)
    s.forward(x, W1, W2, gamma, R3, resid=R3, out_resid=res3)
    torch.cuda.synchronize()
    assert torch.equal(R2, res1) and torch.equal(out2, out1)
    assert torch.equal(R3, out1) and torch.equal(res3, res1)


def _random_cases(n=32, seed=20251203):
    """Seeded random sublayer configurations (drawn once, so the test ids are stable): MLP
    or out-projection + MLP pair, fp32 or bf16, every activation and norm, P 1..8, widths
    that keep every contraction and output a multiple of 8, T from decode batches to a few
    token tiles, any p, with or without the private scaling.  Sized so that the oracle
    finishes each in about a second."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        pair = bool(rng.integers(2))
        dtype = ("bf16", "f32")[int(rng.integers(2))]
        P = int(rng.choice([1, 2, 3, 4, 6, 8]))
        h = 8 * P * int(rng.integers(1, 1024 // (8 * P) + 1)) if pair else 8 * int(rng.integers(4, 129))
        fs = 8 * int(rng.integers(2, 193))
        T = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, 300))]))
        act = ("gelu", "gelu_tanh", "swiglu")[int(rng.integers(3))]
        norm = ("layernorm", "rmsnorm")[int(rng.integers(2))]
        pv = round(float(rng.random()), 3)
        scaled = bool(rng.integers(2))
        F1 = 2 * fs if act == "swiglu" else fs
        if P * T * h * (F1 + h) > 4e8:
            continue
        out.append((pair, dtype, P, h, P * fs, T, act, norm, pv, scaled))
    return out


@pytest.mark.parametrize("pair,dtype,P,h,ffn,T,act,norm,p,scaled", _random_cases())
def test_random_sublayer_configs(pair, dtype, P, h, ffn, T, act, norm, p, scaled):
    """Seeded random configurations through the product path against the oracle (random
    gamma and beta; s_priv = sqrt(P) when scaled)."""
    base = W.PAIR_130M_BF16 if pair else W.TINY_MLP_F32
    w = W.with_(base, name=f"random-{'pair' if pair else 'mlp'}", dtype=dtype, P=P, h=h,
                ffn=ffn, T=T, p=p, act=act, norm=norm, replicated_x=False)
    _run_and_compare(w, s_priv=math.sqrt(P) if scaled else 1.0, norm_params="random")


def _random_fused_cases(n=8, seed=20251204):
    """Seeded random bf16 MLP and pair configurations large enough for the fused path with
    the private rows written by the private GEMM's epilogue (n_s % 8 == 0 and at least 256
    shared-GEMM tiles of 128 x 128), T ragged against the tiles; the oracle runs on 48
    sampled token rows."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        pair = bool(rng.integers(2))
        P = int(rng.choice([2, 4, 8]))
        h = int(rng.choice([1024, 2048, 4096]))
        n_s = 8 * int(rng.integers(1, h // 8))
        T = 128 * int(rng.integers(8, 40)) + int(rng.integers(0, 128))
        if -(-n_s // 128) * -(-T // 128) < 256 or P * T * h > 2 ** 27:
            continue
        fs = 8 * int(rng.integers(8, 129))
        act = ("gelu", "gelu_tanh", "swiglu")[int(rng.integers(3))]
        norm = ("layernorm", "rmsnorm")[int(rng.integers(2))]
        scaled = bool(rng.integers(2))
        out.append((pair, P, h, P * fs, T, n_s / h, act, norm, scaled))
    return out


@pytest.mark.parametrize("pair,P,h,ffn,T,p,act,norm,scaled", _random_fused_cases())
def test_random_fused_configs(pair, P, h, ffn, T, p, act, norm, scaled):
    """The fused path with the epilogue's private rows on seeded random shapes, against the
    oracle on sampled rows (random gamma and beta; s_priv = sqrt(P) when scaled)."""
    base = W.PAIR_130M_BF16 if pair else W.TINY_MLP_F32
    w = W.with_(base, name=f"random-fused-{'pair' if pair else 'mlp'}", dtype="bf16", P=P, h=h,
                ffn=ffn, T=T, p=p, act=act, norm=norm, replicated_x=False)
    hd = caat.Sublayer(h, ffn, P, p, act="none" if pair else act, dtype="bf16")
    assert caat.caat_forward_private_in_epilogue(hd.handle, T)
    if pair:
        hm = caat.Sublayer(h, ffn, P, p, act=act, dtype="bf16")
        assert caat.caat_forward_private_in_epilogue(hm.handle, T)
    _run_and_compare(w, s_priv=math.sqrt(P) if scaled else 1.0, norm_params="random",
                     rows=synth.sample_rows(T, 48))


# ---------------------------------------------------------------------------
# The channel mask, bit-exact; cross-rank identity at p = 1; determinism
# ---------------------------------------------------------------------------
def _code(dtype, P, m):
    """Integer code of rank m's partials: 2^m, whose sum over the ranks, 2^P - 1, is exact
    in the storage dtype for P <= 8 (bf16) or P <= 16 (fp32); for bf16 with P > 8, m + 1
    (sum P (P + 1) / 2 <= 136, exact)."""
    return float(m + 1) if (dtype == "bf16" and P > 8) else 2.0 ** m


def _coded_out_resid(dtype, P, T, h, n_s, s_priv, shared=None):
    """out_resid for integer-coded partials and a zero residual: the sum of the codes on
    the shared channels (or `shared`, when S is given), code(m) * s_priv on the private
    ones (Eq. 22 / 24: l < floor(h p) reduced, §4 private scaling)."""
    want = torch.empty((P, T, h), dtype=torch.float64)
    tot = sum(_code(dtype, P, m) for m in range(P))
    for m in range(P):
        want[m, :, :n_s] = tot if shared is None else shared
        want[m, :, n_s:] = _code(dtype, P, m) * s_priv
    return want


MASK_KERNEL_CASES = [(dt, P, h, T) for dt in ("bf16", "f32") for P in (1, 2, 4, 8)
                     for h in (256, 4096) for T in (3, 100, 1100)
                     if not (h == 4096 and T == 1100 and P < 8)]
# The multi-pass K3 (rows too wide for one register pass): fp32 with P = 16, bf16 with
# P = 16 at h = 8192, at T > 64 (and the per-rank kernel at T <= 64).
MASK_KERNEL_CASES += [("f32", 16, 4096, 100), ("bf16", 16, 8192, 100), ("bf16", 16, 8192, 3),
                      ("f32", 16, 4096, 3)]
# bf16 with 9-16 ranks and rows that fit one register pass: the single-pass K3 with its
# 16-rank register layout (cached and nontemporal forms).
MASK_KERNEL_CASES += [("bf16", 16, 4096, 100), ("bf16", 12, 2048, 100), ("bf16", 16, 4096, 1100)]
# Rows wider than 4096 in one register pass: two or four chunks per thread in the
# single-pass K3 (bf16 P = 8 / 2 / 1, fp32 P = 4 / 2 / 1); the multi-pass K3 with one chunk
# per thread (fp32 rows of 1024 or fewer with more than 8 ranks).
MASK_KERNEL_CASES += [("bf16", 8, 8192, 100), ("bf16", 2, 16384, 100), ("bf16", 1, 16384, 100),
                      ("f32", 4, 8192, 100), ("f32", 2, 16384, 100), ("f32", 1, 16384, 100),
                      ("f32", 16, 1024, 100), ("f32", 9, 256, 100)]


@pytest.mark.parametrize("dtype,P,h,T", MASK_KERNEL_CASES)
def test_mask_bit_exact(dtype, P, h, T):
    """Integer-coded partials Zt_m = code(m), resid = 0, through caat_partial_sync_norm:
    out_resid = the codes' sum on shared channels and code(m) * s_priv on private ones,
    exactly.  T <= 64: one workgroup per (token, rank); T > 64: one per token, with the
    nontemporal row loads past 256 MB per launch (h = 4096, T = 1100)."""
    _say(f"[case] mask K3 {dtype} P={P} h={h} T={T}")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for n_s in sorted({0, 1, 63, 64, 65, 179, h - 1, h}):
        p = n_s / h
        s = caat.Sublayer(h, 8 * P, P, p, norm="rmsnorm", act="gelu", dtype=dtype, s_priv=2.0)
        assert s.n_s == n_s
        Z = torch.stack([torch.full((T, h), _code(dtype, P, m), dtype=dt, device="cuda")
                         for m in range(P)])
        resid = torch.zeros((P, T, h), dtype=dt, device="cuda")
        gamma = torch.ones(h, dtype=dt, device="cuda")
        out = torch.empty_like(resid)
        out_resid = torch.empty_like(resid)
        caat.caat_partial_sync_norm(s.handle, T, Z, resid, gamma, None, out, out_resid)
        torch.cuda.synchronize()
        want = _coded_out_resid(dtype, P, T, h, n_s, 2.0)
        assert torch.equal(out_resid.double().cpu(), want), (P, h, T, n_s)


@pytest.mark.parametrize("dtype,P,h,T", [("bf16", 8, 4096, 3), ("bf16", 8, 4096, 200),
                                         ("bf16", 8, 4096, 1100), ("f32", 16, 4096, 100),
                                         ("bf16", 8, 16384, 100), ("f32", 4, 768, 65)])
def test_sync_norm_mask_bit_exact(dtype, P, h, T):
    """caat_sync_norm (shared channels from S, private ones from the partials) on integer
    codes: out_resid = S on [0, n_s) and code(m) * s_priv on [n_s, h), exactly."""
    _say(f"[case] mask sync_norm {dtype} P={P} h={h} T={T}")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for n_s in sorted({0, 8, 64, h // 2 - 8, h // 2, h // 2 + 8, h - 8, h}):
        s = caat.Sublayer(h, 8 * P, P, n_s / h, norm="layernorm", act="gelu", dtype=dtype,
                          s_priv=2.0)
        assert s.n_s == n_s
        S = torch.full((T, max(n_s, 8)), 100.0, dtype=dt, device="cuda")
        Z = torch.stack([torch.full((T, h), _code(dtype, P, m), dtype=dt, device="cuda")
                         for m in range(P)])
        Z[:, :, :n_s] = float("nan")          # the shared columns must not be read
        resid = torch.zeros((P, T, h), dtype=dt, device="cuda")
        gamma = torch.ones(h, dtype=dt, device="cuda")
        out = torch.empty_like(resid)
        out_resid = torch.empty_like(resid)
        caat.caat_sync_norm(s.handle, T, S if n_s else None, Z if n_s < h else None, resid,
                            gamma, None, out, out_resid)
        torch.cuda.synchronize()
        want = _coded_out_resid(dtype, P, T, h, n_s, 2.0, shared=100.0)
        assert torch.equal(out_resid.double().cpu(), want), (P, h, T, n_s)


@pytest.mark.parametrize("dtype,P,h,T", [("bf16", 8, 4096, 65), ("bf16", 8, 4096, 200),
                                         ("bf16", 4, 768, 300), ("f32", 16, 4096, 100),
                                         ("bf16", 8, 16384, 100)])
def test_row_gemm_reduce_mask_bit_exact(dtype, P, h, T):
    """The fused kernels called directly (caat_row_gemm_reduce, then caat_sync_norm) on
    integer-coded out-projection inputs, for every n_s % 8 == 0 case whatever path the
    forward would take: out_resid is the codes' sum on [0, n_s) and 2 code(m) after."""
    _say(f"[case] mask row_gemm_reduce {dtype} P={P} h={h} T={T}")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    hp = h // P
    H = torch.zeros((P, T, hp), dtype=dt, device="cuda")
    H[:, :, 0] = 1.0
    Wo = torch.full((P, h, hp), 1.5, dtype=dt, device="cuda")
    for m in range(P):
        Wo[m, :, 0] = _code(dtype, P, m)
    resid = torch.zeros((P, T, h), dtype=dt, device="cuda")
    gamma = torch.ones(h, dtype=dt, device="cuda")
    for n_s in sorted({0, 8, 64, h // 2 - 8, h // 2, h // 2 + 8, h - 8, h}):
        s = caat.Sublayer(h, 0, P, n_s / h, norm="rmsnorm", act="none", dtype=dtype, s_priv=2.0)
        assert s.n_s == n_s
        S = torch.full((T, max(n_s, 8)), float("nan"), dtype=dt, device="cuda")
        Z = torch.full((P, T, h), float("nan"), dtype=dt, device="cuda")
        caat.caat_row_gemm_reduce(s.handle, T, H, Wo, S if n_s else None, Z if n_s < h else None)
        out = torch.empty_like(resid)
        out_resid = torch.empty_like(resid)
        caat.caat_sync_norm(s.handle, T, S if n_s else None, Z if n_s < h else None, resid,
                            gamma, None, out, out_resid)
        torch.cuda.synchronize()
        want = _coded_out_resid(dtype, P, T, h, n_s, 2.0)
        assert torch.equal(out_resid.double().cpu(), want), (P, h, T, n_s)


def _forward_mask_cases():
    cases = []
    h = 4096
    # bf16, P = 8: the per-rank path with K3's reduce (n_s % 8 != 0, or too few shared-GEMM
    # tiles) at T > 64, and the decode kernels with the per-rank K3 at T = 3.
    for T in (3, 65, 200):
        for n_s in (0, 8, 64, 2040, 2048, 2056, h - 8, h, 1, 63, 65, 179, h - 1):
            cases.append(("bf16", 8, h, T, n_s))
    # The fused path (S from the K-concatenated GEMM: n_s % 8 == 0 and at least 256
    # shared-GEMM tiles), T = 2048 and a ragged T = 2000.
    for T in (2000, 2048):
        for n_s in (0, 1920, 2040, 2048, 2056, h - 8, h, 2047):
            cases.append(("bf16", 8, h, T, n_s))
    # The nontemporal K3 forms (more than 256 MB per launch); the per-rank row GEMM writing
    # the whole private chunks into out_resid (P T h >= 2^25), with a chunk across n_s.
    cases += [("bf16", 8, h, 1100, n_s) for n_s in (2048, 2047, 1, 65, 4089)]
    # Rows too wide for one register pass: the multi-pass K3.  Off the GPU for now: with
    # the private rows taken from the private GEMM's epilogue, the first of these cases
    # (n_s = 0) hit a memory access fault in the multi-pass K3 whose cause was not found.
    # The library no longer hands that kernel final private rows (these cases now run the
    # stored-partials path), but they stay skipped until the fault is understood.
    for n_s in (0, 8, 8192, 8191, 16383, 16384):
        cases.append(pytest.param("bf16", 8, 16384, 100, n_s, marks=pytest.mark.skip(
            reason="GPU memory fault under investigation (multi-pass K3 with final private rows)")))
    # fp32 with 16 ranks (the multi-pass K3; codes up to 2^15).
    for n_s in (0, 8, 2048, 2047, 4095, 4096):
        cases.append(("f32", 16, h, 100, n_s))
    # bf16 with 16 ranks (the single-pass K3 for up to 16 ranks; codes m + 1).
    for n_s in (0, 8, 2048, 2047, 4095, 4096):
        cases.append(("bf16", 16, h, 100, n_s))
    return cases


@pytest.mark.parametrize("dtype,P,h,T,n_s", _forward_mask_cases())
def test_forward_mask_bit_exact(dtype, P, h, T, n_s):
    """The whole out-projection sublayer through caat_forward_ex on integer codes: the
    head outputs H_m have a 1 in column 0 and zeros elsewhere, and column 0 of O_m is
    code(m), so every partial is exactly code(m) (the other weight columns meet zeros).
    With resid = 0 and s_priv = 2, out_resid must be the codes' sum on [0, n_s) and
    2 code(m) on [n_s, h), bit for bit, on whichever path the library takes."""
    _say(f"[case] mask forward {dtype} P={P} h={h} T={T} n_s={n_s}")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    hp = h // P
    s = caat.Sublayer(h, 0, P, n_s / h, norm="rmsnorm", act="none", dtype=dtype, s_priv=2.0)
    assert s.n_s == n_s
    H = torch.zeros((P, T, hp), dtype=dt, device="cuda")
    H[:, :, 0] = 1.0
    Wo = torch.full((P, h, hp), 1.5, dtype=dt, device="cuda")
    for m in range(P):
        Wo[m, :, 0] = _code(dtype, P, m)
    resid = torch.zeros((P, T, h), dtype=dt, device="cuda")
    gamma = torch.ones(h, dtype=dt, device="cuda")
    out = torch.empty_like(resid)
    out_resid = torch.full_like(resid, float("nan"))
    s.forward(H, None, Wo, gamma, out, resid=resid, out_resid=out_resid)
    torch.cuda.synchronize()
    want = _coded_out_resid(dtype, P, T, h, n_s, 2.0)
    got = out_resid.double().cpu()
    fused = caat.caat_forward_fused(s.handle, T)
    assert fused == (n_s % 8 == 0 and T > 64 and
                     (n_s == 0 or -(-n_s // 128) * -(-T // 128) >= 256)), fused
    if not torch.equal(got, want):
        bad = (got != want).nonzero()[:5].tolist()
        raise AssertionError(f"fused={caat.caat_forward_fused(s.handle, T)} first bad "
                             f"(m, t, l): {bad}")


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


@pytest.mark.parametrize("wname,T", [("7b-prefill-pair-bf16", 520), ("7b-decode-pair-bf16", 64)])
def test_run_to_run_deterministic(wname, T):
    """Repeated forwards are bitwise identical (T = 64: the 64-token MFMA tiles of the
    decode batch)."""
    w = W.with_(W.ALL[wname], T=T)
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



@pytest.mark.parametrize("wname,T,p", [("1.1b-mlp-bf16", 4096, 0.5), ("1.1b-mlp-bf16", 200, 0.0),
                                       ("130m-pair-bf16", 333, 0.0), ("7b-prefill-pair-bf16", 2048, 0.5),
                                       ("7b-prefill-pair-bf16", 384, 0.0),
                                       # the per-rank row GEMM (too few shared-GEMM tiles, or
                                       # n_s % 8 != 0: the chunk across n_s keeps its partials)
                                       ("1.1b-mlp-bf16", 2100, 0.5), ("1.1b-mlp-bf16", 2048, 0.37),
                                       ("7b-prefill-pair-bf16", 1100, 0.61)])
def test_forward_private_rows_from_gemm_epilogue(wname, T, p):
    """With a residual output, the row GEMM adds the residual in its epilogue (out_resid =
    resid + s_priv * Zt on the private channel chunks) and K3 reads those rows.  out_resid
    must equal, bit for bit, what K3 computes from stored partials (fused path:
    caat_row_gemm_reduce, then caat_sync_norm; per-rank path: caat_row_gemm, then
    caat_partial_sync_norm); out (whose private row statistics are now taken from the stored
    bf16 rows) within one bf16 rounding of it.  In place (out_resid = resid) gives the same
    bits."""
    w = W.ALL[wname]
    _say(f"[case] private rows from the epilogue {wname} T={T} p={p}")
    inputs = runner.make_inputs(w, T=T, norm_params="random")
    d = {k: v.cuda() for k, v in inputs.items()}
    dt = runner.torch_dtype(w)
    attn = "ctx" in d
    s = caat.Sublayer(w.h, w.ffn, w.P, p, norm=w.norm, act="none" if attn else w.act,
                      dtype=w.dtype, s_priv=1.75)
    fused = caat.caat_forward_fused(s.handle, T)
    assert caat.caat_forward_private_in_epilogue(s.handle, T), "the case must take that path"
    inp, W1, W2, resid = (d["ctx"], None, d["Wo"], d["x0"]) if attn else (d["x"], d["W1"], d["W2"], d["x"])
    P, h, n_s = w.P, w.h, s.n_s
    out = torch.empty((P, T, h), dtype=dt, device="cuda")
    out_resid = torch.empty_like(out)
    s.forward(inp, W1, W2, d["gamma"], out, resid=resid, beta=d["beta"], out_resid=out_resid)
    # The same sublayer through the per-step calls, partials stored.
    if attn:
        gin = inp
    else:
        gin = torch.empty((P, T, s.f_s), dtype=dt, device="cuda")
        caat.caat_column_gemm_act(s.handle, T, inp, W1, gin)
    Z = torch.empty((P, T, h), dtype=dt, device="cuda")
    out2 = torch.empty_like(out)
    out_resid2 = torch.empty_like(out)
    if fused:
        S = torch.empty((T, max(n_s, 8)), dtype=dt, device="cuda")
        caat.caat_row_gemm_reduce(s.handle, T, gin, W2, S if n_s else None, Z)
        caat.caat_sync_norm(s.handle, T, S if n_s else None, Z, resid, d["gamma"], d["beta"],
                            out2, out_resid2)
    else:
        caat.caat_row_gemm(s.handle, T, gin, W2, Z)
        caat.caat_partial_sync_norm(s.handle, T, Z, resid, d["gamma"], d["beta"], out2, out_resid2)
    # In place: the residual output overwrites the residual.
    r3 = resid.clone()
    out3 = torch.empty_like(out)
    s.forward(inp, W1, W2, d["gamma"], out3, resid=r3, beta=d["beta"], out_resid=r3)
    torch.cuda.synchronize()
    assert torch.equal(out_resid, out_resid2)
    assert torch.equal(r3, out_resid) and torch.equal(out3, out)
    err = ((out.float() - out2.float()).abs().max() / out2.float().abs().max()).item()
    _say(f"   out against the stored-partials path: {err:.2e}")
    assert err <= 2 ** -7


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


def _k3_layout_cases():
    """One (dtype, P, h, T) per register layout the K3 dispatch can reach, for each norm:
    the single-pass kernel (ranks rounded up to a power of two, times chunks per thread,
    within 16 for bf16 and 8 for fp32; cached, and nontemporal past 256 MB per launch), the
    per-rank kernel for T <= 64, and the multi-pass kernel (one to eight chunks per thread)."""
    one_pass = {"bf16": [(1, 256), (1, 4096), (1, 8192), (1, 16384), (2, 4096), (2, 8192),
                         (2, 16384), (3, 4096), (4, 8192), (4, 16384), (8, 4096), (8, 8192),
                         (16, 4096)],
                "f32": [(1, 256), (1, 4096), (1, 8192), (1, 16384), (2, 4096), (2, 8192),
                        (2, 16384), (4, 4096), (4, 8192), (8, 4096)]}
    cases = [(dt, P, h, 65) for dt, l in one_pass.items() for P, h in l]
    # The same layouts with more than 256 MB moved per launch (nontemporal rows).
    esize = {"bf16": 2, "f32": 4}
    cases += [(dt, P, h, 2 ** 26 // (P * h * esize[dt]) + 3) for dt, l in one_pass.items()
              for P, h in l if h >= 4096]
    cases += [(dt, P, h, 5) for dt in ("bf16", "f32")
              for P, h in ((8, 4096), (8, 8192), (16, 4096), (16, 8192), (4, 16384))]
    cases += [("bf16", 16, 8192, 66), ("bf16", 8, 16384, 66), ("f32", 16, 1024, 66),
              ("f32", 16, 4096, 66), ("f32", 16, 8192, 66), ("f32", 8, 16384, 66)]
    return [(dt, P, h, T, nm) for dt, P, h, T in cases for nm in ("layernorm", "rmsnorm")]


@pytest.mark.parametrize("dtype,P,h,T,norm", _k3_layout_cases())
def test_partial_sync_norm_every_layout(dtype, P, h, T, norm):
    _partial_sync_norm_case(dtype, P, h, T, norm)


@pytest.mark.parametrize("dtype,P,h,T", [("bf16", 8, 8192, 100), ("bf16", 2, 16384, 70),
                                         ("bf16", 16, 4096, 100), ("bf16", 16, 8192, 66),
                                         ("f32", 4, 8192, 100), ("f32", 1, 16384, 65),
                                         ("f32", 16, 1024, 100), ("f32", 9, 4096, 65)])
def test_partial_sync_norm_wide_rows_and_many_ranks(dtype, P, h, T):
    """K3 for T > 64 on the register layouts the 7B shapes do not reach: the single-pass
    kernel with two or four chunks per thread and with 16 ranks, and the multi-pass kernel
    (with one, four and two chunks per thread)."""
    _partial_sync_norm_case(dtype, P, h, T)


def _partial_sync_norm_case(dtype, P, h, T, norm="layernorm"):
    """caat_partial_sync_norm with the given norm (LayerNorm with beta), a private scale and
    p = 0.37, against the oracle's reduce + norm."""
    _say(f"[case] partial_sync_norm {dtype} P={P} h={h} T={T} {norm}")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    s = caat.Sublayer(h, 8 * P, P, 0.37, norm=norm, act="gelu", dtype=dtype, s_priv=1.5)
    Z = synth.normal((P, T, h), synth.PARTIALS, dtype=dt)
    R = synth.normal((P, T, h), synth.RESID, dtype=dt)
    gamma = synth.normal((h,), synth.GAMMA, std=0.1, mean=1.0, dtype=dt)
    beta = synth.normal((h,), synth.BETA, std=0.1, dtype=dt) if norm == "layernorm" else None
    out = torch.empty((P, T, h), dtype=dt, device="cuda")
    out_resid = torch.empty_like(out)
    caat.caat_partial_sync_norm(s.handle, T, Z.cuda(), R.cuda(), gamma.cuda(),
                                None if beta is None else beta.cuda(), out, out_resid)
    torch.cuda.synchronize()
    ref_out, ref_res = oracle.partial_sync_norm(
        Z, R, gamma, beta=beta, norm=oracle.LAYERNORM if norm == "layernorm" else oracle.RMSNORM,
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


@pytest.mark.parametrize("p", [0.0, 0.5, 1.0])
def test_forward_fused_ragged(p):
    """The fused row GEMM through the forward (at T = 2000 the shared GEMM has 16 x 16
    tiles: the fused path) with a ragged last token tile, p = 0, 0.5 and 1, against the
    oracle on sampled rows (the last token included)."""
    T = 2000
    w = W.with_(W.PREFILL_7B_BF16, T=T, p=p)
    h = caat.Sublayer(w.h, w.ffn, w.P, p, norm=w.norm, act=w.act)
    assert caat.caat_forward_fused(h.handle, T)
    _run_and_compare(w, norm_params="random", rows=synth.sample_rows(T, 48))


@pytest.mark.parametrize("p", [0.0, 1.0])
def test_forward_per_rank_path_small_tiles(p):
    """T = 70: too few shared-GEMM tiles for the fused path, so the per-rank GEMM and
    K3's reduce run (p = 0 and 1 included)."""
    w = W.with_(W.PREFILL_7B_BF16, T=70, p=p)
    h = caat.Sublayer(w.h, w.ffn, w.P, p, norm=w.norm, act=w.act)
    assert caat.caat_forward_fused(h.handle, 70) == (p == 0.0)
    _run_and_compare(w, norm_params="random")


@pytest.mark.parametrize("T", [8, 64])
def test_graph_replay_matches_eager(T):
    """One decode step captured as a HIP graph: every replay (with eager work between
    replays) reproduces the eager outputs bitwise (T = 64: with the 64-token MFMA tiles)."""
    w = W.with_(W.DECODE_7B_BF16, T=T)
    run = runner.Run(w, runner.make_inputs(w, norm_params="random"))
    run.step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in run.outputs().items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run.step()
    for rep in range(3):
        for v in run.outputs().values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in run.outputs().items():
            assert torch.equal(v, eager[k]), (rep, k)


@pytest.mark.parametrize("T", [8192, 1, 64])
def test_timed_step_is_the_product_path(T):
    """The benchmark's timed step (caat_forward_timed, events after every step) gives
    bitwise the outputs of caat_forward_ex on the same inputs, at the 7B prefill size the
    headline is quoted on and at decode sizes."""
    from bench import timed_steps
    w = W.with_(W.PREFILL_7B_BF16 if T > 64 else W.DECODE_7B_BF16, T=T)
    _say(f"[case] timed step vs caat_forward_ex {w.name} T={T}")
    run = runner.Run(w, runner.make_inputs(w, norm_params="random"))
    run.step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in run.outputs().items()}
    for v in run.outputs().values():
        v.fill_(float("nan"))
    timed_steps(run, 2, 0)
    torch.cuda.synchronize()
    for k, v in run.outputs().items():
        assert torch.equal(v, ref[k]), k
    assert caat.caat_forward_fused(run.mlp.handle, T) == (T > 64)


def test_fault_hook_forces_device_error(monkeypatch):
    """CAAT_FAULT=launch (read on the host) makes a forward return CAAT_EDEVICE with
    nothing enqueued; CAAT_ARCH=gfx942 makes it return CAAT_EUNSUPPORTED.  The GPU does
    not fault: no kernel is launched in either case."""
    w = W.with_(W.MLP_1P1B_BF16, T=70)
    run = runner.Run(w, runner.make_inputs(w))
    run.out.fill_(7.0)
    torch.cuda.synchronize()
    for var, val, code in (("CAAT_FAULT", "launch", caat.EDEVICE),
                           ("CAAT_ARCH", "gfx942", caat.EUNSUPPORTED)):
        monkeypatch.setenv(var, val)
        with pytest.raises(caat.CaatError) as e:
            run.step()
        assert e.value.code == code
        torch.cuda.synchronize()
        assert bool((run.out == 7.0).all()), "an erroring call enqueued work"
        monkeypatch.delenv(var)
    run.step()
    torch.cuda.synchronize()
    assert not bool((run.out == 7.0).all())
