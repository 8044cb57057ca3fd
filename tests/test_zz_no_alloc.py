"""caat_forward_scratch (the entry point that allocates nothing: its workspace is the
library's static device array) against caat_forward_ex on the same inputs, bit for bit,
through the C ABI: two calls in a row, the second with fewer tokens, for an MLP and an
out-projection sublayer.  Also the size check, which needs no launch."""
import pytest
import torch

import partial_activation_sync_amd as caat
from partial_activation_sync_amd import runner, workloads as W

pytestmark = pytest.mark.gpu


def _outputs(sub, d, T, inp, W1, W2, resid, scratch):
    out = torch.full((sub.P, T, sub.h), float("nan"), dtype=sub.torch_dtype, device="cuda")
    out_resid = torch.full_like(out, float("nan"))
    f = caat.caat_forward_scratch if scratch else caat.caat_forward_ex
    f(sub.handle, T, inp, W1, W2, d["gamma"], out, resid=resid, beta=d["beta"],
      out_resid=out_resid)
    torch.cuda.synchronize()
    return out, out_resid


@pytest.mark.parametrize("wname", ["1.1b-mlp-bf16", "130m-pair-bf16", "7b-decode-pair-bf16",
                                   "tiny-mlp-fp32"])
def test_scratch_forward_matches_workspace_forward(wname):
    w = W.ALL[wname]
    # T > 64 takes the fused row GEMM (S in the workspace), T <= 64 the decode kernels.
    Ts = {"1.1b-mlp-bf16": (300, 70), "130m-pair-bf16": (4096, 33),
          "7b-decode-pair-bf16": (64, 8), "tiny-mlp-fp32": (128, 5)}[wname]
    print(f"[case] scratch {wname} T={Ts}", flush=True)
    for T in Ts:
        inputs = runner.make_inputs(w, T=T, norm_params="random")
        d = {k: v.cuda() for k, v in inputs.items()}
        act = "none" if "ctx" in d else w.act
        sub = caat.Sublayer(w.h, w.ffn, w.P, w.p, norm=w.norm, act=act, dtype=w.dtype, eps=w.eps)
        assert caat.caat_workspace_bytes(sub.handle, T) <= caat.SCRATCH_BYTES
        sub.workspace(T)
        if act == "none":
            args = (d["ctx"], None, d["Wo"], d["x0"])
        else:
            args = (d["x"], d["W1"], d["W2"], d["x"])
        want = _outputs(sub, d, T, *args, scratch=False)
        got = _outputs(sub, d, T, *args, scratch=True)
        for g, r in zip(got, want):
            assert torch.equal(g, r), (wname, T)


def test_scratch_rejects_sizes_beyond_its_maximum():
    """A forward whose workspace would exceed CAAT_SCRATCH_BYTES returns CAAT_EWORKSPACE
    before any launch."""
    w = W.MLP_1P1B_BF16
    sub = caat.Sublayer(w.h, w.ffn, w.P, w.p, norm=w.norm, act=w.act, dtype=w.dtype)
    T = 8192
    assert caat.caat_workspace_bytes(sub.handle, T) > caat.SCRATCH_BYTES
    x = torch.zeros((w.P, T, w.h), dtype=torch.bfloat16, device="cuda")
    W1 = torch.zeros((w.P, 2 * w.f_s, w.h), dtype=torch.bfloat16, device="cuda")
    W2 = torch.zeros((w.P, w.h, w.f_s), dtype=torch.bfloat16, device="cuda")
    g = torch.ones(w.h, dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(x, 3.0)
    with pytest.raises(caat.CaatError) as e:
        caat.caat_forward_scratch(sub.handle, T, x, W1, W2, g, out, resid=x)
    assert e.value.code == caat.EWORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
