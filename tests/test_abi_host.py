"""Host-side tests of the C ABI: the library loads, exports every symbol the header
declares, and validates arguments before touching any device (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import oracle
import partial_activation_sync_amd as caat

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "caat.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(caat_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    declared = _declared()
    assert len(declared) >= 13
    nm = subprocess.run(["nm", "-D", "--defined-only", caat.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r"\bT (caat_\w+)", nm))
    missing = [d for d in declared if d not in exported]
    assert not missing, missing
    L = caat.lib()
    for d in declared:
        assert getattr(L, d) is not None


def test_binding_names_match_header():
    for d in _declared():
        assert callable(getattr(caat, d)), d


@pytest.mark.parametrize("h,p", [(4096, 0.5), (2048, 0.25), (768, 0.5), (256, 0.5), (104, 0.29),
                                 (4096, 0.703125), (4096, 1 / 3), (8, 0.0), (8, 1.0), (16, 0.9999999999)])
def test_shared_channels_agree_with_oracle(h, p):
    hd = caat.caat_create(h, 8 * 4, 4, p, caat.LAYERNORM, caat.GELU, caat.BF16)
    try:
        assert caat.caat_shared_channels(hd) == oracle.shared_channels(h, p)
    finally:
        caat.caat_destroy(hd)


@pytest.mark.parametrize("args", [
    (0, 64, 2, 0.5, 0, 0, 1),          # h < 8
    (100, 64, 2, 0.5, 0, 0, 1),        # h % 8
    (16392, 64, 2, 0.5, 0, 0, 1),      # h too large
    (64, 64, 0, 0.5, 0, 0, 1),         # P < 1
    (64, 64 * 17, 17, 0.5, 0, 0, 1),   # P > 16
    (64, 64, 2, -0.1, 0, 0, 1),        # p < 0
    (64, 64, 2, 1.5, 0, 0, 1),         # p > 1
    (64, 64, 2, float("nan"), 0, 0, 1),
    (64, 64, 2, 0.5, 2, 0, 1),         # norm
    (64, 64, 2, 0.5, 0, 4, 1),         # act
    (64, 64, 2, 0.5, 0, 0, 2),         # dtype
    (64, 63, 2, 0.5, 0, 0, 1),         # ffn % P
    (64, 36, 3, 0.5, 0, 0, 1),         # (ffn / P) % 8
    (64, 0, 3, 0.5, 0, 3, 1),          # out-projection: h % P
    (24, 0, 2, 0.5, 0, 3, 1),          # out-projection: (h / P) % 8
])
def test_create_rejects(args):
    handle = ctypes.c_void_p()
    rc = caat.lib().caat_create(ctypes.byref(handle), *args)
    assert rc == caat.EINVAL
    assert not handle.value


def test_setters_and_workspace_size():
    hd = caat.caat_create(256, 1024, 2, 0.5, caat.LAYERNORM, caat.SWIGLU, caat.BF16)
    L = caat.lib()
    assert L.caat_set_eps(hd, -1.0) == caat.EINVAL
    assert L.caat_set_eps(hd, float("nan")) == caat.EINVAL
    assert L.caat_set_private_scale(hd, float("inf")) == caat.EINVAL
    caat.caat_set_eps(hd, 1e-6)
    caat.caat_set_private_scale(hd, 2 ** 0.5)
    # Y [P][T][f_s] + partials [P][T][h] + S [T][n_s] (n_s = 128, a multiple of 8),
    # each rounded up to 256 bytes.
    T = 37
    y = (2 * T * 512 * 2 + 255) // 256 * 256
    z = (2 * T * 256 * 2 + 255) // 256 * 256
    sh = (T * 128 * 2 + 255) // 256 * 256
    assert caat.caat_workspace_bytes(hd, T) == y + z + sh
    assert caat.caat_workspace_bytes(hd, 0) == 0
    assert L.caat_set_workspace(hd, 0x1008, 64) == caat.EINVAL   # misaligned
    caat.caat_destroy(hd)
    att = caat.caat_create(256, 0, 2, 0.5, caat.RMSNORM, caat.NONE, caat.F32)
    assert caat.caat_workspace_bytes(att, T) == ((2 * T * 256 * 4 + 255) // 256 * 256
                                                 + (T * 128 * 4 + 255) // 256 * 256)
    caat.caat_destroy(att)
    # n_s not a multiple of 8: no S buffer (the unfused path)
    odd = caat.caat_create(256, 1024, 2, 0.37, caat.LAYERNORM, caat.GELU, caat.BF16)
    assert caat.caat_shared_channels(odd) == 94
    assert caat.caat_workspace_bytes(odd, T) == y + z
    caat.caat_destroy(odd)


def test_forward_checks_before_any_launch():
    L = caat.lib()
    hd = caat.caat_create(256, 1024, 2, 0.5, caat.LAYERNORM, caat.GELU, caat.BF16)
    fake = 0x10000  # aligned, never dereferenced: every call below fails its checks first
    st = None
    assert L.caat_forward(None, 4, fake, fake, fake, fake, fake, st) == caat.EINVAL
    assert L.caat_forward(hd, 0, fake, fake, fake, fake, fake, st) == caat.EINVAL
    assert L.caat_forward(hd, 4, None, fake, fake, fake, fake, st) == caat.EINVAL
    assert L.caat_forward(hd, 4, fake + 2, fake, fake, fake, fake, st) == caat.EINVAL
    assert L.caat_forward(hd, 4, fake, fake, fake, fake, fake, st) == caat.EWORKSPACE
    caat.caat_set_workspace(hd, fake, 16)
    assert L.caat_forward(hd, 4, fake, fake, fake, fake, fake, st) == caat.EWORKSPACE
    assert L.caat_column_gemm_act(hd, 4, fake, None, fake, st) == caat.EINVAL
    assert L.caat_row_gemm(hd, 0, fake, fake, fake, st) == caat.EINVAL
    assert L.caat_partial_sync_norm(hd, 4, fake, None, fake, None, fake, None, st) == caat.EINVAL
    assert L.caat_partial_sync_norm(hd, 4, fake, fake, fake, fake + 4, fake, None, st) == caat.EINVAL
    caat.caat_destroy(hd)
    att = caat.caat_create(256, 0, 2, 0.5, caat.RMSNORM, caat.NONE, caat.BF16)
    assert L.caat_forward(att, 4, fake, fake, fake, fake, fake, st) == caat.EINVAL   # needs _ex
    assert L.caat_column_gemm_act(att, 4, fake, fake, fake, st) == caat.EINVAL
    a = caat.caat_args(4, fake, None, None, fake, fake, None, fake, None, None)
    assert L.caat_forward_ex(att, ctypes.byref(a)) == caat.EINVAL                     # resid needed
    a = caat.caat_args(4, fake, fake, None, fake, fake, None, fake, None, None)
    assert L.caat_forward_train(att, ctypes.byref(a), fake) == caat.EINVAL          # MLP only
    caat.caat_destroy(att)


def test_fused_steps_check_before_any_launch():
    L = caat.lib()
    fake = 0x10000
    odd = caat.caat_create(256, 1024, 2, 0.37, caat.LAYERNORM, caat.GELU, caat.BF16)  # n_s 94
    assert L.caat_row_gemm_reduce(odd, 4, fake, fake, fake, fake, None) == caat.EUNSUPPORTED
    assert L.caat_sync_norm(odd, 4, fake, fake, fake, fake, None, fake, None, None) == caat.EUNSUPPORTED
    caat.caat_destroy(odd)
    hd = caat.caat_create(256, 1024, 2, 0.5, caat.LAYERNORM, caat.GELU, caat.BF16)
    assert L.caat_row_gemm_reduce(hd, 4, fake, fake, None, fake, None) == caat.EINVAL   # S needed
    assert L.caat_row_gemm_reduce(hd, 4, fake, fake, fake, None, None) == caat.EINVAL   # partials
    assert L.caat_row_gemm_reduce(hd, 0, fake, fake, fake, fake, None) == caat.EINVAL
    assert L.caat_sync_norm(hd, 4, fake, fake, None, fake, None, fake, None, None) == caat.EINVAL
    caat.caat_destroy(hd)
    full = caat.caat_create(256, 1024, 2, 1.0, caat.LAYERNORM, caat.GELU, caat.BF16)   # n_s = h
    none = caat.caat_create(256, 1024, 2, 0.0, caat.LAYERNORM, caat.GELU, caat.BF16)   # n_s = 0
    # (a NULL partials with n_s = h, or a NULL S with n_s = 0, passes the checks; those
    # calls would launch, so they are exercised on the GPU only)
    assert L.caat_row_gemm_reduce(full, 4, fake, fake, None, None, None) == caat.EINVAL
    assert L.caat_row_gemm_reduce(none, 4, fake, fake, None, None, None) == caat.EINVAL
    caat.caat_destroy(full)
    caat.caat_destroy(none)


def test_backward_workspace_and_checks_before_any_launch():
    L = caat.lib()
    fake = 0x10000
    P, h, ffn, T = 2, 256, 1024, 37
    hd = caat.caat_create(h, ffn, P, 0.5, caat.LAYERNORM, caat.SWIGLU, caat.BF16)
    fs, F1, Tp, NB = ffn // P, 2 * ffn // P, 40, T
    a256 = lambda n: (n + 255) // 256 * 256
    # bf16: the weight gradients contract over tokens from the token-major operands, so
    # no transposed activations; fp32 keeps the transposed copies (token count Tp).
    parts = [P * T * h * 2, P * T * h * 2, NB * h * 4, NB * h * 4, P * fs * h * 2,
             P * T * fs * 2,
             P * T * F1 * 2, P * T * F1 * 2, P * T * fs * 2, P * h * F1 * 2]
    assert caat.caat_backward_workspace_bytes(hd, T) == sum(a256(n) for n in parts)
    h32 = caat.caat_create(h, ffn, P, 0.5, caat.LAYERNORM, caat.SWIGLU, caat.F32)
    parts32 = [P * T * h * 4, P * T * h * 4, NB * h * 4, NB * h * 4, P * fs * h * 4,
               P * T * fs * 4, P * h * Tp * 4, P * fs * Tp * 4,
               P * T * F1 * 4, P * T * F1 * 4, P * T * fs * 4, P * h * F1 * 4, P * h * Tp * 4,
               P * F1 * Tp * 4]
    assert caat.caat_backward_workspace_bytes(h32, T) == sum(a256(n) for n in parts32)
    caat.caat_destroy(h32)
    assert caat.caat_backward_workspace_bytes(hd, 0) == 0
    assert caat.caat_backward_workspace_bytes(None, T) == 0
    need = caat.caat_backward_workspace_bytes(hd, T)
    args = lambda **kw: caat.caat_bwd_args(*[kw.get(k, d) for k, d in (
        ("T", T), ("in_", fake), ("W1", fake), ("W2", fake), ("gamma", fake),
        ("out_resid", fake), ("dout", fake), ("dres", None), ("din", fake), ("dresid", None),
        ("dW1", fake), ("dW2", fake), ("dgamma", fake), ("dbeta", None), ("workspace", fake),
        ("workspace_bytes", need), ("stream", None), ("events", None), ("n_events", 0),
        ("preact", None))])
    assert L.caat_backward(None, ctypes.byref(args())) == caat.EINVAL
    assert L.caat_backward(hd, None) == caat.EINVAL
    assert L.caat_backward(hd, ctypes.byref(args(T=0))) == caat.EINVAL
    assert L.caat_backward(hd, ctypes.byref(args(dout=None))) == caat.EINVAL
    assert L.caat_backward(hd, ctypes.byref(args(out_resid=None))) == caat.EINVAL
    assert L.caat_backward(hd, ctypes.byref(args(dW1=None))) == caat.EINVAL
    assert L.caat_backward(hd, ctypes.byref(args(dgamma=fake + 4))) == caat.EINVAL
    assert L.caat_backward(hd, ctypes.byref(args(workspace_bytes=need - 1))) == caat.EWORKSPACE
    assert L.caat_backward(hd, ctypes.byref(args(workspace=None))) == caat.EWORKSPACE
    assert L.caat_backward(hd, ctypes.byref(args(preact=fake + 8))) == caat.EINVAL   # misaligned
    small = 2 * a256(NB * h * 4)
    assert L.caat_partial_sync_norm_backward(hd, T, fake, fake, None, fake, fake, None, fake,
                                             None, fake, small - 1, None) == caat.EWORKSPACE
    assert L.caat_partial_sync_norm_backward(hd, T, fake, None, None, fake, fake, None, fake,
                                             None, fake, small, None) == caat.EINVAL
    caat.caat_destroy(hd)
    att = caat.caat_create(h, 0, P, 0.5, caat.RMSNORM, caat.NONE, caat.BF16)
    need = caat.caat_backward_workspace_bytes(att, T)
    k2 = h // P
    assert need == sum(a256(n) for n in [P * T * h * 2, P * T * h * 2, NB * h * 4, NB * h * 4,
                                        P * k2 * h * 2, P * T * k2 * 2])
    # the out-projection's residual is not its input: dresid is required
    assert L.caat_backward(att, ctypes.byref(args(W1=None, dW1=None, workspace_bytes=need))) == caat.EINVAL
    # a stored pre-activation belongs to an MLP
    assert L.caat_backward(att, ctypes.byref(args(W1=None, dW1=None, dresid=fake, preact=fake,
                                                  workspace_bytes=need))) == caat.EINVAL
    caat.caat_destroy(att)


def test_error_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert caat.caat_error_string(code) != "unknown status"
    assert caat.caat_error_string(7) == "unknown status"
    with pytest.raises(caat.CaatError) as e:
        caat.caat_create(7, 8, 1, 0.5, 0, 0, 1)
    assert e.value.code == caat.EINVAL


def _launching_calls(L, hd, att, fake, ws_bytes):
    """Every entry point that would launch, with arguments that pass their checks."""
    caat.caat_set_workspace(hd, fake, ws_bytes)
    caat.caat_set_workspace(att, fake, ws_bytes)
    a = caat.caat_args(4, fake, fake, fake, fake, fake, None, fake, None, None)
    ev = (ctypes.c_void_p * 1)(None)
    evp = ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p))
    return {
        "caat_forward": lambda: L.caat_forward(hd, 4, fake, fake, fake, fake, fake, None),
        "caat_forward_ex": lambda: L.caat_forward_ex(hd, ctypes.byref(a)),
        "caat_forward_ex (out-projection)": lambda: L.caat_forward_ex(att, ctypes.byref(a)),
        "caat_forward_timed": lambda: L.caat_forward_timed(hd, ctypes.byref(a), evp, 1),
        "caat_forward_train": lambda: L.caat_forward_train(hd, ctypes.byref(a), fake),
        "caat_column_gemm_act": lambda: L.caat_column_gemm_act(hd, 4, fake, fake, fake, None),
        "caat_row_gemm": lambda: L.caat_row_gemm(hd, 4, fake, fake, fake, None),
        "caat_row_gemm_reduce": lambda: L.caat_row_gemm_reduce(hd, 4, fake, fake, fake, fake, None),
        "caat_sync_norm": lambda: L.caat_sync_norm(hd, 4, fake, fake, fake, fake, None, fake,
                                                   None, None),
        "caat_partial_sync_norm": lambda: L.caat_partial_sync_norm(hd, 4, fake, fake, fake, None,
                                                                   fake, None, None),
    }


@pytest.mark.parametrize("var,val,code", [("CAAT_ARCH", "gfx942", caat.EUNSUPPORTED),
                                          ("CAAT_ARCH", "gfx90a", caat.EUNSUPPORTED),
                                          ("CAAT_FAULT", "launch", caat.EDEVICE)])
def test_device_error_hooks(monkeypatch, var, val, code):
    """The host-side hooks drive the device error paths of every launching entry point
    after its argument checks and before any HIP call (no GPU, nothing launched):
    CAAT_ARCH names another architecture -> CAAT_EUNSUPPORTED, CAAT_FAULT=launch ->
    CAAT_EDEVICE.  Argument errors still come first."""
    L = caat.lib()
    fake = 0x10000
    hd = caat.caat_create(256, 1024, 2, 0.5, caat.LAYERNORM, caat.GELU, caat.BF16)
    att = caat.caat_create(256, 0, 2, 0.5, caat.RMSNORM, caat.NONE, caat.BF16)
    try:
        calls = _launching_calls(L, hd, att, fake, 1 << 30)
        monkeypatch.setenv(var, val)
        for name, call in calls.items():
            assert call() == code, name
        assert L.caat_forward(hd, 0, fake, fake, fake, fake, fake, None) == caat.EINVAL
        assert L.caat_row_gemm(hd, 4, fake + 2, fake, fake, None) == caat.EINVAL
        caat.caat_set_workspace(hd, fake, 16)
        assert L.caat_forward(hd, 4, fake, fake, fake, fake, fake, None) == caat.EWORKSPACE
    finally:
        caat.caat_destroy(hd)
        caat.caat_destroy(att)


def test_arch_hook_gfx950_falls_through(monkeypatch):
    """CAAT_ARCH=gfx950 does not force success: the real device query still runs (here,
    with no GPU, it fails with CAAT_EDEVICE; on a GPU it passes)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("needs a host without a GPU")
    L = caat.lib()
    hd = caat.caat_create(256, 1024, 2, 0.5, caat.LAYERNORM, caat.GELU, caat.BF16)
    try:
        caat.caat_set_workspace(hd, 0x10000, 1 << 30)
        monkeypatch.setenv("CAAT_ARCH", "gfx950")
        assert L.caat_forward(hd, 4, 0x10000, 0x10000, 0x10000, 0x10000, 0x10000, None) == caat.EDEVICE
    finally:
        caat.caat_destroy(hd)


def test_forward_path_query():
    """caat_forward_fused: the shared channels are summed inside the row GEMM only for
    n_s % 8 == 0, T > 64 and at least 256 shared-GEMM tiles of 128 x 128 (or n_s = 0),
    and only while the K-concatenated GEMM fits the bf16 kernel's 32-bit offsets
    (P T k2 2 bytes < 2^31); otherwise the per-rank GEMM and K3's reduce."""
    L = caat.lib()
    mlp = caat.caat_create(4096, 11008, 8, 0.5, caat.RMSNORM, caat.SWIGLU, caat.BF16)
    att = caat.caat_create(4096, 0, 8, 0.5, caat.RMSNORM, caat.NONE, caat.BF16)
    odd = caat.caat_create(4096, 11008, 8, 0.37, caat.RMSNORM, caat.SWIGLU, caat.BF16)
    f32 = caat.caat_create(4096, 11008, 8, 0.5, caat.RMSNORM, caat.SWIGLU, caat.F32)
    try:
        assert caat.caat_forward_fused(mlp, 64) is False
        assert caat.caat_forward_fused(mlp, 65) is False            # 16 x 1 tiles
        assert caat.caat_forward_fused(mlp, 1920) is False          # 16 x 15 tiles
        assert caat.caat_forward_fused(mlp, 1921) is True           # 16 x 16 tiles
        assert caat.caat_forward_fused(mlp, 8192) is True
        zero = caat.caat_create(4096, 11008, 8, 0.0, caat.RMSNORM, caat.SWIGLU, caat.BF16)
        small = caat.caat_create(768, 3072, 4, 0.5, caat.LAYERNORM, caat.GELU, caat.BF16)
        try:
            assert caat.caat_forward_fused(zero, 65) is True         # no shared GEMM
            assert caat.caat_forward_fused(zero, 64) is False
            assert caat.caat_forward_fused(small, 4096) is False     # 3 x 32 tiles
            assert caat.caat_forward_fused(small, 128 * 86) is True  # 3 x 86 tiles
        finally:
            caat.caat_destroy(zero)
            caat.caat_destroy(small)
        assert caat.caat_forward_fused(odd, 8192) is False
        limit = (1 << 31) // (8 * 1376 * 2)          # largest T with P T k2 2 < 2^31, + 1
        assert caat.caat_forward_fused(mlp, limit - 1) is True
        assert caat.caat_forward_fused(mlp, limit + 1) is False
        assert caat.caat_forward_fused(att, limit + 1) is True      # k2 = h / P = 512
        assert caat.caat_forward_fused(f32, limit + 1) is True      # the fp32 kernel
        assert L.caat_forward_fused(None, 8) == caat.EINVAL
        assert L.caat_forward_fused(mlp, 0) == caat.EINVAL
    finally:
        for hd in (mlp, att, odd, f32):
            caat.caat_destroy(hd)


def test_private_in_epilogue_query():
    """caat_forward_private_in_epilogue: in bf16 for T > 64, on the fused path or on the
    per-rank path from P T h = 2^25 on, where K3's single-pass kernel handles the rows
    (P = 8: up to 4096 channels), and with whole private chunks of 8 channels left (from
    n_s on when fused, else from n_s rounded up to 8)."""
    L = caat.lib()
    mlp = caat.caat_create(4096, 11008, 8, 0.5, caat.RMSNORM, caat.SWIGLU, caat.BF16)
    full = caat.caat_create(4096, 11008, 8, 1.0, caat.RMSNORM, caat.SWIGLU, caat.BF16)
    odd = caat.caat_create(4096, 11008, 8, 0.37, caat.RMSNORM, caat.SWIGLU, caat.BF16)
    last = caat.caat_create(4096, 11008, 8, 4095 / 4096, caat.RMSNORM, caat.SWIGLU, caat.BF16)
    wide = caat.caat_create(16384, 0, 8, 0.0, caat.RMSNORM, caat.NONE, caat.BF16)
    wide2 = caat.caat_create(16384, 0, 2, 0.0, caat.RMSNORM, caat.NONE, caat.BF16)
    f32 = caat.caat_create(4096, 11008, 8, 0.5, caat.RMSNORM, caat.SWIGLU, caat.F32)
    try:
        assert caat.caat_forward_private_in_epilogue(mlp, 8192) is True   # fused
        assert caat.caat_forward_private_in_epilogue(mlp, 1920) is True   # per-rank GEMM
        assert caat.caat_forward_fused(mlp, 1920) is False
        assert caat.caat_forward_private_in_epilogue(mlp, 1023) is False  # P T h < 2^25
        assert caat.caat_forward_private_in_epilogue(mlp, 1024) is True
        assert caat.caat_forward_private_in_epilogue(mlp, 64) is False    # decode shapes
        assert caat.caat_forward_private_in_epilogue(odd, 8192) is True   # from 1520 on
        assert caat.caat_shared_channels(last) == 4095
        assert caat.caat_forward_private_in_epilogue(last, 8192) is False # no whole chunk
        assert caat.caat_forward_private_in_epilogue(full, 8192) is False # no private channels
        assert caat.caat_forward_private_in_epilogue(wide, 100) is False  # multi-pass K3
        assert caat.caat_forward_fused(wide, 100) is True
        assert caat.caat_forward_private_in_epilogue(wide2, 100) is True  # one pass at P = 2
        assert caat.caat_forward_private_in_epilogue(f32, 8192) is False
        assert L.caat_forward_private_in_epilogue(None, 8) == caat.EINVAL
        assert L.caat_forward_private_in_epilogue(mlp, 0) == caat.EINVAL
    finally:
        for hd in (mlp, full, odd, last, wide, wide2, f32):
            caat.caat_destroy(hd)


def test_forward_timed_checks_events():
    L = caat.lib()
    fake = 0x10000
    hd = caat.caat_create(256, 1024, 2, 0.5, caat.LAYERNORM, caat.GELU, caat.BF16)
    try:
        a = caat.caat_args(4, fake, fake, fake, fake, fake, None, fake, None, None)
        assert L.caat_forward_timed(hd, ctypes.byref(a), None, 2) == caat.EINVAL
        ev = (ctypes.c_void_p * 1)(None)
        evp = ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p))
        assert L.caat_forward_timed(hd, ctypes.byref(a), evp, -1) == caat.EINVAL
        assert L.caat_forward_timed(hd, ctypes.byref(a), evp, 1) == caat.EWORKSPACE
    finally:
        caat.caat_destroy(hd)
