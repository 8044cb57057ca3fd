"""MI355X-native forward of one CAAT tensor-parallel sublayer (partially synchronized
activations), all P ranks emulated on one GPU.

This module is the thin Python binding of ``libcaat.so`` (C ABI in ``include/caat.h``):
the functions carry the C names and only marshal arguments (tensor -> device
pointer, torch's current stream -> hipStream_t).  Every step of the sublayer runs
in the library's HIP kernels; there is no Python or CPU fallback, and every call
raises if the library is missing or returns an error.

Method: "Tensor-Parallelism with Partially Synchronized Activations", App. A.2,
Eq. 22 / Eq. 24 (partial channel-reduce), §4 Eq. 9 (residual + norm), §3.2
(logical devices).
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcaat.so")

GELU, GELU_TANH, SWIGLU, NONE = 0, 1, 2, 3
LAYERNORM, RMSNORM = 0, 1
F32, BF16 = 0, 1
OK, EINVAL, ENOMEM, EWORKSPACE, EDEVICE, EUNSUPPORTED = 0, -1, -2, -3, -4, -5

ACT = {"gelu": GELU, "gelu_tanh": GELU_TANH, "swiglu": SWIGLU, "none": NONE}
NORM = {"layernorm": LAYERNORM, "rmsnorm": RMSNORM}
DTYPE = {"f32": F32, "bf16": BF16}

_lib = None


class CaatError(RuntimeError):
    def __init__(self, what, code):
        super().__init__(f"{what}: {caat_error_string(code)} ({code})")
        self.code = code


class caat_args(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int), ("in_", ctypes.c_void_p), ("resid", ctypes.c_void_p),
                ("W1", ctypes.c_void_p), ("W2", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("beta", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("out_resid", ctypes.c_void_p), ("stream", ctypes.c_void_p)]


class caat_bwd_args(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int), ("in_", ctypes.c_void_p), ("W1", ctypes.c_void_p),
                ("W2", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("out_resid", ctypes.c_void_p), ("dout", ctypes.c_void_p),
                ("dres", ctypes.c_void_p), ("din", ctypes.c_void_p), ("dresid", ctypes.c_void_p),
                ("dW1", ctypes.c_void_p), ("dW2", ctypes.c_void_p), ("dgamma", ctypes.c_void_p),
                ("dbeta", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("stream", ctypes.c_void_p),
                ("events", ctypes.POINTER(ctypes.c_void_p)), ("n_events", ctypes.c_int),
                ("preact", ctypes.c_void_p)]


class caat_block_args(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int), ("S", ctypes.c_int), ("in_", ctypes.c_void_p),
                ("resid", ctypes.c_void_p), ("Wqkv", ctypes.c_void_p), ("Wo", ctypes.c_void_p),
                ("W1", ctypes.c_void_p), ("W2", ctypes.c_void_p),
                ("gamma_attn", ctypes.c_void_p), ("beta_attn", ctypes.c_void_p),
                ("gamma_mlp", ctypes.c_void_p), ("beta_mlp", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("out_resid", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("stream", ctypes.c_void_p), ("events", ctypes.POINTER(ctypes.c_void_p)),
                ("n_events", ctypes.c_int)]


FWD_STEPS = ("K1", "K2", "K2_private", "K3")
BLOCK_STEPS = ("qkv", "vT", "attn", "attn_sublayer", "mlp_sublayer")
BWD_STEPS = ("norm", "W2T", "dY", "a", "act", "W1T", "dx", "daT_xT", "dW1", "YT_dZtT", "dW2")


def lib():
    """The loaded libcaat.so.  torch is imported first so that the library binds to the
    HIP runtime torch already uses (one runtime, shared streams)."""
    global _lib
    if _lib is None:
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.caat_create.argtypes = [ctypes.POINTER(vp), i, i, i, ctypes.c_double, i, i, i]
        L.caat_destroy.argtypes = [vp]
        L.caat_set_eps.argtypes = [vp, ctypes.c_float]
        L.caat_set_private_scale.argtypes = [vp, ctypes.c_float]
        L.caat_shared_channels.argtypes = [vp]
        L.caat_workspace_bytes.argtypes = [vp, i]
        L.caat_workspace_bytes.restype = sz
        L.caat_set_workspace.argtypes = [vp, vp, sz]
        L.caat_forward.argtypes = [vp, i, vp, vp, vp, vp, vp, vp]
        L.caat_forward_ex.argtypes = [vp, ctypes.POINTER(caat_args)]
        L.caat_forward_timed.argtypes = [vp, ctypes.POINTER(caat_args),
                                         ctypes.POINTER(ctypes.c_void_p), i]
        L.caat_forward_fused.argtypes = [vp, i]
        L.caat_forward_private_in_epilogue.argtypes = [vp, i]
        L.caat_forward_scratch.argtypes = [vp, ctypes.POINTER(caat_args)]
        L.caat_forward_train.argtypes = [vp, ctypes.POINTER(caat_args), vp]
        L.caat_column_gemm_act.argtypes = [vp, i, vp, vp, vp, vp]
        L.caat_row_gemm.argtypes = [vp, i, vp, vp, vp, vp]
        L.caat_partial_sync_norm.argtypes = [vp, i, vp, vp, vp, vp, vp, vp, vp]
        L.caat_row_gemm_reduce.argtypes = [vp, i, vp, vp, vp, vp, vp]
        L.caat_sync_norm.argtypes = [vp, i, vp, vp, vp, vp, vp, vp, vp, vp]
        L.caat_backward_workspace_bytes.argtypes = [vp, i]
        L.caat_backward_workspace_bytes.restype = sz
        L.caat_backward.argtypes = [vp, ctypes.POINTER(caat_bwd_args)]
        L.caat_partial_sync_norm_backward.argtypes = [vp, i] + [vp] * 9 + [sz, vp]
        L.caat_attention_workspace_bytes.argtypes = [i, i, i, i]
        L.caat_attention_workspace_bytes.restype = sz
        L.caat_attention.argtypes = [i, i, i, i, i, vp, vp, vp, sz, vp]
        L.caat_block_workspace_bytes.argtypes = [vp, vp, i, i]
        L.caat_block_workspace_bytes.restype = sz
        L.caat_block_forward.argtypes = [vp, vp, i, ctypes.POINTER(caat_block_args)]
        L.caat_error_string.argtypes = [i]
        L.caat_error_string.restype = ctypes.c_char_p
        for name in ("caat_create", "caat_destroy", "caat_set_eps", "caat_set_private_scale",
                     "caat_shared_channels", "caat_set_workspace", "caat_forward",
                     "caat_forward_ex", "caat_forward_timed", "caat_forward_fused",
                     "caat_forward_private_in_epilogue",
                     "caat_forward_scratch",
                     "caat_forward_train",
                     "caat_column_gemm_act",
                     "caat_row_gemm",
                     "caat_partial_sync_norm", "caat_row_gemm_reduce", "caat_sync_norm",
                     "caat_backward", "caat_partial_sync_norm_backward", "caat_attention",
                     "caat_block_forward"):
            getattr(L, name).restype = i
        _lib = L
    return _lib


def _ptr(t):
    """Device pointer of a tensor (None -> NULL; ints pass through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("libcaat takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libcaat takes contiguous tensors")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc, what):
    if rc != OK:
        raise CaatError(what, rc)
    return rc


def caat_error_string(code: int) -> str:
    return lib().caat_error_string(int(code)).decode()


def caat_create(h, ffn, P, p, norm, act, dtype):
    handle = ctypes.c_void_p()
    _check(lib().caat_create(ctypes.byref(handle), int(h), int(ffn), int(P), float(p),
                             int(norm), int(act), int(dtype)), "caat_create")
    return handle


def caat_destroy(handle):
    return _check(lib().caat_destroy(handle), "caat_destroy")


def caat_set_eps(handle, eps):
    return _check(lib().caat_set_eps(handle, float(eps)), "caat_set_eps")


def caat_set_private_scale(handle, s):
    return _check(lib().caat_set_private_scale(handle, float(s)), "caat_set_private_scale")


def caat_shared_channels(handle) -> int:
    n = lib().caat_shared_channels(handle)
    if n < 0:
        raise CaatError("caat_shared_channels", n)
    return n


def caat_workspace_bytes(handle, T) -> int:
    return int(lib().caat_workspace_bytes(handle, int(T)))


def caat_set_workspace(handle, ws, nbytes=None):
    if ws is not None and nbytes is None:
        nbytes = ws.numel() * ws.element_size()
    return _check(lib().caat_set_workspace(handle, _ptr(ws), int(nbytes or 0)), "caat_set_workspace")


def caat_forward(handle, T, x, W1, W2, gamma, out, stream=None):
    return _check(lib().caat_forward(handle, int(T), _ptr(x), _ptr(W1), _ptr(W2), _ptr(gamma),
                                     _ptr(out), _stream(stream)), "caat_forward")


def caat_forward_ex(handle, T, inp, W1, W2, gamma, out, resid=None, beta=None, out_resid=None,
                    stream=None):
    a = caat_args(int(T), _ptr(inp), _ptr(resid), _ptr(W1), _ptr(W2), _ptr(gamma), _ptr(beta),
                  _ptr(out), _ptr(out_resid), _stream(stream))
    return _check(lib().caat_forward_ex(handle, ctypes.byref(a)), "caat_forward_ex")


SCRATCH_BYTES = 64 << 20   # CAAT_SCRATCH_BYTES


def caat_forward_scratch(handle, T, inp, W1, W2, gamma, out, resid=None, beta=None,
                         out_resid=None, stream=None):
    """caat_forward_ex on the library's static device workspace (no allocation; the
    handle's workspace is not used)."""
    a = caat_args(int(T), _ptr(inp), _ptr(resid), _ptr(W1), _ptr(W2), _ptr(gamma), _ptr(beta),
                  _ptr(out), _ptr(out_resid), _stream(stream))
    return _check(lib().caat_forward_scratch(handle, ctypes.byref(a)), "caat_forward_scratch")


def caat_forward_fused(handle, T) -> bool:
    """Whether a forward over T tokens sums the shared channels inside the row GEMM."""
    rc = lib().caat_forward_fused(handle, int(T))
    if rc < 0:
        raise CaatError("caat_forward_fused", rc)
    return bool(rc)


def caat_forward_private_in_epilogue(handle, T) -> bool:
    """Whether a forward over T tokens with a residual output adds the private channels'
    residual in the private GEMM's epilogue (K3 then reads those rows)."""
    rc = lib().caat_forward_private_in_epilogue(handle, int(T))
    if rc < 0:
        raise CaatError("caat_forward_private_in_epilogue", rc)
    return bool(rc)


def caat_forward_timed(handle, T, inp, W1, W2, gamma, out, events, resid=None, beta=None,
                       out_resid=None, stream=None):
    """caat_forward_ex that records raw hipEvent_t handles (ints; None entries skipped)
    after each of FWD_STEPS."""
    a = caat_args(int(T), _ptr(inp), _ptr(resid), _ptr(W1), _ptr(W2), _ptr(gamma), _ptr(beta),
                  _ptr(out), _ptr(out_resid), _stream(stream))
    ev = (ctypes.c_void_p * len(events))(*events)
    return _check(lib().caat_forward_timed(handle, ctypes.byref(a),
                                           ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p)),
                                           len(events)), "caat_forward_timed")


def caat_forward_train(handle, T, inp, W1, W2, gamma, out, preact, resid=None, beta=None,
                       out_resid=None, stream=None):
    """caat_forward_ex that also stores the pre-activation [P][T][F1] in preact."""
    a = caat_args(int(T), _ptr(inp), _ptr(resid), _ptr(W1), _ptr(W2), _ptr(gamma), _ptr(beta),
                  _ptr(out), _ptr(out_resid), _stream(stream))
    return _check(lib().caat_forward_train(handle, ctypes.byref(a), _ptr(preact)),
                  "caat_forward_train")


def caat_column_gemm_act(handle, T, x, W1, Y, stream=None):
    return _check(lib().caat_column_gemm_act(handle, int(T), _ptr(x), _ptr(W1), _ptr(Y),
                                             _stream(stream)), "caat_column_gemm_act")


def caat_row_gemm(handle, T, inp, W2, partials, stream=None):
    return _check(lib().caat_row_gemm(handle, int(T), _ptr(inp), _ptr(W2), _ptr(partials),
                                      _stream(stream)), "caat_row_gemm")


def caat_partial_sync_norm(handle, T, partials, resid, gamma, beta, out, out_resid, stream=None):
    return _check(lib().caat_partial_sync_norm(handle, int(T), _ptr(partials), _ptr(resid),
                                               _ptr(gamma), _ptr(beta), _ptr(out),
                                               _ptr(out_resid), _stream(stream)),
                  "caat_partial_sync_norm")


def caat_row_gemm_reduce(handle, T, inp, W2, S, partials, stream=None):
    return _check(lib().caat_row_gemm_reduce(handle, int(T), _ptr(inp), _ptr(W2), _ptr(S),
                                             _ptr(partials), _stream(stream)),
                  "caat_row_gemm_reduce")


def caat_sync_norm(handle, T, S, partials, resid, gamma, beta, out, out_resid, stream=None):
    return _check(lib().caat_sync_norm(handle, int(T), _ptr(S), _ptr(partials), _ptr(resid),
                                       _ptr(gamma), _ptr(beta), _ptr(out), _ptr(out_resid),
                                       _stream(stream)), "caat_sync_norm")


def caat_backward_workspace_bytes(handle, T) -> int:
    return int(lib().caat_backward_workspace_bytes(handle, int(T)))


def caat_backward(handle, T, inp, W1, W2, gamma, out_resid, dout, din, dW2, dgamma,
                  workspace, dW1=None, dres=None, dresid=None, dbeta=None, stream=None,
                  events=None, preact=None):
    """events: None, or CAAT_BWD_STEPS raw hipEvent_t handles (ints) recorded after
    each step (see BWD_STEPS).  preact: the pre-activation caat_forward_train stored
    (None: the backward recomputes it)."""
    ev = None
    if events is not None:
        ev = (ctypes.c_void_p * len(events))(*events)
    a = caat_bwd_args(int(T), _ptr(inp), _ptr(W1), _ptr(W2), _ptr(gamma), _ptr(out_resid),
                      _ptr(dout), _ptr(dres), _ptr(din), _ptr(dresid), _ptr(dW1), _ptr(dW2),
                      _ptr(dgamma), _ptr(dbeta), _ptr(workspace),
                      workspace.numel() * workspace.element_size(), _stream(stream),
                      ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p)) if ev is not None else None,
                      len(events) if events is not None else 0, _ptr(preact))
    return _check(lib().caat_backward(handle, ctypes.byref(a)), "caat_backward")


def caat_partial_sync_norm_backward(handle, T, out_resid, dout, dres, gamma, dpartials, dresid,
                                    dgamma, dbeta, workspace, stream=None):
    return _check(lib().caat_partial_sync_norm_backward(
        handle, int(T), _ptr(out_resid), _ptr(dout), _ptr(dres), _ptr(gamma), _ptr(dpartials),
        _ptr(dresid), _ptr(dgamma), _ptr(dbeta), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)),
        "caat_partial_sync_norm_backward")


def caat_attention_workspace_bytes(P, T, nh, d) -> int:
    return int(lib().caat_attention_workspace_bytes(int(P), int(T), int(nh), int(d)))


def caat_attention(P, T, S, nh, d, qkv, H, workspace, stream=None):
    return _check(lib().caat_attention(int(P), int(T), int(S), int(nh), int(d), _ptr(qkv), _ptr(H),
                                       _ptr(workspace), workspace.numel() * workspace.element_size(),
                                       _stream(stream)), "caat_attention")


def caat_block_workspace_bytes(attn, mlp, nh, T) -> int:
    return int(lib().caat_block_workspace_bytes(attn, mlp, int(nh), int(T)))


def caat_block_forward(attn, mlp, nh, T, S, inp, resid, Wqkv, Wo, W1, W2, gamma_attn, gamma_mlp,
                       out, out_resid, workspace, beta_attn=None, beta_mlp=None, stream=None,
                       events=None):
    """events: None, or raw hipEvent_t handles recorded after each of BLOCK_STEPS."""
    ev = (ctypes.c_void_p * len(events))(*events) if events is not None else None
    a = caat_block_args(int(T), int(S), _ptr(inp), _ptr(resid), _ptr(Wqkv), _ptr(Wo), _ptr(W1),
                        _ptr(W2), _ptr(gamma_attn), _ptr(beta_attn), _ptr(gamma_mlp),
                        _ptr(beta_mlp), _ptr(out), _ptr(out_resid), _ptr(workspace),
                        workspace.numel() * workspace.element_size(), _stream(stream),
                        ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p)) if ev is not None else None,
                        len(events) if events is not None else 0)
    return _check(lib().caat_block_forward(attn, mlp, int(nh), ctypes.byref(a)),
                  "caat_block_forward")


class Sublayer:
    """One sublayer handle plus a torch-allocated workspace; checks tensor shapes and
    dtypes, then calls the C entry points (no arithmetic here)."""

    def __init__(self, h, ffn, P, p, norm="layernorm", act="gelu", dtype="bf16", eps=1e-5,
                 s_priv=1.0):
        import torch
        self.h, self.P, self.p = int(h), int(P), float(p)
        self.act = ACT[act] if isinstance(act, str) else int(act)
        self.norm = NORM[norm] if isinstance(norm, str) else int(norm)
        self.dtype_code = DTYPE[dtype] if isinstance(dtype, str) else int(dtype)
        self.torch_dtype = torch.bfloat16 if self.dtype_code == BF16 else torch.float32
        self.ffn = 0 if self.act == NONE else int(ffn)
        self.handle = caat_create(self.h, self.ffn, self.P, self.p, self.norm, self.act,
                                  self.dtype_code)
        caat_set_eps(self.handle, eps)
        caat_set_private_scale(self.handle, s_priv)
        self.n_s = caat_shared_channels(self.handle)
        self.f_s = self.ffn // self.P if self.act != NONE else 0
        self.kin = self.h // self.P if self.act == NONE else self.h
        self._ws = None
        self._ws_T = 0

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _lib is not None:
            _lib.caat_destroy(h)
            self.handle = None

    def workspace(self, T, device="cuda"):
        import torch
        if self._ws is None or self._ws_T < T:
            nbytes = caat_workspace_bytes(self.handle, T)
            self._ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
            self._ws_T = T
            caat_set_workspace(self.handle, self._ws)
        return self._ws

    def _expect(self, t, shape, name):
        if t is None:
            return
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.dtype != self.torch_dtype:
            raise ValueError(f"{name}: dtype {t.dtype}, expected {self.torch_dtype}")

    def forward(self, inp, W1, W2, gamma, out, resid=None, beta=None, out_resid=None, stream=None,
                preact=None, events=None):
        """preact (MLP only): a [P][T][F1] tensor that also receives the raw pre-activation
        (caat_forward_train), for a backward that then skips its recompute GEMM.
        events: raw hipEvent_t handles recorded after each of FWD_STEPS
        (caat_forward_timed)."""
        P, h = self.P, self.h
        T = inp.shape[1]
        self._expect(inp, (P, T, self.kin), "in")
        if self.act != NONE:
            F1 = 2 * self.f_s if self.act == SWIGLU else self.f_s
            self._expect(W1, (P, F1, h), "W1")
        self._expect(W2, (P, h, self.f_s if self.act != NONE else self.kin), "W2")
        self._expect(gamma, (h,), "gamma")
        self._expect(beta, (h,), "beta")
        self._expect(resid, (P, T, h), "resid")
        self._expect(out, (P, T, h), "out")
        self._expect(out_resid, (P, T, h), "out_resid")
        self.workspace(T, inp.device)
        if preact is not None:
            if self.act == NONE:
                raise ValueError("preact: the out-projection has no pre-activation")
            self._expect(preact, (P, T, F1), "preact")
            if events is not None:
                raise ValueError("events: not with preact")
            return caat_forward_train(self.handle, T, inp, W1, W2, gamma, out, preact,
                                      resid=resid, beta=beta, out_resid=out_resid, stream=stream)
        if events is not None:
            return caat_forward_timed(self.handle, T, inp, W1 if self.act != NONE else None, W2,
                                      gamma, out, events, resid=resid, beta=beta,
                                      out_resid=out_resid, stream=stream)
        return caat_forward_ex(self.handle, T, inp, W1 if self.act != NONE else None, W2, gamma,
                               out, resid=resid, beta=beta, out_resid=out_resid, stream=stream)

    def backward(self, inp, W1, W2, gamma, out_resid, dout, din, dW2, dgamma, dW1=None,
                 dres=None, dresid=None, dbeta=None, stream=None, events=None, preact=None):
        """Gradients of one sublayer (shape and dtype checks, then caat_backward)."""
        import torch
        P, h = self.P, self.h
        T = inp.shape[1]
        self._expect(inp, (P, T, self.kin), "in")
        self._expect(din, (P, T, self.kin), "din")
        k2 = self.f_s if self.act != NONE else self.kin
        self._expect(W2, (P, h, k2), "W2")
        self._expect(dW2, (P, h, k2), "dW2")
        if self.act != NONE:
            F1 = 2 * self.f_s if self.act == SWIGLU else self.f_s
            self._expect(W1, (P, F1, h), "W1")
            self._expect(dW1, (P, F1, h), "dW1")
            self._expect(preact, (P, T, F1), "preact")
        for name, t in (("out_resid", out_resid), ("dout", dout), ("dres", dres),
                        ("dresid", dresid)):
            self._expect(t, (P, T, h), name)
        self._expect(gamma, (h,), "gamma")
        for name, t in (("dgamma", dgamma), ("dbeta", dbeta)):
            if t is not None and (tuple(t.shape) != (h,) or t.dtype != torch.float32):
                raise ValueError(f"{name}: expected float32 [{h}]")
        nbytes = caat_backward_workspace_bytes(self.handle, T)
        if getattr(self, "_bws", None) is None or self._bws.numel() < nbytes:
            self._bws = torch.empty(nbytes, dtype=torch.uint8, device=inp.device)
        return caat_backward(self.handle, T, inp, W1 if self.act != NONE else None, W2, gamma,
                             out_resid, dout, din, dW2, dgamma, self._bws, dW1=dW1, dres=dres,
                             dresid=dresid, dbeta=dbeta, stream=stream, events=events,
                             preact=preact)


class Block:
    """One transformer block with partially synchronized activations (QKV projection,
    attention core, out-projection sublayer, MLP sublayer), every rank on this device:
    two Sublayer handles plus the block workspace, then caat_block_forward."""

    def __init__(self, h, ffn, P, p, heads_per_rank, norm="rmsnorm", act="swiglu", eps=1e-5,
                 s_priv=1.0):
        self.attn = Sublayer(h, 0, P, p, norm=norm, act="none", dtype="bf16", eps=eps,
                             s_priv=s_priv)
        self.mlp = Sublayer(h, ffn, P, p, norm=norm, act=act, dtype="bf16", eps=eps, s_priv=s_priv)
        self.h, self.P, self.nh = int(h), int(P), int(heads_per_rank)
        self._ws = None

    def forward(self, T, S, inp, resid, Wqkv, Wo, W1, W2, gamma_attn, gamma_mlp, out, out_resid,
                beta_attn=None, beta_mlp=None, stream=None, events=None):
        import torch
        nbytes = caat_block_workspace_bytes(self.attn.handle, self.mlp.handle, self.nh, T)
        if nbytes == 0:
            raise ValueError("these handles and head count do not form a block")
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.empty(nbytes, dtype=torch.uint8, device=inp.device)
        self.attn.workspace(T, inp.device)
        self.mlp.workspace(T, inp.device)
        return caat_block_forward(self.attn.handle, self.mlp.handle, self.nh, T, S, inp, resid,
                                  Wqkv, Wo, W1, W2, gamma_attn, gamma_mlp, out, out_resid,
                                  self._ws, beta_attn=beta_attn, beta_mlp=beta_mlp, stream=stream,
                                  events=events)
