"""Python binding of libkda.so (see include/kda.h for the contract).

Argument marshalling only: every step of the KDA path runs in the library's
HIP kernels. torch supplies device memory and the current stream. There is
no CPU fallback: if the library is missing, loading fails with an error.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_GATE_G = 0
KDA_GATE_RAW = 1
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small",
          4: "device error"}


class KdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class kda_problem(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("H", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("dk", ctypes.c_int32),
        ("dv", ctypes.c_int32),
        ("gate", ctypes.c_int32),
        ("l2norm", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("l2_eps", ctypes.c_float),
    ]


class kda_attn_problem(ctypes.Structure):
    _fields_ = [
        ("Tq", ctypes.c_int64),
        ("Tk", ctypes.c_int64),
        ("num_seqs", ctypes.c_int32),
        ("Hq", ctypes.c_int32),
        ("Hkv", ctypes.c_int32),
        ("D", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


class kda_conv_problem(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("D", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("width", ctypes.c_int32),
        ("has_bias", ctypes.c_int32),
        ("has_halo", ctypes.c_int32),
    ]


_lib = None
EXPORTS = ("kda_saved_bytes", "kda_workspace_bytes", "kda_fwd", "kda_bwd", "kda_fwd_noalloc",
           "kda_set_launch_hook", "kda_status_string", "kda_last_error", "kda_abi_version",
           "kda_conv_workspace_bytes", "kda_conv_silu_fwd", "kda_conv_silu_bwd",
           "kda_attn_workspace_bytes", "kda_attn_fwd", "kda_attn_bwd",
           "kda_fwd_state", "kda_bwd_state", "kda_state_summary_workspace_bytes",
           "kda_state_summary", "kda_state_grad_summary", "kda_state_apply")
ATTN_DKV_BF16, ATTN_DKV_F32, ATTN_DKV_F32_ADD = 0, 1, 2   # kda_attn.h
NOALLOC_SCRATCH_BYTES = 64 << 20   # KDA_NOALLOC_SCRATCH_BYTES in kda.h
LAUNCH_HOOK = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_char_p, ctypes.c_int,
                               ctypes.c_void_p)


def lib():
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m kda_chunked_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        pp = ctypes.POINTER(kda_problem)
        L.kda_saved_bytes.argtypes = [pp]
        L.kda_saved_bytes.restype = sz
        L.kda_workspace_bytes.argtypes = [pp, ctypes.c_int, ctypes.c_int]
        L.kda_workspace_bytes.restype = sz
        L.kda_fwd.argtypes = [pp] + [vp] * 11 + [sz, vp]
        L.kda_fwd.restype = ctypes.c_int
        L.kda_bwd.argtypes = [pp] + [vp] * 18 + [sz, vp]
        L.kda_bwd.restype = ctypes.c_int
        L.kda_fwd_noalloc.argtypes = [pp] + [vp] * 11
        L.kda_fwd_noalloc.restype = ctypes.c_int
        cp = ctypes.POINTER(kda_conv_problem)
        L.kda_conv_workspace_bytes.argtypes = [cp, ctypes.c_int]
        L.kda_conv_workspace_bytes.restype = sz
        L.kda_conv_silu_fwd.argtypes = [cp] + [vp] * 7 + [sz, vp]
        L.kda_conv_silu_fwd.restype = ctypes.c_int
        L.kda_conv_silu_bwd.argtypes = [cp] + [vp] * 11 + [sz, vp]
        L.kda_conv_silu_bwd.restype = ctypes.c_int
        L.kda_fwd_state.argtypes = [pp] + [vp] * 12 + [ctypes.c_int, vp, sz, vp]
        L.kda_fwd_state.restype = ctypes.c_int
        L.kda_bwd_state.argtypes = [pp] + [vp] * 21 + [sz, vp]
        L.kda_bwd_state.restype = ctypes.c_int
        L.kda_state_summary_workspace_bytes.argtypes = [pp]
        L.kda_state_summary_workspace_bytes.restype = sz
        L.kda_state_summary.argtypes = [pp] + [vp] * 12 + [sz, vp]
        L.kda_state_summary.restype = ctypes.c_int
        L.kda_state_grad_summary.argtypes = [pp] + [vp] * 12 + [sz, vp]
        L.kda_state_grad_summary.restype = ctypes.c_int
        L.kda_state_apply.argtypes = [ctypes.c_int32, vp, ctypes.c_int, vp, vp, vp, vp]
        L.kda_state_apply.restype = ctypes.c_int
        ap = ctypes.POINTER(kda_attn_problem)
        L.kda_attn_workspace_bytes.argtypes = [ap, ctypes.c_int, ctypes.c_int64]
        L.kda_attn_workspace_bytes.restype = sz
        L.kda_attn_fwd.argtypes = [ap] + [vp] * 8 + [sz, vp]
        L.kda_attn_fwd.restype = ctypes.c_int
        L.kda_attn_bwd.argtypes = ([ap] + [vp] * 11 + [ctypes.c_int, vp, ctypes.c_int64, vp, sz,
                                                       vp])
        L.kda_attn_bwd.restype = ctypes.c_int
        L.kda_status_string.argtypes = [ctypes.c_int]
        L.kda_status_string.restype = ctypes.c_char_p
        L.kda_last_error.argtypes = []
        L.kda_last_error.restype = ctypes.c_char_p
        L.kda_abi_version.argtypes = []
        L.kda_abi_version.restype = ctypes.c_int
        L.kda_set_launch_hook.argtypes = [LAUNCH_HOOK, ctypes.c_void_p]
        L.kda_set_launch_hook.restype = None
        _lib = L
    return _lib


_hook_ref = None


def set_launch_hook(fn):
    """Install fn(kernel_name: str, end: bool, stream: int) as the library's
    launch hook (None removes it)."""
    global _hook_ref
    if fn is None:
        _hook_ref = None
        lib().kda_set_launch_hook(LAUNCH_HOOK(), None)
        return
    _hook_ref = LAUNCH_HOOK(lambda user, name, end, stream: fn(name.decode(), bool(end), stream))
    lib().kda_set_launch_hook(_hook_ref, None)


def problem(T, H, num_seqs, gate="g", l2norm=False, scale=None, l2_eps=1e-6, dk=128, dv=128):
    if gate not in ("g", "raw"):
        raise ValueError(f"gate must be 'g' or 'raw', got {gate!r}")
    if scale is None:
        scale = dk ** -0.5
    return kda_problem(int(T), int(H), int(num_seqs), int(dk), int(dv),
                       KDA_GATE_RAW if gate == "raw" else KDA_GATE_G, int(bool(l2norm)),
                       float(scale), float(l2_eps))


def saved_bytes(p: kda_problem) -> int:
    return int(lib().kda_saved_bytes(ctypes.byref(p)))


def workspace_bytes(p: kda_problem, backward: bool, replay: bool = False) -> int:
    return int(lib().kda_workspace_bytes(ctypes.byref(p), int(bool(backward)), int(bool(replay))))


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else None


def _check(rc):
    if rc != 0:
        raise KdaError(rc, lib().kda_last_error().decode())


def _stream(device):
    if device is None:
        return None
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(p, tensors):
    """The device of the call. Host tensors are refused for a valid problem (the
    library would hand host addresses to its kernels); for an invalid problem
    the library's own validation reports the error before any launch."""
    ts = [t for t in tensors if t is not None]
    if all(t.is_cuda for t in ts):
        return ts[0].device
    if lib().kda_saved_bytes(ctypes.byref(p)) != 0:
        raise ValueError("every tensor passed to the KDA library must be on the GPU")
    return None


class _nullctx:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


def _device_ctx(dev):
    return torch.cuda.device(dev) if dev is not None else _nullctx()


def kda_fwd(p, q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens, o, saved, workspace):
    """Enqueue the forward on the current stream of q's device (made current)."""
    dev = _dev(p, (q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens, o, saved, workspace))
    with _device_ctx(dev):
        rc = lib().kda_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g_or_a),
                           _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens), _ptr(o), _ptr(saved),
                           _ptr(workspace), workspace.numel() * workspace.element_size(),
                           _stream(dev))
    _check(rc)


def kda_fwd_noalloc(p, q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens, o, saved):
    """kda_fwd without a workspace argument (the library's fixed per-GPU
    scratch serves instead); enqueued on the current stream of q's device."""
    dev = _dev(p, (q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens, o, saved))
    with _device_ctx(dev):
        rc = lib().kda_fwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                   _ptr(g_or_a), _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens),
                                   _ptr(o), _ptr(saved), _stream(dev))
    _check(rc)


def kda_bwd(p, q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens, dO, saved, dq, dk, dv,
            dbeta, dg_or_da, dA_log, ddt_bias, workspace):
    """Enqueue the backward on the current stream of q's device (made current).
    saved=None selects the replay backward."""
    dev = _dev(p, (q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens, dO, saved, dq, dk, dv,
                   dbeta, dg_or_da, dA_log, ddt_bias, workspace))
    with _device_ctx(dev):
        rc = lib().kda_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                           _ptr(g_or_a), _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens), _ptr(dO),
                           _ptr(saved), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbeta),
                           _ptr(dg_or_da), _ptr(dA_log), _ptr(ddt_bias), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream(dev))
    _check(rc)


FWD_PREP_DONE = 1   # kda_fwd_state: the saved set holds kda_state_summary's prep


def kda_fwd_state(p, q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens, s_init, o, s_final,
                  saved, workspace, flags=0):
    """kda_fwd with the state entering document 0 (s_init, None: zero) and the
    state leaving the last document written to s_final (None: not written);
    states fp32 [H,128,128]."""
    dev = _dev(p, (q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens, s_init, o, s_final, saved,
                   workspace))
    with _device_ctx(dev):
        rc = lib().kda_fwd_state(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                 _ptr(g_or_a), _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens),
                                 _ptr(s_init), _ptr(o), _ptr(s_final), _ptr(saved), int(flags),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(dev))
    _check(rc)


def kda_bwd_state(p, q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens, s_init, dO, ds_final,
                  saved, dq, dk, dv, dbeta, dg_or_da, dA_log, ddt_bias, ds_init, workspace):
    """kda_bwd of sum <o, dO> + <s_final, ds_final>, writing ds_init."""
    dev = _dev(p, (q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens, s_init, dO, ds_final,
                   saved, dq, dk, dv, dbeta, dg_or_da, dA_log, ddt_bias, ds_init, workspace))
    with _device_ctx(dev):
        rc = lib().kda_bwd_state(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                 _ptr(g_or_a), _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens),
                                 _ptr(s_init), _ptr(dO), _ptr(ds_final), _ptr(saved), _ptr(dq),
                                 _ptr(dk), _ptr(dv), _ptr(dbeta), _ptr(dg_or_da), _ptr(dA_log),
                                 _ptr(ddt_bias), _ptr(ds_init), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(dev))
    _check(rc)


def state_summary_workspace_bytes(p) -> int:
    return int(lib().kda_state_summary_workspace_bytes(ctypes.byref(p)))


def _nbytes_or0(t):
    return t.numel() * t.element_size() if t is not None else 0


def kda_state_summary(p, q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens, M, B, workspace,
                      saved=None):
    """The fragment's map s_final = M s_init + B (M, B fp32 [H,128,128] or None);
    saved, when given, receives the prep for kda_fwd_state(flags=FWD_PREP_DONE)."""
    dev = _dev(p, (q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens, M, B, saved, workspace))
    with _device_ctx(dev):
        rc = lib().kda_state_summary(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                     _ptr(g_or_a), _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens),
                                     _ptr(M), _ptr(B), _ptr(saved), _ptr(workspace),
                                     _nbytes_or0(workspace), _stream(dev))
    _check(rc)


def kda_state_grad_summary(p, q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens, dO, saved, dB,
                           workspace):
    """dB fp32 [H,128,128]: the gradient w.r.t. s_init with a zero gradient of
    s_final (saved: the saving forward's set, or None to rebuild its panels)."""
    dev = _dev(p, (q, k, v, beta, g_or_a, A_log, dt_bias, cu_seqlens, dO, saved, dB, workspace))
    with _device_ctx(dev):
        rc = lib().kda_state_grad_summary(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                          _ptr(g_or_a), _ptr(A_log), _ptr(dt_bias),
                                          _ptr(cu_seqlens), _ptr(dO), _ptr(saved), _ptr(dB),
                                          _ptr(workspace), _nbytes_or0(workspace), _stream(dev))
    _check(rc)


def kda_state_apply(M, x, B=None, transpose=False, y=None):
    """y = M x + B (or M^T x + B) per head; M, x, B fp32 [H,128,128] on one GPU."""
    if y is None:
        y = torch.empty_like(x)
    if not (M.is_cuda and x.is_cuda and y.is_cuda and (B is None or B.is_cuda)):
        raise ValueError("kda_state_apply takes GPU tensors")
    with _device_ctx(x.device):
        rc = lib().kda_state_apply(int(x.shape[0]), _ptr(M), int(bool(transpose)), _ptr(B),
                                   _ptr(x), _ptr(y), _stream(x.device))
    _check(rc)
    return y


class KDA:
    """Holds the buffers of one problem shape and runs forward / backward.

    Inputs are torch tensors on one GPU: q, k, v [T,H,128] bf16; beta [T,H]
    bf16; gate g [T,H,128] fp32 or a [T,H,128] bf16 with A_log [H] and
    dt_bias [H,128] fp32; cu_seqlens [N+1] int32."""

    def __init__(self, T, H, num_seqs, gate="g", l2norm=False, scale=None, l2_eps=1e-6,
                 device="cuda"):
        self.p = problem(T, H, num_seqs, gate, l2norm, scale, l2_eps)
        self.gate = gate
        self.device = torch.device(device)
        nbytes = max(workspace_bytes(self.p, False, True), workspace_bytes(self.p, True, True))
        u8 = dict(dtype=torch.uint8, device=self.device)
        self.workspace = torch.empty(max(nbytes, 1), **u8)
        self.saved = torch.empty(max(saved_bytes(self.p), 1), **u8)
        self.summary_ws = None     # the state summaries' workspace, made on first use

    def forward(self, q, k, v, beta, gate, cu_seqlens, A_log=None, dt_bias=None, save=True,
                o=None, s_init=None, s_final=None, prep_done=False):
        """o; with s_init / s_final (fp32 [H,128,128]) document 0 enters from
        s_init and the state leaving the last document goes to s_final;
        prep_done: the saved set holds state_summary(keep_prep=True)'s prep."""
        if o is None:
            o = torch.empty_like(v)
        saved = self.saved if save else None
        if prep_done:
            kda_fwd_state(self.p, q, k, v, beta, gate, A_log, dt_bias, cu_seqlens, s_init, o,
                          s_final, saved, self.workspace, flags=FWD_PREP_DONE)
        elif s_init is None and s_final is None:
            kda_fwd(self.p, q, k, v, beta, gate, A_log, dt_bias, cu_seqlens, o, saved,
                    self.workspace)
        else:
            kda_fwd_state(self.p, q, k, v, beta, gate, A_log, dt_bias, cu_seqlens, s_init, o,
                          s_final, saved, self.workspace)
        return o

    def backward(self, q, k, v, beta, gate, cu_seqlens, dO, A_log=None, dt_bias=None,
                 replay=False, out=None, s_init=None, ds_final=None, ds_init=None):
        """Gradients; with s_init / ds_final / ds_init the boundary-state form
        (ds_init, when given, receives the gradient w.r.t. s_init)."""
        if out is None:
            out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                       dbeta=torch.empty_like(beta), dgate=torch.empty_like(gate))
            if self.gate == "raw":
                out["dA_log"] = torch.empty_like(A_log)
                out["ddt_bias"] = torch.empty_like(dt_bias)
        saved = None if replay else self.saved
        if s_init is None and ds_final is None and ds_init is None:
            kda_bwd(self.p, q, k, v, beta, gate, A_log, dt_bias, cu_seqlens, dO, saved,
                    out["dq"], out["dk"], out["dv"], out["dbeta"], out["dgate"],
                    out.get("dA_log"), out.get("ddt_bias"), self.workspace)
        else:
            kda_bwd_state(self.p, q, k, v, beta, gate, A_log, dt_bias, cu_seqlens, s_init, dO,
                          ds_final, saved, out["dq"], out["dk"], out["dv"], out["dbeta"],
                          out["dgate"], out.get("dA_log"), out.get("ddt_bias"), ds_init,
                          self.workspace)
            if ds_init is not None:
                out["ds_init"] = ds_init
        return out

    def _summary_ws(self, device):
        if self.summary_ws is None:
            n = max(state_summary_workspace_bytes(self.p), 16)
            self.summary_ws = torch.empty(n, dtype=torch.uint8, device=device)
        return self.summary_ws

    def state_summary(self, q, k, v, beta, gate, cu_seqlens, A_log=None, dt_bias=None,
                      want_M=True, want_B=True, keep_prep=False):
        """(M, B) fp32 [H,128,128] (None where not wanted): s_final = M s_init + B.
        keep_prep: the prep goes to this object's saved set, for a following
        forward(..., prep_done=True) on the same inputs."""
        st = lambda: torch.empty(self.p.H, 128, 128, dtype=torch.float32, device=q.device)
        M = st() if want_M else None
        B = st() if want_B else None
        kda_state_summary(self.p, q, k, v, beta, gate, A_log, dt_bias, cu_seqlens, M, B,
                          self._summary_ws(q.device), self.saved if keep_prep else None)
        return M, B

    def state_grad_summary(self, q, k, v, beta, gate, cu_seqlens, dO, A_log=None, dt_bias=None,
                           replay=False):
        """dB fp32 [H,128,128]: ds_init with a zero ds_final, from this object's
        saved set (a saving forward ran last) or, with replay, rebuilt."""
        dB = torch.empty(self.p.H, 128, 128, dtype=torch.float32, device=q.device)
        kda_state_grad_summary(self.p, q, k, v, beta, gate, A_log, dt_bias, cu_seqlens, dO,
                               None if replay else self.saved, dB, self._summary_ws(q.device))
        return dB


# ---------------------------------------------------------------- conv1d + SiLU

def conv_problem(T, D, num_seqs, bias=False, halo=False, width=4):
    return kda_conv_problem(int(T), int(D), int(num_seqs), int(width), int(bool(bias)),
                            int(bool(halo)))


def conv_workspace_bytes(p: kda_conv_problem, backward: bool) -> int:
    return int(lib().kda_conv_workspace_bytes(ctypes.byref(p), int(bool(backward))))


def conv_silu_fwd(p, x, w, b, halo, cu_seqlens, y, workspace=None):
    """Enqueue the conv1d + SiLU forward on the current stream of x's device."""
    dev = _dev_conv(p, (x, w, b, halo, cu_seqlens, y, workspace))
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with _device_ctx(dev):
        rc = lib().kda_conv_silu_fwd(ctypes.byref(p), _ptr(x), _ptr(w), _ptr(b), _ptr(halo),
                                     _ptr(cu_seqlens), _ptr(y), _ptr(workspace), nbytes,
                                     _stream(dev))
    _check(rc)


def conv_silu_bwd(p, x, w, b, halo, cu_seqlens, dy, dx, dw, db, dhalo, workspace):
    """Enqueue the conv1d + SiLU backward on the current stream of x's device."""
    dev = _dev_conv(p, (x, w, b, halo, cu_seqlens, dy, dx, dw, db, dhalo, workspace))
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with _device_ctx(dev):
        rc = lib().kda_conv_silu_bwd(ctypes.byref(p), _ptr(x), _ptr(w), _ptr(b), _ptr(halo),
                                     _ptr(cu_seqlens), _ptr(dy), _ptr(dx), _ptr(dw), _ptr(db),
                                     _ptr(dhalo), _ptr(workspace), nbytes, _stream(dev))
    _check(rc)


def _dev_conv(p, tensors):
    ts = [t for t in tensors if t is not None]
    if ts and all(t.is_cuda for t in ts):
        return ts[0].device
    if lib().kda_conv_workspace_bytes(ctypes.byref(p), 0) != 0 or \
            lib().kda_conv_workspace_bytes(ctypes.byref(p), 1) != 0:
        raise ValueError("every tensor passed to the conv op must be on the GPU")
    return None


class ConvSiLU:
    """Width-4 causal conv1d + SiLU over packed documents (optionally after a
    halo of the 3 tokens preceding x[0] in document 0). x, dy [T, D] bf16;
    w [D, 4] fp32; b [D] fp32; halo [3, D] bf16; cu_seqlens [N+1] int32."""

    def __init__(self, T, D, num_seqs, bias=False, halo=False, device="cuda"):
        self.p = conv_problem(T, D, num_seqs, bias, halo)
        self.device = torch.device(device)
        n = max(conv_workspace_bytes(self.p, True), 16)
        self.workspace = torch.empty(n, dtype=torch.uint8, device=self.device)

    def forward(self, x, w, cu_seqlens, b=None, halo=None, y=None):
        if y is None:
            y = torch.empty_like(x)
        conv_silu_fwd(self.p, x, w, b, halo, cu_seqlens, y)
        return y

    def backward(self, x, w, cu_seqlens, dy, b=None, halo=None, out=None):
        if out is None:
            out = dict(dx=torch.empty_like(x), dw=torch.empty_like(w))
            if self.p.has_bias:
                out["db"] = torch.empty_like(b)
            if self.p.has_halo:
                out["dhalo"] = torch.empty_like(halo)
        conv_silu_bwd(self.p, x, w, b, halo, cu_seqlens, dy, out["dx"], out["dw"], out.get("db"),
                      out.get("dhalo"), self.workspace)
        return out


# ---------------------------------------------------------------- GQA attention

def attn_problem(Tq, Tk, num_seqs, Hq, Hkv, D=256, scale=None):
    scale = D ** -0.5 if scale is None else scale
    return kda_attn_problem(int(Tq), int(Tk), int(num_seqs), int(Hq), int(Hkv), int(D),
                            float(scale))


def attn_workspace_bytes(p: kda_attn_problem, stage: int, dst_rows: int = 0) -> int:
    return int(lib().kda_attn_workspace_bytes(ctypes.byref(p), int(stage), int(dst_rows)))


def _dev_attn(p, tensors):
    ts = [t for t in tensors if t is not None]
    if ts and all(t.is_cuda for t in ts):
        return ts[0].device
    if attn_workspace_bytes(p, 0) != 0:
        raise ValueError("every tensor passed to the attention op must be on the GPU")
    return None


def _nbytes(t):
    return t.numel() * t.element_size() if t is not None else 0


def attn_fwd(p, q, k, v, cu_q, cu_k, o, lse, workspace):
    """Enqueue the attention forward on the current stream of q's device."""
    dev = _dev_attn(p, (q, k, v, cu_q, cu_k, o, lse, workspace))
    with _device_ctx(dev):
        rc = lib().kda_attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_q),
                                _ptr(cu_k), _ptr(o), _ptr(lse), _ptr(workspace),
                                _nbytes(workspace), _stream(dev))
    _check(rc)


def attn_bwd(p, q, k, v, cu_q, cu_k, o, lse, dO, dq, dk, dv, form, row_map, dst_rows,
             workspace):
    """Enqueue the attention backward on the current stream of q's device."""
    dev = _dev_attn(p, (q, k, v, cu_q, cu_k, o, lse, dO, dq, dk, dv, row_map, workspace))
    with _device_ctx(dev):
        rc = lib().kda_attn_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_q),
                                _ptr(cu_k), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq), _ptr(dk),
                                _ptr(dv), int(form), _ptr(row_map), int(dst_rows),
                                _ptr(workspace), _nbytes(workspace), _stream(dev))
    _check(rc)


class GQAAttention:
    """Packed-varlen causal GQA attention, head dim 256: q [Tq, Hq, 256] and
    k, v [Tk, Hkv, 256] bf16; cu_q, cu_k [num_seqs + 1] int32 on the device.
    One workspace serves the forward and every backward form; a larger one
    serves smaller problems too."""

    def __init__(self, Tq, Tk, num_seqs, Hq, Hkv, scale=None, dst_rows=None, device="cuda"):
        self.p = attn_problem(Tq, Tk, num_seqs, Hq, Hkv, 256, scale)
        self.device = torch.device(device)
        stage = 2 if dst_rows is not None else 1
        n = max(attn_workspace_bytes(self.p, stage, dst_rows or 0), 16)
        self.workspace = torch.empty(n, dtype=torch.uint8, device=self.device)

    def forward(self, q, k, v, cu_q, cu_k, o=None, lse=None, with_lse=True):
        if o is None:
            o = torch.empty_like(q)
        if lse is None and with_lse:
            lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
        attn_fwd(self.p, q, k, v, cu_q, cu_k, o, lse, self.workspace)
        return o, lse

    def backward(self, q, k, v, cu_q, cu_k, o, lse, dO, form=ATTN_DKV_BF16, dk=None, dv=None,
                 row_map=None, dst_rows=0, dq=None):
        """dq, dk, dv. Form ATTN_DKV_F32_ADD adds into the given fp32 dk, dv
        [dst_rows, Hkv, 256] through row_map [Tk] int32."""
        if dq is None:
            dq = torch.empty_like(q)
        if form != ATTN_DKV_F32_ADD:
            dt = torch.bfloat16 if form == ATTN_DKV_BF16 else torch.float32
            dk = torch.empty(k.shape, dtype=dt, device=k.device) if dk is None else dk
            dv = torch.empty(v.shape, dtype=dt, device=v.device) if dv is None else dv
        attn_bwd(self.p, q, k, v, cu_q, cu_k, o, lse, dO, dq, dk, dv, form, row_map, dst_rows,
                 self.workspace)
        return dq, dk, dv
