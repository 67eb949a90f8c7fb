"""ctypes front end of the FP64 KDA oracle (``kda_oracle.cpp``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``. The product library never
imports, links or runs anything in this directory.

The oracle takes its inputs as exact FP64 copies of the values the GPU path
receives (bf16 and fp32 values widen to FP64 without rounding) and returns
FP64 results. It computes the token-by-token gated delta rule of the
deterministic KDA training package (flashinfer PR #8909, opening section:
gate form g or raw, optional fused Q/K L2 norm) over documents packed by
``cu_seqlens`` (flashinfer PR #7176, opening section), and the hand-derived
reverse recurrence of ``L = sum <o, dO>``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.cpp")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lock = threading.Lock()
_lib = None


class _Problem(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("H", ctypes.c_int32),
        ("N", ctypes.c_int32),
        ("K", ctypes.c_int32),
        ("V", ctypes.c_int32),
        ("gate_raw", ctypes.c_int32),
        ("l2norm", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("l2_eps", ctypes.c_double),
    ]


def compile_source(src: str, out: str) -> str:
    """Compile an oracle source file to a shared library (g++, -O2, no FMA
    contraction, no fast-math)."""
    tmp = out + f".tmp{os.getpid()}"
    subprocess.run(
        ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
         "-shared", "-pthread", src, "-o", tmp],
        check=True,
    )
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile ``kda_oracle.cpp`` next to itself unless an up-to-date build exists."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB)
    return _LIB


def open_library(path: str):
    """Load an oracle build from ``path`` and declare its entry points."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lp = ctypes.POINTER(ctypes.c_int64)
    pp = ctypes.POINTER(_Problem)
    lib.kda_oracle_fwd.argtypes = [pp, lp] + [dp] * 11 + [ctypes.c_int, ctypes.c_int]
    lib.kda_oracle_fwd.restype = ctypes.c_int
    lib.kda_oracle_bwd.argtypes = [pp, lp] + [dp] * 18 + [ctypes.c_int]
    lib.kda_oracle_bwd.restype = ctypes.c_int
    return lib


def _load(lib=None):
    global _lib
    if lib is not None:
        return lib
    with _lock:
        if _lib is None:
            _lib = open_library(build())
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f64(x):
    if x is None:
        return None
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    return a


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


class _Args:
    def __init__(self, cu_seqlens, q, k, v, beta, gate, A_log, dt_bias, gate_form, l2norm,
                 scale, l2_eps):
        self.cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        self.q, self.k, self.v = _f64(q), _f64(k), _f64(v)
        self.beta, self.gate = _f64(beta), _f64(gate)
        T, H, K = self.q.shape
        V = self.v.shape[2]
        if self.k.shape != (T, H, K) or self.v.shape[:2] != (T, H) or self.beta.shape != (T, H):
            raise ValueError("shape mismatch")
        if self.gate.shape != (T, H, K):
            raise ValueError("gate must be [T,H,K]")
        raw = gate_form == "raw"
        if gate_form not in ("g", "raw"):
            raise ValueError(f"unknown gate form {gate_form!r}")
        self.A_log = _f64(A_log) if raw else None
        self.dt_bias = _f64(dt_bias) if raw else None
        if raw and (self.A_log.shape != (H,) or self.dt_bias.shape != (H, K)):
            raise ValueError("A_log must be [H], dt_bias [H,K]")
        if scale is None:
            scale = K ** -0.5
        self.P = _Problem(T, H, len(self.cu) - 1, K, V, int(raw), int(bool(l2norm)),
                          float(scale), float(l2_eps))
        self.T, self.H, self.K, self.V = T, H, K, V
        self.raw = raw


def _state(x, a):
    if x is None:
        return None
    x = _f64(x)
    if x.shape != (a.H, a.K, a.V):
        raise ValueError("a boundary state must be [H,K,V]")
    return x


def fwd(cu_seqlens, q, k, v, beta, gate, A_log=None, dt_bias=None, *, gate_form="g",
        l2norm=False, scale=None, l2_eps=1e-6, chunk=None, threads=None, lib=None,
        s_init=None, final_state=False):
    """Forward. Returns o [T,H,V] (float64), and with ``chunk`` also the
    state at the start of every chunk: [n_chunks, H, K, V], chunks restarting
    at each document start, ordered by document then chunk. ``s_init``
    [H,K,V] is the state entering document 0 (zero if None); with
    ``final_state`` the state leaving the last document is returned last."""
    a = _Args(cu_seqlens, q, k, v, beta, gate, A_log, dt_bias, gate_form, l2norm, scale, l2_eps)
    o = np.zeros((a.T, a.H, a.V))
    states = None
    if chunk:
        lens = np.diff(a.cu)
        nch = int(np.sum((lens + chunk - 1) // chunk))
        states = np.zeros((nch, a.H, a.K, a.V))
    s_in = _state(s_init, a)
    s_fin = np.zeros((a.H, a.K, a.V)) if final_state else None
    lib = _load(lib)
    rc = lib.kda_oracle_fwd(ctypes.byref(a.P), a.cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                            _ptr(a.q), _ptr(a.k), _ptr(a.v), _ptr(a.beta), _ptr(a.gate),
                            _ptr(a.A_log), _ptr(a.dt_bias), _ptr(s_in), _ptr(o), _ptr(s_fin),
                            _ptr(states), int(chunk or 0), int(threads or default_threads()))
    if rc != 0:
        raise ValueError("kda_oracle_fwd rejected its arguments")
    out = (o,) + ((states,) if chunk else ()) + ((s_fin,) if final_state else ())
    return out if len(out) > 1 else o


def bwd(cu_seqlens, q, k, v, beta, gate, dO, A_log=None, dt_bias=None, *, gate_form="g",
        l2norm=False, scale=None, l2_eps=1e-6, threads=None, lib=None, s_init=None,
        ds_final=None):
    """Backward of L = sum(o * dO) + <S_final, ds_final>. Returns a dict with
    dq, dk, dv, dbeta and dg (g form) or da, dA_log, ddt_bias (raw form), and,
    when s_init or ds_final is given, ds_init (the gradient w.r.t. the state
    entering document 0, [H,K,V]), all float64."""
    a = _Args(cu_seqlens, q, k, v, beta, gate, A_log, dt_bias, gate_form, l2norm, scale, l2_eps)
    dO = _f64(dO)
    if dO.shape != (a.T, a.H, a.V):
        raise ValueError("dO must be [T,H,V]")
    dq = np.zeros((a.T, a.H, a.K))
    dk = np.zeros((a.T, a.H, a.K))
    dv = np.zeros((a.T, a.H, a.V))
    dbeta = np.zeros((a.T, a.H))
    dgate = np.zeros((a.T, a.H, a.K))
    dA_log = np.zeros(a.H) if a.raw else None
    ddt = np.zeros((a.H, a.K)) if a.raw else None
    s_in, ds_fin = _state(s_init, a), _state(ds_final, a)
    ds_init = np.zeros((a.H, a.K, a.V)) if a.P.N > 0 else None
    lib = _load(lib)
    rc = lib.kda_oracle_bwd(ctypes.byref(a.P), a.cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                            _ptr(a.q), _ptr(a.k), _ptr(a.v), _ptr(a.beta), _ptr(a.gate),
                            _ptr(a.A_log), _ptr(a.dt_bias), _ptr(s_in), _ptr(dO), _ptr(ds_fin),
                            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbeta), _ptr(dgate), _ptr(dA_log),
                            _ptr(ddt), _ptr(ds_init), int(threads or default_threads()))
    if rc != 0:
        raise ValueError("kda_oracle_bwd rejected its arguments")
    out = {"dq": dq, "dk": dk, "dv": dv, "dbeta": dbeta}
    if s_init is not None or ds_final is not None:
        out["ds_init"] = ds_init
    if a.raw:
        out.update(da=dgate, dA_log=dA_log, ddt_bias=ddt)
    else:
        out["dg"] = dgate
    return out
