"""Plain fp64 CPU oracle of the gated delta rule -- TEST INFRASTRUCTURE ONLY.

This package is the yardstick the HIP library is checked against.  Only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import
it; the library itself never does, and the two share no code.

The arithmetic lives in ``gdr_oracle.c`` (a sequential token recurrence in
double precision, see the header there for the passages it follows).  This
module only builds that file with gcc, loads it with ctypes and converts
numpy arrays to contiguous float64.

Functions
---------
sequence(...)  token recurrence over [B,T,...] inputs (prefill layout)
decode(...)    one token from the packed q|k|v row (decode layout)
sigmoid, softplus, l2norm   the elementwise pieces, exposed for pin tests
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from pathlib import Path

import numpy as np

GATE_CHANNEL = 0
GATE_SCALAR = 1
GATE_SCALAR_FUSED = 2

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "gdr_oracle.c"
_LIB_PATH = _HERE / "libgdr_oracle.so"
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> Path:
    """Compile gdr_oracle.c into libgdr_oracle.so next to it (gcc, -O2, OpenMP)."""
    if force or not _LIB_PATH.exists() or _LIB_PATH.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB_PATH.with_name(f"{_LIB_PATH.name}.tmp{os.getpid()}")
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               str(_SRC), "-o", str(tmp), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(lib):
    """Declare the C signatures on a loaded oracle library and return it."""
    dp = ctypes.POINTER(ctypes.c_double)
    i = ctypes.c_int
    lib.gdr_oracle_sequence.argtypes = [i, i, i, i, i, i, dp, dp, dp, i, dp, dp, dp, dp,
                                        dp, dp, ctypes.c_double, i, i]
    lib.gdr_oracle_sequence.restype = i
    lib.gdr_oracle_decode.argtypes = [i, i, i, i, i, dp, i, dp, dp, dp, dp, dp, dp,
                                      ctypes.c_double, i, i]
    lib.gdr_oracle_decode.restype = i
    lib.orc_sigmoid.argtypes = [ctypes.c_double]
    lib.orc_sigmoid.restype = ctypes.c_double
    lib.orc_softplus.argtypes = [ctypes.c_double]
    lib.orc_softplus.restype = ctypes.c_double
    lib.orc_l2norm.argtypes = [dp, i, dp]
    lib.orc_l2norm.restype = None
    lib.gdr_oracle_threads.argtypes = [i]
    lib.gdr_oracle_threads.restype = i
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            _lib = _bind(ctypes.CDLL(str(_LIB_PATH)))
    return _lib


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def threads_used(threads: int) -> int:
    """Number of OpenMP threads the oracle really runs with for a request."""
    return int(_load().gdr_oracle_threads(int(threads)))


def sequence(q, k, v, gate_kind, gate_in, beta_logit, state0=None, A_log=None, dt_bias=None,
             scale=1.0, l2norm=True, threads=1):
    """Token recurrence over a sequence.

    q, k [B,T,H_qk,dk]; v [B,T,H_v,dv]; beta_logit [B,T,H_v];
    gate_in: g [B,T,H_v,dk] (GATE_CHANNEL), g [B,T,H_v] (GATE_SCALAR) or
    x [B,T,H_v] (GATE_SCALAR_FUSED, with A_log and dt_bias [H_v]);
    state0 [B,H_v,dk,dv] or None for zeros.
    Returns (o [B,T,H_v,dv], final state [B,H_v,dk,dv]) as float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T):
        raise ValueError("q/k/v shapes disagree")
    gate_in, beta_logit = _f64(gate_in), _f64(beta_logit)
    A_log, dt_bias = _f64(A_log), _f64(dt_bias)
    if state0 is None:
        S = np.zeros((B, Hv, dk, dv), np.float64)
    else:
        S = _f64(state0).copy()
    o = np.zeros((B, T, Hv, dv), np.float64)
    rc = _load().gdr_oracle_sequence(B, T, Hqk, Hv, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                     int(gate_kind), _ptr(gate_in), _ptr(A_log), _ptr(dt_bias),
                                     _ptr(beta_logit), _ptr(S), _ptr(o), float(scale),
                                     int(bool(l2norm)), int(threads))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (rc={rc})")
    return o, S


def decode(qkv, H_qk, H_v, dk, dv, gate_kind, gate_in, beta_logit, state, A_log=None,
           dt_bias=None, scale=1.0, l2norm=True, threads=1):
    """One decode token from the packed row qkv [B, 2*H_qk*dk + H_v*dv].

    gate_in: g [B,H_v,dk] | g [B,H_v] | x [B,H_v]; beta_logit [B,H_v];
    state [B,H_v,dk,dv] (not modified).  Returns (o [B,H_v,dv], new state).
    """
    qkv = _f64(qkv)
    B = qkv.shape[0]
    if qkv.shape[1] != 2 * H_qk * dk + H_v * dv:
        raise ValueError("packed row length disagrees with the head sizes")
    gate_in, beta_logit = _f64(gate_in), _f64(beta_logit)
    A_log, dt_bias = _f64(A_log), _f64(dt_bias)
    S = _f64(state).copy()
    o = np.zeros((B, H_v, dv), np.float64)
    rc = _load().gdr_oracle_decode(B, H_qk, H_v, dk, dv, _ptr(qkv), int(gate_kind),
                                   _ptr(gate_in), _ptr(A_log), _ptr(dt_bias), _ptr(beta_logit),
                                   _ptr(S), _ptr(o), float(scale), int(bool(l2norm)),
                                   int(threads))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (rc={rc})")
    return o, S


def sigmoid(x: float) -> float:
    return float(_load().orc_sigmoid(float(x)))


def softplus(x: float) -> float:
    return float(_load().orc_softplus(float(x)))


def l2norm(x) -> np.ndarray:
    x = _f64(x).ravel()
    out = np.empty_like(x)
    _load().orc_l2norm(_ptr(x), x.size, _ptr(out))
    return out
