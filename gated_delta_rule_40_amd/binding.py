"""ctypes binding of libgdr.so (include/gdr.h) for torch device tensors.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  torch supplies device memory and the current
stream.  The binding checks that each tensor matches the sizes it is passed
with (device, dtype, contiguity, element count) before handing raw pointers
over, so that a wrong tensor is a Python error rather than an out-of-bounds
access.  If the library has not been built, every call raises: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

GDR_F32, GDR_BF16 = 0, 1
GDR_GATE_CHANNEL, GDR_GATE_SCALAR, GDR_GATE_SCALAR_FUSED = 0, 1, 2
GDR_OK = 0

LIB_PATH = Path(__file__).resolve().parent / "libgdr.so"
EXPORTED = ("gdr_decode_step", "gdr_prefill_workspace_size", "gdr_prefill_chunked",
            "gdr_prefill_chunked_noalloc", "gdr_strerror")
NOALLOC_SCRATCH_BYTES = 128 << 20   # GDR_NOALLOC_SCRATCH_BYTES


class GdrError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {gdr_strerror(status)} (status {status})")
        self.status = status


class gdr_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "T", "H_qk", "H_v", "dk", "dv", "chunk")]


_lib = None


def load_library(path: Path | str | None = None):
    """Load libgdr.so (once) and declare its signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path else LIB_PATH
    if not p.exists():
        raise RuntimeError(f"{p} is missing: build it with `python -m gated_delta_rule_40_amd.build`")
    lib = ctypes.CDLL(str(p))
    vp, fp, i32 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
    dims_p = ctypes.POINTER(gdr_dims)
    lib.gdr_decode_step.argtypes = [dims_p, i32, i32, vp, fp, fp, fp, fp, fp, vp,
                                    ctypes.c_float, i32, vp]
    lib.gdr_decode_step.restype = i32
    lib.gdr_prefill_workspace_size.argtypes = [dims_p, i32, i32]
    lib.gdr_prefill_workspace_size.restype = ctypes.c_size_t
    lib.gdr_prefill_chunked.argtypes = [dims_p, i32, i32, vp, vp, vp, fp, fp, fp, fp, fp, fp, vp,
                                        ctypes.c_float, i32, vp, ctypes.c_size_t, vp]
    lib.gdr_prefill_chunked.restype = i32
    lib.gdr_prefill_chunked_noalloc.argtypes = [dims_p, i32, i32, vp, vp, vp, fp, fp, fp, fp, fp,
                                                fp, vp, ctypes.c_float, i32, vp]
    lib.gdr_prefill_chunked_noalloc.restype = i32
    lib.gdr_strerror.argtypes = [i32]
    lib.gdr_strerror.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def gdr_strerror(status: int) -> str:
    return load_library().gdr_strerror(int(status)).decode()


def _io_code(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return GDR_F32
    if dtype == torch.bfloat16:
        return GDR_BF16
    raise ValueError(f"io dtype must be float32 or bfloat16, got {dtype}")


def _check(t, name, numel, dtype, device, required=True):
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def gdr_decode_step(qkv, gate_in, beta_logit, state, o, *, H_qk, H_v, dk, dv, gate,
                    A_log=None, dt_bias=None, scale=1.0, l2norm_qk=True, stream=None):
    """One fused decode token.  qkv [B, 2*H_qk*dk + H_v*dv] (float32 or bfloat16),
    gate_in [B,H_v,dk] or [B,H_v], beta_logit [B,H_v], state [B,H_v,dk,dv] fp32
    (updated in place), o [B,H_v,dv] in qkv's dtype."""
    lib = load_library()
    B = qkv.shape[0]
    dev = qkv.device
    io = _io_code(qkv.dtype)
    f32 = torch.float32
    width = 2 * H_qk * dk + H_v * dv
    gate_n = B * H_v * dk if gate == GDR_GATE_CHANNEL else B * H_v
    fused = gate == GDR_GATE_SCALAR_FUSED
    args = (
        _check(qkv, "qkv", B * width, qkv.dtype, dev),
        _check(gate_in, "gate_in", gate_n, f32, dev),
        _check(A_log, "A_log", H_v, f32, dev, required=fused),
        _check(dt_bias, "dt_bias", H_v, f32, dev, required=fused),
        _check(beta_logit, "beta_logit", B * H_v, f32, dev),
        _check(state, "state", B * H_v * dk * dv, f32, dev),
        _check(o, "o", B * H_v * dv, qkv.dtype, dev),
    )
    dims = gdr_dims(B, 1, H_qk, H_v, dk, dv, 0)
    rc = lib.gdr_decode_step(ctypes.byref(dims), io, int(gate), args[0], args[1], args[2],
                             args[3], args[4], args[5], args[6], float(scale), int(bool(l2norm_qk)),
                             _stream(dev, stream))
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_decode_step")


def gdr_prefill_workspace_size(B, T, H_qk, H_v, dk, dv, chunk, io_dtype, gate) -> int:
    dims = gdr_dims(B, T, H_qk, H_v, dk, dv, chunk)
    return int(load_library().gdr_prefill_workspace_size(ctypes.byref(dims), _io_code(io_dtype),
                                                         int(gate)))


def _prefill_args(q, k, v, gate_in, beta_logit, state_in, state_out, o, H_qk, H_v, dk, dv,
                  gate, A_log, dt_bias):
    B, T = q.shape[0], q.shape[1]
    dev = q.device
    f32 = torch.float32
    gate_n = B * T * H_v * dk if gate == GDR_GATE_CHANNEL else B * T * H_v
    fused = gate == GDR_GATE_SCALAR_FUSED
    st = B * H_v * dk * dv
    return (
        _check(q, "q", B * T * H_qk * dk, q.dtype, dev),
        _check(k, "k", B * T * H_qk * dk, q.dtype, dev),
        _check(v, "v", B * T * H_v * dv, q.dtype, dev),
        _check(gate_in, "gate_in", gate_n, f32, dev),
        _check(A_log, "A_log", H_v, f32, dev, required=fused),
        _check(dt_bias, "dt_bias", H_v, f32, dev, required=fused),
        _check(beta_logit, "beta_logit", B * T * H_v, f32, dev),
        _check(state_in, "state_in", st, f32, dev, required=False),
        _check(state_out, "state_out", st, f32, dev),
        _check(o, "o", B * T * H_v * dv, q.dtype, dev),
    )


def gdr_prefill_chunked(q, k, v, gate_in, beta_logit, state_in, state_out, o, workspace, *,
                        H_qk, H_v, dk, dv, chunk, gate, A_log=None, dt_bias=None, scale=1.0,
                        l2norm_qk=True, stream=None):
    """Chunked prefill.  q, k [B,T,H_qk,dk], v [B,T,H_v,dv] (float32 or bfloat16),
    gate_in [B,T,H_v,dk] or [B,T,H_v], beta_logit [B,T,H_v], state_in (or None)
    and state_out [B,H_v,dk,dv] fp32, o [B,T,H_v,dv], workspace a uint8 tensor
    of at least gdr_prefill_workspace_size() bytes."""
    lib = load_library()
    dev = q.device
    if workspace is not None:
        if workspace.device != dev or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the same device")
        ws_ptr = ctypes.c_void_p(workspace.data_ptr())
        ws_bytes = workspace.numel() * workspace.element_size()
    else:
        ws_ptr, ws_bytes = None, 0
    args = _prefill_args(q, k, v, gate_in, beta_logit, state_in, state_out, o, H_qk, H_v, dk, dv,
                         gate, A_log, dt_bias)
    dims = gdr_dims(q.shape[0], q.shape[1], H_qk, H_v, dk, dv, chunk)
    rc = lib.gdr_prefill_chunked(ctypes.byref(dims), _io_code(q.dtype), int(gate), *args,
                                 float(scale), int(bool(l2norm_qk)), ws_ptr,
                                 ctypes.c_size_t(ws_bytes), _stream(dev, stream))
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_prefill_chunked")


def gdr_prefill_chunked_noalloc(q, k, v, gate_in, beta_logit, state_in, state_out, o, *,
                                H_qk, H_v, dk, dv, chunk, gate, A_log=None, dt_bias=None,
                                scale=1.0, l2norm_qk=True, stream=None):
    """gdr_prefill_chunked with the library's own device scratch as workspace
    (nothing is allocated; at most NOALLOC_SCRATCH_BYTES of workspace; calls
    that overlap on one device race on the scratch)."""
    lib = load_library()
    args = _prefill_args(q, k, v, gate_in, beta_logit, state_in, state_out, o, H_qk, H_v, dk, dv,
                         gate, A_log, dt_bias)
    dims = gdr_dims(q.shape[0], q.shape[1], H_qk, H_v, dk, dv, chunk)
    rc = lib.gdr_prefill_chunked_noalloc(ctypes.byref(dims), _io_code(q.dtype), int(gate), *args,
                                         float(scale), int(bool(l2norm_qk)),
                                         _stream(q.device, stream))
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_prefill_chunked_noalloc")
