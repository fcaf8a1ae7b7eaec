"""Seeded synthetic inputs for the gated delta rule.

This module draws random numbers and rounds them to bfloat16; it holds none
of the method's arithmetic (no normalisation, no gates, no recurrence).  The
same arrays feed both the HIP library and the CPU oracle, so both sides see
bit-identical inputs.

Every draw uses ``numpy.random.Generator(PCG64(seed))`` in a fixed order:
q/k/v (or the packed qkv row), then the gate tensors, then beta_logit, then
the initial state.  bf16 tensors are drawn in fp32 and rounded to nearest
even; they are returned as ``uint16`` bit patterns (``bf16_to_f32`` expands
them exactly).

Workload recipes (all sizes are those of the named workloads):

  tiny            B=1, H_qk=H_v=2, dk=dv=16, T=33, chunk 16, fp32;
                  channel log-decay g ~ -U(0.01, 0.5); S0 = 0
  fused_decode    B=1, H_qk=16 -> H_v=32, dk=dv=128, packed bf16 row;
                  scalar gate from A_log ~ U(-1,1), x ~ N(0,1),
                  dt_bias ~ U(-1,1); S0 ~ N(0, 0.02)
  batched_decode  B=64, same heads, channel g ~ -U(0.01, 0.5), fresh
                  inputs per step, S0 ~ N(0, 0.02)
  prefill         B=1, T=4000, chunk 64, bf16 q/k/v, channel
                  g ~ -U(0.001, 0.2), S0 = 0
  long_prefill    B=4, T=32767, chunk 64, bf16, S0 ~ N(0, 0.02), scalar or
                  channel gate with g ~ -U(0.001, 0.2)

q and k are drawn raw from N(0,1); the L2 normalisation is part of the
method and happens in the kernels / oracle (``l2norm_qk=1``).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

GATE_CHANNEL = 0
GATE_SCALAR = 1
GATE_SCALAR_FUSED = 2


def f32_to_bf16(x) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """Expand bfloat16 bit patterns (uint16) to fp32 exactly."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Case:
    """One seeded workload.  Float tensors are fp32 numpy arrays; tensors whose
    io dtype is bf16 are uint16 bit patterns (see ``io``)."""
    name: str
    B: int
    T: int
    H_qk: int
    H_v: int
    dk: int
    dv: int
    chunk: int
    io: str                     # "f32" or "bf16": dtype of q/k/v (qkv) and o
    gate: int                   # GATE_* kind
    tensors: dict = field(default_factory=dict)

    def values(self, key) -> np.ndarray:
        """Tensor as exact fp32 values (bf16 bit patterns expanded)."""
        a = self.tensors[key]
        if a is None:
            return None
        return bf16_to_f32(a) if a.dtype == np.uint16 else a


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _io(rng, shape, io):
    x = rng.standard_normal(shape, dtype=np.float32)
    return f32_to_bf16(x) if io == "bf16" else x


def _neg_uniform(rng, lo, hi, shape):
    return -rng.uniform(lo, hi, size=shape).astype(np.float32)


def _gates(rng, gate, B, T, H_v, dk, g_lo, g_hi):
    """Gate tensors in draw order.  T=None gives the decode layout (no T axis)."""
    lead = (B, H_v) if T is None else (B, T, H_v)
    out = {"A_log": None, "dt_bias": None}
    if gate == GATE_CHANNEL:
        out["gate_in"] = _neg_uniform(rng, g_lo, g_hi, lead + (dk,))
    elif gate == GATE_SCALAR:
        out["gate_in"] = _neg_uniform(rng, g_lo, g_hi, lead)
    elif gate == GATE_SCALAR_FUSED:
        out["A_log"] = rng.uniform(-1.0, 1.0, size=(H_v,)).astype(np.float32)
        out["gate_in"] = rng.standard_normal(lead, dtype=np.float32)
        out["dt_bias"] = rng.uniform(-1.0, 1.0, size=(H_v,)).astype(np.float32)
    else:
        raise ValueError(f"unknown gate kind {gate}")
    return out


def _state(rng, B, H_v, dk, dv, std):
    if std == 0.0:
        return np.zeros((B, H_v, dk, dv), np.float32)
    return (std * rng.standard_normal((B, H_v, dk, dv), dtype=np.float32)).astype(np.float32)


def prefill_case(name, seed, B, T, H_qk, H_v, dk, dv, chunk, io, gate, g_lo, g_hi, s0_std):
    """q, k [B,T,H_qk,dk], v [B,T,H_v,dv], gates, beta_logit [B,T,H_v], S0."""
    rng = _rng(seed)
    t = {}
    t["q"] = _io(rng, (B, T, H_qk, dk), io)
    t["k"] = _io(rng, (B, T, H_qk, dk), io)
    t["v"] = _io(rng, (B, T, H_v, dv), io)
    t.update(_gates(rng, gate, B, T, H_v, dk, g_lo, g_hi))
    t["beta_logit"] = rng.standard_normal((B, T, H_v), dtype=np.float32)
    t["S0"] = _state(rng, B, H_v, dk, dv, s0_std)
    return Case(name, B, T, H_qk, H_v, dk, dv, chunk, io, gate, t)


def decode_case(name, seed, B, steps, H_qk, H_v, dk, dv, io, gate, g_lo, g_hi, s0_std):
    """Per-step packed rows qkv [steps,B,2*H_qk*dk+H_v*dv], gates with a leading
    steps axis, beta_logit [steps,B,H_v] and S0 [B,H_v,dk,dv]."""
    rng = _rng(seed)
    t = {}
    width = 2 * H_qk * dk + H_v * dv
    t["qkv"] = _io(rng, (steps, B, width), io)
    if gate == GATE_SCALAR_FUSED:
        # Static per-head parameters, fresh activation x per step.
        t.update(_gates(rng, gate, steps * B, None, H_v, dk, g_lo, g_hi))
        t["gate_in"] = t["gate_in"].reshape(steps, B, H_v)
    else:
        g = _gates(rng, gate, steps * B, None, H_v, dk, g_lo, g_hi)
        g["gate_in"] = g["gate_in"].reshape((steps, B) + g["gate_in"].shape[1:])
        t.update(g)
    t["beta_logit"] = rng.standard_normal((steps, B, H_v), dtype=np.float32)
    t["S0"] = _state(rng, B, H_v, dk, dv, s0_std)
    return Case(name, B, steps, H_qk, H_v, dk, dv, 0, io, gate, t)


# ---- the named workloads ---------------------------------------------------

def tiny(seed: int = 1, s0_std: float = 0.0, gate: int = GATE_CHANNEL) -> Case:
    return prefill_case("tiny", seed, 1, 33, 2, 2, 16, 16, 16, "f32", gate, 0.01, 0.5, s0_std)


def tiny_decode(seed: int = 1, gate: int = GATE_CHANNEL, s0_std: float = 0.0) -> Case:
    """The tiny shapes as 33 packed decode steps."""
    return decode_case("tiny_decode", seed, 1, 33, 2, 2, 16, 16, "f32", gate, 0.01, 0.5, s0_std)


def fused_decode(seed: int = 2, steps: int = 1) -> Case:
    return decode_case("fused_decode_b1", seed, 1, steps, 16, 32, 128, 128, "bf16",
                       GATE_SCALAR_FUSED, 0.0, 0.0, 0.02)


def batched_decode(seed: int = 3, steps: int = 256, B: int = 64) -> Case:
    return decode_case(f"batched_decode_b{B}", seed, B, steps, 16, 32, 128, 128, "bf16",
                       GATE_CHANNEL, 0.01, 0.5, 0.02)


def prefill(seed: int = 4, T: int = 4000, B: int = 1, gate: int = GATE_CHANNEL) -> Case:
    return prefill_case(f"prefill_t{T}", seed, B, T, 16, 32, 128, 128, 64, "bf16", gate,
                        0.001, 0.2, 0.0)


def long_prefill(gate: int = GATE_CHANNEL, seed: int | None = None, T: int = 32767,
                 B: int = 4) -> Case:
    if seed is None:
        seed = 51 if gate == GATE_SCALAR else 52
    return prefill_case(f"long_prefill_t{T}", seed, B, T, 16, 32, 128, 128, 64, "bf16", gate,
                        0.001, 0.2, 0.02)
