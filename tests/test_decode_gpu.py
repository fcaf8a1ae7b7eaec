"""gdr_decode_step on the GPU against the fp64 oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gated_delta_rule_40_amd as gdr
import oracle
from gated_delta_rule_40_amd import synth
from tests.gpu_util import (DEV, TOL, announce, io_dtype, oracle_threads, rel, require_gpu,
                            to_dev, to_host)

pytestmark = pytest.mark.gpu


def _decode_run(case: synth.Case, steps, rows=None, scale=1.0, l2norm=True, mutate=None):
    """Run `steps` decode steps on the GPU (all batch rows) and on the oracle
    (batch rows `rows` only).  Returns the worst relative errors of o and S."""
    require_gpu()
    t = case.tensors
    B = case.B
    rows = list(range(B)) if rows is None else list(rows)
    dims = dict(H_qk=case.H_qk, H_v=case.H_v, dk=case.dk, dv=case.dv, gate=case.gate)
    S = to_dev(t["S0"])
    A_log, dt_bias = to_dev(t["A_log"]), to_dev(t["dt_bias"])
    o = torch.empty((B, case.H_v, case.dv), dtype=io_dtype(case.io), device=DEV)
    S_ref = t["S0"][rows].astype(np.float64)
    err_o = 0.0
    for s in range(steps):
        raw = t["qkv"][s]
        qkv_np = synth.bf16_to_f32(raw) if case.io == "bf16" else raw
        g_np, bl_np = t["gate_in"][s], t["beta_logit"][s]
        if mutate is not None:
            qkv_np, g_np, bl_np = mutate(qkv_np, g_np, bl_np)
            raw = synth.f32_to_bf16(qkv_np) if case.io == "bf16" else qkv_np
        qkv = to_dev(raw)
        gdr.gdr_decode_step(qkv, to_dev(g_np), to_dev(bl_np), S, o, A_log=A_log,
                            dt_bias=dt_bias, scale=scale, l2norm_qk=l2norm, **dims)
        o_ref, S_ref = oracle.decode(qkv_np[rows], case.H_qk, case.H_v, case.dk, case.dv,
                                     case.gate, g_np[rows], bl_np[rows], S_ref, A_log=t["A_log"],
                                     dt_bias=t["dt_bias"], scale=scale, l2norm=l2norm,
                                     threads=oracle_threads())
        err_o = max(err_o, rel(to_host(o)[rows], o_ref))
    torch.cuda.synchronize()
    err_s = rel(to_host(S)[rows], S_ref)
    return err_o, err_s


@pytest.mark.parametrize("gate", [synth.GATE_CHANNEL, synth.GATE_SCALAR, synth.GATE_SCALAR_FUSED])
def test_decode_tiny_fp32_33_steps(gate):
    case = synth.tiny_decode(seed=1, gate=gate, s0_std=0.0)
    announce(f"decode tiny fp32 gate={gate} B=1 H=2 dk=dv=16 steps=33")
    eo, es = _decode_run(case, 33, scale=1.0)
    print(f"err o={eo:.3e} S={es:.3e}")
    assert eo < TOL["f32"] and es < TOL["f32"]


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_without_l2norm(io):
    """l2norm_qk = 0: q and k are used as given.  They are pre-scaled by
    1/sqrt(dk) so that |k| ~ 1 and the recurrence stays bounded."""
    case = synth.decode_case("nol2", 24, 3, 20, 2, 4, 32, 64, io, synth.GATE_CHANNEL,
                             0.01, 0.5, 0.3)
    nqk = 2 * case.H_qk * case.dk

    def mutate(qkv, g, bl):
        qkv = qkv.copy()
        qkv[:, :nqk] *= np.float32(1.0 / np.sqrt(case.dk))
        if io == "bf16":  # the values the kernel sees
            qkv = synth.bf16_to_f32(synth.f32_to_bf16(qkv))
        return qkv, g, bl

    announce(f"decode no-l2norm io={io} B=3 H 2->4 dk=32 dv=64 steps=20")
    eo, es = _decode_run(case, 20, l2norm=False, mutate=mutate)
    print(f"err o={eo:.3e} S={es:.3e}")
    assert eo < TOL[io] and es < TOL[io]


def test_decode_tiny_fp32_nonzero_state_scale():
    case = synth.tiny_decode(seed=21, gate=synth.GATE_CHANNEL, s0_std=0.5)
    announce("decode tiny fp32 nonzero S0, scale 0.25")
    eo, es = _decode_run(case, 33, scale=0.25)
    assert eo < TOL["f32"] and es < TOL["f32"]


@pytest.mark.parametrize("dk,dv,hqk,hv,B", [(32, 64, 1, 3, 2), (64, 32, 2, 2, 3),
                                            (128, 16, 4, 8, 1), (16, 128, 3, 6, 5)])
def test_decode_shapes_fp32(dk, dv, hqk, hv, B):
    case = synth.decode_case("shapes", 30 + dk + dv, B, 5, hqk, hv, dk, dv, "f32",
                             synth.GATE_CHANNEL, 0.01, 0.5, 0.3)
    announce(f"decode fp32 B={B} H_qk={hqk} H_v={hv} dk={dk} dv={dv}")
    eo, es = _decode_run(case, 5)
    assert eo < TOL["f32"] and es < TOL["f32"]


def test_decode_fused_gate_bf16_b1():
    """Packed bf16 row, scalar fused gate, B=1, H_qk 16 -> H_v 32, dk=dv=128."""
    case = synth.fused_decode(seed=2, steps=8)
    announce("decode fused-gate bf16 B=1 H 16->32 dk=dv=128 steps=8")
    eo, es = _decode_run(case, 8)
    print(f"err o={eo:.3e} S={es:.3e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


@pytest.mark.timeout(900)
def test_decode_batched_channel_b64_256_steps():
    """B=64 channelwise decode, 256 consecutive steps: every output of every
    step and the final state of all 64 batch rows against the oracle."""
    case = synth.batched_decode(seed=3, steps=256, B=64)
    announce("decode batched channel bf16 B=64 H 16->32 dk=dv=128 steps=256 (all rows)")
    eo, es = _decode_run(case, 256)
    print(f"err o={eo:.3e} S={es:.3e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B,rows", [(8, [0, 3, 7]), (160, [0, 77, 159])])
def test_decode_slice_widths_bf16(B, rows):
    """H_qk 16 -> H_v 32, dk=dv=128, bf16, channel gate, 3 steps: B=8 runs
    32-column slices; B=160 (a 320 MiB state, beyond the 256 MiB MALL) whole
    128-column rows, 5120 workgroups.  The oracle follows the sampled batch
    rows."""
    case = synth.decode_case(f"slices{B}", 45 + B, B, 3, 16, 32, 128, 128, "bf16",
                             synth.GATE_CHANNEL, 0.01, 0.5, 0.02)
    announce(f"decode bf16 B={B} H 16->32 dk=dv=128 steps=3")
    eo, es = _decode_run(case, 3, rows=rows)
    print(f"err o={eo:.3e} S={es:.3e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B,io,gate", [
    (80, "f32", synth.GATE_SCALAR),        # 2560 tiles, fp32 rows, scalar gate
    (64, "bf16", synth.GATE_SCALAR_FUSED),  # 2048 tiles, fused gate (full occupancy)
    (72, "bf16", synth.GATE_CHANNEL),       # 2304 tiles, channel gate (at most 3 per CU)
    (36, "f32", synth.GATE_CHANNEL),        # 1152 tiles, below the occupancy cap
])
def test_decode_large_grids(B, io, gate):
    """Whole 128 x 128 tiles (H 16 -> 32, dk=dv=128) on large grids, for each
    launch shape of the step: fp32 or bf16 rows, scalar, fused or channel
    gate, with and without the occupancy cap; 2 steps, sampled batch rows."""
    case = synth.decode_case(f"grid{B}", 60 + B, B, 2, 16, 32, 128, 128, io, gate, 0.01, 0.5,
                             0.02)
    announce(f"decode {io} B={B} gate={gate} H 16->32 dk=dv=128 steps=2")
    eo, es = _decode_run(case, 2, rows=[0, B // 2, B - 1])
    print(f"err o={eo:.3e} S={es:.3e}")
    assert eo < TOL[io] and es < TOL[io]


def test_decode_write_then_read_identity():
    """beta = 1 (large logit), q = k: the value just written is read back."""
    case = synth.decode_case("ident", 41, 3, 3, 2, 4, 64, 64, "f32", synth.GATE_CHANNEL,
                             0.01, 0.5, 0.7)

    def mutate(qkv, g, bl):
        qkv = qkv.copy()
        w = case.H_qk * case.dk
        qkv[:, :w] = qkv[:, w:2 * w]
        return qkv, g, np.full_like(bl, 40.0)

    announce("decode identity q=k beta=1")
    eo, es = _decode_run(case, 3, mutate=mutate)
    assert eo < TOL["f32"] and es < TOL["f32"]


def test_decode_beta_zero_pure_decay():
    case = synth.decode_case("decay", 42, 2, 4, 2, 2, 32, 32, "f32", synth.GATE_CHANNEL,
                             0.01, 0.5, 1.0)

    def mutate(qkv, g, bl):
        return qkv, g, np.full_like(bl, -200.0)

    announce("decode beta=0 pure decay")
    eo, es = _decode_run(case, 4, mutate=mutate)
    assert eo < TOL["f32"] and es < TOL["f32"]


def test_decode_b0_is_noop():
    require_gpu()
    S = torch.zeros((0, 2, 16, 16), device=DEV)
    o = torch.zeros((0, 2, 16), device=DEV)
    qkv = torch.zeros((0, 2 * 16 + 2 * 16), device=DEV)
    gdr.gdr_decode_step(qkv, torch.zeros((0, 2, 16), device=DEV), torch.zeros((0, 2), device=DEV),
                        S, o, H_qk=1, H_v=2, dk=16, dv=16, gate=synth.GATE_CHANNEL)
