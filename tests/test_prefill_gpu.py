"""gdr_prefill_chunked on the GPU against the fp64 oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gated_delta_rule_40_amd as gdr
import oracle
from gated_delta_rule_40_amd import synth
from tests.gpu_util import (DEV, TOL, announce, carry_segments, io_dtype, oracle_threads, rel,
                            require_gpu, run_prefill, to_dev, to_host)

pytestmark = pytest.mark.gpu


def _oracle(case: synth.Case, scale=1.0, l2norm=True, state0="S0", T_slice=None, heads=None):
    """Oracle on the whole case, or on (b, h) units `heads` only (returns dicts)."""
    t = case.tensors
    sl = slice(None) if T_slice is None else T_slice
    S0 = t["S0"] if isinstance(state0, str) else state0
    if heads is None:
        return oracle.sequence(case.values("q")[:, sl], case.values("k")[:, sl],
                               case.values("v")[:, sl], case.gate, t["gate_in"][:, sl],
                               t["beta_logit"][:, sl], S0, A_log=t["A_log"], dt_bias=t["dt_bias"],
                               scale=scale, l2norm=l2norm, threads=oracle_threads())
    rep = case.H_v // case.H_qk
    out = {}
    for b, h in heads:
        hq = h // rep
        q = synth.bf16_to_f32(t["q"][b:b + 1, sl, hq:hq + 1]) if case.io == "bf16" else t["q"][b:b + 1, sl, hq:hq + 1]
        k = synth.bf16_to_f32(t["k"][b:b + 1, sl, hq:hq + 1]) if case.io == "bf16" else t["k"][b:b + 1, sl, hq:hq + 1]
        v = synth.bf16_to_f32(t["v"][b:b + 1, sl, h:h + 1]) if case.io == "bf16" else t["v"][b:b + 1, sl, h:h + 1]
        A = None if t["A_log"] is None else t["A_log"][h:h + 1]
        dt = None if t["dt_bias"] is None else t["dt_bias"][h:h + 1]
        out[(b, h)] = oracle.sequence(q, k, v, case.gate, t["gate_in"][b:b + 1, sl, h:h + 1],
                                      t["beta_logit"][b:b + 1, sl, h:h + 1],
                                      S0[b:b + 1, h:h + 1], A_log=A, dt_bias=dt, scale=scale,
                                      l2norm=l2norm, threads=1)
    return out


@pytest.mark.parametrize("gate", [synth.GATE_CHANNEL, synth.GATE_SCALAR, synth.GATE_SCALAR_FUSED])
@pytest.mark.parametrize("s0", [0.0, 0.5])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_prefill_tiny_fp32(gate, s0, chunk):
    """B=1, H=2, dk=dv=16, T=33 (ragged against every chunk size), fp32."""
    require_gpu()
    case = synth.tiny(seed=1, s0_std=s0, gate=gate)
    announce(f"prefill tiny fp32 gate={gate} s0={s0} chunk={chunk} T=33")
    o, S = run_prefill(case, chunk=chunk, scale=0.75)
    o_ref, S_ref = _oracle(case, scale=0.75)
    print(f"err o={rel(o, o_ref):.3e} S={rel(S, S_ref):.3e}")
    assert rel(o, o_ref) < TOL["f32"] and rel(S, S_ref) < TOL["f32"]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 65, 130, 200])
def test_prefill_ragged_lengths(io, T):
    require_gpu()
    case = synth.prefill_case("ragged", 100 + T, 2, T, 2, 4, 32, 64, 64, io, synth.GATE_CHANNEL,
                              0.01, 0.3, 0.2)
    announce(f"prefill ragged io={io} T={T} B=2 H 2->4 dk=32 dv=64 chunk=64")
    o, S = run_prefill(case)
    o_ref, S_ref = _oracle(case)
    print(f"err o={rel(o, o_ref):.3e} S={rel(S, S_ref):.3e}")
    assert rel(o, o_ref) < TOL[io] and rel(S, S_ref) < TOL[io]


@pytest.mark.parametrize("dk,dv", [(16, 128), (64, 16), (128, 32), (32, 32)])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prefill_head_dims(dk, dv, io):
    require_gpu()
    case = synth.prefill_case("dims", 7 * dk + dv, 1, 77, 1, 2, dk, dv, 32, io,
                              synth.GATE_SCALAR, 0.01, 0.3, 0.3)
    announce(f"prefill dims io={io} dk={dk} dv={dv} T=77 chunk=32")
    o, S = run_prefill(case)
    o_ref, S_ref = _oracle(case)
    assert rel(o, o_ref) < TOL[io] and rel(S, S_ref) < TOL[io]


@pytest.mark.parametrize("B", [1, 2, 4])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prefill_slice_widths(B, io):
    """H 16 -> 32, dk=dv=128 at B=1, 2, 4: the carry splits dv into slices of
    16, 32 and 64 columns respectively (bf16 at B=1: one wave per 16-column
    slice; otherwise one workgroup per CU), so every slice width and its
    fragment schedule is checked against the oracle, with a nonzero initial
    state and a ragged last chunk."""
    require_gpu()
    case = synth.prefill_case("slices", 300 + B, B, 150, 16, 32, 128, 128, 64, io,
                              synth.GATE_CHANNEL, 0.001, 0.2, 0.02)
    announce(f"prefill slices io={io} B={B} T=150 H 16->32 dk=dv=128 chunk=64")
    o, S = run_prefill(case)
    o_ref, S_ref = _oracle(case)
    print(f"err o={rel(o, o_ref):.3e} S={rel(S, S_ref):.3e}")
    assert rel(o, o_ref) < TOL[io] and rel(S, S_ref) < TOL[io]


@pytest.mark.parametrize("B,H_qk,H_v,dk,dv,chunk,T", [
    # one wave per 16-column slice (B * H_v * dv / 16 <= 256)
    (2, 2, 4, 32, 32, 16, 77),
    (2, 2, 4, 16, 32, 64, 77),
    (2, 2, 4, 64, 16, 16, 77),
    (2, 2, 4, 16, 64, 32, 77),
    (1, 1, 2, 128, 16, 16, 77),
    # one workgroup per slice of 32 columns (288 slices of 16) and of 64 (768)
    (3, 4, 12, 16, 128, 64, 70),
    (3, 4, 12, 128, 128, 16, 70),
    (4, 8, 24, 16, 128, 32, 40),
])
def test_prefill_mixed_mfma_shapes(B, H_qk, H_v, dk, dv, chunk, T):
    """bf16 shapes whose two contractions use different MFMA forms (16x16x32
    over a 32-multiple, 16x16x16 over 16): dk = 16 with chunk 32 or 64, or
    chunk 16 with dk >= 32.  The output sums a product of each form, so these
    cases check that neither carry accumulates one form into an accumulator
    the other is still writing.  The last three take the workgroup carry at
    the shapes whose compiled code had put the two products closest together."""
    require_gpu()
    case = synth.prefill_case("mixed", 400 + dk + chunk, B, T, H_qk, H_v, dk, dv, chunk, "bf16",
                              synth.GATE_CHANNEL, 0.01, 0.3, 0.3)
    announce(f"prefill mixed MFMA forms B={B} T={T} H {H_qk}->{H_v} dk={dk} dv={dv} chunk={chunk}")
    o, S = run_prefill(case)
    o_ref, S_ref = _oracle(case)
    print(f"err o={rel(o, o_ref):.3e} S={rel(S, S_ref):.3e}")
    assert rel(o, o_ref) < TOL["bf16"] and rel(S, S_ref) < TOL["bf16"]


@pytest.mark.parametrize("gate", [synth.GATE_CHANNEL, synth.GATE_SCALAR])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prefill_without_l2norm(io, gate):
    """l2norm_qk = 0: q and k are used as given, pre-scaled by 1/sqrt(dk) so
    that |k| ~ 1; ragged against chunk 32, nonzero initial state.  With a
    scalar gate the stored k and q rows are then the inputs as given."""
    require_gpu()
    case = synth.prefill_case("nol2", 81 + gate, 2, 150, 2, 4, 64, 64, 32, io, gate,
                              0.01, 0.3, 0.3)
    t = case.tensors
    for name in ("q", "k"):
        x = case.values(name) * np.float32(1.0 / np.sqrt(case.dk))
        t[name] = synth.f32_to_bf16(x) if io == "bf16" else x.astype(np.float32)
    announce(f"prefill no-l2norm io={io} gate={gate} B=2 T=150 H 2->4 dk=dv=64 chunk=32")
    o, S = run_prefill(case, l2norm=False)
    o_ref, S_ref = _oracle(case, l2norm=False)
    print(f"err o={rel(o, o_ref):.3e} S={rel(S, S_ref):.3e}")
    assert rel(o, o_ref) < TOL[io] and rel(S, S_ref) < TOL[io]


# Scalar gates keep the normalised k and q rows once per (b, qk head, chunk),
# written by the first value head of each qk head and read by all of them.
# Cases: four, one and three value heads per qk head, every slice width of
# the carry (16 to 64 columns), the segmented carry, both io dtypes and both
# scalar gate kinds; outputs NaN-filled beforehand.
@pytest.mark.parametrize("B,H_qk,H_v,dk,dv,chunk,T,io,gate", [
    (3, 2, 8, 64, 64, 32, 150, "bf16", synth.GATE_SCALAR),
    (1, 3, 3, 128, 128, 64, 200, "bf16", synth.GATE_SCALAR_FUSED),
    (2, 1, 3, 32, 64, 16, 77, "f32", synth.GATE_SCALAR),
    (2, 8, 32, 128, 128, 64, 130, "bf16", synth.GATE_SCALAR),
    (4, 16, 32, 128, 128, 64, 130, "bf16", synth.GATE_SCALAR_FUSED),
    (1, 1, 4, 64, 64, 32, 3000, "bf16", synth.GATE_SCALAR),
])
def test_prefill_scalar_gate_shared_qk_rows(B, H_qk, H_v, dk, dv, chunk, T, io, gate):
    require_gpu()
    case = synth.prefill_case("sqk", 460 + H_v + T % 97, B, T, H_qk, H_v, dk, dv, chunk, io, gate,
                              0.01, 0.3, 0.3)
    segs = carry_segments(B, T, H_v, dk, dv, chunk)
    announce(f"prefill scalar gate, shared k/q rows: B={B} T={T} H {H_qk}->{H_v} dk={dk} dv={dv} "
             f"chunk={chunk} io={io} gate={gate} carry segments={segs}")
    o, S = run_prefill(case, o_fill=float("nan"))
    o_ref, S_ref = _oracle(case)
    assert np.isfinite(o).all() and np.isfinite(S).all()
    print(f"err o={rel(o, o_ref):.3e} S={rel(S, S_ref):.3e}")
    assert rel(o, o_ref) < TOL[io] and rel(S, S_ref) < TOL[io]


@pytest.mark.timeout(600)
def test_prefill_t4000_bf16_channel():
    """B=1, T=4000 (62 full chunks of 64 and one of 32), H 16 -> 32, dk=dv=128."""
    require_gpu()
    case = synth.prefill(seed=4)
    announce("prefill bf16 channel B=1 T=4000 H 16->32 dk=dv=128 chunk=64")
    o, S = run_prefill(case)
    o_ref, S_ref = _oracle(case)
    eo, es = rel(o, o_ref), rel(S, S_ref)
    print(f"err o={eo:.3e} S={es:.3e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("gate", [synth.GATE_SCALAR, synth.GATE_CHANNEL])
def test_prefill_t32767_b4_full(gate):
    """B=4, T=32767 (511 full chunks + 63), H 16 -> 32, dk=dv=128, nonzero S0:
    the whole launch on the GPU, then every output and the final state of all
    128 (b, h) units against the oracle, one batch row at a time (about 1 GB
    of fp64 outputs each)."""
    require_gpu()
    case = synth.long_prefill(gate=gate)
    announce(f"prefill bf16 gate={gate} B=4 T=32767 H 16->32 dk=dv=128 chunk=64 (all units)")
    o, S = run_prefill(case, on_device=True)
    t = case.tensors
    worst_o = worst_s = 0.0
    for b in range(case.B):
        sl = slice(b, b + 1)
        o_ref, S_ref = oracle.sequence(
            synth.bf16_to_f32(t["q"][sl]), synth.bf16_to_f32(t["k"][sl]),
            synth.bf16_to_f32(t["v"][sl]), case.gate, t["gate_in"][sl], t["beta_logit"][sl],
            t["S0"][sl], scale=1.0, l2norm=True, threads=oracle_threads())
        eo, es = rel(to_host(o[b]), o_ref[0]), rel(to_host(S[b]), S_ref[0])
        print(f"b={b}: err o={eo:.3e} S={es:.3e}", flush=True)
        worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
        del o_ref, S_ref
    print(f"err o={worst_o:.3e} S={worst_s:.3e}")
    assert worst_o < TOL["bf16"] and worst_s < TOL["bf16"]


# Short sequences (T <= 16 at up to 64 (b, h) units, T <= 24 above) take the
# token-by-token path; the cases cover every head size, gate kind and state
# mode, both io dtypes, and slices of 16 to 128 state columns.
@pytest.mark.parametrize("T,B,H_qk,H_v,dk,dv,gate,io,mode", [
    (2, 1, 2, 4, 32, 32, synth.GATE_CHANNEL, "f32", "S0"),
    (5, 2, 1, 2, 16, 128, synth.GATE_SCALAR, "f32", "S0"),
    (16, 1, 2, 4, 128, 32, synth.GATE_SCALAR_FUSED, "f32", "S0"),
    (13, 3, 2, 2, 64, 16, synth.GATE_CHANNEL, "f32", "inplace"),
    (12, 2, 2, 4, 64, 64, synth.GATE_CHANNEL, "f32", "null"),
    (16, 1, 16, 32, 128, 128, synth.GATE_CHANNEL, "bf16", "S0"),
    (24, 4, 16, 32, 128, 128, synth.GATE_SCALAR, "bf16", "S0"),
    (8, 16, 16, 32, 128, 128, synth.GATE_CHANNEL, "bf16", "S0"),
])
def test_prefill_short_token_path(T, B, H_qk, H_v, dk, dv, gate, io, mode):
    require_gpu()
    s0 = 0.0 if mode == "null" else 0.4
    case = synth.prefill_case(f"short{T}", 80 + T, B, T, H_qk, H_v, dk, dv, 16, io, gate,
                              0.01, 0.3, s0)
    announce(f"prefill short io={io} T={T} B={B} H {H_qk}->{H_v} dk={dk} dv={dv} gate={gate} "
             f"{mode}")
    kw = {"inplace": True} if mode == "inplace" else ({"state_in": None} if mode == "null" else {})
    o, S = run_prefill(case, **kw)
    o_ref, S_ref = _oracle(case)
    eo, es = rel(o, o_ref), rel(S, S_ref)
    print(f"err o={eo:.3e} S={es:.3e}")
    assert eo < TOL[io] and es < TOL[io]


@pytest.mark.timeout(600)
def test_prefill_short_beyond_cache_b160():
    """Token-by-token path with a 320 MiB state (B=160, H 16 -> 32,
    dk=dv=128, bf16, T=4): the final state goes out with streaming stores.
    The oracle follows sampled (b, h) units."""
    require_gpu()
    case = synth.prefill_case("short160", 97, 160, 4, 16, 32, 128, 128, 64, "bf16",
                              synth.GATE_CHANNEL, 0.01, 0.3, 0.4)
    announce("prefill short bf16 B=160 T=4 H 16->32 dk=dv=128 (state beyond the MALL)")
    o, S = run_prefill(case, on_device=True)
    heads = [(0, 0), (77, 13), (159, 31)]
    ref = _oracle(case, heads=heads)
    worst_o = worst_s = 0.0
    for (b, h), (o_ref, S_ref) in ref.items():
        worst_o = max(worst_o, rel(to_host(o[b, :, h]), o_ref[0, :, 0]))
        worst_s = max(worst_s, rel(to_host(S[b, h]), S_ref[0, 0]))
    print(f"err o={worst_o:.3e} S={worst_s:.3e}")
    assert worst_o < TOL["bf16"] and worst_s < TOL["bf16"]


@pytest.mark.parametrize("T", [24, 25])
def test_prefill_short_path_boundary(T):
    """B=8, H 16 -> 32, dk=dv=128, bf16, chunk 64: T=24 is the last length on
    the token-by-token path at 256 (b, h) units, T=25 one ragged chunk on the
    chunked path."""
    require_gpu()
    case = synth.prefill_case(f"edge{T}", 90 + T, 8, T, 16, 32, 128, 128, 64, "bf16",
                              synth.GATE_CHANNEL, 0.01, 0.3, 0.4)
    announce(f"prefill short/chunked boundary bf16 T={T} B=8 H 16->32 dk=dv=128")
    o, S = run_prefill(case)
    o_ref, S_ref = _oracle(case)
    eo, es = rel(o, o_ref), rel(S, S_ref)
    print(f"err o={eo:.3e} S={es:.3e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


# Long sequences at few (b, h) units: 25 to 61 chunks of 16 (ragged last
# chunk) and 25 of 64, with a nonzero, a null and an in-place initial state.
@pytest.mark.parametrize("T,chunk,gate,mode", [
    (389, 16, synth.GATE_CHANNEL, "S0"),
    (600, 16, synth.GATE_CHANNEL, "S0"),
    (967, 16, synth.GATE_CHANNEL, "S0"),
    (600, 16, synth.GATE_SCALAR_FUSED, "S0"),
    (600, 16, synth.GATE_CHANNEL, "inplace"),
    (600, 16, synth.GATE_CHANNEL, "null"),
    (1600, 64, synth.GATE_CHANNEL, "bf16"),
])
def test_prefill_long_few_heads(T, chunk, gate, mode):
    require_gpu()
    io = "bf16" if mode == "bf16" else "f32"
    dkv = 64 if mode == "bf16" else 32
    s0 = 0.0 if mode == "null" else 0.4
    case = synth.prefill_case(f"long{T}", 70 + T % 17, 1, T, 2, 4, dkv, dkv, chunk, io, gate,
                              0.01, 0.3, s0)
    announce(f"prefill long io={io} T={T} chunk={chunk} gate={gate} {mode} B=1 H 2->4 "
             f"dk=dv={dkv}")
    kw = {"inplace": True} if mode == "inplace" else ({"state_in": None} if mode == "null" else {})
    o, S = run_prefill(case, **kw)
    o_ref, S_ref = _oracle(case)
    eo, es = rel(o, o_ref), rel(S, S_ref)
    print(f"err o={eo:.3e} S={es:.3e}")
    assert eo < TOL[io] and es < TOL[io]


@pytest.mark.parametrize("B,H_qk,H_v,dk,dv,chunk,T,io,gate,mode", [
    (1, 1, 2, 128, 128, 64, 3000, "bf16", synth.GATE_CHANNEL, "s0"),
    (1, 1, 4, 64, 32, 32, 2500, "f32", synth.GATE_SCALAR, "null"),
    (1, 2, 4, 64, 64, 16, 1000, "bf16", synth.GATE_SCALAR_FUSED, "inplace"),
    (2, 1, 2, 32, 64, 64, 4100, "bf16", synth.GATE_CHANNEL, "s0"),
    (1, 1, 1, 16, 16, 64, 1700, "f32", synth.GATE_CHANNEL, "s0"),
])
def test_prefill_segmented_carry(B, H_qk, H_v, dk, dv, chunk, T, io, gate, mode):
    """Few (b, h) units and a long sequence: the carry runs as a parallel scan
    of its affine maps over sequence segments (segment 0 beside the maps of
    the middle segments, the start states composed in fp32, then every later
    segment again from its start state).  Checked against the oracle with a
    nonzero, null or in-place initial state and a ragged last chunk."""
    require_gpu()
    P = carry_segments(B, T, H_v, dk, dv, chunk)
    assert P >= 3, "case no longer takes the segmented carry"
    case = synth.prefill_case("seg", 500 + T % 97, B, T, H_qk, H_v, dk, dv, chunk, io, gate,
                              0.01, 0.3, 0.0 if mode == "null" else 0.3)
    announce(f"prefill segmented carry P={P} io={io} B={B} T={T} H {H_qk}->{H_v} dk={dk} "
             f"dv={dv} chunk={chunk} gate={gate} {mode}")
    kw = {"inplace": True} if mode == "inplace" else ({"state_in": None} if mode == "null" else {})
    o, S = run_prefill(case, o_fill=float("nan"), **kw)
    o_ref, S_ref = _oracle(case)
    eo, es = rel(o, o_ref), rel(S, S_ref)
    print(f"err o={eo:.3e} S={es:.3e}")
    assert eo < TOL[io] and es < TOL[io]


@pytest.mark.timeout(600)
def test_prefill_segmented_carry_long():
    """B=1, 4 value heads, dk=dv=128, T=20000 (313 chunks) in bf16 with a
    channel gate: the longest segmented case, every output and the state
    against the oracle."""
    require_gpu()
    B, T, H_qk, H_v = 1, 20000, 1, 4
    P = carry_segments(B, T, H_v, 128, 128, 64)
    assert P >= 3
    case = synth.prefill_case("seglong", 520, B, T, H_qk, H_v, 128, 128, 64, "bf16",
                              synth.GATE_CHANNEL, 0.001, 0.2, 0.02)
    announce(f"prefill segmented carry long P={P} B=1 T=20000 H 1->4 dk=dv=128 bf16")
    o, S = run_prefill(case, o_fill=float("nan"))
    o_ref, S_ref = _oracle(case)
    eo, es = rel(o, o_ref), rel(S, S_ref)
    print(f"err o={eo:.3e} S={es:.3e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("H_v", [2, 40])
def test_prefill_weak_decay_long(H_v):
    """Weak decay (log-decay -U(0.0005, 0.005)) over T=20000 with a nonzero
    initial state: the state carries across the whole sequence, so rounding
    compounds over 313 chunks.  With 2 value heads the carry is segmented (16
    segments, each map's rounding carried through the composed start states);
    with 40 it is one walk.  Both against the oracle, on sampled heads for the
    wider case."""
    require_gpu()
    B, T, dk, dv, C = 1, 20000, 64, 64, 64
    H_qk = H_v // 2
    P = carry_segments(B, T, H_v, dk, dv, C)
    assert (P >= 3) == (H_v == 2)
    case = synth.prefill_case("weak", 530 + H_v, B, T, H_qk, H_v, dk, dv, C, "bf16",
                              synth.GATE_CHANNEL, 0.0005, 0.005, 0.05)
    announce(f"prefill weak decay T=20000 H {H_qk}->{H_v} dk=dv=64 segments={P}")
    o, S = run_prefill(case, o_fill=float("nan"))
    if H_v == 2:
        o_ref, S_ref = _oracle(case)
        eo, es = rel(o, o_ref), rel(S, S_ref)
    else:
        ref = _oracle(case, heads=[(0, 0), (0, 17), (0, 39)])
        eo = max(rel(o[b, :, h], o_r[0, :, 0]) for (b, h), (o_r, _) in ref.items())
        es = max(rel(S[b, h], S_r[0, 0]) for (b, h), (_, S_r) in ref.items())
    print(f"err o={eo:.3e} S={es:.3e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


def test_prefill_split_sequence_equals_whole():
    require_gpu()
    case = synth.prefill_case("split", 61, 2, 150, 2, 2, 64, 64, 32, "f32", synth.GATE_CHANNEL,
                              0.01, 0.3, 0.4)
    announce("prefill split 150 = 70 + 80, fp32")
    o, S = run_prefill(case)
    o1, S1 = run_prefill(case, T_slice=slice(0, 70))
    o2, S2 = run_prefill(case, T_slice=slice(70, 150), state_in=S1)
    assert rel(np.concatenate([o1, o2], axis=1), o) < 1e-5 and rel(S2, S) < 1e-5


def test_prefill_chunk_size_independent():
    require_gpu()
    case = synth.prefill_case("chunks", 62, 1, 190, 2, 4, 64, 64, 64, "f32", synth.GATE_CHANNEL,
                              0.01, 0.3, 0.4)
    announce("prefill chunk-size independence fp32 T=190")
    res = [run_prefill(case, chunk=c) for c in (16, 32, 64)]
    for o, S in res[1:]:
        assert rel(o, res[0][0]) < 1e-5 and rel(S, res[0][1]) < 1e-5


def test_prefill_t1_equals_decode():
    require_gpu()
    case = synth.prefill_case("t1", 63, 3, 1, 2, 4, 32, 32, 16, "f32", synth.GATE_SCALAR_FUSED,
                              0.0, 0.0, 0.5)
    announce("prefill T=1 vs decode, fused gate")
    o_p, S_p = run_prefill(case)
    t = case.tensors
    qkv = np.concatenate([t["q"][:, 0].reshape(3, -1), t["k"][:, 0].reshape(3, -1),
                          t["v"][:, 0].reshape(3, -1)], axis=1)
    S = to_dev(t["S0"])
    o = torch.empty((3, 4, 32), device=DEV)
    gdr.gdr_decode_step(to_dev(qkv), to_dev(t["gate_in"][:, 0]), to_dev(t["beta_logit"][:, 0]),
                        S, o, H_qk=2, H_v=4, dk=32, dv=32, gate=case.gate,
                        A_log=to_dev(t["A_log"]), dt_bias=to_dev(t["dt_bias"]))
    torch.cuda.synchronize()
    assert rel(o_p[:, 0], to_host(o)) < 1e-5 and rel(S_p, to_host(S)) < 1e-5


@pytest.mark.parametrize("gate", [synth.GATE_CHANNEL, synth.GATE_SCALAR_FUSED])
def test_prefill_equals_decode_steps(gate):
    """One prefill over T=37 tokens (chunk 16: 2 full chunks + 5) against 37
    consecutive decode steps from the same state, fp32 io: outputs and final
    state agree to the fp32 tolerance."""
    require_gpu()
    T, B, H_qk, H_v, d = 37, 2, 2, 4, 32
    case = synth.prefill_case("pd", 66, B, T, H_qk, H_v, d, d, 16, "f32", gate, 0.01, 0.3, 0.4)
    announce(f"prefill T=37 vs 37 decode steps, gate={gate}")
    o_p, S_p = run_prefill(case)
    t = case.tensors
    S = to_dev(t["S0"])
    o = torch.empty((B, H_v, d), device=DEV)
    o_d = np.empty((B, T, H_v, d))
    for i in range(T):
        qkv = np.concatenate([t["q"][:, i].reshape(B, -1), t["k"][:, i].reshape(B, -1),
                              t["v"][:, i].reshape(B, -1)], axis=1)
        gdr.gdr_decode_step(to_dev(qkv), to_dev(t["gate_in"][:, i]), to_dev(t["beta_logit"][:, i]),
                            S, o, H_qk=H_qk, H_v=H_v, dk=d, dv=d, gate=gate,
                            A_log=to_dev(t["A_log"]), dt_bias=to_dev(t["dt_bias"]))
        o_d[:, i] = to_host(o)
    S_d = to_host(S)
    assert rel(o_p, o_d) < TOL["f32"] and rel(S_p, S_d) < TOL["f32"]


def test_prefill_inplace_state():
    require_gpu()
    case = synth.prefill_case("inplace", 64, 2, 100, 1, 2, 32, 32, 32, "f32", synth.GATE_CHANNEL,
                              0.01, 0.3, 0.4)
    announce("prefill state_in == state_out")
    o, S = run_prefill(case, inplace=True)
    o_ref, S_ref = _oracle(case)
    assert rel(o, o_ref) < TOL["f32"] and rel(S, S_ref) < TOL["f32"]


def test_prefill_zero_state_in_null():
    require_gpu()
    case = synth.prefill_case("null", 65, 1, 40, 1, 1, 16, 16, 16, "f32", synth.GATE_CHANNEL,
                              0.01, 0.3, 0.0)
    o, S = run_prefill(case, state_in=None)
    o_ref, S_ref = _oracle(case)
    assert rel(o, o_ref) < TOL["f32"] and rel(S, S_ref) < TOL["f32"]


def test_prefill_t0_copies_state():
    require_gpu()
    s_in = torch.randn((2, 2, 16, 16), device=DEV)
    s_out = torch.zeros_like(s_in)
    e = torch.empty((2, 0, 1, 16), device=DEV)
    ev = torch.empty((2, 0, 2, 16), device=DEV)
    gdr.gdr_prefill_chunked(e, e, ev, torch.empty((2, 0, 2, 16), device=DEV),
                            torch.empty((2, 0, 2), device=DEV), s_in, s_out, ev.clone(), None,
                            H_qk=1, H_v=2, dk=16, dv=16, chunk=16, gate=synth.GATE_CHANNEL)
    torch.cuda.synchronize()
    assert torch.equal(s_in, s_out)


# Every byte a chunked prefill writes lies inside the workspace the size query
# asks for: the workspace is a view at the start of a larger buffer whose tail
# (64 KiB) holds a byte pattern that must come back unchanged.  Both gate
# layouts (the channel gate's blocks; the scalar gate's smaller blocks plus
# the per-qk-head rows), the plain and the segmented carry, both io dtypes.
@pytest.mark.parametrize("B,T,H_qk,H_v,dk,dv,chunk,io,gate", [
    (2, 333, 2, 4, 64, 64, 32, "bf16", synth.GATE_CHANNEL),
    (2, 333, 2, 4, 64, 64, 32, "bf16", synth.GATE_SCALAR),
    (1, 2500, 1, 2, 64, 64, 32, "bf16", synth.GATE_CHANNEL),
    (1, 2500, 1, 2, 64, 64, 32, "f32", synth.GATE_SCALAR_FUSED),
    (4, 130, 16, 32, 128, 128, 64, "bf16", synth.GATE_SCALAR),
])
def test_prefill_writes_stay_in_workspace(B, T, H_qk, H_v, dk, dv, chunk, io, gate):
    require_gpu()
    case = synth.prefill_case("canary", 480 + T % 89 + gate, B, T, H_qk, H_v, dk, dv, chunk, io,
                              gate, 0.01, 0.3, 0.3)
    n = gdr.gdr_prefill_workspace_size(B, T, H_qk, H_v, dk, dv, chunk, io_dtype(io), gate)
    pad = 64 << 10
    announce(f"prefill workspace bounds: B={B} T={T} H {H_qk}->{H_v} dk={dk} dv={dv} chunk={chunk} "
             f"io={io} gate={gate} workspace {n} B, carry segments "
             f"{carry_segments(B, T, H_v, dk, dv, chunk)}")
    buf = torch.empty(n + pad, dtype=torch.uint8, device=DEV)
    pattern = (torch.arange(pad, device=DEV, dtype=torch.int32) * 37 + 11).remainder(251).to(torch.uint8)
    buf[n:] = pattern
    t = case.tensors
    S = torch.empty((B, H_v, dk, dv), dtype=torch.float32, device=DEV)
    o = torch.empty((B, T, H_v, dv), dtype=io_dtype(io), device=DEV)
    gdr.gdr_prefill_chunked(to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"]), to_dev(t["gate_in"]),
                            to_dev(t["beta_logit"]), to_dev(t["S0"]), S, o, buf[:n], H_qk=H_qk,
                            H_v=H_v, dk=dk, dv=dv, chunk=chunk, gate=gate,
                            A_log=to_dev(t["A_log"]), dt_bias=to_dev(t["dt_bias"]))
    torch.cuda.synchronize()
    assert torch.equal(buf[n:], pattern), "a prefill wrote past its workspace"
    o_ref, S_ref = _oracle(case)
    assert rel(to_host(o), o_ref) < TOL[io] and rel(to_host(S), S_ref) < TOL[io]
