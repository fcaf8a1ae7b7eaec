"""Parity over a seeded sweep of random shapes and options: batch, length,
head counts and sizes, chunk, gate kind, io dtype, initial state, L2 norm and
output scale, crossed rather than varied one at a time.  Each case runs the
prefill entry point (token-by-token or chunked, whichever it picks) and a few
decode steps, and compares both with the fp64 oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gated_delta_rule_40_amd as gdr
import oracle
from gated_delta_rule_40_amd import synth
from tests.gpu_util import (DEV, TOL, announce, carry_segments, io_dtype, rel, require_gpu,
                            run_prefill, to_dev, to_host)

pytestmark = pytest.mark.gpu

DIMS = (16, 32, 64, 128)
GATES = (synth.GATE_CHANNEL, synth.GATE_SCALAR, synth.GATE_SCALAR_FUSED)


def draw(seed: int) -> dict:
    r = np.random.default_rng(1000 + seed)
    H_qk = int(r.integers(1, 3))
    return dict(
        B=int(r.integers(1, 4)),
        T=int(r.choice([1, 2, int(r.integers(3, 17)), int(r.integers(17, 160))])),
        H_qk=H_qk,
        H_v=H_qk * int(r.integers(1, 4)),
        dk=int(r.choice(DIMS)),
        dv=int(r.choice(DIMS)),
        chunk=int(r.choice([16, 32, 64])),
        gate=int(r.choice(GATES)),
        io=str(r.choice(["f32", "bf16"])),
        s0=float(r.choice([0.0, 0.3])),
        l2norm=bool(r.integers(0, 2)),
        scale_rsqrt=bool(r.integers(0, 2)),
    )


@pytest.mark.parametrize("seed", range(40))
def test_random_shape_prefill_and_decode(seed):
    require_gpu()
    p = draw(seed)
    announce(f"random shape seed={seed}: {p}")
    case = synth.prefill_case(f"rand{seed}", 2000 + seed, p["B"], p["T"], p["H_qk"], p["H_v"],
                              p["dk"], p["dv"], p["chunk"], p["io"], p["gate"], 0.01, 0.4, p["s0"])
    scale = p["dk"] ** -0.5 if p["scale_rsqrt"] else 1.0
    t = case.tensors
    q, k = case.values("q"), case.values("k")
    if not p["l2norm"]:
        # unnormalised rows of a plausible size: the kernels use them as given
        q = q * p["dk"] ** -0.5
        k = k * p["dk"] ** -0.5
        t = dict(t)
        if p["io"] == "bf16":
            t["q"], t["k"] = synth.f32_to_bf16(q), synth.f32_to_bf16(k)
            q, k = synth.bf16_to_f32(t["q"]), synth.bf16_to_f32(t["k"])
        else:
            t["q"], t["k"] = q.astype(np.float32), k.astype(np.float32)
        case = synth.Case(case.name, case.B, case.T, case.H_qk, case.H_v, case.dk, case.dv,
                          case.chunk, case.io, case.gate, t)
    o_ref, S_ref = oracle.sequence(q, k, case.values("v"), case.gate, t["gate_in"],
                                   t["beta_logit"], t["S0"], A_log=t["A_log"],
                                   dt_bias=t["dt_bias"], scale=scale, l2norm=p["l2norm"],
                                   threads=4)
    o, S = run_prefill(case, scale=scale, l2norm=p["l2norm"])
    tol = TOL[p["io"]]
    assert rel(o, o_ref) < tol and rel(S, S_ref) < tol, (rel(o, o_ref), rel(S, S_ref))

    # The first min(T, 3) tokens again as single decode steps from S0.
    steps = min(p["T"], 3)
    S_d = to_dev(t["S0"])
    o_d = torch.empty((p["B"], p["H_v"], p["dv"]), dtype=io_dtype(p["io"]), device=DEV)
    S_o = t["S0"].astype(np.float64)
    for i in range(steps):
        raw = np.concatenate([t["q"][:, i].reshape(p["B"], -1), t["k"][:, i].reshape(p["B"], -1),
                              t["v"][:, i].reshape(p["B"], -1)], axis=1)
        gdr.gdr_decode_step(to_dev(raw), to_dev(t["gate_in"][:, i]),
                            to_dev(t["beta_logit"][:, i]), S_d, o_d, H_qk=p["H_qk"],
                            H_v=p["H_v"], dk=p["dk"], dv=p["dv"], gate=p["gate"],
                            A_log=to_dev(t["A_log"]), dt_bias=to_dev(t["dt_bias"]), scale=scale,
                            l2norm_qk=p["l2norm"])
        vals = synth.bf16_to_f32(raw) if p["io"] == "bf16" else raw
        o_r, S_o = oracle.decode(vals, p["H_qk"], p["H_v"], p["dk"], p["dv"], p["gate"],
                                 t["gate_in"][:, i], t["beta_logit"][:, i], S_o,
                                 A_log=t["A_log"], dt_bias=t["dt_bias"], scale=scale,
                                 l2norm=p["l2norm"])
        assert rel(to_host(o_d), o_r) < tol, (i, rel(to_host(o_d), o_r))
    torch.cuda.synchronize()
    assert rel(to_host(S_d), S_o) < tol


def draw_long(seed: int) -> dict:
    """A long sequence over few (b, h) units: shapes that take the segmented
    carry (the draw is repeated until it does)."""
    r = np.random.default_rng(3000 + seed)
    while True:
        H_qk = int(r.integers(1, 3))
        p = dict(B=int(r.integers(1, 3)), T=int(r.integers(900, 3200)), H_qk=H_qk,
                 H_v=H_qk * int(r.integers(1, 3)), dk=int(r.choice(DIMS)),
                 dv=int(r.choice(DIMS)), chunk=int(r.choice([16, 32, 64])),
                 gate=int(r.choice(GATES)), io=str(r.choice(["f32", "bf16"])),
                 s0=float(r.choice([0.0, 0.3])), inplace=bool(r.integers(0, 2)))
        if carry_segments(p["B"], p["T"], p["H_v"], p["dk"], p["dv"], p["chunk"]) >= 3:
            return p


@pytest.mark.parametrize("seed", range(10))
def test_random_long_few_heads(seed):
    """Seeded long prefills over few heads (segmented carry), crossed over
    head sizes, chunk, gate kind, io dtype and initial state (zero, nonzero,
    in place), every output checked (NaN-filled beforehand) against the
    oracle."""
    require_gpu()
    p = draw_long(seed)
    P = carry_segments(p["B"], p["T"], p["H_v"], p["dk"], p["dv"], p["chunk"])
    announce(f"random long few-head seed={seed} segments={P}: {p}")
    case = synth.prefill_case(f"rlong{seed}", 4000 + seed, p["B"], p["T"], p["H_qk"], p["H_v"],
                              p["dk"], p["dv"], p["chunk"], p["io"], p["gate"], 0.001, 0.2,
                              p["s0"])
    t = case.tensors
    o_ref, S_ref = oracle.sequence(case.values("q"), case.values("k"), case.values("v"),
                                   case.gate, t["gate_in"], t["beta_logit"], t["S0"],
                                   A_log=t["A_log"], dt_bias=t["dt_bias"], threads=4)
    o, S = run_prefill(case, inplace=p["inplace"], o_fill=float("nan"))
    tol = TOL[p["io"]]
    assert rel(o, o_ref) < tol and rel(S, S_ref) < tol, (rel(o, o_ref), rel(S, S_ref))
