"""gdr_prefill_chunked_noalloc on the GPU: the prefill on the library's own
device scratch must give exactly what gdr_prefill_chunked gives with a
caller workspace, call after call on the same scratch (each call smaller than
the one before, so stale contents of a larger call sit beyond the smaller
one's workspace), and it must refuse a call that needs more than the scratch
holds before anything is enqueued."""
from __future__ import annotations

import pytest
import torch

import gated_delta_rule_40_amd as gdr
from gated_delta_rule_40_amd import synth
from tests.gpu_util import (DEV, announce, io_dtype, new_workspace, require_gpu, to_dev)

pytestmark = pytest.mark.gpu


def _inputs(case):
    t = case.tensors
    return dict(q=to_dev(t["q"]), k=to_dev(t["k"]), v=to_dev(t["v"]), g=to_dev(t["gate_in"]),
                bl=to_dev(t["beta_logit"]), s0=to_dev(t["S0"]), A_log=to_dev(t["A_log"]),
                dt_bias=to_dev(t["dt_bias"]))


def _outputs(case):
    o = torch.full((case.B, case.T, case.H_v, case.dv), float("nan"), dtype=io_dtype(case.io),
                   device=DEV)
    s = torch.full((case.B, case.H_v, case.dk, case.dv), float("nan"), device=DEV)
    return o, s


def _both(case):
    """(o, S) from the caller-workspace entry point and from the allocation-free one."""
    x = _inputs(case)
    kw = dict(H_qk=case.H_qk, H_v=case.H_v, dk=case.dk, dv=case.dv, chunk=case.chunk,
              gate=case.gate, A_log=x["A_log"], dt_bias=x["dt_bias"], scale=0.5)
    o_ref, s_ref = _outputs(case)
    ws = new_workspace(case.B, case.T, case.H_qk, case.H_v, case.dk, case.dv, case.chunk, case.io,
                       case.gate)
    gdr.gdr_prefill_chunked(x["q"], x["k"], x["v"], x["g"], x["bl"], x["s0"], s_ref, o_ref, ws,
                            **kw)
    o, s = _outputs(case)
    gdr.gdr_prefill_chunked_noalloc(x["q"], x["k"], x["v"], x["g"], x["bl"], x["s0"], s, o, **kw)
    torch.cuda.synchronize()
    return (o, s), (o_ref, s_ref)


# Three calls in a row on the same scratch, each with a smaller workspace than
# the one before: the largest workload that fits (B=1, T=4032, H 16 -> 32,
# dk=dv=128, chunk 64, bf16: 127 MiB of chunk blocks), a long prefill over two
# heads (the segmented carry, whose fp32 segment states follow the blocks) and
# a short fp32 one.
CASES = [
    ("limit", lambda: synth.prefill_case("na_limit", 601, 1, 4032, 16, 32, 128, 128, 64, "bf16",
                                         synth.GATE_CHANNEL, 0.001, 0.2, 0.02)),
    ("segmented", lambda: synth.prefill_case("na_seg", 602, 1, 3000, 1, 2, 128, 128, 64, "bf16",
                                             synth.GATE_CHANNEL, 0.001, 0.2, 0.02)),
    ("small", lambda: synth.prefill_case("na_small", 603, 2, 200, 2, 4, 64, 64, 32, "f32",
                                         synth.GATE_SCALAR, 0.01, 0.3, 0.3)),
]


def test_noalloc_matches_workspace_entry_point_call_after_call():
    require_gpu()
    sizes = []
    for name, make in CASES:
        case = make()
        sizes.append(gdr.gdr_prefill_workspace_size(case.B, case.T, case.H_qk, case.H_v, case.dk,
                                                    case.dv, case.chunk, io_dtype(case.io),
                                                    case.gate))
        announce(f"noalloc prefill {name}: B={case.B} T={case.T} H {case.H_qk}->{case.H_v} "
                 f"dk={case.dk} dv={case.dv} chunk={case.chunk} io={case.io} gate={case.gate} "
                 f"workspace {sizes[-1]} B")
        assert sizes[-1] <= gdr.binding.NOALLOC_SCRATCH_BYTES
        (o, s), (o_ref, s_ref) = _both(case)
        assert not torch.isnan(o_ref).any() and not torch.isnan(s_ref).any()
        assert torch.equal(o, o_ref), name
        assert torch.equal(s, s_ref), name
    assert sizes[0] > sizes[1] > sizes[2]


def test_noalloc_refuses_more_than_its_scratch():
    require_gpu()
    case = synth.prefill_case("na_big", 604, 1, 4033, 16, 32, 128, 128, 64, "bf16",
                              synth.GATE_CHANNEL, 0.001, 0.2, 0.0)
    announce("noalloc prefill beyond the scratch: B=1 T=4033 H 16->32 (expects GDR_E_SCRATCH)")
    x = _inputs(case)
    o, s = _outputs(case)
    with pytest.raises(gdr.GdrError) as err:
        gdr.gdr_prefill_chunked_noalloc(x["q"], x["k"], x["v"], x["g"], x["bl"], None, s, o,
                                        H_qk=16, H_v=32, dk=128, dv=128, chunk=64,
                                        gate=case.gate)
    assert err.value.status == -9
    torch.cuda.synchronize()
    assert torch.isnan(o).all() and torch.isnan(s).all()   # nothing was enqueued
