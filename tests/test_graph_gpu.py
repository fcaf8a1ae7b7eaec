"""Decode steps and prefills (chunked, segmented and token-by-token) captured
in a HIP graph: every replay must reproduce the eager result exactly (same
kernels, same inputs).  The replays are separated by eager work and
synchronisation."""
from __future__ import annotations

import pytest
import torch

import gated_delta_rule_40_amd as gdr
from gated_delta_rule_40_amd import synth
from tests.gpu_util import DEV, announce, carry_segments, new_workspace, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    require_gpu()
    announce("graph capture: 6 decode steps (B=4) + prefills T=100, T=9 and T=1100 (segmented "
             "carry), 3 replays")
    dec = synth.decode_case("graph", 71, 4, 6, 2, 4, 64, 64, "bf16", synth.GATE_CHANNEL,
                            0.01, 0.5, 0.3)
    td = dec.tensors
    qkv, g, bl = to_dev(td["qkv"]), to_dev(td["gate_in"]), to_dev(td["beta_logit"])
    S0 = to_dev(td["S0"])
    S = S0.clone()
    o = torch.empty((4, 4, 64), dtype=torch.bfloat16, device=DEV)
    kw = dict(H_qk=2, H_v=4, dk=64, dv=64, gate=synth.GATE_CHANNEL)

    pre = synth.prefill_case("graph_p", 72, 2, 100, 2, 4, 64, 64, 32, "bf16", synth.GATE_SCALAR,
                             0.01, 0.3, 0.3)
    tp = pre.tensors
    pq, pk, pv = to_dev(tp["q"]), to_dev(tp["k"]), to_dev(tp["v"])
    pg, pb, ps0 = to_dev(tp["gate_in"]), to_dev(tp["beta_logit"]), to_dev(tp["S0"])
    ps = torch.empty_like(ps0)
    po = torch.empty((2, 100, 4, 64), dtype=torch.bfloat16, device=DEV)
    ws = new_workspace(2, 100, 2, 4, 64, 64, 32, "bf16", synth.GATE_SCALAR)
    pkw = dict(H_qk=2, H_v=4, dk=64, dv=64, chunk=32, gate=synth.GATE_SCALAR)

    # a short prefill (token-by-token path), its state carried in place
    sh = synth.prefill_case("graph_s", 73, 2, 9, 2, 4, 64, 64, 16, "bf16", synth.GATE_CHANNEL,
                            0.01, 0.3, 0.3)
    ts = sh.tensors
    sq, sk, sv = to_dev(ts["q"]), to_dev(ts["k"]), to_dev(ts["v"])
    sg, sb, ss0 = to_dev(ts["gate_in"]), to_dev(ts["beta_logit"]), to_dev(ts["S0"])
    ss = ss0.clone()
    so = torch.empty((2, 9, 4, 64), dtype=torch.bfloat16, device=DEV)
    sws = new_workspace(2, 9, 2, 4, 64, 64, 16, "bf16", synth.GATE_CHANNEL)
    skw = dict(H_qk=2, H_v=4, dk=64, dv=64, chunk=16, gate=synth.GATE_CHANNEL)

    # a long prefill over few heads (segmented carry: maps, scan, re-run)
    lg = synth.prefill_case("graph_l", 74, 1, 1100, 1, 2, 64, 64, 16, "bf16", synth.GATE_CHANNEL,
                            0.01, 0.3, 0.3)
    assert carry_segments(1, 1100, 2, 64, 64, 16) >= 3
    tl = lg.tensors
    lq, lk, lv = to_dev(tl["q"]), to_dev(tl["k"]), to_dev(tl["v"])
    lgi, lb, ls0 = to_dev(tl["gate_in"]), to_dev(tl["beta_logit"]), to_dev(tl["S0"])
    ls = torch.empty_like(ls0)
    lo = torch.empty((1, 1100, 2, 64), dtype=torch.bfloat16, device=DEV)
    lws = new_workspace(1, 1100, 1, 2, 64, 64, 16, "bf16", synth.GATE_CHANNEL)
    lkw = dict(H_qk=1, H_v=2, dk=64, dv=64, chunk=16, gate=synth.GATE_CHANNEL)

    def work():
        for i in range(6):
            gdr.gdr_decode_step(qkv[i], g[i], bl[i], S, o, **kw)
        gdr.gdr_prefill_chunked(pq, pk, pv, pg, pb, ps0, ps, po, ws, **pkw)
        gdr.gdr_prefill_chunked(sq, sk, sv, sg, sb, ss, ss, so, sws, **skw)
        gdr.gdr_prefill_chunked(lq, lk, lv, lgi, lb, ls0, ls, lo, lws, **lkw)

    work()
    torch.cuda.synchronize()
    ref = (S.clone(), o.clone(), ps.clone(), po.clone(), ss.clone(), so.clone(), ls.clone(),
           lo.clone())

    graph = torch.cuda.CUDAGraph()
    S.copy_(S0)
    ss.copy_(ss0)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            work()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for rep in range(3):
        S.copy_(S0)            # eager work between replays
        ss.copy_(ss0)
        ps.zero_()
        po.zero_()
        so.zero_()
        ls.zero_()
        lo.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (S, o, ps, po, ss, so, ls, lo)
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {rep} differs from eager"
