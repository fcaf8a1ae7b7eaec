#!/usr/bin/env python3
"""Benchmark of the gated delta rule on one MI355X.

Three default legs, on seeded synthetic inputs already resident in HBM:

  decode   gdr_decode_step on the batched channelwise workload: B=64,
           H_qk=16 -> H_v=32, dk=dv=128, bf16 packed q|k|v rows, fp32 state
           (128 MiB), fresh inputs every step, the state carried from step to
           step.  One bench step = one decode token for the whole batch.
           The timed steps are captured once in a HIP graph and replayed (as a
           serving loop would issue them); eager per-launch timings are
           reported beside it.  Reported as state-update GB/s: the
           algorithmic bytes of a step (state read + write, qkv, gate, beta,
           o) over its time.
  prefill  gdr_prefill_chunked on B=1, T=4000, chunk 64, H 16 -> 32,
           dk=dv=128, bf16, channelwise gate, zero initial state.  Reported as
           tokens/s, with the fraction of the HBM and bf16 MFMA peaks.
  long     gdr_prefill_chunked on B=4, T=32767, chunk 64, H 16 -> 32,
           dk=dv=128, bf16, carried-in state, scalar and channelwise gates
           (under "prefill_long"), reported like the prefill leg.

Opt-in legs: sweep (T decode steps against one prefill), segmented (B=1,
H 2 -> 4, T=32767: the long prefill over few heads that takes the segmented
carry, under "prefill_segmented") and copy (HBM-counter calibration).

Prints one JSON line.  `value` is the decode GB/s; the prefill figures sit
under "prefill".  Each leg carries its roofline (kernel time from HIP events
recorded around every launch on the launch stream) and the fp64 CPU oracle
timed on a bounded sample of the same workload ("cpu_baseline": all host
cores, with a one-thread figure under "single_thread").
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time
from pathlib import Path

import numpy as np
import torch

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

import gated_delta_rule_40_amd as gdr  # noqa: E402
from gated_delta_rule_40_amd import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "decode state-update GB/s (% of HBM peak); chunked prefill tokens/s"
DEV = "cuda:0"


def up(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


def cpu_threads() -> int:
    # At most 16 host threads: the host's share per GPU, whatever os.cpu_count() reports.
    return max(1, min(16, os.cpu_count() or 1))


_CODE_TOKENS = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/', re.S)


def code_text(src: str) -> str:
    """The source with its comments removed and every run of whitespace made
    one space: what the compiler sees, so a change to comments alone keeps the
    digest."""
    def keep(m):
        t = m.group(0)
        return " " if t.startswith("/") else t
    return " ".join(_CODE_TOKENS.sub(keep, src).split())


def source_digest(*names) -> str:
    """Digest of the code (comments and whitespace aside) of kernel sources."""
    h = hashlib.sha256()
    for n in names:
        src = (ROOT / "gated_delta_rule_40_amd" / "csrc" / n).read_text()
        h.update(code_text(src).encode())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel_key: str, digest: str):
    """HBM bytes per launch measured by rocprofv3 counters, if they were taken
    on the current kernel source (else None)."""
    p = ROOT / "profiles" / "hbm_traffic.json"
    if not p.exists():
        return None
    rec = json.loads(p.read_text()).get(kernel_key)
    if not rec or rec.get("source_digest") != digest:
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
def decode_bytes_per_step(B, H_qk, H_v, dk, dv, fused_gate=False) -> int:
    state = 2 * B * H_v * dk * dv * 4
    qkv = B * (2 * H_qk * dk + H_v * dv) * 2
    # channel gate: g [B,H_v,dk]; fused scalar gate: x [B,H_v] plus A_log, dt_bias [H_v]
    gate = (B * H_v + 2 * H_v) * 4 if fused_gate else B * H_v * dk * 4
    beta = B * H_v * 4
    o = B * H_v * dv * 2
    return state + qkv + gate + beta + o


def host_cpu() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def bench_decode_b1_fused(K=256):
    """The single-sequence fused step: B=1, H_qk=16 -> H_v=32, dk=dv=128, bf16
    packed q|k|v, scalar decay -exp(A_log) softplus(x + dt_bias), fresh inputs
    every step, the state carried; K steps captured in a HIP graph and
    replayed.  At 4.2 MB per step this is a latency figure, not a bandwidth
    one."""
    case = synth.fused_decode(seed=2, steps=K)
    t = case.tensors
    qkv, x, bl = up(t["qkv"]), up(t["gate_in"]), up(t["beta_logit"])
    A_log, dt = up(t["A_log"]), up(t["dt_bias"])
    S0 = up(t["S0"])
    S = S0.clone()
    o = torch.empty((1, case.H_v, case.dv), dtype=torch.bfloat16, device=DEV)
    kw = dict(H_qk=case.H_qk, H_v=case.H_v, dk=case.dk, dv=case.dv, gate=case.gate,
              A_log=A_log, dt_bias=dt)

    def run():
        for i in range(K):
            gdr.gdr_decode_step(qkv[i], x[i], bl[i], S, o, **kw)

    S.copy_(S0)
    us = graph_us(run, reps=3) / K
    nbytes = decode_bytes_per_step(1, case.H_qk, case.H_v, case.dk, case.dv, fused_gate=True)
    return dict(workload="fused_decode_b1: B=1, H_qk=16->H_v=32, dk=dv=128, bf16 packed q|k|v, "
                         "fused scalar gate, fresh inputs per step",
                us_per_step=us, gbs=nbytes / us / 1e3, bytes_per_step=nbytes,
                timing=f"HIP events around graph replays of {K} steps, / steps")


def bench_decode(K, W, B):
    case = synth.batched_decode(seed=3, steps=256, B=B)
    t = case.tensors
    H_qk, H_v, dk, dv = case.H_qk, case.H_v, case.dk, case.dv
    n_in = t["qkv"].shape[0]
    qkv = up(t["qkv"])
    g = up(t["gate_in"])
    bl = up(t["beta_logit"])
    S0 = up(t["S0"])
    S = S0.clone()
    o = torch.empty((B, H_v, dv), dtype=torch.bfloat16, device=DEV)
    kw = dict(H_qk=H_qk, H_v=H_v, dk=dk, dv=dv, gate=case.gate)

    def step(i):
        j = i % n_in
        gdr.gdr_decode_step(qkv[j], g[j], bl[j], S, o, **kw)

    for i in range(W):
        step(i)
    S.copy_(S0)  # pristine state, outside the timed region
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        starts[i].record()
        step(i)
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    eager_region_ms = starts[0].elapsed_time(ends[-1])
    nbytes = decode_bytes_per_step(B, H_qk, H_v, dk, dv)

    # The same K steps captured once in a HIP graph and replayed: the way a
    # serving loop issues decode steps, without per-launch host gaps.
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for i in range(K):
                step(i)
    torch.cuda.current_stream().wait_stream(cap)
    graph.replay()                       # warm replay
    S.copy_(S0)                          # pristine state, outside the timed region
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0.record()
    graph.replay()
    g1.record()
    torch.cuda.synchronize()
    wall_graph = time.perf_counter() - t0
    graph_ms = g0.elapsed_time(g1)
    del graph

    kern_s = graph_ms / K / 1e3          # average launch duration inside the replay
    achieved = nbytes / kern_s / 1e9
    ceiling = inplace_ceiling(S, K)
    digest = source_digest("decode.hip")
    traffic = traffic_from_profile(f"decode_b{B}", digest)
    return dict(
        value=nbytes * K / wall_graph / 1e9,
        wall_s=wall_graph,
        ms_per_step=wall_graph / K * 1e3,
        eager=dict(value=nbytes * K / wall / 1e9, ms_per_step=wall / K * 1e3,
                   region_event_ms=eager_region_ms,
                   launch_event_us_mean=float(np.mean(per_launch_ms)) * 1e3,
                   launch_event_us_median=float(np.median(per_launch_ms)) * 1e3),
        graph_event_ms=graph_ms,
        kernel_us_mean=kern_s * 1e6,
        bytes_per_step=nbytes,
        roofline=dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=achieved / HBM_PEAK_GBS, traffic=traffic,
                      kernel="gdr::decode_kernel (bf16 io, dk=dv=128, channel gate)",
                      timing="HIP events around the graph replay of all timed steps, / steps",
                      source_digest=digest,
                      inplace_ceiling=dict(ceiling, frac=achieved / ceiling["gbs"])),
        case=case,
    )


def inplace_ceiling(S, K):
    """The practical ceiling of an in-place state update: torch's own elementwise
    kernel scaling the same fp32 state buffer in place (read + write of every
    byte, random values), K launches captured in a graph like the decode steps.
    The factors alternate between 2 and 1/2 over an even number of launches,
    which is exact, so S comes back unchanged.  Memory traffic on this part depends on the values moved (an
    all-zero buffer streams markedly faster), so the ceiling is taken on the
    state itself."""
    n = K + K % 2
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for i in range(n):
                S.mul_(2.0 if i % 2 == 0 else 0.5)
    torch.cuda.current_stream().wait_stream(cap)
    graph.replay()                       # warm replay
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    nbytes = 2 * S.numel() * S.element_size()
    del graph
    return dict(gbs=nbytes / us / 1e3, us=us, bytes=nbytes,
                kernel="torch in-place mul_ on the fp32 state (graph replay)")


def _cpu_decode_mode(case, seconds, threads):
    import oracle

    t = case.tensors
    thr = oracle.threads_used(threads)
    S = t["S0"].astype(np.float64)
    steps = 0
    t0 = time.perf_counter()
    while steps < t["qkv"].shape[0]:
        _, S = oracle.decode(synth.bf16_to_f32(t["qkv"][steps]), case.H_qk, case.H_v, case.dk,
                             case.dv, case.gate, t["gate_in"][steps], t["beta_logit"][steps], S,
                             threads=thr)
        steps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    nbytes = decode_bytes_per_step(case.B, case.H_qk, case.H_v, case.dk, case.dv)
    return dict(value=nbytes * steps / el / 1e9, unit="GB/s", cores=thr, kind="oracle",
                sample=f"{steps} consecutive decode steps of the B={case.B} batch "
                       f"({el:.1f} s, fp64 C recurrence"
                       + (", OpenMP over (b,h))" if thr > 1 else ", one thread)"))


def cpu_decode(case, seconds):
    """The fp64 oracle on the decode workload: all host cores (the reported
    baseline) and one thread, each time-boxed."""
    out = _cpu_decode_mode(case, seconds, cpu_threads())
    out["host"] = host_cpu()
    out["nproc"] = os.cpu_count()
    out["single_thread"] = _cpu_decode_mode(case, seconds / 2, 1)
    return out


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------
def prefill_flops(T, B, H_v, dk, dv, C) -> float:
    per = 6 * dk * dv + 2 * C * (3 * dk + 2 * dv) + C * C / 3
    return per * T * B * H_v


def prefill_bytes(T, B, H_qk, H_v, dk, dv, channel=True, state_in=False) -> int:
    per_tok = 2 * H_qk * dk * 2 + H_v * dv * 2 + (H_v * dk if channel else H_v) * 4 \
        + H_v * 4 + H_v * dv * 2
    state = B * H_v * dk * dv * 4 * (2 if state_in else 1)
    return per_tok * T * B + state


def bench_prefill(reps, warm):
    case = synth.prefill(seed=4)
    t = case.tensors
    B, T, C = case.B, case.T, case.chunk
    H_qk, H_v, dk, dv = case.H_qk, case.H_v, case.dk, case.dv
    q, k, v = up(t["q"]), up(t["k"]), up(t["v"])
    g, bl = up(t["gate_in"]), up(t["beta_logit"])
    S = torch.empty((B, H_v, dk, dv), dtype=torch.float32, device=DEV)
    o = torch.empty((B, T, H_v, dv), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(gdr.gdr_prefill_workspace_size(B, T, H_qk, H_v, dk, dv, C, torch.bfloat16,
                                                    case.gate), dtype=torch.uint8, device=DEV)
    kw = dict(H_qk=H_qk, H_v=H_v, dk=dk, dv=dv, chunk=C, gate=case.gate)

    def run():
        gdr.gdr_prefill_chunked(q, k, v, g, bl, None, S, o, ws, **kw)

    for _ in range(warm):
        run()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(reps):
        starts[i].record()
        run()
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    eager_sec = float(np.mean(ms)) / 1e3

    # The same calls captured once in a HIP graph and replayed, as the decode
    # leg does: the launches go back to back without host gaps.
    def run_all():
        for _ in range(reps):
            run()

    sec = graph_us(run_all, reps=3) / reps / 1e6
    flops = prefill_flops(T, B, H_v, dk, dv, C)
    nbytes = prefill_bytes(T, B, H_qk, H_v, dk, dv, channel=True, state_in=False)
    return dict(
        value=B * T / sec,
        unit="tokens/s",
        ms_per_call=sec * 1e3,
        timing=f"HIP events around graph replays of {reps} calls, / calls",
        eager=dict(value=B * T / eager_sec, ms_per_call=eager_sec * 1e3,
                   timing="HIP events around each call, mean"),
        wall_tokens_per_s=B * T * reps / wall,
        workload=f"prefill_t{T}: B={B}, T={T} (62 chunks of 64 + 32), H_qk={H_qk}->H_v={H_v}, "
                 f"dk=dv={dk}, chunk {C}, channelwise gate, bf16 io, zero initial state",
        dtype="bf16",
        roofline=dict(bound="hbm", achieved=nbytes / sec / 1e9, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=nbytes / sec / 1e9 / HBM_PEAK_GBS,
                      mfma_achieved_tflops=flops / sec / 1e12,
                      mfma_peak_tflops=MFMA_BF16_PEAK_TFLOPS,
                      mfma_frac=flops / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                      algorithmic_bytes=nbytes, algorithmic_flops=flops,
                      traffic=traffic_from_profile("prefill_t4000",
                                                   source_digest("prefill.hip"))),
        case=case,
    )


def bench_prefill_long(gate, reps=3, warm=1, seed=None, cpu_seconds=0.0):
    """The long prefill with a carried-in state: B=4, T=32767 (511 chunks of 64
    and one of 63), H_qk=16 -> H_v=32, dk=dv=128, bf16 io, fp32 state with
    S0 ~ N(0, 0.02^2); q, k, v ~ N(0,1) rounded to bf16, log-decay
    g ~ -U(0.001, 0.2) per (b, t, h) (scalar gate) or per (b, t, h, channel)
    (channel gate), beta logits ~ N(0,1).  Drawn on the device from a seeded
    torch generator in that order (the 4 GB of inputs would take a minute to
    draw on the host).  Graph replay of `reps` calls, as in the prefill leg."""
    B, T, H_qk, H_v, dk, dv, C = 4, 32767, 16, 32, 128, 128, 64
    channel = gate == synth.GATE_CHANNEL
    if seed is None:
        seed = 52 if channel else 51
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    bf = torch.bfloat16
    q = torch.randn(B, T, H_qk, dk, device=DEV, generator=gen).to(bf)
    k = torch.randn(B, T, H_qk, dk, device=DEV, generator=gen).to(bf)
    v = torch.randn(B, T, H_v, dv, device=DEV, generator=gen).to(bf)
    gshape = (B, T, H_v, dk) if channel else (B, T, H_v)
    g = -(torch.rand(gshape, device=DEV, generator=gen) * 0.199 + 0.001)
    bl = torch.randn(B, T, H_v, device=DEV, generator=gen)
    S0 = torch.randn(B, H_v, dk, dv, device=DEV, generator=gen) * 0.02
    S = torch.empty_like(S0)
    o = torch.empty((B, T, H_v, dv), dtype=bf, device=DEV)
    ws_bytes = gdr.gdr_prefill_workspace_size(B, T, H_qk, H_v, dk, dv, C, bf, gate)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    kw = dict(H_qk=H_qk, H_v=H_v, dk=dk, dv=dv, chunk=C, gate=gate)

    def run_all():
        for _ in range(reps):
            gdr.gdr_prefill_chunked(q, k, v, g, bl, S0, S, o, ws, **kw)

    for _ in range(warm):
        run_all()
    sec = graph_us(run_all, reps=2) / reps / 1e6
    flops = prefill_flops(T, B, H_v, dk, dv, C)
    nbytes = prefill_bytes(T, B, H_qk, H_v, dk, dv, channel=channel, state_in=True)
    out = dict(
        value=B * T / sec, unit="tokens/s", ms_per_call=sec * 1e3,
        timing=f"HIP events around graph replays of {reps} calls, / calls",
        workload=f"long_prefill_{'channel' if channel else 'scalar'}: B={B}, T={T}, "
                 f"H_qk={H_qk}->H_v={H_v}, dk=dv={dk}, chunk {C}, "
                 f"{'channelwise' if channel else 'scalar'} gate, bf16 io, S0 ~ N(0, 0.02^2)",
        workspace_bytes=ws_bytes,
        roofline=dict(bound="hbm", achieved=nbytes / sec / 1e9, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=nbytes / sec / 1e9 / HBM_PEAK_GBS,
                      mfma_achieved_tflops=flops / sec / 1e12,
                      mfma_peak_tflops=MFMA_BF16_PEAK_TFLOPS,
                      mfma_frac=flops / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                      algorithmic_bytes=nbytes, algorithmic_flops=flops,
                      traffic=traffic_from_profile(
                          f"long_prefill_{'channel' if channel else 'scalar'}",
                          source_digest("prefill.hip"))),
    )
    if cpu_seconds > 0:
        out["cpu_baseline"] = cpu_prefill(device_fetch(q, k, v, g, bl, S0, H_v // H_qk), B, T,
                                          H_qk, H_v, gate, cpu_seconds)
    del q, k, v, g, bl, S0, S, o, ws
    torch.cuda.empty_cache()
    return out


def bench_prefill_segmented(reps=4, warm=1):
    """A long prefill over few heads, where the carry runs as a parallel scan
    of per-segment affine maps: B=1, H_qk=2 -> H_v=4, dk=dv=128, T=32767,
    chunk 64, bf16, channelwise gate with log-decay -U(0.001, 0.2), nonzero
    initial state.  Graph replay of `reps` calls, as in the prefill leg."""
    B, T, H_qk, H_v, dk, dv, C = 1, 32767, 2, 4, 128, 128, 64
    case = synth.prefill_case("bench_seg", 9, B, T, H_qk, H_v, dk, dv, C, "bf16",
                              synth.GATE_CHANNEL, 0.001, 0.2, 0.02)
    t = case.tensors
    q, k, v = up(t["q"]), up(t["k"]), up(t["v"])
    g, bl, S0 = up(t["gate_in"]), up(t["beta_logit"]), up(t["S0"])
    S = torch.empty_like(S0)
    o = torch.empty((B, T, H_v, dv), dtype=torch.bfloat16, device=DEV)
    ws_bytes = gdr.gdr_prefill_workspace_size(B, T, H_qk, H_v, dk, dv, C, torch.bfloat16,
                                              case.gate)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    kw = dict(H_qk=H_qk, H_v=H_v, dk=dk, dv=dv, chunk=C, gate=case.gate)

    def run_all():
        for _ in range(reps):
            gdr.gdr_prefill_chunked(q, k, v, g, bl, S0, S, o, ws, **kw)

    for _ in range(warm):
        run_all()
    sec = graph_us(run_all, reps=2) / reps / 1e6
    return dict(
        value=B * T / sec, unit="tokens/s", ms_per_call=sec * 1e3,
        timing=f"HIP events around graph replays of {reps} calls, / calls",
        workload=f"prefill_few_heads: B={B}, T={T}, H_qk={H_qk}->H_v={H_v}, dk=dv={dk}, "
                 f"chunk {C}, channelwise gate, bf16 io, nonzero initial state "
                 f"(segmented carry)",
        workspace_bytes=ws_bytes,
    )


# ---------------------------------------------------------------------------
# T-sweep: T decode steps against one chunked prefill of the same T tokens
# ---------------------------------------------------------------------------
SWEEP_TS = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4000, 8192, 16384, 32767)


def graph_us(fn, reps=5):
    """Capture fn once in a HIP graph and time its replays with HIP events
    (replays run on the current stream, where the events are recorded)."""
    fn()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            fn()
    torch.cuda.current_stream().wait_stream(cap)
    graph.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) / reps * 1e3


def bench_sweep(batches=(1, 16), ts=SWEEP_TS, seed=11):
    """For each batch B and length T: T consecutive gdr_decode_step calls (one
    token each, graph-replayed as a serving loop would issue them) against one
    gdr_prefill_chunked over the same T tokens, both from the same initial
    state.  H_qk=16 -> H_v=32, dk=dv=128, bf16 io, channelwise gate, chunk 64,
    inputs drawn on the device from a seeded generator (q, k, v ~ N(0,1),
    g ~ -U(0.001, 0.2), beta logits ~ N(0,1), S0 ~ N(0, 0.02)).  `agree` is
    max|o_prefill - o_decode| / max|o_decode| over the T outputs."""
    H_qk, H_v, dk, dv, C = 16, 32, 128, 128, 64
    gate = synth.GATE_CHANNEL
    kw = dict(H_qk=H_qk, H_v=H_v, dk=dk, dv=dv, gate=gate)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    out = []
    for B in batches:
        pts = []
        for T in ts:
            bf = torch.bfloat16
            q = torch.randn(B, T, H_qk, dk, device=DEV, generator=gen).to(bf)
            k = torch.randn(B, T, H_qk, dk, device=DEV, generator=gen).to(bf)
            v = torch.randn(B, T, H_v, dv, device=DEV, generator=gen).to(bf)
            g = -(torch.rand(B, T, H_v, dk, device=DEV, generator=gen) * 0.199 + 0.001)
            bl = torch.randn(B, T, H_v, device=DEV, generator=gen)
            S0 = torch.randn(B, H_v, dk, dv, device=DEV, generator=gen) * 0.02
            # the decode path's per-token inputs: packed q|k|v rows, gates, beta
            qkv = torch.cat([q.transpose(0, 1).reshape(T, B, -1), k.transpose(0, 1).reshape(T, B, -1),
                             v.transpose(0, 1).reshape(T, B, -1)], dim=2).contiguous()
            gd = g.transpose(0, 1).contiguous()
            bd = bl.transpose(0, 1).contiguous()
            Sd = S0.clone()
            od = torch.empty((T, B, H_v, dv), dtype=bf, device=DEV)
            Sp = torch.empty_like(S0)
            op = torch.empty((B, T, H_v, dv), dtype=bf, device=DEV)
            ws = torch.empty(gdr.gdr_prefill_workspace_size(B, T, H_qk, H_v, dk, dv, C, bf, gate),
                             dtype=torch.uint8, device=DEV)

            def decode_all():
                for i in range(T):
                    gdr.gdr_decode_step(qkv[i], gd[i], bd[i], Sd, od[i], **kw)

            def prefill_all():
                gdr.gdr_prefill_chunked(q, k, v, g, bl, S0, Sp, op, ws, chunk=C, **kw)

            Sd.copy_(S0)
            decode_all()
            prefill_all()
            torch.cuda.synchronize()
            ref = od.transpose(0, 1).float()
            agree = float((op.float() - ref).abs().max() / ref.abs().max().clamp_min(1e-30))
            reps = 3 if B * T >= 16384 else 10
            du = graph_us(decode_all, reps)
            pu = graph_us(prefill_all, reps)
            pts.append(dict(T=T, decode_us=du, prefill_us=pu, decode_tok_s=B * T / du * 1e6,
                            prefill_tok_s=B * T / pu * 1e6, agree=agree))
            print(f"[bench] sweep B={B} T={T}: decode {du:.1f} us, prefill {pu:.1f} us, "
                  f"agree {agree:.1e}", file=sys.stderr, flush=True)
            del q, k, v, g, bl, S0, qkv, gd, bd, Sd, od, Sp, op, ws
            torch.cuda.empty_cache()
        cross = next((p["T"] for p in pts if p["prefill_us"] < p["decode_us"]), None)
        out.append(dict(B=B, crossover_T=cross, points=pts))
    return dict(config="H_qk=16->H_v=32, dk=dv=128, bf16 io, channelwise gate, chunk 64, "
                       "S0 ~ N(0, 0.02); decode steps graph-replayed, prefill graph-replayed",
                batches=out)


def _cpu_prefill_mode(fetch, B, T, H_qk, H_v, gate, seconds, threads):
    """The oracle over whole sequences of (b, h) units, `thr` value heads of one
    batch row at a time, until the time box is spent; tokens/s scaled to all
    B * H_v units.  fetch(b, h0, h1) returns (q, k, v, gate_in, beta_logit,
    S0) as host arrays for value heads h0 .. h1 - 1 of batch row b (q and k
    for the query/key heads they use)."""
    import oracle

    thr = oracle.threads_used(threads)
    rep = H_v // H_qk
    step = max(rep, thr - thr % rep)
    units = 0
    t0 = time.perf_counter()
    for b in range(B):
        for h0 in range(0, H_v, step):
            h1 = min(H_v, h0 + step)
            q, k, v, g, bl, s0 = fetch(b, h0, h1)
            oracle.sequence(q, k, v, gate, g, bl, s0, threads=thr)
            units += h1 - h0
            if time.perf_counter() - t0 >= seconds:
                break
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    frac = units / (B * H_v)
    return dict(value=B * T * frac / el, unit="tokens/s", cores=thr, kind="oracle",
                sample=f"{units} of {B * H_v} (b, h) units over all {T} tokens ({el:.1f} s, "
                       f"fp64 token recurrence"
                       + (", OpenMP over heads" if thr > 1 else ", one thread")
                       + "); tokens/s scaled to all units")


def cpu_prefill(fetch, B, T, H_qk, H_v, gate, seconds):
    """All host cores (the reported baseline) and one thread, each time-boxed."""
    out = _cpu_prefill_mode(fetch, B, T, H_qk, H_v, gate, seconds, cpu_threads())
    out["host"] = host_cpu()
    out["nproc"] = os.cpu_count()
    out["single_thread"] = _cpu_prefill_mode(fetch, B, T, H_qk, H_v, gate, seconds / 2, 1)
    return out


def host_fetch(case):
    """fetch() for cpu_prefill from a host-side case (bf16 expanded exactly)."""
    t = case.tensors
    rep = case.H_v // case.H_qk

    def fetch(b, h0, h1):
        sl = slice(b, b + 1)
        f = synth.bf16_to_f32
        return (f(t["q"][sl, :, h0 // rep:(h1 - 1) // rep + 1]),
                f(t["k"][sl, :, h0 // rep:(h1 - 1) // rep + 1]), f(t["v"][sl, :, h0:h1]),
                t["gate_in"][sl, :, h0:h1], t["beta_logit"][sl, :, h0:h1], t["S0"][sl, h0:h1])
    return fetch


def device_fetch(q, k, v, g, bl, s0, rep):
    """fetch() for cpu_prefill from device tensors (copied to the host)."""
    def fetch(b, h0, h1):
        c = lambda x: x.float().cpu().numpy()
        return (c(q[b:b + 1, :, h0 // rep:(h1 - 1) // rep + 1]),
                c(k[b:b + 1, :, h0 // rep:(h1 - 1) // rep + 1]), c(v[b:b + 1, :, h0:h1]),
                c(g[b:b + 1, :, h0:h1]), c(bl[b:b + 1, :, h0:h1]), c(s0[b:b + 1, h0:h1]))
    return fetch


def copy_calibration(reps=8, nbytes=256 << 20):
    """A plain device copy of known size: what HBM byte counters read for it
    calibrates them (FETCH_SIZE ~ nbytes, WRITE_SIZE ~ nbytes per dispatch)."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=DEV)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return nbytes


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256, help="timed decode steps")
    ap.add_argument("--warmup", type=int, default=16, help="untimed decode steps")
    ap.add_argument("--batch", type=int, default=64, help="decode batch (64 is the workload)")
    ap.add_argument("--prefill-reps", type=int, default=20)
    ap.add_argument("--prefill-warmup", type=int, default=3)
    ap.add_argument("--legs", default="decode,prefill,long",
                    help="comma list of decode, prefill, long (B=4, T=32767 with a carried-in "
                         "state, scalar and channel gates), sweep (T-sweep of decode steps "
                         "against one prefill), segmented (a long prefill over few heads: the "
                         "segmented carry), copy (HBM-counter calibration)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time box of each CPU-oracle baseline (0 disables)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the (batch, head) units shard across GPUs without communication, so one GPU's "
              f"figure is the per-GPU figure)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    gdr.load_library()
    legs = set(args.legs.split(","))
    out = {"metric": METRIC}

    dec = None
    if "decode" in legs:
        dec = bench_decode(args.steps, args.warmup, args.batch)
        print(f"[bench] decode done: {dec['value']:.1f} GB/s", file=sys.stderr, flush=True)
        dec["b1_fused"] = bench_decode_b1_fused()
        print(f"[bench] fused B=1 decode done: {dec['b1_fused']['us_per_step']:.2f} us/step",
              file=sys.stderr, flush=True)
    pre = None
    if "prefill" in legs:
        pre = bench_prefill(args.prefill_reps, args.prefill_warmup)
        print(f"[bench] prefill done: {pre['value']:.3e} tok/s", file=sys.stderr, flush=True)

    long_legs = None
    if "long" in legs:
        long_legs = {}
        for name, gate in (("scalar", synth.GATE_SCALAR), ("channel", synth.GATE_CHANNEL)):
            long_legs[name] = bench_prefill_long(gate, cpu_seconds=args.cpu_seconds)
            print(f"[bench] long prefill ({name} gate) done: "
                  f"{long_legs[name]['value']:.3e} tok/s", file=sys.stderr, flush=True)

    sweep = None
    if "sweep" in legs:
        sweep = bench_sweep()
        print("[bench] sweep done", file=sys.stderr, flush=True)

    seg = None
    if "segmented" in legs:
        seg = bench_prefill_segmented()
        print(f"[bench] segmented prefill done: {seg['value']:.3e} tok/s", file=sys.stderr,
              flush=True)

    if "copy" in legs:
        n = copy_calibration()
        print(f"[bench] copy calibration done: {n} bytes per copy", file=sys.stderr, flush=True)

    cpu_dec = cpu_pre = None
    if args.cpu_seconds > 0:
        if dec is not None:
            cpu_dec = cpu_decode(dec["case"], args.cpu_seconds)
        if pre is not None:
            c = pre["case"]
            cpu_pre = cpu_prefill(host_fetch(c), c.B, c.T, c.H_qk, c.H_v, c.gate,
                                  args.cpu_seconds)
        print("[bench] cpu baselines done", file=sys.stderr, flush=True)

    if dec is not None:
        out.update({
            "value": dec["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": dec["ms_per_step"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "io_dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": f"batched_decode_b{args.batch}: B={args.batch}, H_qk=16->H_v=32, "
                                   f"dk=dv=128, channelwise gate, bf16 packed q|k|v, fp32 state, "
                                   f"fresh inputs per step",
                       "batch": args.batch, "bytes_per_step": dec["bytes_per_step"],
                       "hbm_peak_frac_of_wall": dec["value"] / HBM_PEAK_GBS},
            "kernel_us_mean": dec["kernel_us_mean"], "graph_event_ms": dec["graph_event_ms"],
            "eager": dec["eager"],
            "decode_b1_fused": dec["b1_fused"],
            "roofline": dec["roofline"],
            "cpu_baseline": cpu_dec,
        })
    if pre is not None:
        p = {k: v for k, v in pre.items() if k != "case"}
        p["cpu_baseline"] = cpu_pre
        out["prefill"] = p
        if dec is None:
            out.update({"value": pre["value"], "unit": "tokens/s", "n_gpus": 1,
                        "steps": args.prefill_reps, "warmup": args.prefill_warmup,
                        "ms_per_step": pre["ms_per_call"], "higher_is_better": True,
                        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                        "data": "synthetic", "config": {"workload": pre["workload"]},
                        "roofline": pre["roofline"], "cpu_baseline": cpu_pre})
    if long_legs is not None:
        out["prefill_long"] = long_legs
    if sweep is not None:
        out["sweep"] = sweep
    if seg is not None:
        out["prefill_segmented"] = seg
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
