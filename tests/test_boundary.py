"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments with the documented status before
anything is launched."""
from __future__ import annotations

import ctypes
import re
from pathlib import Path

import pytest

import gated_delta_rule_40_amd as gdr
from gated_delta_rule_40_amd.binding import gdr_dims

HEADER = Path(__file__).resolve().parents[1] / "include" / "gdr.h"
E = dict(OK=0, NULL=-1, SHAPE=-2, DTYPE=-3, UNSUPPORTED=-4, WORKSPACE=-5, HIP=-6, ALIAS=-7,
         ALIGN=-8, SCRATCH=-9)
A = 0x10000  # fake, 16-byte aligned device addresses: never dereferenced here


def declared_functions():
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(gdr_\w+)\(", text, re.M)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(gdr.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(str(gdr.binding.LIB_PATH))
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_header_status_values_match():
    text = HEADER.read_text()
    for k, v in E.items():
        assert re.search(rf"GDR_(E_)?{k}\s*=\s*{v}\b", text), k


def test_strerror_covers_every_status():
    msgs = {v: gdr.gdr_strerror(v) for v in E.values()}
    assert len(set(msgs.values())) == len(msgs)
    assert gdr.gdr_strerror(-99) == "unknown gdr status"


def _dims(B=2, T=5, H_qk=2, H_v=4, dk=32, dv=64, chunk=16):
    return gdr_dims(B, T, H_qk, H_v, dk, dv, chunk)


def decode(dims, io=0, gate=0, qkv=A, g=A + 0x100000, Al=None, dt=None, bl=A + 0x200000,
           st=A + 0x300000, o=A + 0x4000000):
    lib = gdr.load_library()
    return lib.gdr_decode_step(ctypes.byref(dims) if dims is not None else None, io, gate, qkv,
                               g, Al, dt, bl, st, o, 1.0, 1, None)


def prefill(dims, io=0, gate=0, q=A, k=A + 0x1000000, v=A + 0x2000000, g=A + 0x3000000, Al=None,
            dt=None, bl=A + 0x4000000, s_in=A + 0x5000000, s_out=A + 0x6000000, o=A + 0x7000000,
            ws=A + 0x10000000, ws_bytes=None):
    lib = gdr.load_library()
    if ws_bytes is None:
        ws_bytes = lib.gdr_prefill_workspace_size(ctypes.byref(dims), io, gate)
    return lib.gdr_prefill_chunked(ctypes.byref(dims) if dims is not None else None, io, gate,
                                   q, k, v, g, Al, dt, bl, s_in, s_out, o, 1.0, 1, ws, ws_bytes,
                                   None)


# Every case must fail validation or have nothing to launch (B = 0, or T = 0
# in place): the addresses are fake, so a case that passed validation would
# launch kernels on them.
@pytest.mark.parametrize("case,expect", [
    (dict(dims=None), "NULL"),
    (dict(io=2), "DTYPE"),
    (dict(gate=3), "DTYPE"),
    (dict(dims=_dims(H_qk=3, H_v=4)), "SHAPE"),
    (dict(dims=_dims(B=-1)), "SHAPE"),
    (dict(dims=_dims(dk=48)), "UNSUPPORTED"),
    (dict(dims=_dims(dv=256)), "UNSUPPORTED"),
    (dict(qkv=None), "NULL"),
    (dict(st=None), "NULL"),
    (dict(g=None), "NULL"),
    (dict(gate=2), "NULL"),                      # fused gate without A_log / dt_bias
    (dict(qkv=A + 8), "ALIGN"),
    (dict(st=A + 0x300004), "ALIGN"),
    (dict(o=A + 0x300000), "ALIAS"),              # o on top of the state
    (dict(o=A), "ALIAS"),                         # o on top of qkv
    (dict(st=A), "ALIAS"),                        # in-place state on top of qkv
    (dict(st=A + 0x100000), "ALIAS"),             # ... on top of the gate
    (dict(st=A + 0x200000 - 0x100), "ALIAS"),     # ... reaching into beta_logit
    (dict(gate=2, Al=A + 0x300040, dt=A + 0x500000), "ALIAS"),   # A_log inside the state
    (dict(gate=2, Al=A + 0x500000, dt=A + 0x4000000), "ALIAS"),  # dt_bias under o
    (dict(dims=_dims(B=0)), "OK"),                # nothing to do, nothing launched
])
def test_decode_validation(case, expect):
    kw = dict(case)
    dims = kw.pop("dims", _dims())
    assert decode(dims, **kw) == E[expect]


@pytest.mark.parametrize("case,expect", [
    (dict(dims=_dims(T=-1)), "SHAPE"),
    (dict(dims=_dims(chunk=8)), "UNSUPPORTED"),
    (dict(dims=_dims(chunk=128)), "UNSUPPORTED"),
    (dict(dims=_dims(dk=8)), "UNSUPPORTED"),
    (dict(q=None), "NULL"),
    (dict(s_out=None), "NULL"),
    (dict(ws=None), "WORKSPACE"),
    (dict(ws_bytes=16), "WORKSPACE"),
    (dict(v=A + 0x2000004), "ALIGN"),
    (dict(o=A + 0x2000000), "ALIAS"),              # o on top of v
    (dict(o=A + 0x10000000), "ALIAS"),             # o on top of the workspace
    (dict(ws=A + 0x1000000), "ALIAS"),             # workspace on top of k
    (dict(ws=A + 0x3000000), "ALIAS"),             # workspace on top of the gate
    (dict(ws=A + 0x5000000), "ALIAS"),             # workspace on top of state_in
    (dict(ws=A + 0x6000000), "ALIAS"),             # workspace on top of state_out
    (dict(s_out=A + 0x5000100), "ALIAS"),          # state_out shifted into state_in
    (dict(s_out=A + 0x5000000 - 0x100), "ALIAS"),  # ... and the other way round
    (dict(s_out=A + 0x2000000), "ALIAS"),          # state_out on top of v
    (dict(s_out=A + 0x1000000), "ALIAS"),          # ... of k
    (dict(s_out=A + 0x4000000), "ALIAS"),          # ... of beta_logit
    (dict(gate=2, Al=A + 0x7000010, dt=A + 0x8000000), "ALIAS"),  # A_log under o
    (dict(gate=2, Al=A + 0x8000000, dt=A + 0x10000000), "ALIAS"),  # dt_bias in the workspace
    (dict(gate=2, Al=A + 0x6000000, dt=A + 0x8000000), "ALIAS"),  # A_log under state_out
    # 64 tokens x 2^19 heads x 128 columns: the carry's 32-bit row offsets would wrap
    (dict(dims=_dims(B=1, H_qk=1, H_v=1 << 19, dv=128, chunk=64)), "SHAPE"),
    (dict(dims=_dims(B=0)), "OK"),
    (dict(dims=_dims(T=0), s_in=A + 0x6000000), "OK"),   # T=0, in place: nothing to copy
    (dict(dims=_dims(T=0), s_out=A + 0x5000100), "ALIAS"),  # T=0, shifted copy
])
def test_prefill_validation(case, expect):
    kw = dict(case)
    dims = kw.pop("dims", _dims())
    assert prefill(dims, **kw) == E[expect]


def prefill_noalloc(dims, io=0, gate=0, q=A, k=A + 0x1000000, v=A + 0x2000000, g=A + 0x3000000,
                    Al=None, dt=None, bl=A + 0x4000000, s_in=A + 0x5000000, s_out=A + 0x6000000,
                    o=A + 0x7000000):
    lib = gdr.load_library()
    return lib.gdr_prefill_chunked_noalloc(ctypes.byref(dims) if dims is not None else None, io,
                                           gate, q, k, v, g, Al, dt, bl, s_in, s_out, o, 1.0, 1,
                                           None)


def _big(T):
    return gdr_dims(1, T, 16, 32, 128, 128, 64)


G = 1 << 30
# fake addresses 1 GiB apart, so that tensors of the large cases do not overlap
SPREAD = dict(q=A, k=A + G, v=A + 2 * G, g=A + 3 * G, bl=A + 4 * G, s_in=A + 5 * G,
              s_out=A + 6 * G, o=A + 7 * G)


# As above: only cases that fail validation or have nothing to launch.
@pytest.mark.parametrize("case,expect", [
    (dict(dims=None), "NULL"),
    (dict(io=2), "DTYPE"),
    (dict(dims=_dims(chunk=8)), "UNSUPPORTED"),
    (dict(q=None), "NULL"),
    (dict(s_out=None), "NULL"),
    (dict(o=A + 0x2000000), "ALIAS"),
    (dict(s_out=A + 0x5000100), "ALIAS"),
    (dict(v=A + 0x2000004), "ALIGN"),
    (dict(dims=_big(4033), io=1, **SPREAD), "SCRATCH"),   # 64 chunks x 32 heads x 66,048 B
    (dict(dims=_big(32767), io=1, **SPREAD), "SCRATCH"),
    (dict(dims=_big(4032), io=0, **SPREAD), "SCRATCH"),   # fp32 operands: twice the bytes
    (dict(dims=_dims(B=0)), "OK"),
    (dict(dims=_dims(T=0), s_in=A + 0x6000000), "OK"),
])
def test_prefill_noalloc_validation(case, expect):
    kw = dict(case)
    dims = kw.pop("dims", _dims())
    assert prefill_noalloc(dims, **kw) == E[expect]


def test_noalloc_limit_is_the_workspace_of_the_t4000_workload():
    """The scratch holds the workspace of B=1, H 16 -> 32, dk=dv=128, chunk 64,
    bf16 up to T=4032 and no more."""
    lib = gdr.load_library()
    assert gdr.binding.NOALLOC_SCRATCH_BYTES == 128 << 20
    text = HEADER.read_text()
    assert re.search(r"#define GDR_NOALLOC_SCRATCH_BYTES \(\(size_t\)128 << 20\)", text)
    size = lambda T: lib.gdr_prefill_workspace_size(ctypes.byref(_big(T)), 1, 0)
    assert size(4032) <= gdr.binding.NOALLOC_SCRATCH_BYTES < size(4033)


def _al(x, n):
    return -(-x // n) * n


def block_bytes(dk, chunk, es, scalar_gate=False):
    """One (b, h, chunk) block: Kt, Qt, Ke^T (chunk x dk each), Tb and P (chunk x
    chunk each) in the operand type, then e^Gamma_L (dk fp32), 16-byte aligned.
    Scalar gates leave out Kt and Qt (row scalings of the normalised k and q
    rows, which are stored once per qk head instead) and add one fp32 row factor
    per chunk row."""
    if scalar_gate:
        return _al((chunk * dk + 2 * chunk * chunk) * es + 4 * dk + 4 * chunk, 16)
    return _al((3 * chunk * dk + 2 * chunk * chunk) * es + 4 * dk, 16)


def qk_bytes(B, H_qk, nc, dk, chunk, es):
    """Scalar gates: the normalised k and q rows of each (b, qk head, chunk)."""
    return B * H_qk * nc * 2 * chunk * dk * es


def layout_bytes(units, nc, bb, seg=0, qk=0):
    """Chunk blocks; for scalar gates the qk rows at the next 256-byte boundary;
    the segmented carry's buffers (if any) at the next 256-byte boundary."""
    end = units * nc * bb
    if qk:
        end = _al(end, 256) + qk
    return _al(end, 256) + seg if seg else end


def test_workspace_size_query():
    lib = gdr.load_library()
    size = lambda io=1, gate=0, **kw: lib.gdr_prefill_workspace_size(ctypes.byref(_dims(**kw)), io, gate)
    assert size(T=0) == 0 and size(B=0) == 0
    assert size(dk=48) == 0 and size(chunk=8) == 0
    units = 2 * 4                                  # B=2, H_v=4 (the _dims defaults)
    for io, es in ((1, 2), (0, 4)):
        for T, C in ((1, 16), (16, 16), (17, 16), (100, 32), (129, 64)):
            nc = -(-T // C)
            for gate in (0, 1, 2):
                sg = gate != 0
                expect = layout_bytes(units, nc, block_bytes(32, C, es, scalar_gate=sg),
                                      qk=qk_bytes(2, 2, nc, 32, C, es) if sg else 0)
                assert size(io=io, gate=gate, T=T, chunk=C) == expect, (io, T, C, gate)
    assert size(T=16) == size(T=1) > 0            # one chunk either way
    # the long prefill's blocks: 66,048 B with a channel gate; 33,536 B with a
    # scalar one, plus 32 KiB of k and q rows per qk head (two value heads each)
    assert block_bytes(128, 64, 2) == 66048 and block_bytes(128, 64, 2, True) == 33536
    two = dict(B=1, T=64, H_qk=1, H_v=2, dk=128, dv=128, chunk=64)
    assert size(gate=0, **two) == 2 * 66048
    assert size(gate=1, **two) == size(gate=2, **two) == _al(2 * 33536, 256) + 32768


def test_workspace_size_segmented_carry():
    """Long prefills over few units take the segmented carry: the size query
    adds its fp32 segment states and maps (S and N: P x units x dk x dv, M:
    P x units x dk x dk) after the chunk blocks, aligned to 256 bytes, for P
    from 3 to 16 segments of at least 8 chunks each; many units keep one walk
    and the chunk blocks alone."""
    lib = gdr.load_library()

    def size(**kw):
        return lib.gdr_prefill_workspace_size(ctypes.byref(_dims(**kw)), 1, 0)

    kw = dict(B=1, H_qk=1, H_v=2, dk=128, dv=128, chunk=64)
    bb = block_bytes(128, 64, 2)
    assert bb == 66048
    per_seg = 2 * 128 * (2 * 128 + 128) * 4
    for T in (3000, 20000):
        nc = -(-T // 64)
        extra = size(T=T, **kw) - layout_bytes(2, nc, bb, 1) + 1
        assert extra > 0 and extra % per_seg == 0, (T, extra)
        P = extra // per_seg
        assert 3 <= P <= 16 and -(-nc // P) >= 8, (T, P)
    # many units: one walk, chunk blocks only
    assert size(T=3000, B=1, H_qk=16, H_v=32, dk=128, dv=128, chunk=64) == layout_bytes(32, 47, bb)
    # the GPU tests' reading of the plan agrees with the same query
    from tests.gpu_util import carry_segments
    assert carry_segments(1, 3000, 32, 128, 128, 64) == 1
    assert carry_segments(1, 20000, 2, 128, 128, 64) >= 3


def test_missing_library_raises(tmp_path):
    with pytest.raises(RuntimeError):
        gdr.load_library(tmp_path / "libgdr.so")
