"""gated_delta_rule_40_amd -- the gated delta rule (GatedDeltaNet, scalar and
channelwise decay) for AMD Instinct MI355X (gfx950).

The computation lives in ``libgdr.so`` (hand-written HIP kernels behind the C
ABI of ``include/gdr.h``); this package holds its build script, a thin ctypes
binding with the same entry-point names, and the seeded input generator.

    gdr_decode_step             one fused token (T = 1), state updated in place
    gdr_prefill_chunked         T tokens, chunkwise WY/UT form
    gdr_prefill_workspace_size  bytes of workspace the prefill needs
    gdr_prefill_chunked_noalloc the prefill on the library's own device scratch
                                (for callers that cannot allocate)
    gdr_strerror                text of a status code
"""
from .binding import (  # noqa: F401
    GDR_BF16,
    GDR_F32,
    GDR_GATE_CHANNEL,
    GDR_GATE_SCALAR,
    GDR_GATE_SCALAR_FUSED,
    EXPORTED,
    GdrError,
    gdr_decode_step,
    gdr_prefill_chunked,
    gdr_prefill_chunked_noalloc,
    gdr_prefill_workspace_size,
    gdr_strerror,
    load_library,
)
