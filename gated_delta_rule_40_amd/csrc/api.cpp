// api.cpp -- the C ABI declared in include/gdr.h: host-side argument
// validation and dispatch to the kernel launchers.  Nothing here allocates,
// frees or synchronises; errors are returned before anything is enqueued.
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "gdr.h"
#include "gdr_internal.h"

static_assert(GDR_NOALLOC_SCRATCH_BYTES == gdr::kNoallocScratchBytes,
              "the header's scratch limit is the size of the device array");

namespace {

bool supported_head_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool supported_chunk(int c) { return c == 16 || c == 32 || c == 64; }

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, size_t bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + bytes};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

bool overlaps_any(Range a, const Range* others, int n) {
  for (int i = 0; i < n; ++i)
    if (overlap(a, others[i])) return true;
  return false;
}

int check_sizes(const gdr_dims* d, gdr_dtype io, gdr_gate gate, bool prefill) {
  if (!d) return GDR_E_NULL;
  if (io != GDR_F32 && io != GDR_BF16) return GDR_E_DTYPE;
  if (gate != GDR_GATE_CHANNEL && gate != GDR_GATE_SCALAR && gate != GDR_GATE_SCALAR_FUSED)
    return GDR_E_DTYPE;
  if (d->B < 0 || d->H_qk <= 0 || d->H_v <= 0 || d->dk <= 0 || d->dv <= 0) return GDR_E_SHAPE;
  if (prefill && d->T < 0) return GDR_E_SHAPE;
  if (d->H_v % d->H_qk != 0) return GDR_E_SHAPE;
  if (!supported_head_dim(d->dk) || !supported_head_dim(d->dv)) return GDR_E_UNSUPPORTED;
  if (prefill && !supported_chunk(d->chunk)) return GDR_E_UNSUPPORTED;
  // Grid sizes and element offsets must stay within 32-bit workgroup counts.
  const long long units = static_cast<long long>(d->B) * d->H_v;
  if (units * d->dv > INT32_MAX) return GDR_E_SHAPE;
  if (prefill) {
    const long long chunks = (static_cast<long long>(d->T) + d->chunk - 1) / d->chunk;
    if (units * chunks > INT32_MAX) return GDR_E_SHAPE;
    // The carry reaches a chunk's v and o rows through 32-bit element offsets
    // from the chunk's first row (token stride H_v * dv).
    if (static_cast<long long>(d->chunk) * d->H_v * d->dv > UINT32_MAX) return GDR_E_SHAPE;
  }
  return GDR_OK;
}

int check_gate_ptrs(gdr_gate gate, const float* gate_in, const float* A_log,
                    const float* dt_bias) {
  if (!gate_in) return GDR_E_NULL;
  if (gate == GDR_GATE_SCALAR_FUSED && (!A_log || !dt_bias)) return GDR_E_NULL;
  if (!aligned(gate_in, 16)) return GDR_E_ALIGN;
  if (gate == GDR_GATE_SCALAR_FUSED && (!aligned(A_log, 4) || !aligned(dt_bias, 4)))
    return GDR_E_ALIGN;
  return GDR_OK;
}

// The arguments of one prefill call (everything but the workspace and stream).
struct PrefillCall {
  const gdr_dims* dims;
  gdr_dtype io;
  gdr_gate gate;
  const void *q, *k, *v;
  const float *gate_in, *A_log, *dt_bias, *beta_logit, *state_in;
  float* state_out;
  void* o;
  float scale;
  int l2norm_qk;
};

// Validates a prefill call.  own_scratch: the workspace is the library's own
// scratch array (workspace and workspace_bytes are then ignored).  *need
// receives the workspace bytes the call uses (0 when nothing is launched).
int check_prefill(const PrefillCall& c, bool own_scratch, const void* workspace,
                  size_t workspace_bytes, size_t* need) {
  *need = 0;
  int rc = check_sizes(c.dims, c.io, c.gate, true);
  if (rc != GDR_OK) return rc;
  const gdr_dims& d = *c.dims;
  if (d.B == 0) return GDR_OK;
  if (!c.state_out) return GDR_E_NULL;
  if (!aligned(c.state_out, 16) || (c.state_in && !aligned(c.state_in, 16))) return GDR_E_ALIGN;
  const size_t B = d.B, T = d.T, Hv = d.H_v;
  const size_t state_bytes = B * Hv * d.dk * d.dv * sizeof(float);
  if (T > 0) {
    if (!c.q || !c.k || !c.v || !c.beta_logit || !c.o) return GDR_E_NULL;
    rc = check_gate_ptrs(c.gate, c.gate_in, c.A_log, c.dt_bias);
    if (rc != GDR_OK) return rc;
    if (!aligned(c.q, 16) || !aligned(c.k, 16) || !aligned(c.v, 16) || !aligned(c.o, 16) ||
        !aligned(c.beta_logit, 4))
      return GDR_E_ALIGN;
    *need = gdr::prefill_workspace_bytes(d.B, d.T, d.H_qk, d.H_v, d.dk, d.dv, d.chunk,
                                         c.io == GDR_BF16, c.gate);
    if (!own_scratch) {
      if (!workspace || workspace_bytes < *need) return GDR_E_WORKSPACE;
      if (!aligned(workspace, 16)) return GDR_E_ALIGN;
    }
    const size_t es = c.io == GDR_BF16 ? 2 : 4;
    const size_t gate_elems = c.gate == GDR_GATE_CHANNEL ? B * T * Hv * d.dk : B * T * Hv;
    // Read-only inputs; o, the workspace and state_out are written while
    // they (and state_in) are still being read.
    Range ins[8] = {range_of(c.q, B * T * d.H_qk * d.dk * es),
                    range_of(c.k, B * T * d.H_qk * d.dk * es),
                    range_of(c.v, B * T * Hv * d.dv * es),
                    range_of(c.gate_in, gate_elems * sizeof(float)),
                    range_of(c.beta_logit, B * T * Hv * sizeof(float)),
                    c.state_in ? range_of(c.state_in, state_bytes) : Range{0, 0},
                    Range{0, 0}, Range{0, 0}};
    if (c.gate == GDR_GATE_SCALAR_FUSED) {
      ins[6] = range_of(c.A_log, Hv * sizeof(float));
      ins[7] = range_of(c.dt_bias, Hv * sizeof(float));
    }
    const Range ro = range_of(c.o, B * T * Hv * d.dv * es);
    const Range rw = own_scratch ? Range{0, 0} : range_of(workspace, *need);
    const Range rso = range_of(c.state_out, state_bytes);
    if (overlap(ro, rw) || overlap(ro, rso) || overlap(rw, rso) || overlaps_any(ro, ins, 8) ||
        overlaps_any(rw, ins, 8))
      return GDR_E_ALIAS;
    // state_out may be state_in itself (every state slice is read before it
    // is rewritten), but no other input.
    ins[5] = Range{0, 0};
    if (overlaps_any(rso, ins, 8)) return GDR_E_ALIAS;
  }
  // state_out either is state_in or lies apart from it: a shifted overlap
  // would have one workgroup read a state row that another has rewritten.
  if (c.state_in && c.state_in != c.state_out &&
      overlap(range_of(c.state_in, state_bytes), range_of(c.state_out, state_bytes)))
    return GDR_E_ALIAS;
  return GDR_OK;
}

int launch(const PrefillCall& c, void* workspace, hipStream_t stream) {
  const gdr_dims& d = *c.dims;
  if (d.B == 0) return GDR_OK;
  gdr::PrefillArgs a;
  a.q = c.q;
  a.k = c.k;
  a.v = c.v;
  a.gate_in = c.gate_in;
  a.A_log = c.A_log;
  a.dt_bias = c.dt_bias;
  a.beta_logit = c.beta_logit;
  a.state_in = c.state_in;
  a.state_out = c.state_out;
  a.o = c.o;
  a.ws = workspace;
  a.ws_qk = nullptr;  // placed inside the workspace by the chunked launch
  a.B = d.B;
  a.T = d.T;
  a.H_qk = d.H_qk;
  a.H_v = d.H_v;
  a.dk = d.dk;
  a.dv = d.dv;
  a.chunk = d.chunk;
  a.gate = c.gate;
  a.l2norm = c.l2norm_qk != 0;
  a.scale = c.scale;
  return gdr::launch_prefill(a, c.io == GDR_BF16, stream) == hipSuccess ? GDR_OK : GDR_E_HIP;
}

}  // namespace

extern "C" {

const char* gdr_strerror(int status) {
  switch (status) {
    case GDR_OK: return "ok";
    case GDR_E_NULL: return "a required pointer is NULL";
    case GDR_E_SHAPE: return "invalid shape (negative size, H_v not a multiple of H_qk, or too large)";
    case GDR_E_DTYPE: return "unknown io dtype or gate kind";
    case GDR_E_UNSUPPORTED: return "dk/dv must be 16, 32, 64 or 128 and chunk 16, 32 or 64";
    case GDR_E_WORKSPACE: return "workspace is NULL or smaller than gdr_prefill_workspace_size()";
    case GDR_E_HIP: return "HIP runtime error at kernel launch";
    case GDR_E_ALIAS: return "an output, the state or the workspace overlaps a buffer it must not";
    case GDR_E_ALIGN: return "tensor pointer is not 16-byte aligned";
    case GDR_E_SCRATCH:
      return "the call needs more workspace than the allocation-free entry point holds";
    default: return "unknown gdr status";
  }
}

int gdr_decode_step(const gdr_dims* dims, gdr_dtype io, gdr_gate gate, const void* qkv,
                    const float* gate_in, const float* A_log, const float* dt_bias,
                    const float* beta_logit, float* state, void* o, float scale,
                    int l2norm_qk, hipStream_t stream) {
  int rc = check_sizes(dims, io, gate, false);
  if (rc != GDR_OK) return rc;
  const gdr_dims& d = *dims;
  if (d.B == 0) return GDR_OK;
  if (!qkv || !beta_logit || !state || !o) return GDR_E_NULL;
  rc = check_gate_ptrs(gate, gate_in, A_log, dt_bias);
  if (rc != GDR_OK) return rc;
  if (!aligned(qkv, 16) || !aligned(state, 16) || !aligned(o, 16) || !aligned(beta_logit, 4))
    return GDR_E_ALIGN;

  const size_t es = io == GDR_BF16 ? 2 : 4;
  const size_t B = d.B, Hv = d.H_v;
  const Range ro = range_of(o, B * Hv * d.dv * es);
  const Range rs = range_of(state, B * Hv * d.dk * d.dv * sizeof(float));
  const size_t gate_elems = gate == GDR_GATE_CHANNEL ? B * Hv * d.dk : B * Hv;
  // Inputs the kernel reads while o and the state are being written.
  Range ins[5] = {range_of(qkv, B * (2 * d.H_qk * d.dk + Hv * d.dv) * es),
                  range_of(gate_in, gate_elems * sizeof(float)),
                  range_of(beta_logit, B * Hv * sizeof(float)), Range{0, 0}, Range{0, 0}};
  if (gate == GDR_GATE_SCALAR_FUSED) {
    ins[3] = range_of(A_log, Hv * sizeof(float));
    ins[4] = range_of(dt_bias, Hv * sizeof(float));
  }
  if (overlap(ro, rs) || overlaps_any(ro, ins, 5) || overlaps_any(rs, ins, 5)) return GDR_E_ALIAS;

  gdr::DecodeArgs a;
  a.qkv = qkv;
  a.gate_in = gate_in;
  a.A_log = A_log;
  a.dt_bias = dt_bias;
  a.beta_logit = beta_logit;
  a.state = state;
  a.o = o;
  a.B = d.B;
  a.H_qk = d.H_qk;
  a.H_v = d.H_v;
  a.dk = d.dk;
  a.dv = d.dv;
  a.gate = gate;
  a.l2norm = l2norm_qk != 0;
  a.scale = scale;
  const int dvs = gdr::decode_dv_slice(d.B, d.H_v, d.dv);
  return gdr::launch_decode(a, io == GDR_BF16, dvs, stream) == hipSuccess ? GDR_OK : GDR_E_HIP;
}

size_t gdr_prefill_workspace_size(const gdr_dims* dims, gdr_dtype io, gdr_gate gate) {
  if (check_sizes(dims, io, gate, true) != GDR_OK) return 0;
  return gdr::prefill_workspace_bytes(dims->B, dims->T, dims->H_qk, dims->H_v, dims->dk,
                                      dims->dv, dims->chunk, io == GDR_BF16, gate);
}

int gdr_prefill_chunked(const gdr_dims* dims, gdr_dtype io, gdr_gate gate, const void* q,
                        const void* k, const void* v, const float* gate_in, const float* A_log,
                        const float* dt_bias, const float* beta_logit, const float* state_in,
                        float* state_out, void* o, float scale, int l2norm_qk, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  const PrefillCall c{dims, io, gate, q, k, v, gate_in, A_log, dt_bias, beta_logit, state_in,
                      state_out, o, scale, l2norm_qk};
  size_t need = 0;
  int rc = check_prefill(c, false, workspace, workspace_bytes, &need);
  if (rc != GDR_OK) return rc;
  return launch(c, workspace, stream);
}

int gdr_prefill_chunked_noalloc(const gdr_dims* dims, gdr_dtype io, gdr_gate gate,
                                const void* q, const void* k, const void* v,
                                const float* gate_in, const float* A_log, const float* dt_bias,
                                const float* beta_logit, const float* state_in, float* state_out,
                                void* o, float scale, int l2norm_qk, hipStream_t stream) {
  const PrefillCall c{dims, io, gate, q, k, v, gate_in, A_log, dt_bias, beta_logit, state_in,
                      state_out, o, scale, l2norm_qk};
  size_t need = 0;
  int rc = check_prefill(c, true, nullptr, 0, &need);
  if (rc != GDR_OK) return rc;
  if (need > gdr::kNoallocScratchBytes) return GDR_E_SCRATCH;
  if (dims->B == 0) return GDR_OK;
  void* ws = nullptr;
  if (need > 0 && gdr::noalloc_scratch(&ws) != hipSuccess) return GDR_E_HIP;
  return launch(c, ws, stream);
}

}  // extern "C"
