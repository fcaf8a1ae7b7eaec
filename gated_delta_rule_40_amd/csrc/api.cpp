// api.cpp -- the C ABI declared in include/gdr.h: host-side argument
// validation and dispatch to the kernel launchers.  Nothing here allocates,
// frees or synchronises; errors are returned before anything is enqueued.
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "gdr.h"
#include "gdr_internal.h"

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
  return gdr::prefill_workspace_bytes(dims->B, dims->T, dims->H_v, dims->dk, dims->dv,
                                      dims->chunk, io == GDR_BF16);
}

int gdr_prefill_chunked(const gdr_dims* dims, gdr_dtype io, gdr_gate gate, const void* q,
                        const void* k, const void* v, const float* gate_in, const float* A_log,
                        const float* dt_bias, const float* beta_logit, const float* state_in,
                        float* state_out, void* o, float scale, int l2norm_qk, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  int rc = check_sizes(dims, io, gate, true);
  if (rc != GDR_OK) return rc;
  const gdr_dims& d = *dims;
  if (d.B == 0) return GDR_OK;
  if (!state_out) return GDR_E_NULL;
  if (!aligned(state_out, 16) || (state_in && !aligned(state_in, 16))) return GDR_E_ALIGN;
  const size_t B = d.B, T = d.T, Hv = d.H_v;
  const size_t state_bytes = B * Hv * d.dk * d.dv * sizeof(float);
  if (T > 0) {
    if (!q || !k || !v || !beta_logit || !o) return GDR_E_NULL;
    rc = check_gate_ptrs(gate, gate_in, A_log, dt_bias);
    if (rc != GDR_OK) return rc;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(beta_logit, 4))
      return GDR_E_ALIGN;
    const size_t need = gdr::prefill_workspace_bytes(d.B, d.T, d.H_v, d.dk, d.dv, d.chunk,
                                                     io == GDR_BF16);
    if (!workspace || workspace_bytes < need) return GDR_E_WORKSPACE;
    if (!aligned(workspace, 16)) return GDR_E_ALIGN;
    const size_t es = io == GDR_BF16 ? 2 : 4;
    const size_t gate_elems = gate == GDR_GATE_CHANNEL ? B * T * Hv * d.dk : B * T * Hv;
    // Read-only inputs; o, the workspace and state_out are written while
    // they (and state_in) are still being read.
    Range ins[8] = {range_of(q, B * T * d.H_qk * d.dk * es),
                    range_of(k, B * T * d.H_qk * d.dk * es),
                    range_of(v, B * T * Hv * d.dv * es),
                    range_of(gate_in, gate_elems * sizeof(float)),
                    range_of(beta_logit, B * T * Hv * sizeof(float)),
                    state_in ? range_of(state_in, state_bytes) : Range{0, 0},
                    Range{0, 0}, Range{0, 0}};
    if (gate == GDR_GATE_SCALAR_FUSED) {
      ins[6] = range_of(A_log, Hv * sizeof(float));
      ins[7] = range_of(dt_bias, Hv * sizeof(float));
    }
    const Range ro = range_of(o, B * T * Hv * d.dv * es);
    const Range rw = range_of(workspace, need);
    const Range rso = range_of(state_out, state_bytes);
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
  if (state_in && state_in != state_out &&
      overlap(range_of(state_in, state_bytes), range_of(state_out, state_bytes)))
    return GDR_E_ALIAS;

  gdr::PrefillArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.gate_in = gate_in;
  a.A_log = A_log;
  a.dt_bias = dt_bias;
  a.beta_logit = beta_logit;
  a.state_in = state_in;
  a.state_out = state_out;
  a.o = o;
  a.ws = workspace;
  a.B = d.B;
  a.T = d.T;
  a.H_qk = d.H_qk;
  a.H_v = d.H_v;
  a.dk = d.dk;
  a.dv = d.dv;
  a.chunk = d.chunk;
  a.gate = gate;
  a.l2norm = l2norm_qk != 0;
  a.scale = scale;
  return gdr::launch_prefill(a, io == GDR_BF16, stream) == hipSuccess ? GDR_OK : GDR_E_HIP;
}

}  // extern "C"
