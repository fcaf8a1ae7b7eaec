// gdr_internal.h -- argument blocks and launchers shared by the C-ABI layer
// (api.cpp) and the kernel sources.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace gdr {

// Argument block of the fused decode kernel.  Pointers are device pointers.
struct DecodeArgs {
  const void* qkv;          // [B, 2*H_qk*dk + H_v*dv] io dtype
  const float* gate_in;     // channel [B,H_v,dk] | scalar/fused [B,H_v]
  const float* A_log;       // [H_v] (fused gate only)
  const float* dt_bias;     // [H_v] (fused gate only)
  const float* beta_logit;  // [B,H_v]
  float* state;             // [B,H_v,dk,dv] in place
  void* o;                  // [B,H_v,dv] io dtype
  int B, H_qk, H_v, dk, dv;
  int gate;                 // gdr_gate value
  int l2norm;
  float scale;
};

// Launch the decode kernel; dv_slice columns of the state per workgroup.
hipError_t launch_decode(const DecodeArgs& a, int io_bf16, int dv_slice, hipStream_t stream);

// Columns of the state one decode workgroup owns, for these sizes.
int decode_dv_slice(int B, int H_v, int dv);

// Argument block of the chunked prefill kernels.
struct PrefillArgs {
  const void* q;            // [B,T,H_qk,dk]
  const void* k;            // [B,T,H_qk,dk]
  const void* v;            // [B,T,H_v,dv]
  const float* gate_in;     // channel [B,T,H_v,dk] | scalar/fused [B,T,H_v]
  const float* A_log;       // [H_v]
  const float* dt_bias;     // [H_v]
  const float* beta_logit;  // [B,T,H_v]
  const float* state_in;    // [B,H_v,dk,dv] or nullptr
  float* state_out;         // [B,H_v,dk,dv]
  void* o;                  // [B,T,H_v,dv]
  void* ws;                 // workspace
  void* ws_qk;              // scalar gates: the normalised k and q rows per (b, qk head, chunk),
                            // inside the workspace (set by the chunked launch)
  int B, T, H_qk, H_v, dk, dv, chunk;
  int gate;
  int l2norm;
  float scale;
};

// Workspace bytes of a chunked prefill; scalar gates (any gate but
// GDR_GATE_CHANNEL) take smaller chunk blocks plus the normalised k and q rows
// once per qk head.
size_t prefill_workspace_bytes(int B, int T, int H_qk, int H_v, int dk, int dv, int chunk,
                               int io_bf16, int gate);
hipError_t launch_prefill(const PrefillArgs& a, int io_bf16, hipStream_t stream);

// The allocation-free prefill takes its workspace from a device array of this
// many bytes (one per device, held until the process ends).
constexpr size_t kNoallocScratchBytes = static_cast<size_t>(128) << 20;
// Device address of the current device's array (resolved on the first call
// on that device).
hipError_t noalloc_scratch(void** ptr);

// Short sequences token by token (the state tile held in registers over all
// T tokens; the workspace is not used).  The prefill takes this path for
// T <= recurrent_max_t(B, H_v) when the per-token vectors fit
// kRecurrentMaxLds bytes of LDS per workgroup.
constexpr size_t kRecurrentMaxLds = 64 * 1024;
int recurrent_max_t(int B, int H_v);
int recurrent_dv_slice(int B, int H_v, int dv);
size_t recurrent_lds_bytes(int T, int dk, int dv_slice);
hipError_t launch_recurrent(const PrefillArgs& a, int io_bf16, hipStream_t stream);

}  // namespace gdr
