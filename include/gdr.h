/*
 * gdr.h -- C ABI of the gated delta rule library for AMD Instinct MI355X (gfx950).
 *
 * The gated delta rule is the GatedDeltaNet linear-attention recurrence.  Per
 * batch row b and value head h it keeps a state S (dk x dv, fp32) and, for each
 * token with query q, key k (dk), value v (dv), write strength beta in (0,1) and
 * log-decay g <= 0 (one per key channel, or one per token for the scalar gate):
 *
 *     S   <- diag(exp(g)) S                       decay
 *     S   <- S + beta * k * (v - S^T k)^T         delta-rule write
 *     o    = scale * S^T q                        read the updated state
 *
 * Sources: the fused decode step (Q/K/V split, L2 normalisation, head repeat,
 * gating, recurrent update) is the one described on the page "Add fused
 * GatedDeltaNet decode Triton kernel" (executorch PR #18865, summary); the
 * two-pass state update on "Two-pass optimization for channelwise gated delta
 * rule kernel" (executorch PR #21020, Summary); routing by sequence length and
 * the chunkwise WY/UT prefill with a ragged final chunk on "Add parallel
 * chunked prefill for channelwise gated delta rule" (executorch PR #21061,
 * Summary).  The pages print no formulas; the conventions below are the
 * library's reading of them and are fixed:
 *
 *   - L2 normalisation (when l2norm_qk != 0): x / sqrt(sum x^2 + 1e-6);
 *   - head repeat: value head h uses query/key head h / (H_v / H_qk);
 *   - beta = sigmoid(beta_logit), computed in the kernel;
 *   - gates (gdr_gate): channel g per key channel; scalar g per token/head;
 *     fused g = -exp(A_log[h]) * softplus(x + dt_bias[h]);
 *   - output from the post-update state, times `scale`.
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, row-major (last index fastest), in device memory,
 *     16-byte aligned, owned by the caller.  The library never allocates,
 *     frees or synchronises; it only enqueues kernels on `stream` (a
 *     hipStream_t; NULL means the default stream) and returns.
 *   - fp32 tensors are `float`; bf16 tensors are IEEE bfloat16 bit patterns.
 *     The state is always fp32.  q/k/v (or qkv) and o use the io dtype.
 *   - Return value: GDR_OK or a negative gdr_status.  Arguments are validated
 *     on the host before any launch; on error nothing is enqueued and no
 *     buffer is touched.  GDR_E_HIP reports a failed launch.
 *   - Supported sizes: dk, dv in {16, 32, 64, 128}; H_v a multiple of H_qk;
 *     chunk in {16, 32, 64}.  B = 0 (and T = 0 for prefill) is a valid no-op.
 *     GDR_E_SHAPE also reports sizes past the 32-bit limits of the launch:
 *     B * H_v * dv and, for prefill, B * H_v * ceil(T / chunk) at most
 *     2^31 - 1, and chunk * H_v * dv at most 2^32 - 1.
 */
#ifndef GDR_H_
#define GDR_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype of q/k/v (or the packed qkv row) and of o. */
typedef enum gdr_dtype { GDR_F32 = 0, GDR_BF16 = 1 } gdr_dtype;

/* How the log-decay g is given.  Shapes are listed as [decode] / [prefill].
 *   GDR_GATE_CHANNEL      gate_in = g  [B,H_v,dk] / [B,T,H_v,dk]
 *   GDR_GATE_SCALAR       gate_in = g  [B,H_v]    / [B,T,H_v]
 *   GDR_GATE_SCALAR_FUSED gate_in = x  [B,H_v]    / [B,T,H_v], with A_log and
 *                         dt_bias [H_v]: g = -exp(A_log[h]) * softplus(x + dt_bias[h])
 * All gate tensors are fp32.  A_log and dt_bias must be NULL for the other kinds
 * or are ignored.  Channel and scalar g must be <= 0 (a decay, not a growth);
 * any strength of decay is supported: the chunked prefill evaluates only
 * exponentials of non-positive arguments (it forms the chunk's causal terms
 * exactly once a chunk decays by more than e^-64 on some channel). */
typedef enum gdr_gate {
  GDR_GATE_CHANNEL = 0,
  GDR_GATE_SCALAR = 1,
  GDR_GATE_SCALAR_FUSED = 2
} gdr_gate;

/* Problem sizes.  Decode ignores T and chunk. */
typedef struct gdr_dims {
  int32_t B, T, H_qk, H_v, dk, dv, chunk;
} gdr_dims;

typedef enum gdr_status {
  GDR_OK = 0,
  GDR_E_NULL = -1,        /* a required pointer is NULL                         */
  GDR_E_SHAPE = -2,       /* negative size, H_v % H_qk != 0, ...                */
  GDR_E_DTYPE = -3,       /* unknown io dtype or gate kind                      */
  GDR_E_UNSUPPORTED = -4, /* dk/dv/chunk outside the compiled set               */
  GDR_E_WORKSPACE = -5,   /* workspace NULL or smaller than the size query      */
  GDR_E_HIP = -6,         /* the HIP runtime reported an error at launch        */
  GDR_E_ALIAS = -7,       /* o, the state or the workspace overlaps a buffer    */
                          /* it must not (see each entry point)                 */
  GDR_E_ALIGN = -8,       /* a tensor is not 16-byte aligned                    */
  GDR_E_SCRATCH = -9      /* the call needs more workspace than the             */
                          /* allocation-free entry point holds                  */
} gdr_status;

/*
 * gdr_decode_step -- one token (T = 1) for every (batch row, value head), one kernel.
 *
 * Fuses, per the page "Add fused GatedDeltaNet decode Triton kernel" (PR #18865,
 * summary): the Q/K/V split of the packed row, L2 normalisation of q and k, the
 * head repeat H_qk -> H_v, the gates (beta and the decay) and the state update.
 * The update reads and writes the state once each, in the two-pass order of
 * "Two-pass optimization for channelwise gated delta rule kernel" (PR #21020,
 * Summary): pass 1 forms vhat = (diag(a) S)^T k with the decay a = exp(g)
 * folded in; pass 2 writes S = diag(a) S + beta k (v - vhat)^T and accumulates
 * o = scale S^T q.
 *
 *   dims        B, H_qk, H_v, dk, dv (T and chunk ignored)
 *   io          dtype of qkv and o
 *   gate        see gdr_gate; gate_in shape [B,H_v,dk] or [B,H_v]
 *   qkv         [B, 2*H_qk*dk + H_v*dv]: q heads, then k heads, then v heads,
 *               each head's channels contiguous
 *   A_log, dt_bias  [H_v] fp32 for GDR_GATE_SCALAR_FUSED, else ignored
 *   beta_logit  [B,H_v] fp32
 *   state       [B,H_v,dk,dv] fp32, read and updated IN PLACE; must not
 *               overlap qkv, gate_in, A_log, dt_bias or beta_logit
 *   o           [B,H_v,dv] io dtype, written; must not overlap the state or
 *               any input
 *   scale       output multiplier
 *   l2norm_qk   nonzero: normalise q and k rows; zero: use them as given
 */
int gdr_decode_step(const gdr_dims* dims, gdr_dtype io, gdr_gate gate, const void* qkv,
                    const float* gate_in, const float* A_log, const float* dt_bias,
                    const float* beta_logit, float* state, void* o, float scale,
                    int l2norm_qk, hipStream_t stream);

/*
 * gdr_prefill_workspace_size -- bytes of device workspace gdr_prefill_chunked
 * needs for these sizes and this gate kind (0 when B or T is 0).  Returns 0 as
 * well for unsupported arguments; gdr_prefill_chunked then reports the reason.
 * Scalar gates need less per value head: with one decay per token the decayed
 * keys and queries are row scalings of the normalised k and q rows, which are
 * kept once per qk head.
 */
size_t gdr_prefill_workspace_size(const gdr_dims* dims, gdr_dtype io, gdr_gate gate);

/*
 * gdr_prefill_chunked -- T tokens per (batch row, value head), chunkwise WY/UT form.
 *
 * Follows "Add parallel chunked prefill for channelwise gated delta rule"
 * (PR #21061, Summary): per chunk of `chunk` tokens (the last chunk may be
 * shorter and runs through the same code), per-channel log-decay prefix sums,
 * the causal query/key and key/key terms, the beta-folded unit-lower-triangular
 * transform, WY pseudo-keys / pseudo-values, and the carry of the state from
 * chunk to chunk.  Independent (batch, head) units run in parallel, each with a
 * disjoint slice of the caller's workspace.  The result equals T applications
 * of the token update (up to rounding).
 *
 * Short sequences (T <= 16 at up to 64 (batch, head) units, T <= 24 above)
 * are run token by token instead, each token the two-pass update above, with
 * the state held on chip across the tokens: the fixed cost of the chunked form
 * does not pay off there.  The workspace is then not touched, but the same
 * size is still required.
 *
 * Long sequences over few units (at most 128 sixteen-column state slices,
 * B * H_v * dv / 16, and segments of at least 8 chunks) carry the state by a
 * parallel scan instead of one walk: the carry over a range of chunks is an
 * affine map of the state, S_out = M S_in + N, so the sequence is cut into
 * segments whose maps are formed side by side, composed in fp32, and each
 * segment is then run from its start state.  The workspace then also holds
 * fp32 segment states and maps, which the size query includes.  The result
 * matches the single walk to rounding.
 *
 *   dims        B, T, H_qk, H_v, dk, dv, chunk
 *   io          dtype of q, k, v and o
 *   gate        see gdr_gate; gate_in shape [B,T,H_v,dk] or [B,T,H_v]
 *   q, k        [B,T,H_qk,dk]
 *   v           [B,T,H_v,dv]
 *   A_log, dt_bias  [H_v] fp32 for GDR_GATE_SCALAR_FUSED, else ignored
 *   beta_logit  [B,T,H_v] fp32
 *   state_in    [B,H_v,dk,dv] fp32 initial state, or NULL for zeros
 *   state_out   [B,H_v,dk,dv] fp32 final state; either equal to state_in
 *               (in place) or not overlapping it, and not overlapping any
 *               other input
 *   o           [B,T,H_v,dv] io dtype; must not overlap any input or the state
 *   workspace   device memory of at least gdr_prefill_workspace_size() bytes,
 *               16-byte aligned, contents need not be initialised; it must not
 *               overlap any input, o or the state, and may be reused once the
 *               enqueued work has finished
 *   T == 0      copies state_in to state_out (zeros when state_in is NULL)
 */
int gdr_prefill_chunked(const gdr_dims* dims, gdr_dtype io, gdr_gate gate, const void* q,
                        const void* k, const void* v, const float* gate_in, const float* A_log,
                        const float* dt_bias, const float* beta_logit, const float* state_in,
                        float* state_out, void* o, float scale, int l2norm_qk, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * gdr_prefill_chunked_noalloc -- gdr_prefill_chunked without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 *
 * Same arguments, results, validation and status codes as
 * gdr_prefill_chunked, minus workspace / workspace_bytes.  The workspace is a
 * device array inside the library, GDR_NOALLOC_SCRATCH_BYTES bytes on each
 * device it runs on, held until the process ends; the library allocates and
 * frees nothing on any call.  The first call on a device (the current device)
 * looks up that device's array address.
 *
 *   - A call whose gdr_prefill_workspace_size() exceeds
 *     GDR_NOALLOC_SCRATCH_BYTES returns GDR_E_SCRATCH and enqueues nothing
 *     (B = 1, H_v = 32, dk = dv = 128, chunk 64, bf16 fits up to T = 4032).
 *   - Every call on a device shares that device's array and leaves its
 *     contents behind; no content needs to be cleared between calls.  Calls
 *     that may run at the same time on one device (other streams, other
 *     threads) RACE on the array: order them on one stream, or use
 *     gdr_prefill_chunked with a workspace per concurrent call.
 */
#define GDR_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int gdr_prefill_chunked_noalloc(const gdr_dims* dims, gdr_dtype io, gdr_gate gate,
                                const void* q, const void* k, const void* v,
                                const float* gate_in, const float* A_log, const float* dt_bias,
                                const float* beta_logit, const float* state_in, float* state_out,
                                void* o, float scale, int l2norm_qk, hipStream_t stream);

/* Static, human-readable text for a gdr_status value. */
const char* gdr_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H_ */
