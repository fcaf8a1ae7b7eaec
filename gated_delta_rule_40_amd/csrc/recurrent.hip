// recurrent.hip -- a short sequence token by token, the state tile held in
// registers from the first token to the last.
//
// The chunked form ("Add parallel chunked prefill for channelwise gated delta
// rule", PR #21061, Summary) pays a fixed cost per call -- the chunk-parallel
// preparation and a dependent step per chunk -- that a few tokens do not
// amortise, while repeated single-token steps read and write the whole state
// once per token.  Here one workgroup owns a (b, h, slice of DVS state columns)
// tile for the whole sequence, so the state crosses HBM once in each direction
// whatever T is, and each token is the two-pass update of "Two-pass
// optimization for channelwise gated delta rule kernel" (PR #21020, Summary):
//   pass 1: vhat[j] = sum_i a_i k_i S[i][j]
//   pass 2: S[i][j] = a_i S[i][j] + k_i u_j,  u = beta (v - vhat)
//           o[j]    = scale sum_i q_i S[i][j]
// with the fused split, L2 norm, head repeat and gating of "Add fused
// GatedDeltaNet decode Triton kernel" (PR #18865, summary) applied per token.
//
// Nothing a token needs depends on the state except the two passes, so a
// pre-pass builds every token's normalised k and q, decay a, v slice, beta and
// q.k in LDS (all waves, tokens spread over the waves, each wave's loads for a
// batch of tokens in flight together).  The token loop then reads only LDS.
// The output needs no reduction of its own: since S' = diag(a) S + k u^T,
//   o[j] = scale (sum_i q_i a_i S[i][j] + (q.k) u_j),
// and the first sum runs over the same rows as vhat, so per token one
// reduction (8 column sums per thread, one barrier) serves both.
//
// Thread layout as in the decode step: C4 = DVS/4 lanes cover a row slice as
// float4s, RG = NT/C4 row groups each own RPT = DK/RG consecutive rows.
#include "device_common.hpp"
#include "gdr_internal.h"
#include "gdr.h"

namespace gdr {
namespace {

typedef unsigned int u32x4_t __attribute__((__vector_size__(16)));
constexpr int kBufferWord3 = 0x00020000;  // gfx9 buffer descriptor, raw 32-bit elements

__device__ __forceinline__ float4 rtile_load(__amdgpu_buffer_rsrc_t r, unsigned voff,
                                             unsigned soff) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// kNt: the store carries the non-temporal cache policy (bit 1 of the gfx9
// buffer cache-policy operand).
template <bool kNt>
__device__ __forceinline__ void rtile_store(__amdgpu_buffer_rsrc_t r, unsigned voff,
                                            unsigned soff, float4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, voff, soff,
                                         kNt ? 2 : 0);
}
constexpr size_t kMallBytes = size_t{256} << 20;  // MI355X Infinity Cache

template <int DK, int DVS>
struct RecShape {
  static constexpr int C4 = DVS / 4;                          // float4 columns
  static constexpr int RG = (DK < 256 / C4) ? DK : 256 / C4;  // row groups
  static constexpr int NT = C4 * RG;                          // threads
  static constexpr int RPT = DK / RG;                         // rows per thread
  static constexpr int NW = NT / 64;                          // waves
  static constexpr int NE = (DK + 63) / 64;                   // head elements per lane
  static constexpr int NV = (DVS + 63) / 64;                  // v elements per lane
  static constexpr int G = DVS >= 64 ? 4 : 8;                 // tokens per wave per load batch
  // LDS per token: k, q, a (3 DK floats), the v slice (DVS floats), beta, q.k.
  static constexpr size_t kTokenBytes = (3 * DK + DVS + 2) * sizeof(float);
  static_assert(NT % 64 == 0 && NT <= 256, "workgroup must be whole waves");
};

// kNtStore: the final state is written with the non-temporal cache policy,
// as the decode step does once the state exceeds the 256 MiB MALL (B=256,
// T=4 at dk=dv=128: 229 -> 184 us; B=64 unchanged).
template <typename IoT, int DK, int DVS, bool kChannel, bool kNtStore>
__global__ __launch_bounds__((RecShape<DK, DVS>::NT)) void recurrent_kernel(PrefillArgs a) {
  using Sh = RecShape<DK, DVS>;
  constexpr int C4 = Sh::C4, RPT = Sh::RPT, NW = Sh::NW, NE = Sh::NE, NV = Sh::NV, G = Sh::G;
  extern __shared__ __attribute__((aligned(16))) float rsm[];
  __shared__ float4 red[2][2][NW][C4];  // [token parity][vhat, o part][wave][column quad]

  const int T = a.T;
  float* hv = rsm;                 // [T][3][DK]: normalised k, normalised q, decay a
  float* vS = rsm + T * 3 * DK;    // [T][DVS]
  float* bS = vS + T * DVS;        // [T] beta
  float* qkS = bS + T;             // [T] q.k

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c4 = tid % C4;
  const int rg = tid / C4;
  const int row0 = rg * RPT;

  const int n_slices = a.dv / DVS;
  const int wg = blockIdx.x;
  const int slice = wg % n_slices;
  const int h = (wg / n_slices) % a.H_v;
  const int b = wg / (n_slices * a.H_v);
  const int hq = h / (a.H_v / a.H_qk);  // head repeat (repeat-interleave)
  const int jb = slice * DVS;
  const int j0 = jb + c4 * 4;
  const size_t bh = static_cast<size_t>(b) * a.H_v + h;

  // ---- the state tile, through buffer descriptors (one 32-bit lane offset,
  //      a scalar offset per row) ----
  const unsigned boff = (static_cast<unsigned>(row0) * a.dv + j0) * 4u;
  const unsigned rstep = static_cast<unsigned>(a.dv) * 4u;
  const int tile_bytes = static_cast<int>(DK * a.dv * sizeof(float));
  float4 s[RPT];
  if (a.state_in) {
    const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.state_in) + bh * DK * a.dv, 0, tile_bytes, kBufferWord3);
#pragma unroll
    for (int m = 0; m < RPT; ++m) s[m] = rtile_load(src, boff, m * rstep);
  } else {
#pragma unroll
    for (int m = 0; m < RPT; ++m) s[m] = make_float4(0.f, 0.f, 0.f, 0.f);
  }

  // ---- pre-pass: every token's head vectors, v slice, beta and q.k into LDS ----
  // Wave w takes tokens w, w + NW, ...; a batch of G of them has all its loads
  // issued before any is used.  Indices past the end are clamped (loaded,
  // then not written).
  const IoT* qg = static_cast<const IoT*>(a.q);
  const IoT* kg = static_cast<const IoT*>(a.k);
  const IoT* vg = static_cast<const IoT*>(a.v);
  float A_log = 0.f, dt_bias = 0.f;
  if (!kChannel && a.gate == GDR_GATE_SCALAR_FUSED) {
    A_log = a.A_log[h];
    dt_bias = a.dt_bias[h];
  }
  for (int t0 = wave; t0 < T; t0 += NW * G) {
    IoT rk[G][NE], rq[G][NE], rv[G][NV];
    float rgate[G][NE], rb[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int t = min(t0 + i * NW, T - 1);
      const size_t qk_row = (static_cast<size_t>(b) * T + t) * a.H_qk + hq;
      const size_t v_row = (static_cast<size_t>(b) * T + t) * a.H_v + h;
#pragma unroll
      for (int u = 0; u < NE; ++u) {
        const int e = min(lane + 64 * u, DK - 1);
        rk[i][u] = kg[qk_row * DK + e];
        rq[i][u] = qg[qk_row * DK + e];
        if constexpr (kChannel) rgate[i][u] = a.gate_in[v_row * DK + e];
      }
      if constexpr (!kChannel) rgate[i][0] = a.gate_in[v_row];
#pragma unroll
      for (int u = 0; u < NV; ++u) rv[i][u] = vg[v_row * a.dv + jb + min(lane + 64 * u, DVS - 1)];
      rb[i] = a.beta_logit[v_row];
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int t = t0 + i * NW;
      if (t < T) {  // wave-uniform
        float ek[NE], eq[NE];
        float sk = 0.f, sq = 0.f, skq = 0.f;
#pragma unroll
        for (int u = 0; u < NE; ++u) {
          ek[u] = to_f32(rk[i][u]);
          eq[u] = to_f32(rq[i][u]);
          const float msk = lane + 64 * u < DK ? 1.0f : 0.0f;
          sk += msk * ek[u] * ek[u];
          sq += msk * eq[u] * eq[u];
          skq += msk * ek[u] * eq[u];
        }
        sk = wave_sum(sk);
        sq = wave_sum(sq);
        skq = wave_sum(skq);
        const float inv_nk = a.l2norm ? 1.0f / sqrtf(sk + kL2Eps) : 1.0f;
        const float inv_nq = a.l2norm ? 1.0f / sqrtf(sq + kL2Eps) : 1.0f;
        float d1 = 0.f;
        if constexpr (!kChannel) {
          const float g = a.gate == GDR_GATE_SCALAR ? rgate[i][0]
                                                    : fused_log_decay(rgate[i][0], A_log, dt_bias);
          d1 = expf(g);
        }
        float* ht = hv + static_cast<size_t>(t) * 3 * DK;
#pragma unroll
        for (int u = 0; u < NE; ++u) {
          const int e = lane + 64 * u;
          if (e < DK) {
            ht[e] = ek[u] * inv_nk;
            ht[DK + e] = eq[u] * inv_nq;
            ht[2 * DK + e] = kChannel ? expf(rgate[i][u]) : d1;
          }
        }
#pragma unroll
        for (int u = 0; u < NV; ++u)
          if (lane + 64 * u < DVS) vS[t * DVS + lane + 64 * u] = to_f32(rv[i][u]);
        if (lane == 0) {
          bS[t] = sigmoidf(rb[i]);
          qkS[t] = skq * inv_nk * inv_nq;
        }
      }
    }
  }
  __syncthreads();

  // ---- the tokens, in order ----
  // Per token: column sums of a*k (vhat) and a*q (o part) weighted by the
  // state, over this thread's rows, then over the row groups of the wave and
  // across waves (LDS, one barrier); then u and o, and the rank-one update.
  // red is double-buffered by token parity: a wave writes token t + 1's sums
  // while another may still read token t's, and no wave reaches token t + 2
  // before every wave has passed token t + 1's barrier.
  // With few rows per thread (few workgroups, latency-bound) the next
  // token's rows of k, q and a are read from LDS before the barrier, so that
  // their latency hides behind it; with many (many workgroups, throughput-
  // bound) the registers this takes cost more than it hides.
  constexpr bool kAhead = RPT <= 4;
  IoT* og = static_cast<IoT*>(a.o);
  float kn[RPT], qn[RPT], dn[RPT];
  auto read_rows = [&](int t) __attribute__((always_inline)) {
    const float* kS = hv + static_cast<size_t>(t) * 3 * DK;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {  // same address across the row group: broadcast
      kn[m] = kS[row0 + m];
      qn[m] = kS[DK + row0 + m];
      dn[m] = kS[2 * DK + row0 + m];
    }
  };
  if constexpr (kAhead) read_rows(0);
  for (int t = 0; t < T; ++t) {
    if constexpr (!kAhead) read_rows(t);
    float dd[RPT], kk[RPT];
    float pv[4] = {0.f, 0.f, 0.f, 0.f}, po[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      dd[m] = dn[m];
      kk[m] = kn[m];
      const float ak = dd[m] * kk[m], aq = dd[m] * qn[m];
      const float sv[4] = {s[m].x, s[m].y, s[m].z, s[m].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        pv[c] += ak * sv[c];
        po[c] += aq * sv[c];
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      pv[c] = lane_class_sum<C4>(pv[c]);
      po[c] = lane_class_sum<C4>(po[c]);
    }
    const int par = t & 1;
    if (lane < C4) {
      red[par][0][wave][c4] = make_float4(pv[0], pv[1], pv[2], pv[3]);
      red[par][1][wave][c4] = make_float4(po[0], po[1], po[2], po[3]);
    }
    if constexpr (kAhead) read_rows(min(t + 1, T - 1));
    __syncthreads();
    // Every thread reads both sums (LDS broadcasts); only the store of o is
    // left to the first row group, so no wave waits on a read of its own.
    float4 vh4 = red[par][0][0][c4], oh = red[par][1][0][c4];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      const float4 x = red[par][0][w][c4], y = red[par][1][w][c4];
      vh4.x += x.x;
      vh4.y += x.y;
      vh4.z += x.z;
      vh4.w += x.w;
      oh.x += y.x;
      oh.y += y.y;
      oh.z += y.z;
      oh.w += y.w;
    }
    const float beta = bS[t], qk = qkS[t];
    const float4 vv = *reinterpret_cast<const float4*>(vS + t * DVS + c4 * 4);
    const float u[4] = {beta * (vv.x - vh4.x), beta * (vv.y - vh4.y), beta * (vv.z - vh4.z),
                        beta * (vv.w - vh4.w)};
    const float o0 = a.scale * (oh.x + qk * u[0]), o1 = a.scale * (oh.y + qk * u[1]);
    const float o2 = a.scale * (oh.z + qk * u[2]), o3 = a.scale * (oh.w + qk * u[3]);
    if (tid < C4) {
      IoT* op = og + ((static_cast<size_t>(b) * T + t) * a.H_v + h) * a.dv + j0;
      store4<IoT>(op, o0, o1, o2, o3);
    }
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      s[m].x = dd[m] * s[m].x + kk[m] * u[0];
      s[m].y = dd[m] * s[m].y + kk[m] * u[1];
      s[m].z = dd[m] * s[m].z + kk[m] * u[2];
      s[m].w = dd[m] * s[m].w + kk[m] * u[3];
    }
  }

  // ---- final state ----
  const __amdgpu_buffer_rsrc_t dst = __builtin_amdgcn_make_buffer_rsrc(
      a.state_out + bh * DK * a.dv, 0, tile_bytes, kBufferWord3);
#pragma unroll
  for (int m = 0; m < RPT; ++m) rtile_store<kNtStore>(dst, boff, m * rstep, s[m]);
}

template <typename IoT, int DK, int DVS, bool kNtStore>
hipError_t launch_nt(const PrefillArgs& a, hipStream_t stream) {
  using Sh = RecShape<DK, DVS>;
  const unsigned grid = static_cast<unsigned>(a.B) * a.H_v * (a.dv / DVS);
  const size_t lds = static_cast<size_t>(a.T) * Sh::kTokenBytes;
  if (a.gate == GDR_GATE_CHANNEL)
    hipLaunchKernelGGL((recurrent_kernel<IoT, DK, DVS, true, kNtStore>), dim3(grid), dim3(Sh::NT),
                       lds, stream, a);
  else
    hipLaunchKernelGGL((recurrent_kernel<IoT, DK, DVS, false, kNtStore>), dim3(grid),
                       dim3(Sh::NT), lds, stream, a);
  return hipGetLastError();
}

template <typename IoT, int DK, int DVS>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
  const size_t state_bytes =
      static_cast<size_t>(a.B) * a.H_v * static_cast<size_t>(a.dk) * a.dv * sizeof(float);
  return state_bytes > kMallBytes ? launch_nt<IoT, DK, DVS, true>(a, stream)
                                  : launch_nt<IoT, DK, DVS, false>(a, stream);
}

template <typename IoT, int DK>
hipError_t launch_dk(const PrefillArgs& a, int dvs, hipStream_t stream) {
  switch (dvs) {
    case 16: return launch_t<IoT, DK, 16>(a, stream);
    case 32: return launch_t<IoT, DK, 32>(a, stream);
    case 64: return launch_t<IoT, DK, 64>(a, stream);
    case 128: return launch_t<IoT, DK, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename IoT>
hipError_t launch_io(const PrefillArgs& a, int dvs, hipStream_t stream) {
  switch (a.dk) {
    case 16: return launch_dk<IoT, 16>(a, dvs, stream);
    case 32: return launch_dk<IoT, 32>(a, dvs, stream);
    case 64: return launch_dk<IoT, 64>(a, dvs, stream);
    case 128: return launch_dk<IoT, 128>(a, dvs, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int recurrent_max_t(int B, int H_v) {
  // Where the token loop stops beating the chunked path (H 16 -> 32,
  // dk = dv = 128, bf16, kernel times): at B = 1 the chunked path costs about
  // 16 us for any T up to a chunk and the loop passes it after 16 tokens; at
  // B = 16 and 64 (throughput-bound chunked launches) after about 24.
  return static_cast<long>(B) * H_v <= 64 ? 16 : 24;
}

int recurrent_dv_slice(int B, int H_v, int dv) {
  // The widest slice that still gives 256 workgroups (one per CU), down to
  // 16 columns: each workgroup rebuilds its head's per-token vectors, so
  // fewer, wider slices repeat less of that work.
  const long units = static_cast<long>(B) * H_v;
  int dvs = dv;
  while (dvs > 16 && units * (dv / dvs) < 256) dvs /= 2;
  return dvs;
}

size_t recurrent_lds_bytes(int T, int dk, int dv_slice) {
  return static_cast<size_t>(T) * (3 * static_cast<size_t>(dk) + dv_slice + 2) * sizeof(float);
}

hipError_t launch_recurrent(const PrefillArgs& a, int io_bf16, hipStream_t stream) {
  const int dvs = recurrent_dv_slice(a.B, a.H_v, a.dv);
  return io_bf16 ? launch_io<bf16>(a, dvs, stream) : launch_io<float>(a, dvs, stream);
}

}  // namespace gdr
