// decode.hip -- fused single-token gated-delta-rule step for gfx950.
//
// One workgroup owns a (batch row b, value head h, slice of DVS state columns)
// tile.  The columns of the state are independent in the update (column j of
// the new state and of o depends only on column j of S and v), so slicing dv
// only costs the recomputation of the small per-head prologue.
//
// The step follows "Add fused GatedDeltaNet decode Triton kernel" (executorch
// PR #18865, summary) for what is fused -- Q/K/V split of the packed row, L2
// normalisation, head repeat, gating and the recurrent update -- and the
// two-pass order of "Two-pass optimization for channelwise gated delta rule
// kernel" (PR #21020, Summary) for the state traffic:
//   pass 1: vhat[j] = sum_i a_i k_i S[i][j]         (decay folded in)
//   pass 2: S[i][j] = a_i S[i][j] + k_i u_j,  u = beta (v - vhat)
//           o[j]    = scale sum_i q_i S[i][j]
// The tile is held in registers between the passes, so the state crosses HBM
// exactly once in each direction.  The kernel is bandwidth bound (well under
// one flop per byte) and uses no matrix cores.
//
// Thread layout: C4 = DVS/4 lanes cover a row slice as float4s (a wave reads
// whole 512-byte rows when DVS = 128), RG = NT/C4 row groups each own
// RPT = dk/RG consecutive rows.  Column sums over rows are reduced first
// across the row groups inside a wave (lane xor), then across waves in LDS.
#include "device_common.hpp"
#include "gdr_internal.h"
#include "gdr.h"

namespace gdr {
namespace {

template <int DK, int DVS>
struct DecodeShape {
  static constexpr int C4 = DVS / 4;                          // float4 columns
  static constexpr int RG = (DK < 256 / C4) ? DK : 256 / C4;  // row groups
  static constexpr int NT = C4 * RG;                          // threads
  static constexpr int RPT = DK / RG;                         // rows per thread
  static constexpr int NW = NT / 64;                          // waves
  static_assert(NT % 64 == 0 && NT <= 256, "workgroup must be whole waves");
  static_assert(DK % RG == 0, "rows must split evenly");
};

// kChannel: per-channel log-decays; otherwise one per (b, h), plain or fused.
template <typename IoT, int DK, int DVS, bool kChannel>
__global__ __launch_bounds__((DecodeShape<DK, DVS>::NT)) void decode_kernel(DecodeArgs a) {
  using Sh = DecodeShape<DK, DVS>;
  constexpr int C4 = Sh::C4, RPT = Sh::RPT, NW = Sh::NW;
  __shared__ float4 red[2][NW][C4];

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
  const int j0 = slice * DVS + c4 * 4;

  // ---- every load first: the small per-head inputs, then the state tile ----
  // Waits are in issue order, so with the small loads ahead of the 64 KiB
  // tile the norms and gates are computed while the tile is still arriving;
  // nothing is computed (and so nothing waits) before the tile is requested.
  const IoT* row = static_cast<const IoT*>(a.qkv) +
                   static_cast<size_t>(b) * (2 * a.H_qk * DK + a.H_v * a.dv);
  const IoT* qh = row + hq * DK;
  const IoT* kh = row + a.H_qk * DK + hq * DK;
  const IoT* vh = row + 2 * a.H_qk * DK + h * a.dv;
  const size_t bh = static_cast<size_t>(b) * a.H_v + h;

  float kr[RPT], qr[RPT];
  load_row<IoT, RPT>(kh + row0, kr);
  load_row<IoT, RPT>(qh + row0, qr);
  float vv[4];
  load_row<IoT, 4>(vh + j0, vv);
  float g[kChannel ? RPT : 1];
  float A_log = 0.0f, dt_bias = 0.0f;
  if constexpr (kChannel) {
    load_row<float, RPT>(a.gate_in + bh * DK + row0, g);
  } else {
    g[0] = a.gate_in[bh];
    if (a.gate == GDR_GATE_SCALAR_FUSED) {
      A_log = a.A_log[h];
      dt_bias = a.dt_bias[h];
    }
  }
  const float beta_x = a.beta_logit[bh];
  // Whole-head k and q for the L2 norms (every wave reduces the head itself);
  // lanes past dk read element dk - 1 and are masked.
  constexpr int NE = (DK + 63) / 64;
  float ek[NE], eq[NE];
#pragma unroll
  for (int u = 0; u < NE; ++u) {
    const int e = min(lane + 64 * u, DK - 1);
    ek[u] = to_f32(kh[e]);
    eq[u] = to_f32(qh[e]);
  }

  float* S = a.state + bh * DK * a.dv;
  float4 s[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m)
    s[m] = *reinterpret_cast<const float4*>(S + static_cast<size_t>(row0 + m) * a.dv + j0);

  // (computed unconditionally, so the element loads stay ahead of the tile)
  float sk = 0.0f, sq = 0.0f;
#pragma unroll
  for (int u = 0; u < NE; ++u) {
    const float m = lane + 64 * u < DK ? 1.0f : 0.0f;
    sk += m * ek[u] * ek[u];
    sq += m * eq[u] * eq[u];
  }
  sk = wave_sum(sk);
  sq = wave_sum(sq);
  const float inv_nk = a.l2norm ? 1.0f / sqrtf(sk + kL2Eps) : 1.0f;
  const float inv_nq = a.l2norm ? 1.0f / sqrtf(sq + kL2Eps) : 1.0f;

  // ---- gates ----
  const float beta = sigmoidf(beta_x);
  float ak[RPT], dec[RPT];
  if constexpr (kChannel) {
#pragma unroll
    for (int m = 0; m < RPT; ++m) dec[m] = expf(g[m]);
  } else {
    const float g1 =
        a.gate == GDR_GATE_SCALAR_FUSED ? fused_log_decay(g[0], A_log, dt_bias) : g[0];
    const float d = expf(g1);
#pragma unroll
    for (int m = 0; m < RPT; ++m) dec[m] = d;
  }
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    kr[m] *= inv_nk;
    qr[m] *= inv_nq;
    ak[m] = dec[m] * kr[m];
  }

  // ---- pass 1: vhat = (diag(a) S)^T k ----
  float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    p0 += ak[m] * s[m].x;
    p1 += ak[m] * s[m].y;
    p2 += ak[m] * s[m].z;
    p3 += ak[m] * s[m].w;
  }
#pragma unroll
  for (int off = C4; off < 64; off <<= 1) {
    p0 += __shfl_xor(p0, off, 64);
    p1 += __shfl_xor(p1, off, 64);
    p2 += __shfl_xor(p2, off, 64);
    p3 += __shfl_xor(p3, off, 64);
  }
  if (lane < C4) red[0][wave][c4] = make_float4(p0, p1, p2, p3);
  __syncthreads();
  float4 vh4 = red[0][0][c4];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    float4 t = red[0][w][c4];
    vh4.x += t.x;
    vh4.y += t.y;
    vh4.z += t.z;
    vh4.w += t.w;
  }
  const float u0 = beta * (vv[0] - vh4.x), u1 = beta * (vv[1] - vh4.y);
  const float u2 = beta * (vv[2] - vh4.z), u3 = beta * (vv[3] - vh4.w);

  // ---- pass 2: decay + rank-one write, accumulate o = S^T q ----
  float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    float4 t = s[m];
    t.x = dec[m] * t.x + kr[m] * u0;
    t.y = dec[m] * t.y + kr[m] * u1;
    t.z = dec[m] * t.z + kr[m] * u2;
    t.w = dec[m] * t.w + kr[m] * u3;
    *reinterpret_cast<float4*>(S + static_cast<size_t>(row0 + m) * a.dv + j0) = t;
    o0 += qr[m] * t.x;
    o1 += qr[m] * t.y;
    o2 += qr[m] * t.z;
    o3 += qr[m] * t.w;
  }
#pragma unroll
  for (int off = C4; off < 64; off <<= 1) {
    o0 += __shfl_xor(o0, off, 64);
    o1 += __shfl_xor(o1, off, 64);
    o2 += __shfl_xor(o2, off, 64);
    o3 += __shfl_xor(o3, off, 64);
  }
  if (lane < C4) red[1][wave][c4] = make_float4(o0, o1, o2, o3);
  __syncthreads();
  if (tid < C4) {
    float4 acc = red[1][0][c4];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      float4 t = red[1][w][c4];
      acc.x += t.x;
      acc.y += t.y;
      acc.z += t.z;
      acc.w += t.w;
    }
    IoT* op = static_cast<IoT*>(a.o) + bh * a.dv + j0;
    store4<IoT>(op, a.scale * acc.x, a.scale * acc.y, a.scale * acc.z, a.scale * acc.w);
  }
}

template <typename IoT, int DK, int DVS>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(a.B) * a.H_v * (a.dv / DVS);
  if (a.gate == GDR_GATE_CHANNEL)
    hipLaunchKernelGGL((decode_kernel<IoT, DK, DVS, true>), dim3(grid),
                       dim3(DecodeShape<DK, DVS>::NT), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<IoT, DK, DVS, false>), dim3(grid),
                       dim3(DecodeShape<DK, DVS>::NT), 0, stream, a);
  return hipGetLastError();
}

template <typename IoT, int DK>
hipError_t launch_dk(const DecodeArgs& a, int dvs, hipStream_t stream) {
  switch (dvs) {
    case 16: return launch_t<IoT, DK, 16>(a, stream);
    case 32: return launch_t<IoT, DK, 32>(a, stream);
    case 64: return launch_t<IoT, DK, 64>(a, stream);
    case 128: return launch_t<IoT, DK, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename IoT>
hipError_t launch_io(const DecodeArgs& a, int dvs, hipStream_t stream) {
  switch (a.dk) {
    case 16: return launch_dk<IoT, 16>(a, dvs, stream);
    case 32: return launch_dk<IoT, 32>(a, dvs, stream);
    case 64: return launch_dk<IoT, 64>(a, dvs, stream);
    case 128: return launch_dk<IoT, 128>(a, dvs, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int decode_dv_slice(int B, int H_v, int dv) {
  // Enough workgroups to cover the 256 CUs several times over; never below
  // 16 columns (one float4 lane group per row needs at least 4 lanes).
  long units = static_cast<long>(B) * H_v;
  int slices = 1;
  while (units * slices < 1024 && dv / (slices * 2) >= 16) slices *= 2;
  return dv / slices;
}

hipError_t launch_decode(const DecodeArgs& a, int io_bf16, int dv_slice, hipStream_t stream) {
  return io_bf16 ? launch_io<bf16>(a, dv_slice, stream) : launch_io<float>(a, dv_slice, stream);
}

}  // namespace gdr
