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
// across the row groups inside a wave (row rotations and lane exchanges), then
// across waves in LDS.
#include "device_common.hpp"
#include "gdr_internal.h"
#include "gdr.h"

namespace gdr {
namespace {

// The state tile goes through a buffer descriptor (gfx9 family: third word
// 0x00020000, raw 32-bit elements): one 32-bit lane offset serves every row,
// and each row's offset is a scalar, so the tile's 16 rows per thread need no
// per-row 64-bit addresses in vector registers.
typedef unsigned int u32x4_t __attribute__((__vector_size__(16)));
constexpr int kBufferWord3 = 0x00020000;
constexpr size_t kMallBytes = size_t{256} << 20;  // MI355X Infinity Cache

__device__ __forceinline__ float4 tile_load(__amdgpu_buffer_rsrc_t r, unsigned voff,
                                            unsigned soff) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// kNt: the store carries the non-temporal cache policy (bit 1 of the gfx9
// buffer cache-policy operand).
template <bool kNt>
__device__ __forceinline__ void tile_store(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff,
                                           float4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, voff, soff,
                                         kNt ? 2 : 0);
}

// NTM: threads per workgroup at most (256, or 64 for one wave per tile).
template <int DK, int DVS, int NTM = 256>
struct DecodeShape {
  static constexpr int C4 = DVS / 4;                          // float4 columns
  static constexpr int RG = (DK < NTM / C4) ? DK : NTM / C4;  // row groups
  static constexpr int NT = C4 * RG;                          // threads
  static constexpr int RPT = DK / RG;                         // rows per thread
  static constexpr int NW = NT / 64;                          // waves
  static_assert(NT % 64 == 0 && NT <= 256, "workgroup must be whole waves");
  static_assert(DK % RG == 0, "rows must split evenly");
};

// kChannel: per-channel log-decays; otherwise one per (b, h), plain or fused.
// kNtStore: the new state is written with the non-temporal cache policy.
// While the whole state fits the 256 MiB MALL, plain stores keep it there
// for the next step; beyond it, write-allocating every line of the new state
// only evicts what the rest of the step needs, and streaming stores are
// faster (B=160, 192, 256 at dk=dv=128: 12%, 19%, 18%; B=64 and 128: plain
// 6% and 2% faster).
template <typename IoT, int DK, int DVS, bool kChannel, bool kNtStore, int NTM>
__global__ __launch_bounds__((DecodeShape<DK, DVS, NTM>::NT))
__attribute__((amdgpu_waves_per_eu(sizeof(IoT) == 4 && !kChannel ? 4 : 5))) void decode_kernel(
    DecodeArgs a) {
  using Sh = DecodeShape<DK, DVS, NTM>;
  constexpr int C4 = Sh::C4, RPT = Sh::RPT, NW = Sh::NW;
  constexpr int NE = (DK + 63) / 64;  // head elements per lane of wave 0
  // Per-row vectors of the head, shared by the C4 lanes of each row group:
  // normalised k and q, the decay a, and a*k.  One copy per wave: every wave
  // builds the whole set, writes only its own copy and reads it after its own
  // writes have completed, so no workgroup barrier is needed before pass 1 and
  // no two waves touch the same words.
  __shared__ __attribute__((aligned(16))) float kS_w[NW][DK], qS_w[NW][DK], dS_w[NW][DK],
      akS_w[NW][DK];
  __shared__ float4 red[2][NW][C4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  float* const kS = kS_w[wave];
  float* const qS = qS_w[wave];
  float* const dS = dS_w[wave];
  float* const akS = akS_w[wave];
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
  const size_t bh = static_cast<size_t>(b) * a.H_v + h;

  // ---- every load first: the small per-head inputs, then the state tile ----
  // Waits are in issue order, so with the small loads ahead of the 64 KiB
  // tile the per-head vectors are built while the tile is still arriving.
  const IoT* row = static_cast<const IoT*>(a.qkv) +
                   static_cast<size_t>(b) * (2 * a.H_qk * DK + a.H_v * a.dv);
  const IoT* qh = row + hq * DK;
  const IoT* kh = row + a.H_qk * DK + hq * DK;
  const IoT* vh = row + 2 * a.H_qk * DK + h * a.dv;
  float vv[4];
  load_row<IoT, 4>(vh + j0, vv);
  const float beta = sigmoidf(a.beta_logit[bh]);
  // Every wave reads the whole head's k, q (and channel gate) and keeps them
  // raw until the tile has been requested, so that nothing waits on them
  // before that.
  // kVec (bf16 rows, channel gate): one 16-byte load per lane covers all
  // three -- lanes 0-15 k, 16-31 q (8 values a lane), 32-63 the gate (4 a
  // lane) -- so each norm is a sum over one 16-lane row.  Otherwise every
  // lane reads element lane (+64) of each (lanes past dk read element dk - 1,
  // masked).
  constexpr bool kVec = kChannel && sizeof(IoT) == 2 && DK <= 128;
  constexpr int KL = DK / 8, GL = DK / 4;  // lanes holding k (or q), the gate
  const int vrow = lane >> 4, vpos = lane & 15;
  uint4 rv4 = make_uint4(0u, 0u, 0u, 0u);
  IoT rk[NE], rq[NE];
  float eg[NE];
  if constexpr (kVec) {
    const void* src;
    if (vrow == 0) src = kh + 8 * min(vpos, KL - 1);
    else if (vrow == 1) src = qh + 8 * min(vpos, KL - 1);
    else src = a.gate_in + bh * DK + 4 * min(lane - 32, GL - 1);
    rv4 = *static_cast<const uint4*>(src);
  } else {
#pragma unroll
    for (int u = 0; u < NE; ++u) {
      const int e = min(lane + 64 * u, DK - 1);
      rk[u] = kh[e];
      rq[u] = qh[e];
      if constexpr (kChannel) eg[u] = a.gate_in[bh * DK + e];
    }
  }

  // The state tile (dk x dv fp32, at most 64 KiB) through a buffer descriptor.
  float* S = a.state + bh * DK * a.dv;
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      S, 0, static_cast<int>(DK * a.dv * sizeof(float)), kBufferWord3);
  const unsigned boff = (static_cast<unsigned>(row0) * a.dv + j0) * 4u;  // lane, bytes
  const unsigned rstep = static_cast<unsigned>(a.dv) * 4u;                // row, bytes
  float4 s[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) s[m] = tile_load(srs, boff, m * rstep);
  __builtin_amdgcn_sched_barrier(0);

  // Every wave builds the whole head's vectors into its own LDS copy.
  if constexpr (kVec) {
    if (vrow < 2) {
      const IoT* e8 = reinterpret_cast<const IoT*>(&rv4);
      float x[8];
      float ss = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[j] = to_f32(e8[j]);
        ss += x[j] * x[j];
      }
      ss = row16_sum(vpos < KL ? ss : 0.0f);
      const float inv = a.l2norm ? 1.0f / sqrtf(ss + kL2Eps) : 1.0f;
      if (vpos < KL) {
        float* dst = (vrow == 0 ? kS : qS) + 8 * vpos;
        *reinterpret_cast<float4*>(dst) = make_float4(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
        *reinterpret_cast<float4*>(dst + 4) =
            make_float4(x[4] * inv, x[5] * inv, x[6] * inv, x[7] * inv);
      }
    } else if (lane - 32 < GL) {
      const float4 g = *reinterpret_cast<const float4*>(&rv4);
      *reinterpret_cast<float4*>(dS + 4 * (lane - 32)) =
          make_float4(expf(g.x), expf(g.y), expf(g.z), expf(g.w));
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): k and the decays are in LDS
    __builtin_amdgcn_wave_barrier();
    if (lane < DK / 4) {
      const float4 k4 = *reinterpret_cast<const float4*>(kS + 4 * lane);
      const float4 d4 = *reinterpret_cast<const float4*>(dS + 4 * lane);
      *reinterpret_cast<float4*>(akS + 4 * lane) =
          make_float4(d4.x * k4.x, d4.y * k4.y, d4.z * k4.z, d4.w * k4.w);
    }
  } else {
    float ek[NE], eq[NE];
#pragma unroll
    for (int u = 0; u < NE; ++u) {
      ek[u] = to_f32(rk[u]);
      eq[u] = to_f32(rq[u]);
    }
    float sk = 0.0f, sq = 0.0f;
#pragma unroll
    for (int u = 0; u < NE; ++u) {
      const float msk = lane + 64 * u < DK ? 1.0f : 0.0f;
      sk += msk * ek[u] * ek[u];
      sq += msk * eq[u] * eq[u];
    }
    sk = wave_sum(sk);
    sq = wave_sum(sq);
    const float inv_nk = a.l2norm ? 1.0f / sqrtf(sk + kL2Eps) : 1.0f;
    const float inv_nq = a.l2norm ? 1.0f / sqrtf(sq + kL2Eps) : 1.0f;
    float d1 = 0.0f;
    if constexpr (!kChannel) {
      const float g = a.gate == GDR_GATE_SCALAR
                          ? a.gate_in[bh]
                          : fused_log_decay(a.gate_in[bh], a.A_log[h], a.dt_bias[h]);
      d1 = expf(g);
    }
#pragma unroll
    for (int u = 0; u < NE; ++u) {
      const int e = lane + 64 * u;
      if (e < DK) {
        const float d = kChannel ? expf(eg[u]) : d1;
        const float kk = ek[u] * inv_nk;
        kS[e] = kk;
        qS[e] = eq[u] * inv_nq;
        dS[e] = d;
        akS[e] = d * kk;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
  __builtin_amdgcn_wave_barrier();

  // ---- pass 1: vhat = (diag(a) S)^T k ----
  float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const float ak = akS[row0 + m];  // same address across the row group: broadcast
    p0 += ak * s[m].x;
    p1 += ak * s[m].y;
    p2 += ak * s[m].z;
    p3 += ak * s[m].w;
  }
  p0 = lane_class_sum<C4>(p0);  // over the row groups of the wave
  p1 = lane_class_sum<C4>(p1);
  p2 = lane_class_sum<C4>(p2);
  p3 = lane_class_sum<C4>(p3);
  float4 vh4 = make_float4(p0, p1, p2, p3);  // one wave: every lane holds its columns' sums
  if constexpr (NW > 1) {
    if (lane < C4) red[0][wave][c4] = vh4;
    __syncthreads();
    vh4 = red[0][0][c4];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      float4 t = red[0][w][c4];
      vh4.x += t.x;
      vh4.y += t.y;
      vh4.z += t.z;
      vh4.w += t.w;
    }
  }
  const float u0 = beta * (vv[0] - vh4.x), u1 = beta * (vv[1] - vh4.y);
  const float u2 = beta * (vv[2] - vh4.z), u3 = beta * (vv[3] - vh4.w);

  // ---- pass 2: decay + rank-one write, accumulate o = S^T q ----
  float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const float d = dS[row0 + m], kk = kS[row0 + m], qq = qS[row0 + m];
    float4 t = s[m];
    t.x = d * t.x + kk * u0;
    t.y = d * t.y + kk * u1;
    t.z = d * t.z + kk * u2;
    t.w = d * t.w + kk * u3;
    tile_store<kNtStore>(srs, boff, m * rstep, t);
    o0 += qq * t.x;
    o1 += qq * t.y;
    o2 += qq * t.z;
    o3 += qq * t.w;
  }
  o0 = lane_class_sum<C4>(o0);  // over the row groups of the wave
  o1 = lane_class_sum<C4>(o1);
  o2 = lane_class_sum<C4>(o2);
  o3 = lane_class_sum<C4>(o3);
  float4 acc = make_float4(o0, o1, o2, o3);
  if constexpr (NW > 1) {
    if (lane < C4) red[1][wave][c4] = acc;
    __syncthreads();
  }
  if (tid < C4) {
    if constexpr (NW > 1) {
      acc = red[1][0][c4];
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        float4 t = red[1][w][c4];
        acc.x += t.x;
        acc.y += t.y;
        acc.z += t.z;
        acc.w += t.w;
      }
    }
    IoT* op = static_cast<IoT*>(a.o) + bh * a.dv + j0;
    store4<IoT>(op, a.scale * acc.x, a.scale * acc.y, a.scale * acc.z, a.scale * acc.w);
  }
}

// Occupancy cap for large grids of whole 128 x 128 tiles with a channel gate,
// written with plain stores: LDS the kernel does not use, so that at most
// three workgroups share a CU (160 KiB of LDS over more than 40 KiB each; the
// kernel's own LDS, 12 KiB at four waves, comes on top).
// Fewer tiles in flight contend less for the memory system there (graph
// replay, bf16: B=64 41.5 -> 41.1 us, B=128 80.7 -> 78.8 us).  Smaller grids
// lose by it (B=16: 9.5 -> 10.9 us), with streaming stores (B=256) it is
// neutral, and with a scalar gate (one decay per tile, lighter loads) it costs
// 0.4-0.9%.
constexpr unsigned kOccupancyPadBytes = 40 * 1024;
constexpr unsigned kOccupancyPadMinGrid = 2048;

// Grids of at most this many tiles (one per CU or fewer: the step is a
// latency chain) run one wave per tile, so that both column sums stay within
// the wave (no LDS exchange, no barrier).
constexpr unsigned kOneWaveMaxGrid = 256;

template <typename IoT, int DK, int DVS, bool kNtStore, int NTM>
hipError_t launch_ntm(const DecodeArgs& a, unsigned grid, unsigned pad, hipStream_t stream) {
  if (a.gate == GDR_GATE_CHANNEL)
    hipLaunchKernelGGL((decode_kernel<IoT, DK, DVS, true, kNtStore, NTM>), dim3(grid),
                       dim3(DecodeShape<DK, DVS, NTM>::NT), pad, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<IoT, DK, DVS, false, kNtStore, NTM>), dim3(grid),
                       dim3(DecodeShape<DK, DVS, NTM>::NT), pad, stream, a);
  return hipGetLastError();
}

template <typename IoT, int DK, int DVS, bool kNtStore>
hipError_t launch_nt(const DecodeArgs& a, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(a.B) * a.H_v * (a.dv / DVS);
  if (grid <= kOneWaveMaxGrid) return launch_ntm<IoT, DK, DVS, kNtStore, 64>(a, grid, 0, stream);
  const unsigned pad = (DK == 128 && DVS == 128 && !kNtStore && a.gate == GDR_GATE_CHANNEL &&
                        grid >= kOccupancyPadMinGrid)
                           ? kOccupancyPadBytes
                           : 0;
  return launch_ntm<IoT, DK, DVS, kNtStore, 256>(a, grid, pad, stream);
}

template <typename IoT, int DK, int DVS>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const size_t state_bytes =
      static_cast<size_t>(a.B) * a.H_v * static_cast<size_t>(a.dk) * a.dv * sizeof(float);
  return state_bytes > kMallBytes ? launch_nt<IoT, DK, DVS, true>(a, stream)
                                  : launch_nt<IoT, DK, DVS, false>(a, stream);
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
