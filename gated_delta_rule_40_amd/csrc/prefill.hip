// prefill.hip -- chunkwise WY/UT prefill of the gated delta rule for gfx950.
//
// Follows "Add parallel chunked prefill for channelwise gated delta rule"
// (executorch PR #21061, Summary): per chunk, per-channel log-decay prefix
// sums, causal query/key terms, the beta-folded triangular transform, WY
// pseudo-keys/values and the inter-chunk state carry; the last chunk may be
// short and goes through the same code (its missing rows are zeros, which
// leave the result unchanged: k = q = v = 0, beta = 0, g = 0).
//
// For a chunk of C tokens entered with state S (dk x dv), with
// Gamma_r = sum_{s<=r} g_s per key channel:
//   Kt = K e^Gamma, Kh = K e^-Gamma, Qt = Q e^Gamma, Ke = K e^(Gamma_L - Gamma)
//   A  = strict_lower(diag(beta) Kt Kh^T),   Tb = (I + A)^-1 diag(beta)
//   P  = lower(Qt Kh^T)
//   U  = Tb (V - Kt S)                       (the WY pseudo-values minus the
//                                             pseudo-keys applied to S)
//   O  = scale (Qt S + P U)
//   S' = diag(e^Gamma_L) S + Ke^T U
// which is T token updates regrouped exactly.
//
// Two kernels:
//   chunk_prep   one workgroup per (b, h, chunk), all chunks in parallel:
//                everything that does not depend on S -- Kt, Qt, Ke^T, Tb, P
//                and e^Gamma_L -- written to the caller's workspace, one
//                disjoint block per (b, h, chunk).
//   chunk_carry  one workgroup per (b, h, slice of DVS state columns), walking
//                the chunks in order with its state slice held in MFMA
//                accumulators; the columns of S are independent, so slices
//                need no communication.  The next chunk's operands are
//                prefetched into registers while the current one computes.
// Dense products use MFMA (bf16 operands with fp32 accumulation for bf16 io,
// fp32 MFMA for fp32 io); the triangular solve runs in fp32 in LDS.
#include "device_common.hpp"
#include "gdr_internal.h"
#include "gdr.h"

namespace gdr {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

template <typename T>
constexpr int pad_of() {
  return 16 / static_cast<int>(sizeof(T));  // keeps LDS rows 16-byte aligned
}

// ---------------------------------------------------------------------------
// 16x16 MFMA tiles.  Every product is written as  acc += X Z^T  with X and Z
// stored row-major with the contraction index contiguous: lane l supplies
// row (l % 16) of X and row (l % 16) of Z, each with its slice of k, and gets
// back D[4*(l/16) + e][l % 16] for e = 0..3.
// ---------------------------------------------------------------------------
template <typename OpT, int KD>
__device__ __forceinline__ f32x4 mma_xzt(const OpT* __restrict__ X, int ldx, int x0,
                                         const OpT* __restrict__ Z, int ldz, int z0, f32x4 acc,
                                         int lane) {
  const int r = lane & 15;
  const int kg = lane >> 4;
  if constexpr (sizeof(OpT) == 4) {
#pragma unroll
    for (int k = 0; k < KD; k += 4) {
      float a = X[(x0 + r) * ldx + k + kg];
      float b = Z[(z0 + r) * ldz + k + kg];
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
  } else if constexpr (KD % 32 == 0) {
#pragma unroll
    for (int k = 0; k < KD; k += 32) {
      bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(X + (x0 + r) * ldx + k + 8 * kg);
      bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(Z + (z0 + r) * ldz + k + 8 * kg);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
  } else {
    static_assert(KD % 16 == 0, "contraction must be a multiple of 16");
#pragma unroll
    for (int k = 0; k < KD; k += 16) {
      bf16x4_t a = *reinterpret_cast<const bf16x4_t*>(X + (x0 + r) * ldx + k + 4 * kg);
      bf16x4_t b = *reinterpret_cast<const bf16x4_t*>(Z + (z0 + r) * ldz + k + 4 * kg);
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
    }
  }
  return acc;
}

// Store a tile's 4 accumulator values transposed: lane l holds D[4g+e][c]
// (g = l/16, c = l%16), written to Y[c][4g + e] of a row-major buffer.
template <typename OpT>
__device__ __forceinline__ void store_tile_t(OpT* Y, int ldy, int y_row0, int y_col0,
                                             const float (&v)[4], int lane) {
  OpT* p = Y + (y_row0 + (lane & 15)) * ldy + y_col0 + 4 * (lane >> 4);
  if constexpr (sizeof(OpT) == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    bf16x4_t t = {static_cast<bf16>(v[0]), static_cast<bf16>(v[1]), static_cast<bf16>(v[2]),
                  static_cast<bf16>(v[3])};
    *reinterpret_cast<bf16x4_t*>(p) = t;
  }
}

// Layout of one (b, h, chunk) block of the workspace.
template <typename OpT, int DK, int C>
struct ChunkBlock {
  static constexpr int kKt = 0;                  // [C][DK]  K e^Gamma
  static constexpr int kQt = C * DK;             // [C][DK]  Q e^Gamma
  static constexpr int kKeT = 2 * C * DK;        // [DK][C]  (K e^(Gamma_L - Gamma))^T
  static constexpr int kTb = 3 * C * DK;         // [C][C]   (I + A)^-1 diag(beta)
  static constexpr int kP = 3 * C * DK + C * C;  // [C][C]   lower(Qt Kh^T)
  static constexpr int kOpElems = 3 * C * DK + 2 * C * C;
  static constexpr size_t kGammaByte = static_cast<size_t>(kOpElems) * sizeof(OpT);  // [DK] f32
  static constexpr size_t kBytes = (kGammaByte + DK * sizeof(float) + 15) / 16 * 16;
};

// ---------------------------------------------------------------------------
// chunk_prep
// ---------------------------------------------------------------------------
template <typename OpT, int DK, int C>
struct PrepSmem {
  static constexpr int LDK = DK + pad_of<OpT>();
  static constexpr int LDA = C + 1;  // fp32 [C][C+1] for the solve
  static constexpr int LDP = C + pad_of<OpT>();
  static constexpr int PARTS = kThreads / DK;  // threads per key channel
  static constexpr int RPP = C / PARTS;         // rows per part
  static_assert(kThreads % DK == 0 && C % PARTS == 0 && RPP >= 1, "prep split");
  // The decayed operands and, once they are consumed, the triangular
  // transform share storage.
  static constexpr size_t kOps = 3 * static_cast<size_t>(C) * LDK * sizeof(OpT);
  static constexpr size_t kTm = static_cast<size_t>(C) * LDA * sizeof(float);
  static constexpr size_t kUnion = kOps > kTm ? kOps : kTm;
};

template <typename OpT, int DK, int C>
__global__ __launch_bounds__(kThreads) void chunk_prep_kernel(PrefillArgs a) {
  using Sm = PrepSmem<OpT, DK, C>;
  using Blk = ChunkBlock<OpT, DK, C>;
  constexpr int LDK = Sm::LDK, LDA = Sm::LDA, LDP = Sm::LDP;
  constexpr int PARTS = Sm::PARTS, RPP = Sm::RPP;

  __shared__ __attribute__((aligned(16))) unsigned char u_raw[Sm::kUnion];
  __shared__ float A_s[C * LDA];  // strict-lower beta-scaled key/key terms
  __shared__ __attribute__((aligned(16))) OpT P_s[C * LDP];  // lower(Qt Kh^T)
  __shared__ float inv_nk[C], inv_nq[C], beta_s[C], gsc[C];
  __shared__ float gpart[PARTS][DK];

  OpT* Kt_s = reinterpret_cast<OpT*>(u_raw);
  OpT* Kh_s = Kt_s + C * LDK;
  OpT* Qt_s = Kh_s + C * LDK;
  float* T_s = reinterpret_cast<float*>(u_raw);  // after the operands are consumed

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int NC = (a.T + C - 1) / C;
  const int n = blockIdx.x % NC;
  const int bh = blockIdx.x / NC;
  const int h = bh % a.H_v;
  const int b = bh / a.H_v;
  const int hq = h / (a.H_v / a.H_qk);
  const int t0 = n * C;
  const int L = min(C, a.T - t0);
  const OpT* qg = static_cast<const OpT*>(a.q);
  const OpT* kg = static_cast<const OpT*>(a.k);
  OpT* blk = reinterpret_cast<OpT*>(static_cast<unsigned char*>(a.ws) +
                                    static_cast<size_t>(blockIdx.x) * Blk::kBytes);

  // ---- per-row scalars: L2 norms, beta, scalar gate ----
  for (int r = wave; r < C; r += kThreads / 64) {
    float sk = 0.f, sq = 0.f;
    const bool valid = r < L;
    if (valid && a.l2norm) {
      const size_t base = ((static_cast<size_t>(b) * a.T + t0 + r) * a.H_qk + hq) * DK;
      for (int e = lane; e < DK; e += 64) {
        float x = to_f32(kg[base + e]);
        float y = to_f32(qg[base + e]);
        sk += x * x;
        sq += y * y;
      }
      sk = wave_sum(sk);
      sq = wave_sum(sq);
    }
    if (lane == 0) {
      inv_nk[r] = a.l2norm ? 1.0f / sqrtf(sk + kL2Eps) : 1.0f;
      inv_nq[r] = a.l2norm ? 1.0f / sqrtf(sq + kL2Eps) : 1.0f;
      const size_t gi = (static_cast<size_t>(b) * a.T + t0 + r) * a.H_v + h;
      beta_s[r] = valid ? sigmoidf(a.beta_logit[gi]) : 0.0f;
      float g = 0.0f;
      if (valid && a.gate == GDR_GATE_SCALAR) g = a.gate_in[gi];
      if (valid && a.gate == GDR_GATE_SCALAR_FUSED)
        g = fused_log_decay(a.gate_in[gi], a.A_log[h], a.dt_bias[h]);
      gsc[r] = g;
    }
  }
  __syncthreads();

  // ---- per-channel log-decay prefix sums and decayed operands ----
  const int c = tid % DK;
  const int part = tid / DK;
  const int rlo = part * RPP;
  auto g_at = [&](int r) -> float {
    if (r >= L) return 0.0f;
    if (a.gate == GDR_GATE_CHANNEL)
      return a.gate_in[((static_cast<size_t>(b) * a.T + t0 + r) * a.H_v + h) * DK + c];
    return gsc[r];
  };
  {
    float s = 0.f;
    for (int r = rlo; r < rlo + RPP; ++r) s += g_at(r);
    gpart[part][c] = s;
  }
  __syncthreads();
  float gam = 0.f, total = 0.f;
  for (int p = 0; p < PARTS; ++p) {
    const float x = gpart[p][c];
    if (p < part) gam += x;
    total += x;
  }
  // gam is now Gamma just before row rlo; total is Gamma_L.
  OpT* KeT_g = blk + Blk::kKeT + c * C;
  for (int r = rlo; r < rlo + RPP; ++r) {
    gam += g_at(r);
    float kv = 0.f, qv = 0.f;
    if (r < L) {
      const size_t base = ((static_cast<size_t>(b) * a.T + t0 + r) * a.H_qk + hq) * DK + c;
      kv = to_f32(kg[base]) * inv_nk[r];
      qv = to_f32(qg[base]) * inv_nq[r];
    }
    const float e_pos = expf(gam), e_neg = expf(-gam);
    const OpT kt = from_f32<OpT>(kv * e_pos);
    const OpT qt = from_f32<OpT>(qv * e_pos);
    Kt_s[r * LDK + c] = kt;
    Kh_s[r * LDK + c] = from_f32<OpT>(kv * e_neg);
    Qt_s[r * LDK + c] = qt;
    blk[Blk::kKt + r * DK + c] = kt;
    blk[Blk::kQt + r * DK + c] = qt;
    KeT_g[r] = from_f32<OpT>(kv * expf(total - gam));
  }
  if (part == 0)
    reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(blk) + Blk::kGammaByte)[c] =
        expf(total);
  __syncthreads();

  // ---- A = strict_lower(diag(beta) Kt Kh^T) and P = lower(Qt Kh^T) by MFMA ----
  constexpr int NB = C / 16;
  constexpr int NL = NB * (NB + 1) / 2;  // lower-triangular 16x16 tiles
  for (int job = wave; job < 2 * NL; job += kThreads / 64) {
    const int tl = job % NL;
    int R = 0;
    while ((R + 1) * (R + 2) / 2 <= tl) ++R;
    const int S = tl - R * (R + 1) / 2;
    const bool isP = job >= NL;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = mma_xzt<OpT, DK>(isP ? Qt_s : Kt_s, LDK, 16 * R, Kh_s, LDK, 16 * S, acc, lane);
    const int col = 16 * S + (lane & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * R + 4 * (lane >> 4) + e;
      if (isP)
        P_s[row * LDP + col] = from_f32<OpT>(row >= col ? acc[e] : 0.0f);
      else
        A_s[row * LDA + col] = row > col ? beta_s[row] * acc[e] : 0.0f;
    }
  }
  // Upper tiles of P are zero.
  for (int idx = tid; idx < C * C; idx += kThreads) {
    const int row = idx / C, col = idx % C;
    if ((row >> 4) < (col >> 4)) P_s[row * LDP + col] = from_f32<OpT>(0.0f);
  }
  __syncthreads();  // Kt/Kh/Qt are dead from here; their storage becomes T_s

  // ---- (I + A)^-1 by forward substitution, one column per thread ----
  if (tid < C) {
    const int s = tid;
    for (int r = 0; r < s; ++r) T_s[r * LDA + s] = 0.0f;
    T_s[s * LDA + s] = 1.0f;
    for (int r = s + 1; r < C; ++r) {
      float acc = 0.0f;
      for (int m = s; m < r; ++m) acc += A_s[r * LDA + m] * T_s[m * LDA + s];
      T_s[r * LDA + s] = -acc;
    }
  }
  __syncthreads();

  // ---- write Tb = T diag(beta) and P to the workspace ----
  OpT* Tb_g = blk + Blk::kTb;
  OpT* P_g = blk + Blk::kP;
  for (int idx = tid; idx < C * C; idx += kThreads) {
    const int row = idx / C, col = idx % C;
    Tb_g[idx] = from_f32<OpT>(row >= col ? T_s[row * LDA + col] * beta_s[col] : 0.0f);
    P_g[idx] = P_s[row * LDP + col];
  }
}

// ---------------------------------------------------------------------------
// chunk_carry
// ---------------------------------------------------------------------------
template <typename OpT, int DK, int DVS, int C>
struct CarryShape {
  using Blk = ChunkBlock<OpT, DK, C>;
  static constexpr int P = pad_of<OpT>();
  static constexpr int LDK = DK + P;  // rows of Kt, Qt, St
  static constexpr int LDC = C + P;   // rows of KeT, Tb, P, Rt, Ut
  static constexpr int LDV = DVS + 1;
  static constexpr int NW = kThreads / 64;
  static constexpr int NST = (DK / 16) * (DVS / 16);  // state tiles
  static constexpr int SPW = (NST + NW - 1) / NW;      // state tiles per wave
  static constexpr int NOT = (C / 16) * (DVS / 16);   // output tiles
  static constexpr int OPW = (NOT + NW - 1) / NW;
  static constexpr int kPieces = static_cast<int>(Blk::kBytes / 16);  // 16-byte pieces
  static constexpr int kPF = (kPieces + kThreads - 1) / kThreads;
  static constexpr int kVPer = 16 / static_cast<int>(sizeof(OpT));   // elements per piece
  static constexpr int kVPieces = C * DVS / kVPer;
  static constexpr int kVPF = (kVPieces + kThreads - 1) / kThreads;
  static constexpr size_t kSmem =
      sizeof(OpT) * (2 * C * LDK + DK * LDC + 2 * C * LDC + DVS * LDK + 2 * DVS * LDC) +
      sizeof(float) * (C * LDV + DK);
};

template <typename OpT, int DK, int DVS, int C>
__global__ __launch_bounds__(kThreads) void chunk_carry_kernel(PrefillArgs a) {
  using Sh = CarryShape<OpT, DK, DVS, C>;
  using Blk = typename Sh::Blk;
  constexpr int LDK = Sh::LDK, LDC = Sh::LDC, LDV = Sh::LDV;
  constexpr int SPW = Sh::SPW, OPW = Sh::OPW, NST = Sh::NST, NOT = Sh::NOT;
  constexpr int DVT = DVS / 16;

  __shared__ __attribute__((aligned(16))) OpT Kt_s[C * LDK];
  __shared__ __attribute__((aligned(16))) OpT Qt_s[C * LDK];
  __shared__ __attribute__((aligned(16))) OpT KeT_s[DK * LDC];
  __shared__ __attribute__((aligned(16))) OpT Tb_s[C * LDC];
  __shared__ __attribute__((aligned(16))) OpT P_s[C * LDC];
  __shared__ __attribute__((aligned(16))) OpT St_s[DVS * LDK];
  __shared__ __attribute__((aligned(16))) OpT Rt_s[DVS * LDC];
  __shared__ __attribute__((aligned(16))) OpT Ut_s[DVS * LDC];
  __shared__ float V_s[C * LDV];
  __shared__ __attribute__((aligned(16))) float gam_s[DK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n_sl = a.dv / DVS;

  // XCD-aware order: workgroups w, w+8, w+16, ... run on one XCD (and share its
  // L2); give them consecutive (head, slice) units so that the slices of one
  // head read that head's chunk blocks through the same L2.
  const int G = gridDim.x;
  int unit = blockIdx.x;
  if (G % 8 == 0) unit = (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;
  const int slice = unit % n_sl;
  const int bh = unit / n_sl;
  const int h = bh % a.H_v;
  const int b = bh / a.H_v;
  const int jb = slice * DVS;
  const int NC = (a.T + C - 1) / C;

  const size_t st_off = static_cast<size_t>(bh) * DK * a.dv;
  const unsigned char* ws_head =
      static_cast<const unsigned char*>(a.ws) + static_cast<size_t>(bh) * NC * Blk::kBytes;
  const OpT* vg = static_cast<const OpT*>(a.v);
  OpT* og = static_cast<OpT*>(a.o);

  // ---- state tiles owned by this wave, in accumulator layout ----
  f32x4 sacc[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int t = wave * SPW + i;
    sacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (t < NST && a.state_in) {
      const int I = t / DVT, J = t % DVT;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * I + 4 * (lane >> 4) + e;
        sacc[i][e] = a.state_in[st_off + static_cast<size_t>(row) * a.dv + jb + 16 * J +
                                (lane & 15)];
      }
    }
  }

  // ---- prefetch registers for one chunk block and one V slice ----
  uint4 pf[Sh::kPF];
  uint4 vpf[Sh::kVPF];
  auto fetch = [&](int nn) __attribute__((always_inline)) {
    const uint4* src = reinterpret_cast<const uint4*>(ws_head + static_cast<size_t>(nn) * Blk::kBytes);
#pragma unroll
    for (int i = 0; i < Sh::kPF; ++i) {
      const int piece = tid + i * kThreads;
      if (piece < Sh::kPieces) pf[i] = src[piece];
    }
    const int t0 = nn * C;
#pragma unroll
    for (int i = 0; i < Sh::kVPF; ++i) {
      const int piece = tid + i * kThreads;
      vpf[i] = uint4{0u, 0u, 0u, 0u};
      if (piece < Sh::kVPieces) {
        const int r = piece / (DVS / Sh::kVPer);
        const int col = (piece % (DVS / Sh::kVPer)) * Sh::kVPer;
        if (t0 + r < a.T)
          vpf[i] = *reinterpret_cast<const uint4*>(
              vg + ((static_cast<size_t>(b) * a.T + t0 + r) * a.H_v + h) * a.dv + jb + col);
      }
    }
  };
  auto stage = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < Sh::kPF; ++i) {
      const int piece = tid + i * kThreads;
      if (piece >= Sh::kPieces) continue;
      const int byte = piece * 16;
      unsigned char* dst;
      if (byte < static_cast<int>(Blk::kGammaByte)) {
        const int e = byte / static_cast<int>(sizeof(OpT));
        if (e < Blk::kQt) {
          dst = reinterpret_cast<unsigned char*>(Kt_s + (e / DK) * LDK + e % DK);
        } else if (e < Blk::kKeT) {
          const int f = e - Blk::kQt;
          dst = reinterpret_cast<unsigned char*>(Qt_s + (f / DK) * LDK + f % DK);
        } else if (e < Blk::kTb) {
          const int f = e - Blk::kKeT;
          dst = reinterpret_cast<unsigned char*>(KeT_s + (f / C) * LDC + f % C);
        } else if (e < Blk::kP) {
          const int f = e - Blk::kTb;
          dst = reinterpret_cast<unsigned char*>(Tb_s + (f / C) * LDC + f % C);
        } else {
          const int f = e - Blk::kP;
          dst = reinterpret_cast<unsigned char*>(P_s + (f / C) * LDC + f % C);
        }
      } else {
        const int f = (byte - static_cast<int>(Blk::kGammaByte)) / 4;
        if (f >= DK) continue;  // tail padding of the block
        dst = reinterpret_cast<unsigned char*>(gam_s + f);
      }
      *reinterpret_cast<uint4*>(dst) = pf[i];
    }
#pragma unroll
    for (int i = 0; i < Sh::kVPF; ++i) {
      const int piece = tid + i * kThreads;
      if (piece >= Sh::kVPieces) continue;
      const int r = piece / (DVS / Sh::kVPer);
      const int col = (piece % (DVS / Sh::kVPer)) * Sh::kVPer;
      const OpT* e = reinterpret_cast<const OpT*>(&vpf[i]);
#pragma unroll
      for (int u = 0; u < Sh::kVPer; ++u) V_s[r * LDV + col + u] = to_f32(e[u]);
    }
  };

  if (NC > 0) fetch(0);
  for (int nn = 0; nn < NC; ++nn) {
    const int t0 = nn * C;
    const int L = min(C, a.T - t0);

    // S^T in the operand type, for Kt S and Qt S.
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int t = wave * SPW + i;
      if (t < NST) {
        const int I = t / DVT, J = t % DVT;
        float v[4] = {sacc[i][0], sacc[i][1], sacc[i][2], sacc[i][3]};
        store_tile_t<OpT>(St_s, LDK, 16 * J, 16 * I, v, lane);
      }
    }
    stage();
    __syncthreads();
    if (nn + 1 < NC) fetch(nn + 1);

    // R = V - Kt S  (stored transposed),  O = Qt S (kept in registers).
    f32x4 oacc[OPW];
#pragma unroll
    for (int i = 0; i < OPW; ++i) {
      const int t = wave * OPW + i;
      oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (t < NOT) {
        const int R = t / DVT, J = t % DVT;
        f32x4 ks = {0.f, 0.f, 0.f, 0.f};
        ks = mma_xzt<OpT, DK>(Kt_s, LDK, 16 * R, St_s, LDK, 16 * J, ks, lane);
        oacc[i] = mma_xzt<OpT, DK>(Qt_s, LDK, 16 * R, St_s, LDK, 16 * J, oacc[i], lane);
        float rv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          rv[e] = V_s[(16 * R + 4 * (lane >> 4) + e) * LDV + 16 * J + (lane & 15)] - ks[e];
        store_tile_t<OpT>(Rt_s, LDC, 16 * J, 16 * R, rv, lane);
      }
    }
    __syncthreads();

    // U = Tb R  (stored transposed).
#pragma unroll
    for (int i = 0; i < OPW; ++i) {
      const int t = wave * OPW + i;
      if (t < NOT) {
        const int R = t / DVT, J = t % DVT;
        f32x4 u = {0.f, 0.f, 0.f, 0.f};
        u = mma_xzt<OpT, C>(Tb_s, LDC, 16 * R, Rt_s, LDC, 16 * J, u, lane);
        float uv[4] = {u[0], u[1], u[2], u[3]};
        store_tile_t<OpT>(Ut_s, LDC, 16 * J, 16 * R, uv, lane);
      }
    }
    __syncthreads();

    // O = scale (Qt S + P U) -> o rows of this chunk.
#pragma unroll
    for (int i = 0; i < OPW; ++i) {
      const int t = wave * OPW + i;
      if (t < NOT) {
        const int R = t / DVT, J = t % DVT;
        oacc[i] = mma_xzt<OpT, C>(P_s, LDC, 16 * R, Ut_s, LDC, 16 * J, oacc[i], lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * R + 4 * (lane >> 4) + e;
          if (r < L)
            og[((static_cast<size_t>(b) * a.T + t0 + r) * a.H_v + h) * a.dv + jb + 16 * J +
               (lane & 15)] = from_f32<OpT>(a.scale * oacc[i][e]);
        }
      }
    }
    // S = diag(e^Gamma_L) S + Ke^T U.
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int t = wave * SPW + i;
      if (t < NST) {
        const int I = t / DVT, J = t % DVT;
#pragma unroll
        for (int e = 0; e < 4; ++e) sacc[i][e] *= gam_s[16 * I + 4 * (lane >> 4) + e];
        sacc[i] = mma_xzt<OpT, C>(KeT_s, LDC, 16 * I, Ut_s, LDC, 16 * J, sacc[i], lane);
      }
    }
    __syncthreads();
  }

  // ---- final state ----
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int t = wave * SPW + i;
    if (t < NST) {
      const int I = t / DVT, J = t % DVT;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * I + 4 * (lane >> 4) + e;
        a.state_out[st_off + static_cast<size_t>(row) * a.dv + jb + 16 * J + (lane & 15)] =
            sacc[i][e];
      }
    }
  }
}

// T = 0: state_out = state_in (or zeros).
__global__ void state_copy_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                  size_t n) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    dst[i] = src ? src[i] : 0.0f;
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
template <typename OpT, int DK, int C>
size_t block_bytes() {
  return ChunkBlock<OpT, DK, C>::kBytes;
}

template <typename OpT>
size_t block_bytes_rt(int dk, int chunk) {
#define GDR_BB(DKV, CV) \
  if (dk == DKV && chunk == CV) return block_bytes<OpT, DKV, CV>();
  GDR_BB(16, 16) GDR_BB(16, 32) GDR_BB(16, 64)
  GDR_BB(32, 16) GDR_BB(32, 32) GDR_BB(32, 64)
  GDR_BB(64, 16) GDR_BB(64, 32) GDR_BB(64, 64)
  GDR_BB(128, 16) GDR_BB(128, 32) GDR_BB(128, 64)
#undef GDR_BB
  return 0;
}

constexpr size_t kSmemLimit = 160 * 1024;

// Widest state slice whose carry workgroup fits in LDS and that still gives
// at least `want` workgroups.
template <typename OpT, int DK, int C>
int carry_slice(int units, int dv) {
  constexpr int cand[4] = {128, 64, 32, 16};
  int best = 0;
  for (int dvs : cand) {
    if (dvs > dv) continue;
    size_t smem = 0;
    switch (dvs) {
      case 128: smem = CarryShape<OpT, DK, 128, C>::kSmem; break;
      case 64: smem = CarryShape<OpT, DK, 64, C>::kSmem; break;
      case 32: smem = CarryShape<OpT, DK, 32, C>::kSmem; break;
      default: smem = CarryShape<OpT, DK, 16, C>::kSmem; break;
    }
    if (smem > kSmemLimit) continue;
    best = dvs;
    if (static_cast<long>(units) * (dv / dvs) >= 256) break;
  }
  return best;
}

template <typename OpT, int DK, int DVS, int C>
hipError_t launch_carry(const PrefillArgs& a, hipStream_t stream) {
  if constexpr (CarryShape<OpT, DK, DVS, C>::kSmem > kSmemLimit) {
    return hipErrorInvalidConfiguration;
  } else {
    const unsigned grid = static_cast<unsigned>(a.B) * a.H_v * (a.dv / DVS);
    hipLaunchKernelGGL((chunk_carry_kernel<OpT, DK, DVS, C>), dim3(grid), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
  }
}

template <typename OpT, int DK, int C>
hipError_t launch_dk_c(const PrefillArgs& a, hipStream_t stream) {
  const int NC = (a.T + C - 1) / C;
  const unsigned prep_grid = static_cast<unsigned>(a.B) * a.H_v * NC;
  hipLaunchKernelGGL((chunk_prep_kernel<OpT, DK, C>), dim3(prep_grid), dim3(kThreads), 0, stream,
                     a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int dvs = carry_slice<OpT, DK, C>(a.B * a.H_v, a.dv);
  switch (dvs) {
    case 128: return launch_carry<OpT, DK, 128, C>(a, stream);
    case 64: return launch_carry<OpT, DK, 64, C>(a, stream);
    case 32: return launch_carry<OpT, DK, 32, C>(a, stream);
    case 16: return launch_carry<OpT, DK, 16, C>(a, stream);
    default: return hipErrorInvalidConfiguration;
  }
}

template <typename OpT, int DK>
hipError_t launch_dk(const PrefillArgs& a, hipStream_t stream) {
  switch (a.chunk) {
    case 16: return launch_dk_c<OpT, DK, 16>(a, stream);
    case 32: return launch_dk_c<OpT, DK, 32>(a, stream);
    case 64: return launch_dk_c<OpT, DK, 64>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename OpT>
hipError_t launch_io(const PrefillArgs& a, hipStream_t stream) {
  switch (a.dk) {
    case 16: return launch_dk<OpT, 16>(a, stream);
    case 32: return launch_dk<OpT, 32>(a, stream);
    case 64: return launch_dk<OpT, 64>(a, stream);
    case 128: return launch_dk<OpT, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t prefill_workspace_bytes(int B, int T, int H_v, int dk, int dv, int chunk, int io_bf16) {
  (void)dv;
  if (B <= 0 || T <= 0) return 0;
  const size_t nc = (static_cast<size_t>(T) + chunk - 1) / chunk;
  const size_t bb = io_bf16 ? block_bytes_rt<bf16>(dk, chunk) : block_bytes_rt<float>(dk, chunk);
  return static_cast<size_t>(B) * H_v * nc * bb;
}

hipError_t launch_prefill(const PrefillArgs& a, int io_bf16, hipStream_t stream) {
  if (a.T == 0) {
    const size_t n = static_cast<size_t>(a.B) * a.H_v * a.dk * a.dv;
    if (a.state_in == a.state_out || n == 0) return hipSuccess;
    const unsigned grid = static_cast<unsigned>(std::min<size_t>((n + 255) / 256, 4096));
    hipLaunchKernelGGL(state_copy_kernel, dim3(grid), dim3(256), 0, stream, a.state_in,
                       a.state_out, n);
    return hipGetLastError();
  }
  return io_bf16 ? launch_io<bf16>(a, stream) : launch_io<float>(a, stream);
}

}  // namespace gdr
