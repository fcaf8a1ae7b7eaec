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
// Gamma_r = sum_{s<=r} g_s per key channel (non-increasing along the rows,
// since g <= 0) and D_rs = e^(Gamma_r - Gamma_s) per channel:
//   A  = strict_lower(diag(beta) (K K^T o D)),   Tb = (I + A)^-1 diag(beta)
//   P  = lower(Q K^T o D)                        (o D: each product over
//                                                 channel i weighted by D_rs,i)
//   Kt = K e^Gamma, Qt = Q e^Gamma, Ke = K e^(Gamma_L - Gamma)
//   U  = Tb (V - Kt S)                       (the WY pseudo-values minus the
//                                             pseudo-keys applied to S)
//   O  = scale (Qt S + P U)
//   S' = diag(e^Gamma_L) S + Ke^T U
// which is C token updates regrouped exactly.  Every exponent above is <= 0
// in the entries that are used.  How A and P are formed depends on the gate:
//   scalar gate   D is one number per (r, s): the plain products K K^T and
//                 Q K^T on MFMA, each entry times D_rs;
//   channel gate  while the chunk's decay stays moderate (-Gamma_L <= 64 on
//                 every channel), the factorised form (K e^Gamma)(K e^-Gamma)^T
//                 on MFMA; past that, an exact routine that refers each 16x16
//                 tile below the diagonal to the start of its row block (all
//                 exponents <= 0, on MFMA) and sums the diagonal blocks entry
//                 by entry.
//
// Kernels:
//   chunk_prep   one workgroup per (b, h, chunk), all chunks in parallel:
//                everything that does not depend on S -- Kt, Qt, Ke^T, Tb, P
//                and e^Gamma_L -- written to the caller's workspace, one
//                disjoint block per (b, h, chunk).  With a scalar gate Kt
//                and Qt are row scalings: the block holds the row factors
//                instead, and the normalised k and q rows go once per
//                (b, qk head, chunk) to a region of their own.
//   chunk_carry  one workgroup per (b, h, slice of DVS state columns), walking
//                the chunks in order with its state slice held in MFMA
//                accumulators; the columns of S are independent, so slices
//                need no communication.  Operand fragments go straight from
//                the workspace into registers: as soon as a phase has used
//                its fragments, the same registers load that phase's
//                fragments of the next chunk.
//   carry_scan   for long sequences over few (b, h) units only: the carry is
//                cut into sequence segments whose affine maps (M, N) are
//                formed by the carry side by side, this kernel composes the
//                segments' start states, and the segments then run in
//                parallel (the segmented carry, below).
// Dense products use MFMA (bf16 operands with fp32 accumulation for bf16 io,
// fp32 MFMA for fp32 io); the triangular solve runs in fp32 in LDS.
#include <mutex>
#include <type_traits>

#include "device_common.hpp"
#include "gdr_internal.h"
#include "gdr.h"

namespace gdr {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr float kLog2e = 1.44269504088896340736f;

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

// MFMA fragment of one operand for a contraction of length KD: the 16x16x32
// bf16 form (8 values per lane) when KD is a multiple of 32, 16x16x16 bf16
// (4 values) for KD = 16, 16x16x4 fp32 (1 value) for fp32 operands.  Lane l
// supplies row (l % 16) and k-values step*KS + (l / 16)*VL ... + VL - 1.
template <typename OpT, int KD>
struct FragT {
  static constexpr int KS = sizeof(OpT) == 4 ? 4 : (KD % 32 == 0 ? 32 : 16);
  static constexpr int VL = KS / 4;
  static constexpr int STEPS = KD / KS;
  using T = std::conditional_t<sizeof(OpT) == 4, float,
                               std::conditional_t<KS == 32, bf16x8_t, bf16x4_t>>;
  __device__ static __forceinline__ f32x4 mma(T a, T b, f32x4 c) {
    if constexpr (sizeof(OpT) == 4)
      return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    else if constexpr (KS == 32)
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  // Workspace blocks hold every operand region in fragment order: for each
  // 16-row tile and contraction step, the 64 lanes' VL-element slices back
  // to back, so a fragment is one contiguous read of 64 * VL elements.
  // Slot d (VL elements) holds row slot_row(d) at columns slot_col(d) ...
  // slot_col(d) + VL - 1 of the region.
  __host__ __device__ static constexpr int slot_row(int d) {
    return 16 * (d / (64 * STEPS)) + d % 16;
  }
  __host__ __device__ static constexpr int slot_col(int d) {
    return ((d / 64) % STEPS) * KS + ((d / 16) % 4) * VL;
  }
  // The fragment of rows row0 ... row0 + 15 (row0 a multiple of 16), `step`.
  __device__ static __forceinline__ T load(const OpT* region, int row0, int step, int lane) {
    return *reinterpret_cast<const T*>(region + ((row0 / 16 * STEPS + step) * 64 + lane) * VL);
  }
  // A fragment from a padded row-major LDS buffer.
  __device__ static __forceinline__ T load_pad(const OpT* buf, int ld, int row0, int step,
                                               int lane) {
    return *reinterpret_cast<const T*>(buf + (row0 + (lane & 15)) * ld + step * KS +
                                       (lane >> 4) * VL);
  }
};

// Layout of one (b, h, chunk) block of the workspace.  The operand regions are
// in fragment order (FragT::slot_row / slot_col): Kt and Qt for a
// contraction over DK, the others over C.
//
// kScalarGate (scalar gates): with one decay per row, Kt = diag(e^Gamma) K and
// Qt = diag(e^Gamma) Q are row scalings of the normalised k and q rows, which
// do not depend on the value head.  The block of a value head then leaves Kt
// and Qt out and holds the row factor e^Gamma_r instead (0 on the rows past
// the end of a ragged last chunk); the normalised rows are stored once per
// (b, qk head, chunk) in a QKRegion, and the carry scales its products row by
// row.  With two value heads per qk head that is a quarter fewer bytes.
template <typename OpT, int DK, int C, bool kScalarGate>
struct ChunkBlock {
  static constexpr int kKt = 0;                         // [C][DK] K e^Gamma (channel gates)
  static constexpr int kQt = C * DK;                    // [C][DK] Q e^Gamma (channel gates)
  static constexpr int kKeT = kScalarGate ? 0 : 2 * C * DK;  // [DK][C] (K e^(Gamma_L - Gamma))^T
  static constexpr int kTb = kKeT + C * DK;             // [C][C]  (I + A)^-1 diag(beta)
  static constexpr int kP = kTb + C * C;                // [C][C]  lower(Q K^T o D)
  static constexpr int kOpElems = kP + C * C;
  static constexpr size_t kGammaByte = static_cast<size_t>(kOpElems) * sizeof(OpT);  // [DK] f32
  static constexpr size_t kFacByte = kGammaByte + DK * sizeof(float);  // scalar: e^Gamma [C] f32
  static constexpr size_t kBytes =
      (kFacByte + (kScalarGate ? C * sizeof(float) : 0) + 15) / 16 * 16;
};

// Scalar gates: the normalised k rows and q rows of one (b, qk head, chunk),
// each [C][DK] in fragment order (contraction over DK).
template <typename OpT, int DK, int C>
struct QKRegion {
  static constexpr int kK = 0;
  static constexpr int kQ = C * DK;
  static constexpr size_t kBytes = 2 * static_cast<size_t>(C) * DK * sizeof(OpT);
};

// The workspace is chunk-major: block (b, chunk n, value head h) is number
// (b * NC + n) * H_v + h, and the QKRegion of (b, n, qk head hq) number
// (b * NC + n) * H_qk + hq.  The blocks that one chunk step of the carry reads
// (chunk n of every head) and that neighbouring prep units write then lie
// side by side.
template <typename Blk>
__device__ __forceinline__ size_t block_offset(int b, int n, int h, int NC, int H_v) {
  return ((static_cast<size_t>(b) * NC + n) * H_v + h) * Blk::kBytes;
}

// ---------------------------------------------------------------------------
// chunk_prep
//
// Per (b, h, chunk):
//   1. every global load of the chunk is issued up front (per-thread channel
//      quads of k, q, g over a part of the rows; beta once per row);
//   2. row norms through LDS partial sums;
//   3. per-channel prefix sums (each channel split into row parts, combined
//      through LDS);
//   4. A and P (prep_causal_scalar, prep_causal_factored or
//      prep_causal_exact), computed transposed so that each lane holds four
//      consecutive columns of a row; the carry's operands Kt, Qt and Ke^T,
//      built in fp32 and rounded once into row-major LDS, then copied to the
//      block, consecutive threads writing consecutive lane slices (Ke^T read
//      down the columns of Ke);
//   5. (I + A)^-1 blocked by 16: the diagonal 16x16 blocks by forward
//      substitution in registers (one lane per column), then the off-diagonal
//      blocks level by level, T_ij = -T_ii sum_k A_ik T_kj, with fp32 MFMA;
//   6. Tb = T diag(beta) leaves for the block in coalesced lane slices.
// LDS holds regions that are reused phase by phase (PrepSmem): three with a
// channel gate (three workgroups per CU at dk = 128, C = 64, bf16), two and
// the solve scratch with a scalar gate (four per CU).
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma_f32x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename OpT, int DK, int C, bool kScalarGate = false>
struct PrepSmem {
  static constexpr int LDK = DK + pad_of<OpT>();  // rows of Kt, Kh, Ke, Qt
  static constexpr int LDT = C + 4;               // fp32 A (row-major), T (column-major)
  static constexpr int LDX = 20;                  // fp32 16x16 scratch of the solve
  static constexpr int NB = C / 16;
  // Channel phase: a thread owns a quad of key channels and RPP consecutive
  // rows (one row part); the NQ threads of a part are consecutive lanes.
  static constexpr int NQ = DK / 4;                                    // channel quads
  static constexpr int PARTS = (4 * kThreads / DK) < C ? 4 * kThreads / DK : C;
  static constexpr int NTA = PARTS * NQ;                               // active threads
  static constexpr int RPP = C / PARTS;                                // rows per part
  static_assert(NTA <= kThreads && NTA % 64 == 0 && C % PARTS == 0, "prep split");
  static_assert(NB <= kThreads / 64, "one wave per diagonal block of the solve");
  static constexpr int LDN = 2 * NQ + 1;  // row-norm partials: [C][2 NQ + 1]
  static constexpr size_t al16(size_t x) { return (x + 15) / 16 * 16; }
  static constexpr size_t mx(size_t x, size_t y) { return x > y ? x : y; }
  static constexpr size_t kOpRows = static_cast<size_t>(C) * LDK * sizeof(OpT);
  static constexpr size_t kTm = static_cast<size_t>(C) * LDT * sizeof(float);
  static constexpr size_t kX = 4 * 16 * LDX * sizeof(float);
  static constexpr size_t kN = static_cast<size_t>(C) * LDN * sizeof(float);
  static constexpr size_t kG = static_cast<size_t>(PARTS) * DK * sizeof(float);
  // Channel gates: three regions, each reused as the chunk moves on (a
  // barrier between uses):
  //   R0: row-norm partials -> operand rows (Kt, Qt, K, ...) -> solve scratch
  //   R1: operand rows (Kh, Ke, Q, ...) -> T, column-major
  //   R2: per-part channel sums of the prefix -> A
  // (R0 + R1 also stage the exact routine's fp32 passes.)
  // Scalar gates need only the K and Q rows at once (P goes straight to the
  // block and A waits in registers until the Q rows are dead), so two regions
  // and the solve scratch do: 40,960 bytes in all at dk = 128, C = 64, bf16,
  // which lets four workgroups share a CU instead of three.
  //   R0: row-norm partials -> K rows -> Ke rows -> T, column-major
  //   R1: Q rows -> A
  //   X:  per-part sums of the prefix -> solve scratch
  static constexpr size_t oR0 = 0;
  static constexpr size_t oR1 = al16(mx(mx(kOpRows, kN), kScalarGate ? kTm : kX));
  static constexpr size_t oR2 = oR1 + al16(mx(kOpRows, kTm));
  static constexpr size_t oX = kScalarGate ? oR2 : oR0;  // solve scratch
  static constexpr size_t oT = kScalarGate ? oR0 : oR1;  // T, column-major
  static constexpr size_t oA = kScalarGate ? oR1 : oR2;  // A, row-major
  static constexpr size_t oG = oR2;                      // prefix partials
  static constexpr size_t kBytes = oR2 + al16(kScalarGate ? mx(kX, kG) : mx(kTm, kG));
  static constexpr size_t oBeta = kBytes;  // beta of the chunk's rows
  static constexpr size_t oGam = oBeta + al16(static_cast<size_t>(C) * sizeof(float));  // scalar gate: Gamma per row
  static constexpr size_t oNrm = oGam + al16(static_cast<size_t>(C) * sizeof(float));   // 1/|k|, 1/|q| per row
  static constexpr size_t kAll = oNrm + al16(2 * static_cast<size_t>(C) * sizeof(float));
  // Register arrays of a thread's channel quad over its rows.
  using RowsF = float[RPP][4];
  using RowsOp = OpT[RPP][4];
};

// A half-open range [n0, n1) of chunk indices.
struct ChunkRange {
  int n0, n1;
};

// Element offset of (row, col) in a region held in fragment order.
template <typename OpT, int KD>
__device__ __forceinline__ int frag_off(int row, int col) {
  using F = FragT<OpT, KD>;
  return (((row / 16 * F::STEPS + col / F::KS) * 4 + (col % F::KS) / F::VL) * 16 + row % 16) *
             F::VL +
         col % F::VL;
}

// Store N consecutive values of one row, columns col0 ... col0 + N - 1 (col0 a
// multiple of N), into a region held in fragment order: runs of up to one
// lane slice are contiguous there and go out as single vector stores.
template <typename OpT, int KD, int N>
__device__ __forceinline__ void frag_store(OpT* region, int row, int col0, const OpT (&v)[N]) {
  constexpr int VL = FragT<OpT, KD>::VL;
  constexpr int G = N < VL ? N : VL;
  constexpr int kB = G * static_cast<int>(sizeof(OpT));
  static_assert(kB == 2 || kB == 4 || kB == 8 || kB == 16, "store width");
  using W = std::conditional_t<
      kB == 2, unsigned short,
      std::conditional_t<kB == 4, unsigned, std::conditional_t<kB == 8, uint2, uint4>>>;
#pragma unroll
  for (int j = 0; j < N / G; ++j) {
    W w;
    __builtin_memcpy(&w, &v[j * G], kB);
    *reinterpret_cast<W*>(region + frag_off<OpT, KD>(row, col0 + j * G)) = w;
  }
}

// Copy a ROWS x KD region held row-major in LDS (row pitch ld, rows 16-byte
// aligned) to a block region in fragment order.  Thread t writes slots t,
// t + kThreads, ...: consecutive lanes write consecutive lane slices, so each
// wave store covers one contiguous run of 64 slices (1 KiB in bf16) instead of
// pieces scattered over the fragment layout.
template <typename OpT, int KD, int ROWS>
__device__ __forceinline__ void lds_to_frag(OpT* region, const OpT* src, int ld, int tid) {
  using F = FragT<OpT, KD>;
  using V = typename F::T;
  constexpr int N = ROWS * KD / F::VL;  // slots
#pragma unroll
  for (int i = 0; i < (N + kThreads - 1) / kThreads; ++i) {
    const int d = tid + i * kThreads;
    if (N % kThreads == 0 || d < N) {
      const V v = *reinterpret_cast<const V*>(src + F::slot_row(d) * ld + F::slot_col(d));
      *reinterpret_cast<V*>(region + d * F::VL) = v;
    }
  }
}

// The same for the transpose of a row-major LDS buffer: region row r (of
// ROWS), column c (of KD) is src[c * ld + r].
template <typename OpT, int KD, int ROWS>
__device__ __forceinline__ void lds_to_frag_t(OpT* region, const OpT* src, int ld, int tid) {
  using F = FragT<OpT, KD>;
  using V = typename F::T;
  constexpr int N = ROWS * KD / F::VL;  // slots
#pragma unroll
  for (int i = 0; i < (N + kThreads - 1) / kThreads; ++i) {
    const int d = tid + i * kThreads;
    if (N % kThreads == 0 || d < N) {
      const int r = F::slot_row(d), c = F::slot_col(d);
      OpT v[F::VL];
#pragma unroll
      for (int j = 0; j < F::VL; ++j) v[j] = src[(c + j) * ld + r];
      V w;
      __builtin_memcpy(&w, v, sizeof(V));
      *reinterpret_cast<V*>(region + d * F::VL) = w;
    }
  }
}

// Chunks whose largest per-channel decay over the chunk, -Gamma_L, is at most
// this take the factorised causal terms (Kt Kh^T with Kh = K e^-Gamma, so Kh
// is at most e^64 K and every product stays far inside fp32); chunks with a
// stronger decay on any channel take the exact routine.
constexpr float kFastChunkDecay = 64.0f;

// A thread's rows of its channel quad (registers) to a row-major LDS buffer.
template <typename OpT, int RPP>
__device__ __forceinline__ void rows_to_lds(OpT* dst, int ld, int rlo, int c4,
                                            const OpT (&v)[RPP][4]) {
#pragma unroll
  for (int i = 0; i < RPP; ++i) store_vec4<OpT>(dst + (rlo + i) * ld + 4 * c4, v[i]);
}

// The carry's operands Kt = K e^Gamma, Ke = K e^(Gamma_L - Gamma) and
// Qt = Q e^Gamma, held as the thread's rows, to the block: through LDS rows
// (R0, R1) and coalesced copies (Ke transposed).  R0 and R1 must be free on
// entry and are free again on return.
template <typename OpT, int DK, int C>
__device__ __forceinline__ void emit_carry_operands(
    const typename PrepSmem<OpT, DK, C>::RowsOp& ktr, const typename PrepSmem<OpT, DK, C>::RowsOp& ker,
    const typename PrepSmem<OpT, DK, C>::RowsOp& qtr, int rlo, bool active, int c4, OpT* out,
    unsigned char* sm, int tid) {
  using Sm = PrepSmem<OpT, DK, C>;
  using Blk = ChunkBlock<OpT, DK, C, false>;
  OpT* r0 = reinterpret_cast<OpT*>(sm + Sm::oR0);
  OpT* r1 = reinterpret_cast<OpT*>(sm + Sm::oR1);
  if (active) {
    rows_to_lds<OpT, Sm::RPP>(r0, Sm::LDK, rlo, c4, ktr);
    rows_to_lds<OpT, Sm::RPP>(r1, Sm::LDK, rlo, c4, ker);
  }
  __syncthreads();
  lds_to_frag<OpT, DK, C>(out + Blk::kKt, r0, Sm::LDK, tid);
  lds_to_frag_t<OpT, C, DK>(out + Blk::kKeT, r1, Sm::LDK, tid);
  __syncthreads();
  if (active) rows_to_lds<OpT, Sm::RPP>(r0, Sm::LDK, rlo, c4, qtr);
  __syncthreads();
  lds_to_frag<OpT, DK, C>(out + Blk::kQt, r0, Sm::LDK, tid);
  __syncthreads();
}

// Row and column of lower-triangular 16x16 tile `job` (row-major order over
// the tiles with S <= R).
__device__ __forceinline__ void lower_tile(int job, int& R, int& S) {
  R = 0;
  while ((R + 1) * (R + 2) / 2 <= job) ++R;
  S = job - R * (R + 1) / 2;
}

// Causal terms for a scalar gate (one decay per row): the decays leave the
// contraction, so A and P come from the plain products K K^T and Q K^T on
// MFMA, each entry scaled by e^(Gamma_r - Gamma_s) <= 1 -- exact for any
// decay.  Ke is a per-row scaling with exponents <= 0; Kt and Qt are not
// stored: the block gets the row factor e^Gamma_r, and qk_out (the QKRegion of
// this chunk's qk head, written by the first of its value heads; null for the
// others) the normalised k and q rows.
template <typename OpT, int DK, int C>
__device__ __forceinline__ void prep_causal_scalar(
    const typename PrepSmem<OpT, DK, C>::RowsF& kq, const typename PrepSmem<OpT, DK, C>::RowsF& qq,
    const typename PrepSmem<OpT, DK, C>::RowsF& gq, float gam0, float total, int L, int rlo,
    bool active, int c4, OpT* out, OpT* qk_out, unsigned char* sm, int tid, int lane, int wave) {
  using Sm = PrepSmem<OpT, DK, C, true>;
  using Blk = ChunkBlock<OpT, DK, C, true>;
  constexpr int LDK = Sm::LDK, LDT = Sm::LDT, NB = Sm::NB, RPP = Sm::RPP;
  OpT* Kr_s = reinterpret_cast<OpT*>(sm + Sm::oR0);  // K rows as given, then the Ke rows
  OpT* Qr_s = reinterpret_cast<OpT*>(sm + Sm::oR1);  // Q rows as given
  float* A_s = reinterpret_cast<float*>(sm + Sm::oA);  // where the Q rows were
  float* gam_s = reinterpret_cast<float*>(sm + Sm::oGam);
  const float* beta_s = reinterpret_cast<const float*>(sm + Sm::oBeta);

  OpT ker[RPP][4];
  if (active) {
    float gam = gam0;
#pragma unroll
    for (int i = 0; i < RPP; ++i) {
      const int r = rlo + i;
      gam += gq[i][0];
      const float ef = __builtin_amdgcn_exp2f((total - gam) * kLog2e);
      OpT kr[4], qr[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        kr[u] = from_f32<OpT>(kq[i][u]);
        qr[u] = from_f32<OpT>(qq[i][u]);
        ker[i][u] = from_f32<OpT>(kq[i][u] * ef);
      }
      store_vec4<OpT>(Kr_s + r * LDK + 4 * c4, kr);
      store_vec4<OpT>(Qr_s + r * LDK + 4 * c4, qr);
      if (c4 == 0) gam_s[r] = gam;
    }
  }
  __syncthreads();
  if (tid < C) {
    float* fac = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(out) + Blk::kFacByte);
    fac[tid] = tid < L ? __builtin_amdgcn_exp2f(gam_s[tid] * kLog2e) : 0.0f;
  }
  if (qk_out) {
    lds_to_frag<OpT, DK, C>(qk_out + QKRegion<OpT, DK, C>::kK, Kr_s, LDK, tid);
    lds_to_frag<OpT, DK, C>(qk_out + QKRegion<OpT, DK, C>::kQ, Qr_s, LDK, tid);
  }

  // Lower tiles: A and P of a tile by one wave, computed transposed (each
  // lane holds four consecutive columns of one row) with one shared decay
  // factor per entry; tiles above the diagonal of P are zeros.  P goes
  // straight to the block; a wave's A tiles stay in registers until the Q
  // rows are dead.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  constexpr int NW = kThreads / 64;
  constexpr int NL = NB * (NB + 1) / 2;
  constexpr int NJ = (NL + NW - 1) / NW;  // lower tiles per wave, at most
  float av[NJ][4];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int job = wv + j * NW;
    if (job < NL) {
      int R, S;
      lower_tile(job, R, S);
      f32x4 ga = {0.f, 0.f, 0.f, 0.f}, gp = {0.f, 0.f, 0.f, 0.f};
      ga = mma_xzt<OpT, DK>(Kr_s, LDK, 16 * S, Kr_s, LDK, 16 * R, ga, lane);
      gp = mma_xzt<OpT, DK>(Kr_s, LDK, 16 * S, Qr_s, LDK, 16 * R, gp, lane);
      const int row = 16 * R + (lane & 15);
      const int col = 16 * S + 4 * (lane >> 4);
      const float gr = gam_s[row], br = beta_s[row];
      OpT pv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = col + e;
        const float f = row >= c ? __builtin_amdgcn_exp2f((gr - gam_s[c]) * kLog2e) : 0.0f;
        av[j][e] = row > c ? br * f * ga[e] : 0.0f;
        pv[e] = from_f32<OpT>(f * gp[e]);
      }
      frag_store<OpT, C, 4>(out + Blk::kP, row, col, pv);
    }
  }
  for (int job = wv; job < NB * NB; job += kThreads / 64) {
    const int R = job / NB, S = job % NB;
    if (S > R) {
      const OpT z[4] = {from_f32<OpT>(0.f), from_f32<OpT>(0.f), from_f32<OpT>(0.f),
                        from_f32<OpT>(0.f)};
      frag_store<OpT, C, 4>(out + Blk::kP, 16 * R + (lane & 15), 16 * S + 4 * (lane >> 4), z);
    }
  }
  __syncthreads();  // K and Q rows are dead: A where the Q rows were, Ke^T through R0
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int job = wv + j * NW;
    if (job < NL) {
      int R, S;
      lower_tile(job, R, S);
      const int row = 16 * R + (lane & 15);
      const int col = 16 * S + 4 * (lane >> 4);
      *reinterpret_cast<float4*>(A_s + row * LDT + col) =
          make_float4(av[j][0], av[j][1], av[j][2], av[j][3]);
    }
  }
  if (active) rows_to_lds<OpT, RPP>(Kr_s, LDK, rlo, c4, ker);
  __syncthreads();
  lds_to_frag_t<OpT, C, DK>(out + Blk::kKeT, Kr_s, LDK, tid);
  __syncthreads();
}

// Causal terms for a channel gate whose chunk decays by at most
// kFastChunkDecay on every channel: factorised as Kt Kh^T and Qt Kh^T with
// Kt = K e^Gamma, Qt = Q e^Gamma and Kh = K e^-Gamma, two exponentials per
// key element.  Kt goes to LDS for A and to the block; Qt replaces it for P;
// Ke = Kh e^Gamma_L replaces Kh once P is done.  `strong`: this thread's
// channels decay by more over the chunk.  The workgroup votes at the barrier
// after the operand rows; if any thread is strong the routine stops there
// (the rows only went to LDS) and returns false: the chunk is then left to
// prep_causal_exact.
template <typename OpT, int DK, int C>
__device__ __forceinline__ bool prep_causal_factored(
    const typename PrepSmem<OpT, DK, C>::RowsF& kq, const typename PrepSmem<OpT, DK, C>::RowsF& qq,
    const typename PrepSmem<OpT, DK, C>::RowsF& gq, const float (&gam0)[4],
    const float (&total)[4], bool strong, int rlo, bool active, int c4, OpT* out,
    unsigned char* sm, int tid, int lane, int wave) {
  using Sm = PrepSmem<OpT, DK, C>;
  using Blk = ChunkBlock<OpT, DK, C, false>;
  constexpr int LDK = Sm::LDK, LDT = Sm::LDT, NB = Sm::NB, RPP = Sm::RPP;
  OpT* Kt_s = reinterpret_cast<OpT*>(sm + Sm::oR0);
  OpT* Qt_s = Kt_s;  // once A is done
  OpT* Kh_s = reinterpret_cast<OpT*>(sm + Sm::oR1);
  OpT* Ke_s = Kh_s;  // once P is done
  float* A_s = reinterpret_cast<float*>(sm + Sm::oR2);
  const float* beta_s = reinterpret_cast<const float*>(sm + Sm::oBeta);

  OpT qtr[RPP][4], ker[RPP][4];
  if (active) {
    float eL[4], gam[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      eL[u] = __builtin_amdgcn_exp2f(total[u] * kLog2e);
      gam[u] = gam0[u];
    }
#pragma unroll
    for (int i = 0; i < RPP; ++i) {
      const int r = rlo + i;
      OpT kt[4], kh[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        gam[u] += gq[i][u];
        // e^(+-x) as 2^(+-x log2 e): one scaling serves both signs.
        const float x = gam[u] * kLog2e;
        const float e_pos = __builtin_amdgcn_exp2f(x), e_neg = __builtin_amdgcn_exp2f(-x);
        kt[u] = from_f32<OpT>(kq[i][u] * e_pos);
        kh[u] = from_f32<OpT>(kq[i][u] * e_neg);
        qtr[i][u] = from_f32<OpT>(qq[i][u] * e_pos);
        ker[i][u] = from_f32<OpT>(kq[i][u] * (e_neg * eL[u]));
      }
      store_vec4<OpT>(Kt_s + r * LDK + 4 * c4, kt);
      store_vec4<OpT>(Kh_s + r * LDK + 4 * c4, kh);
    }
  }
  // The vote is the barrier; readfirstlane tells the compiler that its
  // result is the same in every lane (so that the two routines sit on the
  // two sides of a plain branch, not in sequence).
  if (__builtin_amdgcn_readfirstlane(__syncthreads_or(strong)) != 0) return false;

  // A = strict_lower(diag(beta) Kt Kh^T), one lower 16x16 tile per job,
  // computed transposed (Kh Kt^T): each lane then holds four consecutive
  // columns of one row of A, one 16-byte LDS store.
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // jobs are wave-uniform
  constexpr int NL = NB * (NB + 1) / 2;
  for (int job = wv; job < NL; job += kThreads / 64) {
    int R, S;
    lower_tile(job, R, S);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = mma_xzt<OpT, DK>(Kh_s, LDK, 16 * S, Kt_s, LDK, 16 * R, acc, lane);
    const int row = 16 * R + (lane & 15);
    const int col = 16 * S + 4 * (lane >> 4);
    const float br = beta_s[row];
    *reinterpret_cast<float4*>(A_s + row * LDT + col) =
        make_float4(row > col ? br * acc[0] : 0.0f, row > col + 1 ? br * acc[1] : 0.0f,
                    row > col + 2 ? br * acc[2] : 0.0f, row > col + 3 ? br * acc[3] : 0.0f);
  }
  lds_to_frag<OpT, DK, C>(out + Blk::kKt, Kt_s, LDK, tid);
  __syncthreads();  // Kt is dead: its storage takes Qt
  if (active) rows_to_lds<OpT, RPP>(Qt_s, LDK, rlo, c4, qtr);
  __syncthreads();

  // P = lower(Qt Kh^T), transposed like A, straight to the block in fragment
  // order; tiles above the diagonal are written as zeros.
  for (int job = wv; job < NB * NB; job += kThreads / 64) {
    const int R = job / NB, S = job % NB;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (S <= R) acc = mma_xzt<OpT, DK>(Kh_s, LDK, 16 * S, Qt_s, LDK, 16 * R, acc, lane);
    const int row = 16 * R + (lane & 15);
    const int col = 16 * S + 4 * (lane >> 4);
    OpT v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = from_f32<OpT>(row >= col + e ? acc[e] : 0.0f);
    frag_store<OpT, C, 4>(out + Blk::kP, row, col, v);
  }
  lds_to_frag<OpT, DK, C>(out + Blk::kQt, Qt_s, LDK, tid);
  __syncthreads();  // Kh and Qt are dead: Ke takes Kh's storage
  if (active) rows_to_lds<OpT, RPP>(Ke_s, LDK, rlo, c4, ker);
  __syncthreads();
  lds_to_frag_t<OpT, C, DK>(out + Blk::kKeT, Ke_s, LDK, tid);
  __syncthreads();
  return true;
}

// Staging of the exact routine: the channels go in passes of KP, each pass
// holding K, Q and Gamma of every row of the chunk in fp32 LDS (R0 + R1).
template <typename OpT, int DK, int C>
struct ExactPass {
  using Sm = PrepSmem<OpT, DK, C>;
  static constexpr bool fits(int kp) { return 3 * C * (kp + 4) * 4 <= static_cast<int>(Sm::oR2); }
  static constexpr int KP = DK < 32 ? DK : (fits(32) ? 32 : 16);
  static constexpr int LDP = KP + 4;
  static constexpr int NPASS = DK / KP;
  static constexpr int NB = C / 16;
  static constexpr int NOFF = NB * (NB - 1) / 2;              // tiles below the diagonal
  static constexpr int JPW = NOFF > 0 ? (NOFF + 3) / 4 : 1;    // of them per wave
  static constexpr int NDE = NB * 136;                          // diagonal-block entries, r >= s
  static constexpr int EPT = (NDE + kThreads - 1) / kThreads;   // of them per thread
  static constexpr int LDPB = C + pad_of<OpT>();                // P staged row-major in LDS
  static_assert(fits(KP), "pass staging fits R0 + R1");
  static_assert(static_cast<size_t>(C) * LDPB * sizeof(OpT) <= Sm::oR2, "P staging fits R0 + R1");
  static_assert(KP % 4 == 0 && DK % KP == 0, "pass width");
};

// The lane's MFMA fragment (contraction over a pass's KP channels) of the 16
// rows row0 ... row0 + 15: X[row][ch] e^(sgn (G[row][ch] - E[ch])), where E
// is the reference row of Gamma; sgn = +1 for rows at or after the reference
// row, -1 for rows at or before it, so that the exponent is <= 0.  With two
// sources the exponential is shared.
template <typename OpT, int KP, int LDP, int NSRC>
__device__ __forceinline__ void exact_frags(const float* X0, const float* X1, const float* G,
                                            const float* E, int row0, int step, int lane,
                                            float sgn, typename FragT<OpT, KP>::T (&f)[NSRC]) {
  using F = FragT<OpT, KP>;
  const int row = row0 + (lane & 15);
  const int ch0 = step * F::KS + (lane >> 4) * F::VL;
  OpT v0[F::VL], v1[F::VL];
#pragma unroll
  for (int j = 0; j < F::VL; ++j) {
    const int ch = ch0 + j;
    const float d = __builtin_amdgcn_exp2f(sgn * (G[row * LDP + ch] - E[ch]) * kLog2e);
    v0[j] = from_f32<OpT>(X0[row * LDP + ch] * d);
    if constexpr (NSRC > 1) v1[j] = from_f32<OpT>(X1[row * LDP + ch] * d);
  }
  __builtin_memcpy(&f[0], v0, sizeof(f[0]));
  if constexpr (NSRC > 1) __builtin_memcpy(&f[1], v1, sizeof(f[1]));
}

// Entry `idx` (< NB * 136) of the diagonal 16x16 blocks, r >= s, as absolute
// chunk rows.
__device__ __forceinline__ void diag_entry(int idx, int& r, int& s) {
  const int blk = idx / 136, loc = idx % 136;
  int rl = 0;
  while ((rl + 1) * (rl + 2) / 2 <= loc) ++rl;
  r = 16 * blk + rl;
  s = 16 * blk + loc - rl * (rl + 1) / 2;
}

// k, q (normalised with the 1/norms in nrm_s, io dtype widened to fp32) and
// g of the thread's channel quad at chunk row r, read again from the inputs;
// zero past the chunk's end.
template <typename OpT, int DK>
__device__ __forceinline__ void reload_quad_row(const PrefillArgs& a, size_t qk_row0,
                                                size_t g_row0, int L, int r, int c4, bool live,
                                                const float* nrm_s, float (&k4)[4],
                                                float (&q4)[4], float (&g4)[4]) {
  const int rr = min(r, L - 1);
  const size_t off = (qk_row0 + static_cast<size_t>(rr) * a.H_qk) * DK + 4 * c4;
  load_row<OpT, 4>(static_cast<const OpT*>(a.k) + off, k4);
  load_row<OpT, 4>(static_cast<const OpT*>(a.q) + off, q4);
  const size_t gi = g_row0 + static_cast<size_t>(rr) * a.H_v;
  load_row<float, 4>(a.gate_in + gi * DK + 4 * c4, g4);
  live = live && r < L;
  const float nk = live ? nrm_s[2 * r] : 0.0f, nq = live ? nrm_s[2 * r + 1] : 0.0f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    k4[u] *= nk;
    q4[u] *= nq;
    g4[u] = live ? g4[u] : 0.0f;
  }
}

// Causal terms for a channel gate with a strong decay somewhere in the chunk:
// exact, with every exponent <= 0.  Per pass of KP channels (fp32 K, Q and
// Gamma of all rows staged in LDS by the threads whose channel quads lie in
// the pass, read again from the inputs so that nothing of the chunk is held
// in registers across the passes):
//   - the tiles below the diagonal, (R, S < R), on MFMA, referred to the end
//     of row block R - 1: E = Gamma at row 16R - 1, rows r of block R scaled
//     by e^(Gamma_r - E) and rows s < 16R by e^(E - Gamma_s);
//   - the diagonal 16x16 blocks entry by entry, with e^(Gamma_r - Gamma_s).
// A and P are accumulated over the passes in registers, then written to A_s
// and, through a row-major LDS tile, to the block.
template <typename OpT, int DK, int C>
__device__ __forceinline__ void prep_causal_exact(const PrefillArgs& a, size_t qk_row0,
                                                  size_t g_row0, int L, const float (&gam0)[4],
                                                  const float (&total)[4], int rlo, bool active,
                                                  int c4, OpT* out, unsigned char* sm, int tid,
                                                  int lane, int wave) {
  using Sm = PrepSmem<OpT, DK, C>;
  using Blk = ChunkBlock<OpT, DK, C, false>;
  using X = ExactPass<OpT, DK, C>;
  using F = FragT<OpT, X::KP>;
  constexpr int LDT = Sm::LDT, RPP = Sm::RPP, KP = X::KP, LDP = X::LDP;
  float* Kp = reinterpret_cast<float*>(sm + Sm::oR0);  // [C][LDP] per pass
  float* Qp = Kp + C * LDP;
  float* Gp = Qp + C * LDP;
  float* A_s = reinterpret_cast<float*>(sm + Sm::oR2);
  const float* beta_s = reinterpret_cast<const float*>(sm + Sm::oBeta);
  const float* nrm_s = reinterpret_cast<const float*>(sm + Sm::oNrm);
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  f32x4 accA[X::JPW], accP[X::JPW];
#pragma unroll
  for (int j = 0; j < X::JPW; ++j) accA[j] = accP[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dA[X::EPT], dP[X::EPT];
#pragma unroll
  for (int e = 0; e < X::EPT; ++e) dA[e] = dP[e] = 0.0f;

#pragma unroll 1
  for (int pass = 0; pass < X::NPASS; ++pass) {
    // the threads whose channel quad lies in this pass stage their rows
    if (active && (4 * c4) / KP == pass) {
      const int cc = 4 * c4 - pass * KP;
      float g[4] = {gam0[0], gam0[1], gam0[2], gam0[3]};
#pragma unroll 2
      for (int i = 0; i < RPP; ++i) {
        const int r = rlo + i;
        float k4[4], q4[4], g4[4];
        reload_quad_row<OpT, DK>(a, qk_row0, g_row0, L, r, c4, true, nrm_s, k4, q4, g4);
#pragma unroll
        for (int u = 0; u < 4; ++u) g[u] += g4[u];
        *reinterpret_cast<float4*>(Kp + r * LDP + cc) = make_float4(k4[0], k4[1], k4[2], k4[3]);
        *reinterpret_cast<float4*>(Qp + r * LDP + cc) = make_float4(q4[0], q4[1], q4[2], q4[3]);
        *reinterpret_cast<float4*>(Gp + r * LDP + cc) = make_float4(g[0], g[1], g[2], g[3]);
      }
    }
    __syncthreads();
    // tiles below the diagonal, computed transposed as in the other routines
#pragma unroll
    for (int j = 0; j < X::JPW; ++j) {
      const int job = wv + j * (kThreads / 64);
      if (job < X::NOFF) {
        int R = 1, S = job;
        while (S >= R) {
          S -= R;
          ++R;
        }
        const float* E = Gp + (16 * R - 1) * LDP;
#pragma unroll
        for (int st = 0; st < F::STEPS; ++st) {
          typename F::T zc[1], zr[2];
          exact_frags<OpT, KP, LDP, 1>(Kp, nullptr, Gp, E, 16 * S, st, lane, -1.0f, zc);
          exact_frags<OpT, KP, LDP, 2>(Kp, Qp, Gp, E, 16 * R, st, lane, 1.0f, zr);
          accA[j] = F::mma(zc[0], zr[0], accA[j]);
          accP[j] = F::mma(zc[0], zr[1], accP[j]);
        }
      }
    }
    // diagonal blocks, entry by entry
#pragma unroll
    for (int e = 0; e < X::EPT; ++e) {
      const int idx = tid + e * kThreads;
      if (idx < X::NDE) {
        int r, s;
        diag_entry(idx, r, s);
        float sa = 0.f, sp = 0.f;
#pragma unroll 2
        for (int ch = 0; ch < KP; ch += 4) {
          const float4 kr = *reinterpret_cast<const float4*>(Kp + r * LDP + ch);
          const float4 qr = *reinterpret_cast<const float4*>(Qp + r * LDP + ch);
          const float4 gr = *reinterpret_cast<const float4*>(Gp + r * LDP + ch);
          const float4 ks = *reinterpret_cast<const float4*>(Kp + s * LDP + ch);
          const float4 gs = *reinterpret_cast<const float4*>(Gp + s * LDP + ch);
          const float kra[4] = {kr.x, kr.y, kr.z, kr.w}, qra[4] = {qr.x, qr.y, qr.z, qr.w};
          const float gra[4] = {gr.x, gr.y, gr.z, gr.w}, ksa[4] = {ks.x, ks.y, ks.z, ks.w};
          const float gsa[4] = {gs.x, gs.y, gs.z, gs.w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float t = ksa[u] * __builtin_amdgcn_exp2f((gra[u] - gsa[u]) * kLog2e);
            sa += kra[u] * t;
            sp += qra[u] * t;
          }
        }
        dA[e] += sa;
        dP[e] += sp;
      }
    }
    __syncthreads();  // the next pass overwrites the staging
  }

  // A to A_s (times beta of the row, strictly below the diagonal); P row-major
  // into LDS (zeros above the diagonal), then to the block in fragment order.
  OpT* Pb = reinterpret_cast<OpT*>(sm + Sm::oR0);
  for (int i = tid; i < C * C; i += kThreads) {
    const int r = i / C, c = i % C;
    if (c > r) {
      Pb[r * X::LDPB + c] = from_f32<OpT>(0.0f);
      if (c / 16 == r / 16) A_s[r * LDT + c] = 0.0f;
    }
  }
#pragma unroll
  for (int j = 0; j < X::JPW; ++j) {
    const int job = wv + j * (kThreads / 64);
    if (job < X::NOFF) {
      int R = 1, S = job;
      while (S >= R) {
        S -= R;
        ++R;
      }
      const int row = 16 * R + (lane & 15);
      const int col = 16 * S + 4 * (lane >> 4);
      const float br = beta_s[row];
      *reinterpret_cast<float4*>(A_s + row * LDT + col) =
          make_float4(br * accA[j][0], br * accA[j][1], br * accA[j][2], br * accA[j][3]);
      const OpT pv[4] = {from_f32<OpT>(accP[j][0]), from_f32<OpT>(accP[j][1]),
                         from_f32<OpT>(accP[j][2]), from_f32<OpT>(accP[j][3])};
      store_vec4<OpT>(Pb + row * X::LDPB + col, pv);
    }
  }
#pragma unroll
  for (int e = 0; e < X::EPT; ++e) {
    const int idx = tid + e * kThreads;
    if (idx < X::NDE) {
      int r, s;
      diag_entry(idx, r, s);
      A_s[r * LDT + s] = r > s ? beta_s[r] * dA[e] : 0.0f;
      Pb[r * X::LDPB + s] = from_f32<OpT>(dP[e]);
    }
  }
  __syncthreads();
  lds_to_frag<OpT, C, C>(out + Blk::kP, Pb, X::LDPB, tid);
  __syncthreads();

  // Kt, Ke and Qt: exponents Gamma and Gamma_L - Gamma, both <= 0.  Kt and
  // Ke rows go to LDS row by row; Qt waits in registers.
  constexpr int LDK = Sm::LDK;
  OpT* Kt_s = reinterpret_cast<OpT*>(sm + Sm::oR0);
  OpT* Ke_s = reinterpret_cast<OpT*>(sm + Sm::oR1);
  OpT qtr[RPP][4];
  if (active) {
    float g[4] = {gam0[0], gam0[1], gam0[2], gam0[3]};
#pragma unroll
    for (int i = 0; i < RPP; ++i) {
      const int r = rlo + i;
      float k4[4], q4[4], g4[4];
      reload_quad_row<OpT, DK>(a, qk_row0, g_row0, L, r, c4, true, nrm_s, k4, q4, g4);
      OpT kt[4], ke[4], qt[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        g[u] += g4[u];
        const float ep = __builtin_amdgcn_exp2f(g[u] * kLog2e);
        const float ef = __builtin_amdgcn_exp2f((total[u] - g[u]) * kLog2e);
        kt[u] = from_f32<OpT>(k4[u] * ep);
        ke[u] = from_f32<OpT>(k4[u] * ef);
        qt[u] = from_f32<OpT>(q4[u] * ep);
      }
      store_vec4<OpT>(Kt_s + r * LDK + 4 * c4, kt);
      store_vec4<OpT>(Ke_s + r * LDK + 4 * c4, ke);
#pragma unroll
      for (int u = 0; u < 4; ++u) qtr[i][u] = qt[u];
    }
  }
  __syncthreads();
  lds_to_frag<OpT, DK, C>(out + Blk::kKt, Kt_s, LDK, tid);
  lds_to_frag_t<OpT, C, DK>(out + Blk::kKeT, Ke_s, LDK, tid);
  __syncthreads();
  if (active) rows_to_lds<OpT, RPP>(Kt_s, LDK, rlo, c4, qtr);
  __syncthreads();
  lds_to_frag<OpT, DK, C>(out + Blk::kQt, Kt_s, LDK, tid);
  __syncthreads();
}

// kChannel: per-channel log-decays (one per key channel and row); otherwise one
// per row (plain or fused), broadcast over the channels.
// One work unit (b, h, chunk) per workgroup, over the chunks of cr; wg is the
// workgroup's index among the G that do this work, and sm its LDS (kAll bytes).
template <typename OpT, int DK, int C, bool kChannel>
__device__ __forceinline__ void prep_body(const PrefillArgs& a, ChunkRange cr, int wg, int G,
                                          unsigned char* sm) {
  using Sm = PrepSmem<OpT, DK, C, !kChannel>;
  using Blk = ChunkBlock<OpT, DK, C, !kChannel>;
  constexpr int LDT = Sm::LDT, LDX = Sm::LDX, NB = Sm::NB;
  constexpr int PARTS = Sm::PARTS, RPP = Sm::RPP;

  float* beta_s = reinterpret_cast<float*>(sm + Sm::oBeta);

  float* X_s = reinterpret_cast<float*>(sm + Sm::oX);    // solve scratch
  float* TT_s = reinterpret_cast<float*>(sm + Sm::oT);   // T column-major: TT[s][r] = T[r][s]
  float* gpart = reinterpret_cast<float*>(sm + Sm::oG);  // [PARTS][DK]
  float* A_s = reinterpret_cast<float*>(sm + Sm::oA);    // A row-major

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int NC = (a.T + C - 1) / C;
  const int NCr = cr.n1 - cr.n0;
  // Work order: every value head of one (b, chunk) is a run of consecutive
  // units, the rep = H_v / H_qk heads that share a qk head next to each other,
  // and consecutive units run on one XCD (workgroups w, w + 8, ... share an
  // XCD).  One cache line of beta (and of a per-head gate) holds every head's
  // value for a token, and the rep heads read the same q and k rows, so those
  // lines come from HBM about once and from the XCD's L2 after that.
  int unit = wg;
  if (G % 8 == 0) unit = (wg % 8) * (G / 8) + wg / 8;
  const int rep = a.H_v / a.H_qk;
  const int r_in = unit % rep;
  const int hq = (unit / rep) % a.H_qk;
  const int bn = unit / a.H_v;  // b * NCr + (n - n0)
  const int n = cr.n0 + bn % NCr;
  const int b = bn / NCr;
  const int h = hq * rep + r_in;
  const int t0 = n * C;
  const int L = min(C, a.T - t0);
  const OpT* qg = static_cast<const OpT*>(a.q);
  const OpT* kg = static_cast<const OpT*>(a.k);
  unsigned char* blk_bytes =
      static_cast<unsigned char*>(a.ws) + block_offset<Blk>(b, n, h, NC, a.H_v);
  const size_t qk_row0 = (static_cast<size_t>(b) * a.T + t0) * a.H_qk + hq;  // row t0
  const size_t g_row0 = (static_cast<size_t>(b) * a.T + t0) * a.H_v + h;

  // ---- 1. loads: this thread's channel quad over its rows ----
  // Every load of the phase is issued before any value is used: the row
  // loops hold no branch (the gate kind is decided around them) and beta is
  // read by one thread per row afterwards, so all loads are in flight at
  // once.  Rows past the end load a valid row and are then multiplied by zero.
  static_assert(C <= kThreads, "one thread per row reads beta");
  const int c4 = tid % Sm::NQ;
  const int part = tid / Sm::NQ;
  const bool active = part < PARTS;
  const int rlo = active ? part * RPP : 0;
  float kq[RPP][4], qq[RPP][4], gq[RPP][4];
  // beta first: its wait then covers no other load
  const float beta_x =
      tid < C ? a.beta_logit[g_row0 + static_cast<size_t>(min(tid, L - 1)) * a.H_v] : 0.0f;
#pragma unroll
  for (int i = 0; i < RPP; ++i) {
    const int rr = min(rlo + i, L - 1);
    const size_t off = (qk_row0 + static_cast<size_t>(rr) * a.H_qk) * DK + 4 * c4;
    load_row<OpT, 4>(kg + off, kq[i]);
    load_row<OpT, 4>(qg + off, qq[i]);
  }
  if constexpr (kChannel) {
#pragma unroll
    for (int i = 0; i < RPP; ++i) {
      const size_t gi = g_row0 + static_cast<size_t>(min(rlo + i, L - 1)) * a.H_v;
      load_row<float, 4>(a.gate_in + gi * DK + 4 * c4, gq[i]);
    }
  } else {
    float g1[RPP];
#pragma unroll
    for (int i = 0; i < RPP; ++i)
      g1[i] = a.gate_in[g_row0 + static_cast<size_t>(min(rlo + i, L - 1)) * a.H_v];
    if (a.gate == GDR_GATE_SCALAR_FUSED) {
      const float A_log = a.A_log[h], dt_bias = a.dt_bias[h];
#pragma unroll
      for (int i = 0; i < RPP; ++i) g1[i] = fused_log_decay(g1[i], A_log, dt_bias);
    }
#pragma unroll
    for (int i = 0; i < RPP; ++i)
#pragma unroll
      for (int u = 0; u < 4; ++u) gq[i][u] = g1[i];
  }
  if (tid < C) beta_s[tid] = tid < L ? sigmoidf(beta_x) : 0.0f;
#pragma unroll
  for (int i = 0; i < RPP; ++i) {
    const float m = (active && rlo + i < L) ? 1.0f : 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      kq[i][u] *= m;
      qq[i][u] *= m;
      gq[i][u] *= m;
    }
  }

  // ---- 2. row L2 norms: each thread leaves its quad's partial sums in LDS,
  //         one thread per row adds them up ----
  float* nrm = reinterpret_cast<float*>(sm + Sm::oR0);  // [C][2 NQ + 1] partials, then 1/norms
  float* nrm_s = reinterpret_cast<float*>(sm + Sm::oNrm);
  if (!a.l2norm && tid < C) {
    nrm_s[2 * tid] = 1.0f;
    nrm_s[2 * tid + 1] = 1.0f;
  }
  if (a.l2norm) {
    if (active) {
#pragma unroll
      for (int i = 0; i < RPP; ++i) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          sk += kq[i][u] * kq[i][u];
          sq += qq[i][u] * qq[i][u];
        }
        nrm[(rlo + i) * Sm::LDN + c4] = sk;
        nrm[(rlo + i) * Sm::LDN + Sm::NQ + c4] = sq;
      }
    }
    __syncthreads();
    if (tid < C) {
      float sk = 0.f, sq = 0.f;
      for (int q = 0; q < Sm::NQ; ++q) {
        sk += nrm[tid * Sm::LDN + q];
        sq += nrm[tid * Sm::LDN + Sm::NQ + q];
      }
      nrm[tid * Sm::LDN] = 1.0f / sqrtf(sk + kL2Eps);
      nrm[tid * Sm::LDN + 1] = 1.0f / sqrtf(sq + kL2Eps);
      // kept for the exact routine, which reads k and q again, and for the
      // scalar gate's row factors
      nrm_s[2 * tid] = nrm[tid * Sm::LDN];
      nrm_s[2 * tid + 1] = nrm[tid * Sm::LDN + 1];
    }
    __syncthreads();
    if (active) {
#pragma unroll
      for (int i = 0; i < RPP; ++i) {
        const float ik = nrm[(rlo + i) * Sm::LDN], iq = nrm[(rlo + i) * Sm::LDN + 1];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          kq[i][u] *= ik;
          qq[i][u] *= iq;
        }
      }
    }
  }

  // ---- 3. per-channel prefix sums: each channel's rows are split into
  //         parts, whose sums are combined through LDS.  gam0: Gamma just
  //         before row rlo; total: Gamma_L, per channel of the thread's quad ----
  OpT* out = reinterpret_cast<OpT*>(blk_bytes);
  float gam0[4] = {0.f, 0.f, 0.f, 0.f}, total[4] = {0.f, 0.f, 0.f, 0.f};
  if (active) {
    float sp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPP; ++i)
#pragma unroll
      for (int u = 0; u < 4; ++u) sp[u] += gq[i][u];
    *reinterpret_cast<float4*>(gpart + part * DK + 4 * c4) = make_float4(sp[0], sp[1], sp[2], sp[3]);
  }
  __syncthreads();
  if (active) {
    for (int p = 0; p < PARTS; ++p) {
      const float4 x = *reinterpret_cast<const float4*>(gpart + p * DK + 4 * c4);
      const float xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (p < part) gam0[u] += xv[u];
        total[u] += xv[u];
      }
    }
    if (part == 0)
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(blk_bytes + Blk::kGammaByte) + 4 * c4) =
          make_float4(expf(total[0]), expf(total[1]), expf(total[2]), expf(total[3]));
  }

  // ---- 4. the causal terms A = strict_lower(diag(beta) (K K^T o D)) and
  //         P = lower(Q K^T o D), D_rs = e^(Gamma_r - Gamma_s) per channel,
  //         into A_s (fp32) and the block; and the carry's operands Kt, Qt,
  //         Ke^T into the block.  Every exponent that these need is <= 0
  //         (Gamma falls along the rows) except in the factorised form, which
  //         is used only where its e^-Gamma stays small ----
  if constexpr (!kChannel) {
    OpT* qk_out = r_in == 0 ? static_cast<OpT*>(a.ws_qk) +
                                  ((static_cast<size_t>(b) * NC + n) * a.H_qk + hq) * (2 * C * DK)
                            : nullptr;
    prep_causal_scalar<OpT, DK, C>(kq, qq, gq, gam0[0], total[0], L, rlo, active, c4, out, qk_out,
                                   sm, tid, lane, wave);
  } else {
    bool strong = false;
#pragma unroll
    for (int u = 0; u < 4; ++u) strong |= active && -total[u] > kFastChunkDecay;
    if (!prep_causal_factored<OpT, DK, C>(kq, qq, gq, gam0, total, strong, rlo, active, c4, out,
                                          sm, tid, lane, wave))
      prep_causal_exact<OpT, DK, C>(a, qk_row0, g_row0, L, gam0, total, rlo, active, c4, out, sm,
                                    tid, lane, wave);
  }

  // ---- 5a. diagonal 16x16 blocks of (I + A)^-1: lane = column ----
  // x_r = -sum_{m<r} A_rm x_m, with four independent partial sums per row
  // and each row of A read as broadcast float4s.
  if (wave < NB && lane < 16) {
    const int o = 16 * wave;
    const int s = lane;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = r == s ? 1.0f : 0.0f;
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      const float* arow = A_s + (o + r) * LDT + o;
      float part_sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m4 = 0; m4 < r; m4 += 4) {
        const float4 av = *reinterpret_cast<const float4*>(arow + m4);
        const float aa[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (m4 + u < r) part_sum[u] += aa[u] * x[m4 + u];
      }
      const float acc = (part_sum[0] + part_sum[1]) + (part_sum[2] + part_sum[3]);
      if (r > s) x[r] = -acc;
    }
    float* col = TT_s + (o + s) * LDT + o;
#pragma unroll
    for (int r = 0; r < 16; r += 4)
      *reinterpret_cast<float4*>(col + r) = make_float4(x[r], x[r + 1], x[r + 2], x[r + 3]);
  }
  __syncthreads();

  // ---- 5b. off-diagonal blocks, by distance from the diagonal ----
#pragma unroll
  for (int d = 1; d < NB; ++d) {
    const int jobs = NB - d;
    const int j = wave, i = wave + d;
    float* Xw = X_s + wave * 16 * LDX;  // column-major 16x16: Xw[c][r]
    if (wave < jobs) {
      // X = sum_{k=j}^{i-1} A_ik T_kj
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int kb = j; kb < i; ++kb) {
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) {
          const float xa = A_s[(16 * i + (lane & 15)) * LDT + 16 * kb + k0 + (lane >> 4)];
          const float zb = TT_s[(16 * j + (lane & 15)) * LDT + 16 * kb + k0 + (lane >> 4)];
          acc = mfma_f32x4(xa, zb, acc);
        }
      }
      *reinterpret_cast<float4*>(Xw + (lane & 15) * LDX + 4 * (lane >> 4)) =
          make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
    __syncthreads();
    if (wave < jobs) {
      // T_ij = -T_ii X
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < 16; k0 += 4) {
        const float xa = TT_s[(16 * i + k0 + (lane >> 4)) * LDT + 16 * i + (lane & 15)];
        const float zb = Xw[(lane & 15) * LDX + k0 + (lane >> 4)];
        acc = mfma_f32x4(xa, zb, acc);
      }
      *reinterpret_cast<float4*>(TT_s + (16 * j + (lane & 15)) * LDT + 16 * i + 4 * (lane >> 4)) =
          make_float4(-acc[0], -acc[1], -acc[2], -acc[3]);
    }
    __syncthreads();
  }

  // ---- 6. Tb = T diag(beta) out, in fragment order ----
  {
    using FC = FragT<OpT, C>;
    using SC = typename FC::T;
    constexpr int VL = FC::VL;
    for (int d = tid; d < C * C / VL; d += kThreads) {
      const int r = FC::slot_row(d), c = FC::slot_col(d);
      OpT v[VL];
#pragma unroll
      for (int u = 0; u < VL; ++u) {
        const int s = c + u;
        v[u] = from_f32<OpT>(r >= s ? TT_s[s * LDT + r] * beta_s[s] : 0.0f);
      }
      *reinterpret_cast<SC*>(out + Blk::kTb + d * VL) = *reinterpret_cast<const SC*>(v);
    }
  }
}

template <typename OpT, int DK, int C, bool kChannel>
__global__ __launch_bounds__(kThreads) void chunk_prep_kernel(PrefillArgs a, ChunkRange cr) {
  __shared__ __attribute__((aligned(16))) unsigned char sm[PrepSmem<OpT, DK, C, !kChannel>::kAll];
  prep_body<OpT, DK, C, kChannel>(a, cr, blockIdx.x, gridDim.x, sm);
}

// ---------------------------------------------------------------------------
// chunk_carry
//
// One workgroup per (b, h, slice of DVS state columns) and chunk range (the
// whole sequence, or one segment of the segmented carry); the slice of S lives
// in MFMA accumulators for the whole range.  Every operand the workspace block
// holds is an A operand of some product, and each wave reads exactly the rows
// of them its tiles need straight from global memory into registers (each
// fragment one contiguous read, the block being in fragment order), ahead of
// their use (scalar gates: the Kt and Qt fragments from the qk head's region
// of normalised rows, the products then scaled row by row).  LDS only
// carries what the waves exchange: S^T, R^T and U^T.  Per chunk, three
// barriers:
//   [B1]  S^T (operand type) written
//   c:    R = V - Kt S (to LDS, transposed), O = Qt S (registers)      [B2]
//   d:    U = Tb R (to LDS, transposed)                                  [B3]
//   e:    O += P U -> o;  S = e^Gamma_L . S + Ke^T U
// ---------------------------------------------------------------------------


// An optional scheduling fence: the compiler does not move instructions across it.
template <bool kOn>
__device__ __forceinline__ void pin_order() {
  if constexpr (kOn) __builtin_amdgcn_sched_barrier(0);
}

template <typename OpT, int DK, int DVS, int C, bool kScalarGate>
struct CarryShape {
  using Blk = ChunkBlock<OpT, DK, C, kScalarGate>;
  using FK = FragT<OpT, DK>;  // contraction over key channels
  using FC = FragT<OpT, C>;   // contraction over the chunk's tokens
  static constexpr int P = pad_of<OpT>();
  static constexpr int LDK = DK + P;  // rows of St
  static constexpr int LDC = C + P;   // rows of Rt, Ut
  // Four waves, one per SIMD, at every width: the output tiles of one row
  // block go to one wave, so each fragment of Kt, Qt, Tb and P is loaded once
  // per workgroup.  With eight waves two of them shared each row block and
  // loaded its fragments twice (B=2, T=4000: 262 -> 242 us per prefill; B=4,
  // T=32767: 2.90 -> 2.82 ms).
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int DVT = DVS / 16;
  static constexpr int NST = (DK / 16) * DVT;         // state tiles
  static constexpr int SPW = (NST + NW - 1) / NW;      // state tiles per wave
  static constexpr int NOT = (C / 16) * DVT;          // output tiles
  static constexpr int OPW = (NOT + NW - 1) / NW;
  static constexpr size_t kSmem = sizeof(OpT) * (DVS * LDK + 2 * DVS * LDC);
  // Keep each next-chunk load where it is written (right after the MFMA that
  // last reads its registers) when a wave owns one output tile; with more the
  // pinned order costs more registers than it saves (64-column slices:
  // 3.8 ms against 3.4 ms at B=4, T=32767, measured with eight waves;
  // 16 columns: 148 us against 166 us unpinned at B=1, T=4000).
  static constexpr bool kPinLoads = OPW == 1;
  // With 16-column slices each o store is a 16 C-byte piece (32 bytes in
  // bf16) of a row that the 8 slices of the head share; written with the
  // non-temporal policy these partial lines go to memory without being
  // allocated in the caches (B=1, T=4000: 150 -> 126 us per prefill).  With
  // wider slices the pieces are 64 bytes or more and plain stores are
  // faster (B=2 and B=4: 1-3%).
  static constexpr bool kNtO = DVS == 16;
};

// What a carry workgroup computes over its chunk range:
//   kCarryFull  the o rows and the final state, from the given start state;
//   kCarryMapN  the final state only, from a zero start state: the constant
//               part N of the range's affine map S_out = M S_in + N;
//   kCarryMapM  the final state only, from the identity (dk columns) with
//               V = 0: the linear part M.  Neither map reads Qt or P or
//               writes o.
enum CarryMode { kCarryFull = 0, kCarryMapN = 1, kCarryMapM = 2 };

template <typename OpT, int DK, int DVS, int C, bool kScalarGate>
struct CarryFrags {
  using Sh = CarryShape<OpT, DK, DVS, C, kScalarGate>;
  typename Sh::FK::T kt[Sh::OPW][Sh::FK::STEPS], qt[Sh::OPW][Sh::FK::STEPS];
  typename Sh::FC::T tb[Sh::OPW][Sh::FC::STEPS], p[Sh::OPW][Sh::FC::STEPS];
  typename Sh::FC::T ke[Sh::SPW][Sh::FC::STEPS];
  OpT v[Sh::OPW][4];  // as loaded (widened to fp32 where used, so the load is not waited for early)
  float gam[Sh::SPW][4];
  float fk[Sh::OPW][4];  // scalar gates: e^Gamma of the four rows of each output tile of the lane
  float fq[Sh::OPW];     // scalar gates: e^Gamma of the output row this lane stores
};

// kScalarGate: the QKRegion of chunk nn of (b, qk head hq).
template <typename OpT, int DK, int C>
__device__ __forceinline__ const OpT* qk_region(const PrefillArgs& a, int b, int hq, int nn) {
  const int NC = (a.T + C - 1) / C;
  return static_cast<const OpT*>(a.ws_qk) +
         ((static_cast<size_t>(b) * NC + nn) * a.H_qk + hq) * (2 * C * DK);
}

// kScalarGate: the row factors e^Gamma of output tile row-block R in accumulator
// layout (rows 16 R + 4 (lane / 16) ... + 3) from the block at blk.
template <typename OpT, int DK, int DVS, int C, bool kScalarGate>
__device__ __forceinline__ void carry_load_fk(CarryFrags<OpT, DK, DVS, C, kScalarGate>& F,
                                              const OpT* blk, int i, int R, int lane) {
  using Blk = typename CarryShape<OpT, DK, DVS, C, kScalarGate>::Blk;
  const float* fac =
      reinterpret_cast<const float*>(reinterpret_cast<const unsigned char*>(blk) + Blk::kFacByte);
  const float4 f4 = *reinterpret_cast<const float4*>(fac + 16 * R + 4 * (lane >> 4));
  F.fk[i][0] = f4.x;
  F.fk[i][1] = f4.y;
  F.fk[i][2] = f4.z;
  F.fk[i][3] = f4.w;
}

// kScalarGate: the row factor e^Gamma of output row 16 R + lane % 16 (the row this
// lane stores).
template <typename OpT, int DK, int DVS, int C, bool kScalarGate>
__device__ __forceinline__ void carry_load_fq(CarryFrags<OpT, DK, DVS, C, kScalarGate>& F,
                                              const OpT* blk, int i, int R, int lane) {
  using Blk = typename CarryShape<OpT, DK, DVS, C, kScalarGate>::Blk;
  const float* fac =
      reinterpret_cast<const float*>(reinterpret_cast<const unsigned char*>(blk) + Blk::kFacByte);
  F.fq[i] = fac[16 * R + (lane & 15)];
}

// Issue the loads of chunk nn's fragments for this wave's tiles, by phase:
// phase c needs Kt, Qt and V; phase d Tb; phase e P, Ke^T and e^Gamma_L.
// Where the loop pins its reloads (kPinLoads), each load here is fenced in
// place too, so that these first loads go out in the order the chunk loop
// issues its reloads: the compiler's wait counts at the top of the loop take
// the worse of the entry path and the loop's own, and a reordered entry (a Qt
// fragment requested among the last) made every loop trip wait for nearly all
// of the previous step's loads.
template <typename OpT, int DK, int DVS, int C, bool kScalarGate, int PHASE, int MODE>
__device__ __forceinline__ void carry_load(CarryFrags<OpT, DK, DVS, C, kScalarGate>& F,
                                           const PrefillArgs& a, const unsigned char* ws_head,
                                           int nn, int b, int h, int jb, int wave, int lane) {
  using Sh = CarryShape<OpT, DK, DVS, C, kScalarGate>;
  using Blk = typename Sh::Blk;
  using FK = typename Sh::FK;
  using FC = typename Sh::FC;
  const unsigned char* blk_bytes = ws_head + static_cast<size_t>(nn) * a.H_v * Blk::kBytes;
  const OpT* blk = reinterpret_cast<const OpT*>(blk_bytes);
  const OpT* vg = static_cast<const OpT*>(a.v);
  const int t0 = nn * C;
  const OpT* qkr = kScalarGate ? qk_region<OpT, DK, C>(a, b, h / (a.H_v / a.H_qk), nn) : nullptr;
#pragma unroll
  for (int i = 0; i < Sh::OPW; ++i) {
    const int t = wave * Sh::OPW + i;
    if (Sh::NOT % Sh::NW == 0 || t < Sh::NOT) {
      const int R = t / Sh::DVT, J = t % Sh::DVT;
      if constexpr (PHASE == 0) {
#pragma unroll
        for (int s = 0; s < FK::STEPS; ++s) {
          if constexpr (kScalarGate)
            F.kt[i][s] = FK::load(qkr + QKRegion<OpT, DK, C>::kK, 16 * R, s, lane);
          else
            F.kt[i][s] = FK::load(blk + Blk::kKt, 16 * R, s, lane);
          pin_order<Sh::kPinLoads>();
          if constexpr (MODE == kCarryFull) {
            if constexpr (kScalarGate)
              F.qt[i][s] = FK::load(qkr + QKRegion<OpT, DK, C>::kQ, 16 * R, s, lane);
            else
              F.qt[i][s] = FK::load(blk + Blk::kQt, 16 * R, s, lane);
          }
          pin_order<Sh::kPinLoads>();
        }
        if constexpr (kScalarGate) {
          carry_load_fk<OpT, DK, DVS, C, kScalarGate>(F, blk, i, R, lane);
          if constexpr (MODE == kCarryFull)
            carry_load_fq<OpT, DK, DVS, C, kScalarGate>(F, blk, i, R, lane);
          pin_order<Sh::kPinLoads>();
        }
        if constexpr (MODE != kCarryMapM) {
          // Uniform row base plus 32-bit lane offsets; rows past the end
          // re-read the last row and are zeroed when used.
          const OpT* vrow = vg + ((static_cast<size_t>(b) * a.T + t0) * a.H_v + h) * a.dv + jb;
          const unsigned rs = static_cast<unsigned>(a.H_v) * a.dv;
          const int last = a.T - 1 - t0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = min(16 * R + 4 * (lane >> 4) + e, last);
            F.v[i][e] = vrow[static_cast<unsigned>(r) * rs + 16 * J + (lane & 15)];
          }
          pin_order<Sh::kPinLoads>();
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) F.v[i][e] = from_f32<OpT>(0.0f);
        }
      }
      if constexpr (PHASE == 1) {
#pragma unroll
        for (int s = 0; s < FC::STEPS; ++s) {
          F.tb[i][s] = FC::load(blk + Blk::kTb, 16 * R, s, lane);
          pin_order<Sh::kPinLoads>();
        }
      }
      if constexpr (PHASE == 2 && MODE == kCarryFull) {
#pragma unroll
        for (int s = 0; s < FC::STEPS; ++s) {
          F.p[i][s] = FC::load(blk + Blk::kP, 16 * R, s, lane);
          pin_order<Sh::kPinLoads>();
        }
      }
    }
  }
  if constexpr (PHASE == 2) {
    const float* gam = reinterpret_cast<const float*>(blk_bytes + Blk::kGammaByte);
#pragma unroll
    for (int j = 0; j < Sh::SPW; ++j) {
      const int t = wave * Sh::SPW + j;
      if (Sh::NST % Sh::NW == 0 || t < Sh::NST) {
        const int I = t / Sh::DVT;
#pragma unroll
        for (int s = 0; s < FC::STEPS; ++s) {
          F.ke[j][s] = FC::load(blk + Blk::kKeT, 16 * I, s, lane);
          pin_order<Sh::kPinLoads>();
        }
        const float4 g4 = *reinterpret_cast<const float4*>(gam + 16 * I + 4 * (lane >> 4));
        F.gam[j][0] = g4.x;
        F.gam[j][1] = g4.y;
        F.gam[j][2] = g4.z;
        F.gam[j][3] = g4.w;
      }
    }
  }
}

// V rows of output tile (R, J) of chunk nn, in accumulator layout.
template <typename OpT, int DK, int DVS, int C, bool kScalarGate>
__device__ __forceinline__ void carry_load_v(CarryFrags<OpT, DK, DVS, C, kScalarGate>& F,
                                             const PrefillArgs& a, int nn, int b, int h, int jb,
                                             int i, int R, int J, int lane) {
  // Uniform row base plus 32-bit lane offsets; rows past the end re-read the
  // last row and are zeroed when used.
  const int t0 = nn * C;
  const OpT* vrow = static_cast<const OpT*>(a.v) +
                    ((static_cast<size_t>(b) * a.T + t0) * a.H_v + h) * a.dv + jb;
  const unsigned rs = static_cast<unsigned>(a.H_v) * a.dv;
  const int last = a.T - 1 - t0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = min(16 * R + 4 * (lane >> 4) + e, last);
    F.v[i][e] = vrow[static_cast<unsigned>(r) * rs + 16 * J + (lane & 15)];
  }
}

// e^Gamma_L for the rows of state tile row-block I of the block at blk.
template <typename OpT, int DK, int DVS, int C, bool kScalarGate>
__device__ __forceinline__ void carry_load_gam(CarryFrags<OpT, DK, DVS, C, kScalarGate>& F,
                                               const OpT* blk, int i, int I, int lane) {
  using Blk = typename CarryShape<OpT, DK, DVS, C, kScalarGate>::Blk;
  const float* gam =
      reinterpret_cast<const float*>(reinterpret_cast<const unsigned char*>(blk) + Blk::kGammaByte);
  const float4 g4 = *reinterpret_cast<const float4*>(gam + 16 * I + 4 * (lane >> 4));
  F.gam[i][0] = g4.x;
  F.gam[i][1] = g4.y;
  F.gam[i][2] = g4.z;
  F.gam[i][3] = g4.w;
}

template <typename OpT, int DK, int DVS, int C, bool kScalarGate, int MODE>
__device__ __forceinline__ void carry_load_all(CarryFrags<OpT, DK, DVS, C, kScalarGate>& F,
                                               const PrefillArgs& a, const unsigned char* ws_head,
                                               int nn, int b, int h, int jb, int wave, int lane) {
  carry_load<OpT, DK, DVS, C, kScalarGate, 0, MODE>(F, a, ws_head, nn, b, h, jb, wave, lane);
  carry_load<OpT, DK, DVS, C, kScalarGate, 1, MODE>(F, a, ws_head, nn, b, h, jb, wave, lane);
  carry_load<OpT, DK, DVS, C, kScalarGate, 2, MODE>(F, a, ws_head, nn, b, h, jb, wave, lane);
}

// One workgroup per (b, h, slice), over the chunks of cr: the state slice
// starts from s_src (zeros when it is null; the identity for kCarryMapM) and ends
// in s_dst (not written when it is null).  a.dv is the number of state
// columns (dk for kCarryMapM).  wg is the workgroup's index among the G that do
// this work, and sm its LDS (kSmem bytes).
template <typename OpT, int DK, int DVS, int C, bool kScalarGate, int MODE>
__device__ __forceinline__ void carry_body(const PrefillArgs& a, ChunkRange cr,
                                           const float* s_src, float* s_dst, int wg, int G,
                                           unsigned char* sm) {
  using Sh = CarryShape<OpT, DK, DVS, C, kScalarGate>;
  using Blk = typename Sh::Blk;
  using FK = typename Sh::FK;
  using FC = typename Sh::FC;
  using Frags = CarryFrags<OpT, DK, DVS, C, kScalarGate>;
  constexpr int LDK = Sh::LDK, LDC = Sh::LDC, DVT = Sh::DVT;
  constexpr int SPW = Sh::SPW, OPW = Sh::OPW, NST = Sh::NST, NOT = Sh::NOT;

  OpT* St_s = reinterpret_cast<OpT*>(sm);
  OpT* Rt_s = St_s + DVS * LDK;
  OpT* Ut_s = Rt_s + DVS * LDC;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n_sl = a.dv / DVS;

  // XCD-aware order: workgroups w, w+8, w+16, ... run on one XCD (and share its
  // L2); give them consecutive (head, slice) units so that the slices of one
  // head read that head's chunk blocks through the same L2.
  int unit = wg;
  if (G % 8 == 0) unit = (wg % 8) * (G / 8) + wg / 8;
  const int slice = unit % n_sl;
  const int bh = unit / n_sl;
  const int h = bh % a.H_v;
  const int b = bh / a.H_v;
  const int hq = h / (a.H_v / a.H_qk);  // qk head of value head h
  const int jb = slice * DVS;
  const int NC = (a.T + C - 1) / C;

  const size_t st_off = static_cast<size_t>(bh) * DK * a.dv;
  const unsigned char* ws_head =
      static_cast<const unsigned char*>(a.ws) + block_offset<Blk>(b, 0, h, NC, a.H_v);
  OpT* og = static_cast<OpT*>(a.o);

  // ---- state tiles owned by this wave, in accumulator layout ----
  f32x4 sacc[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int t = wave * SPW + i;
    sacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (MODE == kCarryMapM) {
      const int I = t / DVT, J = t % DVT;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sacc[i][e] = 16 * I + 4 * (lane >> 4) + e == jb + 16 * J + (lane & 15) ? 1.0f : 0.0f;
    } else if ((NST % Sh::NW == 0 || t < NST) && s_src) {
      const int I = t / DVT, J = t % DVT;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * I + 4 * (lane >> 4) + e;
        sacc[i][e] = s_src[st_off + static_cast<size_t>(row) * a.dv + jb + 16 * J +
                                (lane & 15)];
      }
    }
  }

  // One register set of fragments: as soon as a phase has consumed its
  // fragments, the same registers start loading that phase's fragments of
  // the next chunk, so each load has most of a chunk step to arrive.  The
  // range's last chunk re-reads itself (in bounds, unused), keeping every load
  // unconditional so that the wait counters stay exact across iterations.
  // kFull: the chunk has all C rows (every chunk but a ragged last one), so
  // the o stores need no row guard and the loop body holds no branch around
  // memory operations, which keeps the compiler's wait counts exact.
  auto compute = [&](Frags& F, int nn, auto full) __attribute__((always_inline)) {
    constexpr bool kFull = decltype(full)::value;
    constexpr bool kPin = Sh::kPinLoads;
    const int t0 = nn * C;
    const int L = kFull ? C : min(C, a.T - t0);
    const int nx = min(nn + 1, cr.n1 - 1);
    const OpT* nblk =
        reinterpret_cast<const OpT*>(ws_head + static_cast<size_t>(nx) * a.H_v * Blk::kBytes);
    const OpT* nqk = kScalarGate ? qk_region<OpT, DK, C>(a, b, hq, nx) : nullptr;
    // S^T in the operand type, for Kt S and Qt S.
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int t = wave * SPW + i;
      if (NST % Sh::NW == 0 || t < NST) {
        const int I = t / DVT, J = t % DVT;
        float v[4] = {sacc[i][0], sacc[i][1], sacc[i][2], sacc[i][3]};
        store_tile_t<OpT>(St_s, LDK, 16 * J, 16 * I, v, lane);
      }
    }
    __syncthreads();  // [B1]

    // R = V - Kt S  (stored transposed),  O = Qt S (kept in registers).
    f32x4 oacc[OPW];
#pragma unroll
    for (int i = 0; i < OPW; ++i) {
      const int t = wave * OPW + i;
      oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (NOT % Sh::NW == 0 || t < NOT) {
        const int R = t / DVT, J = t % DVT;
        f32x4 ks = {0.f, 0.f, 0.f, 0.f};
        typename FK::T z[FK::STEPS];
        z[0] = FK::load_pad(St_s, LDK, 16 * J, 0, lane);
#pragma unroll
        for (int s = 0; s < FK::STEPS; ++s) {
          if (s + 1 < FK::STEPS) z[s + 1] = FK::load_pad(St_s, LDK, 16 * J, s + 1, lane);
          ks = FK::mma(F.kt[i][s], z[s], ks);
          // O is accumulated transposed (S^T Qt^T): each lane then holds four
          // consecutive columns of one output row, stored with one wide write.
          if constexpr (MODE == kCarryFull) oacc[i] = FK::mma(z[s], F.qt[i][s], oacc[i]);
          // The next chunk's fragments go out one pair per step, each as soon
          // as its registers have been read.
          pin_order<kPin>();  // the reloads below may then reuse the consumed registers
          if constexpr (kScalarGate) {
            F.kt[i][s] = FK::load(nqk + QKRegion<OpT, DK, C>::kK, 16 * R, s, lane);
            if constexpr (MODE == kCarryFull)
              F.qt[i][s] = FK::load(nqk + QKRegion<OpT, DK, C>::kQ, 16 * R, s, lane);
          } else {
            F.kt[i][s] = FK::load(nblk + Blk::kKt, 16 * R, s, lane);
            if constexpr (MODE == kCarryFull)
              F.qt[i][s] = FK::load(nblk + Blk::kQt, 16 * R, s, lane);
          }
          pin_order<kPin>();
        }
        float rv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * R + 4 * (lane >> 4) + e;
          const float kts = kScalarGate ? F.fk[i][e] * ks[e] : ks[e];
          rv[e] = (r < L ? to_f32(F.v[i][e]) : 0.0f) - kts;
        }
        store_tile_t<OpT>(Rt_s, LDC, 16 * J, 16 * R, rv, lane);
        if constexpr (kScalarGate) carry_load_fk<OpT, DK, DVS, C, kScalarGate>(F, nblk, i, R, lane);
        if constexpr (MODE != kCarryMapM)
          carry_load_v<OpT, DK, DVS, C, kScalarGate>(F, a, nx, b, h, jb, i, R, J, lane);
      }
    }
    __syncthreads();  // [B2]

    // U = Tb R  (stored transposed).
#pragma unroll
    for (int i = 0; i < OPW; ++i) {
      const int t = wave * OPW + i;
      if (NOT % Sh::NW == 0 || t < NOT) {
        const int R = t / DVT, J = t % DVT;
        f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < FC::STEPS; ++s) {
          u = FC::mma(F.tb[i][s], FC::load_pad(Rt_s, LDC, 16 * J, s, lane), u);
          pin_order<kPin>();
          F.tb[i][s] = FC::load(nblk + Blk::kTb, 16 * R, s, lane);
          pin_order<kPin>();
        }
        float uv[4] = {u[0], u[1], u[2], u[3]};
        store_tile_t<OpT>(Ut_s, LDC, 16 * J, 16 * R, uv, lane);
      }
    }
    __syncthreads();  // [B3]

    // O = scale (Qt S + P U) -> o rows of this chunk.  When the contractions
    // over dk and over the chunk use different MFMA shapes (16x16x32 and
    // 16x16x16), P U goes to accumulators of its own: the compiler may sink the
    // Qt S product (it touches no memory) next to this one, and it puts no wait
    // states between an accumulator written by one shape and read as the
    // addend of the other, which then reads two of its four values too early.
    // Scalar gates: Q S is scaled by e^Gamma row by row, so P U goes to
    // accumulators of its own as well.
    constexpr bool kSplitO = kScalarGate || FK::KS != FC::KS;
    f32x4 pacc[OPW];
#pragma unroll
    for (int i = 0; i < OPW; ++i) {
      const int t = wave * OPW + i;
      pacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (MODE == kCarryFull && (NOT % Sh::NW == 0 || t < NOT)) {
        const int R = t / DVT, J = t % DVT;
#pragma unroll
        for (int s = 0; s < FC::STEPS; ++s) {
          if constexpr (kSplitO)
            pacc[i] = FC::mma(FC::load_pad(Ut_s, LDC, 16 * J, s, lane), F.p[i][s], pacc[i]);
          else
            oacc[i] = FC::mma(FC::load_pad(Ut_s, LDC, 16 * J, s, lane), F.p[i][s], oacc[i]);
          pin_order<kPin>();
          F.p[i][s] = FC::load(nblk + Blk::kP, 16 * R, s, lane);
          pin_order<kPin>();
        }
      }
    }
    // S = diag(e^Gamma_L) S + Ke^T U.
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int t = wave * SPW + i;
      if (NST % Sh::NW == 0 || t < NST) {
        const int I = t / DVT, J = t % DVT;
        // Ke^T U from zero, so that the products do not wait for the decay.
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < FC::STEPS; ++s) {
          t = FC::mma(F.ke[i][s], FC::load_pad(Ut_s, LDC, 16 * J, s, lane), t);
          pin_order<kPin>();
          F.ke[i][s] = FC::load(nblk + Blk::kKeT, 16 * I, s, lane);
          pin_order<kPin>();
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sacc[i][e] = F.gam[i][e] * sacc[i][e] + t[e];
        carry_load_gam<OpT, DK, DVS, C, kScalarGate>(F, nblk, i, I, lane);
      }
    }
    // Scalar gates: O = e^Gamma (Q S) + P U per row; then the next chunk's factors.
    if constexpr (kScalarGate && MODE == kCarryFull) {
#pragma unroll
      for (int i = 0; i < OPW; ++i) {
        const int t = wave * OPW + i;
        if (NOT % Sh::NW == 0 || t < NOT) {
#pragma unroll
          for (int e = 0; e < 4; ++e) oacc[i][e] = F.fq[i] * oacc[i][e] + pacc[i][e];
          carry_load_fq<OpT, DK, DVS, C, kScalarGate>(F, nblk, i, t / DVT, lane);
        }
      }
    }
    // The o rows go out last, after every load of the step.  On gfx9 stores
    // and loads share one in-order completion counter, so a wait for a load
    // issued after a store also waits for that store's write acknowledgement;
    // with the stores last, the first load issued after them is waited for
    // two chunk steps later.
#pragma unroll
    for (int i = 0; i < OPW; ++i) {
      const int t = wave * OPW + i;
      if (MODE == kCarryFull && (NOT % Sh::NW == 0 || t < NOT)) {
        const int R = t / DVT, J = t % DVT;
        // lane (c, g): row 16 R + c, columns 16 J + 4 g ... + 3 of the chunk's o
        OpT* obase = og + ((static_cast<size_t>(b) * a.T + t0) * a.H_v + h) * a.dv + jb;
        const unsigned rs = static_cast<unsigned>(a.H_v) * a.dv;
        const int r = 16 * R + (lane & 15);
        OpT* op = obase + (static_cast<unsigned>(r) * rs + 16 * J + 4 * (lane >> 4));
        if constexpr (kSplitO && !kScalarGate) {
#pragma unroll
          for (int e = 0; e < 4; ++e) oacc[i][e] += pacc[i][e];
        }
        if (kFull || r < L) {
          if constexpr (Sh::kNtO)
            store4_nt<OpT>(op, a.scale * oacc[i][0], a.scale * oacc[i][1], a.scale * oacc[i][2],
                           a.scale * oacc[i][3]);
          else
            store4<OpT>(op, a.scale * oacc[i][0], a.scale * oacc[i][1], a.scale * oacc[i][2],
                        a.scale * oacc[i][3]);
        }
      }
    }
  };

  Frags F;
  carry_load_all<OpT, DK, DVS, C, kScalarGate, MODE>(F, a, ws_head, cr.n0, b, h, jb, wave, lane);
  const int NF = a.T / C;  // full chunks
  const int nf_end = min(cr.n1, NF);
  int nn = cr.n0;
  for (; nn + 1 < nf_end; nn += 2) {
    compute(F, nn, std::true_type{});
    compute(F, nn + 1, std::true_type{});
  }
  if (nn < nf_end) compute(F, nn, std::true_type{});
  if (cr.n1 > NF) compute(F, NF, std::false_type{});  // the ragged last chunk

  // ---- final state ----
  if (!s_dst) return;
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int t = wave * SPW + i;
    if (NST % Sh::NW == 0 || t < NST) {
      const int I = t / DVT, J = t % DVT;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * I + 4 * (lane >> 4) + e;
        s_dst[st_off + static_cast<size_t>(row) * a.dv + jb + 16 * J + (lane & 15)] = sacc[i][e];
      }
    }
  }
}

// A carry launch runs up to three jobs side by side, each over nseg
// consecutive sequence segments of seg_len chunks (the last segment of the
// sequence may be shorter).  Workgroups are job-major, then segment-major.
struct CarryJob {
  int mode;           // CarryMode
  int first, nseg;    // segments first ... first + nseg - 1
  int per;            // workgroups per segment: (b, h) units x column slices
  int cols;           // state columns: dv, or dk for kCarryMapM
  const float* src;   // start state of segment first + i at src + i * src_stride (null: zeros)
  size_t src_stride;
  float* dst;         // final state of segment first + i at dst + i * dst_stride (null: none)
  size_t dst_stride;
};
struct CarryJobs {
  CarryJob job[3];
  int n;
  int seg_len;
};

// kMaps: the launch may hold kCarryMapN / kCarryMapM jobs (instantiated for the one
// slice width the segmented schedule uses); otherwise every job is kCarryFull.
template <typename OpT, int DK, int DVS, int C, bool kScalarGate, bool kMaps>
__global__ __launch_bounds__((CarryShape<OpT, DK, DVS, C, kScalarGate>::NT)) void
chunk_carry_kernel(PrefillArgs a, CarryJobs J) {
  using Sh = CarryShape<OpT, DK, DVS, C, kScalarGate>;
  __shared__ __attribute__((aligned(16))) unsigned char sm[Sh::kSmem];
  int w = blockIdx.x, k = 0;
  while (k + 1 < J.n && w >= J.job[k].nseg * J.job[k].per) {
    w -= J.job[k].nseg * J.job[k].per;
    ++k;
  }
  const CarryJob& jb = J.job[k];
  const int i = w / jb.per;
  const int p = jb.first + i;
  const int NC = (a.T + C - 1) / C;
  const ChunkRange cr{p * J.seg_len, min((p + 1) * J.seg_len, NC)};
  PrefillArgs ap = a;
  ap.dv = jb.cols;
  const float* src = jb.src ? jb.src + i * jb.src_stride : nullptr;
  float* dst = jb.dst ? jb.dst + i * jb.dst_stride : nullptr;
  if constexpr (kMaps) {
    if (jb.mode == kCarryMapN) {
      carry_body<OpT, DK, DVS, C, kScalarGate, kCarryMapN>(ap, cr, src, dst, w % jb.per, jb.per,
                                                           sm);
      return;
    }
    if (jb.mode == kCarryMapM) {
      carry_body<OpT, DK, DVS, C, kScalarGate, kCarryMapM>(ap, cr, src, dst, w % jb.per, jb.per,
                                                           sm);
      return;
    }
  }
  carry_body<OpT, DK, DVS, C, kScalarGate, kCarryFull>(ap, cr, src, dst, w % jb.per, jb.per, sm);
}

// Start states of segments p0 + 1 ... p1 + 1 of the segmented carry:
// S[p + 1] = M[p] S[p] + N[p] per (b, h) unit, in fp32.  S and N are
// [segment][unit][DK][dv], M is [segment][unit][DK][DK].  One workgroup per
// unit and 16-column block; the product runs on fp32 MFMA (16x16x4), wave w
// owning row tiles TPW w ... TPW w + TPW - 1.  Lane (g, n) holds row
// 16 I + n of M at k = g KG ... g KG + KG - 1 in registers, so k-step t
// contracts k = g KG + t over the four lane groups, and S[k][n] comes from
// LDS (double buffered across segments).  The next segment's M rows and N
// are loaded while the current product runs.
template <int DK>
__global__ __launch_bounds__(256) void carry_scan_kernel(const float* __restrict__ M,
                                                         const float* __restrict__ N,
                                                         float* __restrict__ S, int units, int dv,
                                                         int p0, int p1) {
  constexpr int NI = DK / 16;          // row tiles
  constexpr int TPW = (NI + 3) / 4;    // row tiles per wave
  constexpr int KG = DK / 4;           // k-values per lane group
  constexpr bool kAllWaves = NI % 4 == 0;  // every wave owns TPW row tiles
  __shared__ float Ss[2][DK][16];
  const int nb = dv / 16;
  const int u = blockIdx.x / nb;
  const int c0 = (blockIdx.x % nb) * 16;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, n = lane & 15;
  const size_t sv = static_cast<size_t>(units) * DK * dv;  // segment stride of S and N
  const size_t sm = static_cast<size_t>(units) * DK * DK;  // segment stride of M
  const size_t uv = static_cast<size_t>(u) * DK * dv;
  const size_t um = static_cast<size_t>(u) * DK * DK;

  static_assert(DK * 16 % 256 == 0, "start state: whole passes of the workgroup");
  {
    float s0[DK * 16 / 256];  // every load issued before any is used
#pragma unroll
    for (int i = 0; i < DK * 16 / 256; ++i) {
      const int x = threadIdx.x + 256 * i;
      s0[i] = S[p0 * sv + uv + static_cast<size_t>(x / 16) * dv + c0 + x % 16];
    }
#pragma unroll
    for (int i = 0; i < DK * 16 / 256; ++i) {
      const int x = threadIdx.x + 256 * i;
      Ss[0][x / 16][x % 16] = s0[i];
    }
  }

  // Two register sets: segment p + 1's M rows and N are in flight while
  // segment p's product runs.  Fetches are unconditional (the last segment is
  // fetched again, unused) so that the wait counts stay exact.
  float m[2][TPW][KG];
  float na[2][TPW][4];
  auto fetch = [&](int p, auto buf) __attribute__((always_inline)) {
    constexpr int B = decltype(buf)::value;
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) {
      const int I = wave * TPW + ti;
      if (kAllWaves || I < NI) {
        const float* mr = M + p * sm + um + static_cast<size_t>(16 * I + n) * DK + g * KG;
#pragma unroll
        for (int k4 = 0; k4 < KG / 4; ++k4) {
          const float4 v = *reinterpret_cast<const float4*>(mr + 4 * k4);
          m[B][ti][4 * k4] = v.x;
          m[B][ti][4 * k4 + 1] = v.y;
          m[B][ti][4 * k4 + 2] = v.z;
          m[B][ti][4 * k4 + 3] = v.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          na[B][ti][e] = N[p * sv + uv + static_cast<size_t>(16 * I + 4 * g + e) * dv + c0 + n];
      }
    }
  };
  int cur = 0;
  auto step = [&](int p, auto buf) __attribute__((always_inline)) {
    constexpr int B = decltype(buf)::value;
    f32x4 acc[TPW];
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti)
      acc[ti] = f32x4{na[B][ti][0], na[B][ti][1], na[B][ti][2], na[B][ti][3]};
    float bv[KG];  // this lane group's k-values of column n, all read before the products
#pragma unroll
    for (int t = 0; t < KG; ++t) bv[t] = Ss[cur][g * KG + t][n];
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) {
      if (kAllWaves || wave * TPW + ti < NI) {
#pragma unroll
        for (int t = 0; t < KG; ++t) acc[ti] = mfma_f32x4(m[B][ti][t], bv[t], acc[ti]);
      }
    }
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) {
      const int I = wave * TPW + ti;
      if (kAllWaves || I < NI) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * I + 4 * g + e;
          Ss[cur ^ 1][row][n] = acc[ti][e];
          S[(p + 1) * sv + uv + static_cast<size_t>(row) * dv + c0 + n] = acc[ti][e];
        }
      }
    }
    __syncthreads();
    cur ^= 1;
  };
  fetch(p0, std::integral_constant<int, 0>{});
  __syncthreads();
  // Segments in pairs, each fetch one product ahead of its use; the
  // scheduling fences keep every fetch ahead of the product it overlaps.
  int p = p0;
  for (; p + 1 <= p1; p += 2) {
    fetch(p + 1, std::integral_constant<int, 1>{});
    __builtin_amdgcn_sched_barrier(0);
    step(p, std::integral_constant<int, 0>{});
    fetch(min(p + 2, p1), std::integral_constant<int, 0>{});
    __builtin_amdgcn_sched_barrier(0);
    step(p + 1, std::integral_constant<int, 1>{});
  }
  if (p <= p1) step(p, std::integral_constant<int, 0>{});  // an odd last segment
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
size_t block_bytes(bool scalar_gate) {
  return scalar_gate ? ChunkBlock<OpT, DK, C, true>::kBytes : ChunkBlock<OpT, DK, C, false>::kBytes;
}

// Scalar gates take the smaller block without Kt and Qt.
template <typename OpT>
size_t block_bytes_rt(int dk, int chunk, bool scalar_gate) {
#define GDR_BB(DKV, CV) \
  if (dk == DKV && chunk == CV) return block_bytes<OpT, DKV, CV>(scalar_gate);
  GDR_BB(16, 16) GDR_BB(16, 32) GDR_BB(16, 64)
  GDR_BB(32, 16) GDR_BB(32, 32) GDR_BB(32, 64)
  GDR_BB(64, 16) GDR_BB(64, 32) GDR_BB(64, 64)
  GDR_BB(128, 16) GDR_BB(128, 32) GDR_BB(128, 64)
#undef GDR_BB
  return 0;
}

template <typename OpT, int DK, int DVS, int C, bool kScalarGate, bool kMaps>
hipError_t launch_carry_jobs(const PrefillArgs& a, const CarryJobs& J, hipStream_t stream) {
  unsigned grid = 0;
  for (int k = 0; k < J.n; ++k) grid += static_cast<unsigned>(J.job[k].nseg) * J.job[k].per;
  hipLaunchKernelGGL((chunk_carry_kernel<OpT, DK, DVS, C, kScalarGate, kMaps>), dim3(grid),
                     dim3(CarryShape<OpT, DK, DVS, C, kScalarGate>::NT), 0, stream, a, J);
  return hipGetLastError();
}

// The plain carry: one job, the whole sequence as one segment.
template <typename OpT, int DK, int DVS, int C, bool kScalarGate>
hipError_t launch_carry(const PrefillArgs& a, hipStream_t stream) {
  CarryJobs J{};
  J.n = 1;
  J.seg_len = (a.T + C - 1) / C;
  J.job[0] = CarryJob{kCarryFull, 0, 1, a.B * a.H_v * (a.dv / DVS), a.dv, a.state_in, 0, a.state_out, 0};
  return launch_carry_jobs<OpT, DK, DVS, C, kScalarGate, false>(a, J, stream);
}

// Slice width: the narrowest (from 16 columns) that keeps the number of
// (b, h, slice) workgroups within one per CU, and at most 64 columns (wider
// slices would not fit their fragments in registers).  A chunk step of a
// workgroup costs more the wider its slice, but a second workgroup on a CU
// costs more still: the carry is a chain of dependent steps, so two chains
// sharing a CU's load path and matrix cores each run slower.
int carry_slice_width(const PrefillArgs& a) {
  const long units = static_cast<long>(a.B) * a.H_v;
  int dvs = a.dv < 16 ? a.dv : 16;
  while (dvs < a.dv && dvs < 64 && units * (a.dv / dvs) > 256) dvs *= 2;
  return dvs;
}

template <typename OpT, int DK, int C, bool kScalarGate>
hipError_t launch_carry_any(const PrefillArgs& a, hipStream_t stream) {
  switch (carry_slice_width(a)) {
    case 16: return launch_carry<OpT, DK, 16, C, kScalarGate>(a, stream);
    case 32: return launch_carry<OpT, DK, 32, C, kScalarGate>(a, stream);
    default: return launch_carry<OpT, DK, 64, C, kScalarGate>(a, stream);
  }
}

// ---------------------------------------------------------------------------
// Segmented carry: a parallel scan of the carry's affine maps.
//
// Over a range of chunks the carry maps each state column affinely,
// S_out = M S_in + N: N is the range run from a zero state, M (dk x dk) the
// range run from the identity with V = 0.  When the plain carry would leave
// most CUs idle (few (b, h) units) and the sequence is long, it is cut into P
// segments of seg_len chunks and run in three launches:
//   1. segment 0 in full, side by side with the maps (N, M) of segments
//      1 ... P-2 (the last segment's map is never needed);
//   2. the start states S_2 ... S_{P-1} by S_{p+1} = M_p S_p + N_p, with S_1
//      the final state of segment 0 (fp32, a few small products per unit);
//   3. segments 1 ... P-1 in full from their start states, side by side; the
//      last one's final state is the result.
// That is about three times the carry's work for segments 1 ... P-2, spread
// over P times more workgroups, and two segment lengths of chained steps
// instead of P.  The maps use the same bf16 (or fp32) operands as the plain
// carry, so the result matches it to rounding.
// ---------------------------------------------------------------------------
// Limits measured at B=1, dk=dv=128 (eager prefills): a side-by-side launch of
// up to 512 workgroups pays at any length; up to 1024 pays from 256 chunks
// (H_v=8, T=32767: 495 -> 452 us; H_v=16: 938 -> 830 us) but not at 125
// (H_v=8, T=8000: 103 -> 115 us).
constexpr long kSegMaxPlainWgs = 128;   // plain carry workgroups (16-column slices) at most
constexpr int kSegMinChunks = 8;        // chunks per segment at least
constexpr int kSegMaxSegments = 16;
constexpr long kSegMaxWgs = 512;        // workgroups of the side-by-side launch at most ...
constexpr long kSegMaxWgsLong = 1024;   // ... from kSegLongChunks chunks on
constexpr int kSegLongChunks = 256;

struct SegPlan {
  int P;        // segments (1: the plain carry)
  int seg_len;  // chunks per segment
};

SegPlan carry_segments(int B, int T, int H_v, int dk, int dv, int chunk) {
  const int NC = (T + chunk - 1) / chunk;
  const SegPlan plain{1, NC};
  const long units = static_cast<long>(B) * H_v;
  const long w_n = units * (dv / 16);  // workgroups per segment of a dv-column job
  const long w_m = units * (dk / 16);  // of a dk-column (linear part) job
  if (dv < 16 || dk < 16 || w_n > kSegMaxPlainWgs) return plain;
  const long max_wgs = NC >= kSegLongChunks ? kSegMaxWgsLong : kSegMaxWgs;
  SegPlan best = plain;
  for (int P = 3; P <= kSegMaxSegments; ++P) {
    const int L = (NC + P - 1) / P;
    if (L < kSegMinChunks) break;
    const int Pe = (NC + L - 1) / L;  // segments actually formed
    if (Pe < 3) continue;
    if (w_n + (Pe - 2) * (w_n + w_m) > max_wgs) break;
    best = SegPlan{Pe, L};
  }
  return best;
}

// Bytes of the segmented carry's buffers (S and N: [P][units][dk][dv],
// M: [P][units][dk][dk], fp32).
size_t seg_bytes(SegPlan sp, long units, int dk, int dv) {
  if (sp.P < 3) return 0;
  return static_cast<size_t>(sp.P) * units * dk * (2 * static_cast<size_t>(dv) + dk) *
         sizeof(float);
}
size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace layout: the chunk blocks (chunk-major: (b, chunk, h), see
// block_offset); at the next 256-byte boundary, for scalar gates, the
// QKRegions ((b, chunk, qk head)); at the next 256-byte boundary, the
// segmented carry's buffers (if it runs).
struct WsLayout {
  size_t qk, seg, total;
};
WsLayout ws_layout(long units, size_t nc, size_t block_bytes, size_t qk, size_t seg) {
  const size_t blocks = static_cast<size_t>(units) * nc * block_bytes;
  WsLayout w;
  w.qk = align256(blocks);
  const size_t end = qk ? w.qk + qk : blocks;
  w.seg = align256(end);
  w.total = seg ? w.seg + seg : end;
  return w;
}

// Bytes of the QKRegions of a prefill (scalar gates).
size_t qk_region_bytes(bool scalar_gate, int B, int H_qk, size_t nc, int dk, int chunk, size_t es) {
  return scalar_gate ? static_cast<size_t>(B) * H_qk * nc * 2 * chunk * dk * es : 0;
}

template <typename OpT, int DK, int C, bool kScalarGate>
hipError_t launch_carry_segmented(const PrefillArgs& a, SegPlan sp, hipStream_t stream) {
  const long units = static_cast<long>(a.B) * a.H_v;
  const int NC = (a.T + C - 1) / C;
  const int P = sp.P;
  const size_t sv = static_cast<size_t>(units) * DK * a.dv;  // one segment's S or N
  const size_t smm = static_cast<size_t>(units) * DK * DK;   // one segment's M
  const size_t qk = qk_region_bytes(kScalarGate, a.B, a.H_qk, NC, DK, C, sizeof(OpT));
  const WsLayout wl = ws_layout(units, NC, ChunkBlock<OpT, DK, C, kScalarGate>::kBytes, qk, 1);
  float* Sb = reinterpret_cast<float*>(static_cast<unsigned char*>(a.ws) + wl.seg);
  float* Nb = Sb + P * sv;
  float* Mb = Nb + P * sv;
  const int per_n = static_cast<int>(units) * (a.dv / 16);
  const int per_m = static_cast<int>(units) * (DK / 16);

  CarryJobs J{};
  J.n = 3;
  J.seg_len = sp.seg_len;
  J.job[0] = CarryJob{kCarryFull, 0, 1, per_n, a.dv, a.state_in, 0, Sb + sv, 0};
  J.job[1] = CarryJob{kCarryMapN, 1, P - 2, per_n, a.dv, nullptr, 0, Nb + sv, sv};
  J.job[2] = CarryJob{kCarryMapM, 1, P - 2, per_m, DK, nullptr, 0, Mb + smm, smm};
  hipError_t err = launch_carry_jobs<OpT, DK, 16, C, kScalarGate, true>(a, J, stream);
  if (err != hipSuccess) return err;

  hipLaunchKernelGGL(carry_scan_kernel<DK>, dim3(static_cast<unsigned>(per_n)), dim3(256), 0,
                     stream, Mb, Nb, Sb, static_cast<int>(units), a.dv, 1, P - 2);
  err = hipGetLastError();
  if (err != hipSuccess) return err;

  CarryJobs R{};
  R.n = 2;
  R.seg_len = sp.seg_len;
  R.job[0] = CarryJob{kCarryFull, 1, P - 2, per_n, a.dv, Sb + sv, sv, nullptr, 0};
  R.job[1] = CarryJob{kCarryFull, P - 1, 1, per_n, a.dv, Sb + (P - 1) * sv, 0, a.state_out, 0};
  return launch_carry_jobs<OpT, DK, 16, C, kScalarGate, false>(a, R, stream);
}

template <typename OpT, int DK, int C>
hipError_t launch_prep(const PrefillArgs& a, ChunkRange cr, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(a.B) * a.H_v * (cr.n1 - cr.n0);
  if (a.gate == GDR_GATE_CHANNEL)
    hipLaunchKernelGGL((chunk_prep_kernel<OpT, DK, C, true>), dim3(grid), dim3(kThreads), 0,
                       stream, a, cr);
  else
    hipLaunchKernelGGL((chunk_prep_kernel<OpT, DK, C, false>), dim3(grid), dim3(kThreads), 0,
                       stream, a, cr);
  return hipGetLastError();
}

template <typename OpT, int DK, int C>
hipError_t launch_dk_c(const PrefillArgs& a0, hipStream_t stream) {
  const int NC = (a0.T + C - 1) / C;
  const ChunkRange all{0, NC};
  PrefillArgs a = a0;
  if (a.gate != GDR_GATE_CHANNEL) {
    const WsLayout wl = ws_layout(static_cast<long>(a.B) * a.H_v, NC,
                                  ChunkBlock<OpT, DK, C, true>::kBytes, 0, 0);
    a.ws_qk = static_cast<unsigned char*>(a.ws) + wl.qk;  // right after the blocks
  }
  const hipError_t err = launch_prep<OpT, DK, C>(a, all, stream);
  if (err != hipSuccess) return err;
  const SegPlan sp = carry_segments(a.B, a.T, a.H_v, DK, a.dv, C);
  if (a.gate == GDR_GATE_CHANNEL) {
    if (sp.P >= 3) return launch_carry_segmented<OpT, DK, C, false>(a, sp, stream);
    return launch_carry_any<OpT, DK, C, false>(a, stream);
  }
  if (sp.P >= 3) return launch_carry_segmented<OpT, DK, C, true>(a, sp, stream);
  return launch_carry_any<OpT, DK, C, true>(a, stream);
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

size_t prefill_workspace_bytes(int B, int T, int H_qk, int H_v, int dk, int dv, int chunk,
                               int io_bf16, int gate) {
  if (B <= 0 || T <= 0) return 0;
  const size_t nc = (static_cast<size_t>(T) + chunk - 1) / chunk;
  const bool scalar_gate = gate != GDR_GATE_CHANNEL;
  const size_t bb = io_bf16 ? block_bytes_rt<bf16>(dk, chunk, scalar_gate)
                            : block_bytes_rt<float>(dk, chunk, scalar_gate);
  const size_t qk = qk_region_bytes(scalar_gate, B, H_qk, nc, dk, chunk, io_bf16 ? 2 : 4);
  const SegPlan sp = carry_segments(B, T, H_v, dk, dv, chunk);
  const long units = static_cast<long>(B) * H_v;
  return ws_layout(units, nc, bb, qk, seg_bytes(sp, units, dk, dv)).total;
}

// Scratch of the allocation-free prefill entry point: the workspace of one
// call at a time on each device (every call on a device shares it, so calls
// that overlap on one device race).  In host code `scratch` names a host-side
// stand-in, not device memory: its device address is resolved once per device
// with hipGetSymbolAddress and only that address is ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

hipError_t noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (!p) return hipErrorInvalidSymbol;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
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
  if (a.T <= recurrent_max_t(a.B, a.H_v) &&
      recurrent_lds_bytes(a.T, a.dk, recurrent_dv_slice(a.B, a.H_v, a.dv)) <= kRecurrentMaxLds)
    return launch_recurrent(a, io_bf16, stream);
  return io_bf16 ? launch_io<bf16>(a, stream) : launch_io<float>(a, stream);
}

}  // namespace gdr
