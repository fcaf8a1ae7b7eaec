// device_common.hpp -- small gfx950 device helpers: bf16 <-> fp32, vector
// loads/stores of io-dtype rows, wave64 reductions and the gate functions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

using bf16 = __bf16;

constexpr float kL2Eps = 1e-6f;  // x / sqrt(sum x^2 + eps)

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// Load N contiguous io-dtype values (16-byte aligned when N*sizeof(T) >= 16)
// and widen them to fp32.
template <typename T, int N>
__device__ __forceinline__ void load_row(const T* __restrict__ p, float (&out)[N]) {
  constexpr int kBytes = N * static_cast<int>(sizeof(T));
  if constexpr (kBytes % 16 == 0) {
    constexpr int kPer = 16 / static_cast<int>(sizeof(T));
#pragma unroll
    for (int c = 0; c < N / kPer; ++c) {
      uint4 raw = reinterpret_cast<const uint4*>(p)[c];
      const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int u = 0; u < kPer; ++u) out[c * kPer + u] = to_f32(e[u]);
    }
  } else if constexpr (kBytes % 8 == 0) {
    constexpr int kPer = 8 / static_cast<int>(sizeof(T));
#pragma unroll
    for (int c = 0; c < N / kPer; ++c) {
      uint2 raw = reinterpret_cast<const uint2*>(p)[c];
      const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int u = 0; u < kPer; ++u) out[c * kPer + u] = to_f32(e[u]);
    }
  } else {
#pragma unroll
    for (int u = 0; u < N; ++u) out[u] = to_f32(p[u]);
  }
}

// Store 4 fp32 values as io dtype (8 or 16 bytes, aligned).
template <typename T>
__device__ __forceinline__ void store4(T* __restrict__ p, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  } else {
    T e[4] = {from_f32<T>(a), from_f32<T>(b), from_f32<T>(c), from_f32<T>(d)};
    *reinterpret_cast<uint2*>(p) = *reinterpret_cast<const uint2*>(e);
  }
}

// store4 with the non-temporal cache policy (the value goes to memory
// without being kept in the caches).
typedef unsigned nt_u32x2 __attribute__((ext_vector_type(2)));
typedef float nt_f32x4 __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ void store4_nt(T* __restrict__ p, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 4) {
    const nt_f32x4 v = {a, b, c, d};
    __builtin_nontemporal_store(v, reinterpret_cast<nt_f32x4*>(p));
  } else {
    const T e[4] = {from_f32<T>(a), from_f32<T>(b), from_f32<T>(c), from_f32<T>(d)};
    nt_u32x2 w;
    __builtin_memcpy(&w, e, sizeof(w));
    __builtin_nontemporal_store(w, reinterpret_cast<nt_u32x2*>(p));
  }
}

// Store 4 io-dtype values held as T (8 or 16 bytes, aligned).
template <typename T>
__device__ __forceinline__ void store_vec4(T* __restrict__ p, const T (&v)[4]) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<uint4*>(p) = *reinterpret_cast<const uint4*>(v);
  } else {
    *reinterpret_cast<uint2*>(p) = *reinterpret_cast<const uint2*>(v);
  }
}

// Sum of x over the lanes of a wave that share lane % OFF (OFF a power of two
// below 64); every such lane gets the sum.  Inside each 16-lane row the sum
// is taken by row rotations (DPP row_ror by OFF, 2 OFF, ... 8: after them a
// lane holds its row's sum over its residue class), across rows by lane
// exchanges (xor 16, 32).  A rotation step costs one VALU instruction, a lane
// exchange a round trip through the LDS crossbar.
template <int OFF>
__device__ __forceinline__ float lane_class_sum(float x) {
  if constexpr (OFF >= 64) {
    return x;
  } else {
    if constexpr (OFF < 16)
      x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         0u, __builtin_bit_cast(unsigned, x), 0x120 + OFF,
                                         0xf, 0xf, false));  // row_ror:OFF
    else
      x += __shfl_xor(x, OFF, 64);
    return lane_class_sum<2 * OFF>(x);
  }
}

// Sum over each 16-lane row of a wave (DPP row rotations only); every lane
// gets its row's total.
__device__ __forceinline__ float row16_sum(float x) {
#define GDR_ROR(n)                                                                      \
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(                           \
                                     0u, __builtin_bit_cast(unsigned, x), 0x120 + (n), \
                                     0xf, 0xf, false))
  GDR_ROR(1);
  GDR_ROR(2);
  GDR_ROR(4);
  GDR_ROR(8);
#undef GDR_ROR
  return x;
}

// Sum over the 64 lanes of a wave; every lane gets the total.
__device__ __forceinline__ float wave_sum(float x) { return lane_class_sum<1>(x); }

__device__ __forceinline__ float sigmoidf(float x) { return 1.0f / (1.0f + expf(-x)); }

// softplus(z) = log(1 + e^z), written so that large |z| neither overflows nor
// loses the linear tail.
__device__ __forceinline__ float softplusf(float z) {
  return z > 0.0f ? z + log1pf(expf(-z)) : log1pf(expf(z));
}

// Fused GatedDeltaNet scalar log-decay: -exp(A_log) * softplus(x + dt_bias).
__device__ __forceinline__ float fused_log_decay(float x, float A_log, float dt_bias) {
  return -expf(A_log) * softplusf(x + dt_bias);
}

}  // namespace gdr
