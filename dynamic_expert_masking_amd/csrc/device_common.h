// Device-side building blocks shared by the BEAM kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace beam {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Exact widening of a bf16 bit pattern.
__device__ __forceinline__ float bf16_to_f32(u16 b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bf16, round to nearest even (inputs here are finite).
__device__ __forceinline__ u16 f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u16(u >> 16);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Streaming load for weights that are read once per call.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ u32x4 zero16() { return u32x4{0u, 0u, 0u, 0u}; }

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).
// Operand lane layout (v_mfma_f32_16x16x32_bf16): lane l supplies row/column
// (l % 16) and the 8 consecutive k values 8*(l/16) .. 8*(l/16)+7; lane l
// receives D[4*(l/16) + i][l % 16] in element i.  Any permutation of k that
// is applied identically to both operands leaves the product unchanged.
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float silu_f32(float a) { return a / (1.0f + expf(-a)); }

// Order-preserving map from float to uint32 (-0 and +0 map together).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    unsigned long long o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

}  // namespace beam
