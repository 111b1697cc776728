// Device-side building blocks shared by the BEAM kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace beam {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Load through the constant address space, for data that nothing writes
// while the kernel runs (e.g. the routing plan, written by an earlier
// kernel).  A wave-uniform address then becomes a scalar load, which is
// counted apart from the vector loads in flight, so waiting for it does not
// drain them.
template <class T>
__device__ __forceinline__ T ld_const(const T* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) T*>(reinterpret_cast<uintptr_t>(p));
}

constexpr int kWave = 64;

// Exact widening of a bf16 bit pattern.
__device__ __forceinline__ float bf16_to_f32(u16 b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bf16, round to nearest even (inputs here are finite).
__device__ __forceinline__ u16 f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u16(u >> 16);
}

// Four consecutive elements at base[elem], as floats: bf16 (BF16) or fp32.
template <bool BF16>
__device__ __forceinline__ float4 ld4_f32(const void* base, size_t elem) {
  if (BF16) {
    const ushort4 v = *reinterpret_cast<const ushort4*>(static_cast<const u16*>(base) + elem);
    return make_float4(bf16_to_f32(v.x), bf16_to_f32(v.y), bf16_to_f32(v.z), bf16_to_f32(v.w));
  }
  return *reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
}

// Four floats rounded to bf16 and stored at base[elem] (8 bytes).
__device__ __forceinline__ void st4_bf16(u16* base, size_t elem, float a, float b, float c, float d) {
  ushort4 v;
  v.x = f32_to_bf16(a);
  v.y = f32_to_bf16(b);
  v.z = f32_to_bf16(c);
  v.w = f32_to_bf16(d);
  *reinterpret_cast<ushort4*>(base + elem) = v;
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Streaming load for weights that are read once per call.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ u32x4 zero16() { return u32x4{0u, 0u, 0u, 0u}; }

// Eight OCP FP8 E4M3 codes (the bytes of w0 then w1, in memory order) widened
// to eight bf16 values in the same order.  Every E4M3 value, subnormals
// included, is exactly representable in bf16, so the conversion is exact
// (scale operand 1.0: no exponent adjustment).
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true))};
}

// Scales of 16 consecutive rows starting at p (wave-uniform, 16-byte
// aligned), read with scalar loads; lane l receives those of rows
// 4*(l/16) .. 4*(l/16)+3, the rows of its MFMA accumulator elements.
__device__ __forceinline__ f32x4 row_scales16(const float* p, int lane) {
  const f32x4* q = reinterpret_cast<const f32x4*>(p);
  const f32x4 s0 = ld_const(q), s1 = ld_const(q + 1), s2 = ld_const(q + 2), s3 = ld_const(q + 3);
  const int g = lane >> 4;
  return g == 0 ? s0 : g == 1 ? s1 : g == 2 ? s2 : s3;
}

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

// Order-preserving map from float to uint32: a larger float has a larger
// key, and -0 and +0 map together (logits are never NaN).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Inverse of float_key (-0 comes back as +0).
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// ---- wave-wide sums without LDS round trips --------------------------------
// Within each 16-lane row, rotations by 8, 4, 2, 1 (DPP row_ror) leave every
// lane holding the row's sum; the four row results are then read with
// v_readlane and combined in row order 0..3, so every lane receives the same,
// order-fixed result.

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;

__device__ __forceinline__ float dpp_f32_ror(float v, int step) {
  const uint32_t u = __float_as_uint(v);
  uint32_t r;
  switch (step) {
    case 8: r = dpp_u32<kRowRor8>(u); break;
    case 4: r = dpp_u32<kRowRor4>(u); break;
    case 2: r = dpp_u32<kRowRor2>(u); break;
    default: r = dpp_u32<kRowRor1>(u); break;
  }
  return __uint_as_float(r);
}

// Sum over the wave; identical in every lane.
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32_ror(v, 8);
  v += dpp_f32_ror(v, 4);
  v += dpp_f32_ror(v, 2);
  v += dpp_f32_ror(v, 1);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Inclusive prefix sum over the wave (lane l gets v_0 + ... + v_l).
__device__ __forceinline__ int32_t wave_inclusive_scan_i32(int32_t v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

}  // namespace beam
