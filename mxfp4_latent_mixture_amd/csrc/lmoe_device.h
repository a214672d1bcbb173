// Device-side building blocks shared by the LatentMoE kernels (gfx950 only).
//
// MXFP4 element decode: an E2M1 code c (sign bit 3, magnitudes 0, 0.5, 1, 1.5,
// 2, 3, 4, 6) times 2^(b - 127) for the E8M0 byte b of its 32-wide block
// (infervisor.ai "Bringing up Kimi-K3 on day zero", section "The model we
// hadn't run"). CDNA4 converts two packed E2M1 codes and applies an fp32 scale
// in one instruction (v_cvt_scalef32_pk_bf16_fp4); every product is exact in
// bf16 for the exponent range the layer uses, so decode is bit-exact.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmoe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// 2^(b-127) as fp32; b = 0 is the fp32 subnormal 2^-127, b = 255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  uint32_t bits = (b == 0u) ? 0x00400000u : ((b == 255u) ? 0x7FC00000u : (b << 23));
  return __uint_as_float(bits);
}

// Eight consecutive MXFP4 elements (one dword: element 2m in the low nibble of
// byte m) scaled by `scale`, as eight bf16 in element order.
__device__ __forceinline__ bf16x8_t dequant8(uint32_t w, float scale) {
  bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  bf16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ u32x4_t load16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ u32x4_t zero16() {
  u32x4_t z = {0u, 0u, 0u, 0u};
  return z;
}

// D[16x16] += A[16x32] * B[32x16], bf16 inputs, fp32 accumulate.
// Lane l supplies A row (l % 16) and B column (l % 16), eight K values of
// K-slot (l / 16); D comes back as column (l % 16), rows 4*(l/16) + 0..3.
__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ float silu(float z) {
  return z / (1.0f + __expf(-z));
}

}  // namespace lmoe
