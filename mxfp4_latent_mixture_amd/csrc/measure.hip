// Measurement hook: the sustained bf16 MFMA rate of this GPU under full load,
// the practical ceiling the MFMA-bound prefill GEMMs are held against (at
// prefill sizes the layer is bound by the matrix cores: dev48.org "Kimi K3 on
// AMD Instinct GPUs with TokenSpeed", section 4.4). With every matrix core
// busy the clock settles below the one the 2.5 PFLOP/s figure assumes; this
// kernel measures the rate at that clock.
//
// Each wave runs `iters` rounds of eight independent v_mfma_f32_32x32x16_bf16
// (32768 flops each) on register operands. The accumulators are folded into
// one word per workgroup, so no MFMA is dead.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmoe {

namespace {
typedef __bf16 mr_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float mr_f32x16_t __attribute__((ext_vector_type(16)));
}  // namespace

// Operand bits are random (a per-lane hash): the power a matrix core draws,
// and so the clock it sustains, depends on how many operand bits toggle, and
// the GEMMs multiply random-looking data. Four operand sets are rotated so
// consecutive MFMAs see different operands. Values lie in [2^-7, 2) in
// magnitude, so no sum overflows.
__device__ __forceinline__ uint32_t mr_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(256, 2) void mfma_rate_kernel(int iters, uint32_t* __restrict__ sink) {
  const uint32_t id = blockIdx.x * 256 + threadIdx.x;
  mr_bf16x8_t a[4], b[4];
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t ra = mr_hash(id * 64 + v * 16 + i), rb = mr_hash(id * 64 + v * 16 + 8 + i);
      // sign, exponent 120..127, random mantissa
      a[v][i] = __builtin_bit_cast(__bf16, (uint16_t)((ra & 0x807Fu) | ((120u + ((ra >> 8) & 7u)) << 7)));
      b[v][i] = __builtin_bit_cast(__bf16, (uint16_t)((rb & 0x807Fu) | ((120u + ((rb >> 8) & 7u)) << 7)));
    }
  mr_f32x16_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 3], b[(j + (j >> 2)) & 3], acc[j], 0, 0, 0);
  }
  float x = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) x += acc[j][i];
  uint32_t w = __float_as_uint(x);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) w ^= __shfl_xor(w, off, 64);
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = w;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

hipError_t launch_mfma_rate(int iters, uint32_t* sink, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace lmoe
