// Dense bf16 GEMMs of the MoE block around the layer (dev48.org "Kimi K3 on
// AMD Instinct GPUs with TokenSpeed", sections 4.2-4.4): the packed input
// projection (router scores, latent input and the shared experts' gate/up in
// one multiply, the shared activation in its epilogue), the shared experts'
// down projection, and the tail's latent -> hidden up-projection that adds
// the shared output and the residual. Plus the routed RMSNorm.
//
// C = A B^T with A bf16 [M][K] (token rows) and B bf16 [N][K] (weight rows,
// the storage the pages describe: matrices one after another, row-major).
// A workgroup computes a BM x 128 tile of C over its K range in chunks of 64,
// with both operands staged in LDS by global-to-LDS loads: one load
// instruction moves 1 KB, 8 rows x 128 contiguous bytes, so weight rows are
// streamed with full cache lines. The 16-byte segments of a staged row are
// XOR-swizzled by the row's low three bits, so the eight rows an MFMA operand
// read serves at once sit in eight different bank groups. Four waves; each
// computes its part of the tile with v_mfma_f32_32x32x16_bf16 from operands
// read out of LDS. NS chunks are in flight (one LDS array per slot: a read of
// one slot never waits for the copy into another).
//
// Small M (decode) splits K over blockIdx.y so that the weight stream is
// spread over enough workgroups; the fp32 partial tiles are then summed in a
// fixed order by a finishing kernel that applies the epilogue, so results do
// not depend on timing.

#include "lmoe_internal.h"
#include "lmoe_device.h"

namespace lmoe {

constexpr int kDnBK = 64;    // K per chunk

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Epilogue of one output element (non-GLU columns) and of one GLU pair.
// extra: the second product's bf16-rounded sum (launch_dense_pair), else 0;
// zo: the output offset of problem blockIdx.z (launch_dense_batched).
__device__ __forceinline__ void dense_store(const DenseArgs& a, int m, int n, float v,
                                            float extra = 0.f, int64_t zo = 0) {
  if (n < a.n_f32) {
    a.f32_out[zo + (int64_t)m * a.ld_f32 + n] = v;
  } else if (n < a.n_f32 + a.n_bf16) {
    const int c = n - a.n_f32;
    float r = v + extra;
    if (a.add0) r += bf16_bits_to_f32(a.add0[(int64_t)m * a.ld_add + c]);
    if (a.add1) r += bf16_bits_to_f32(a.add1[(int64_t)m * a.ld_add + c]);
    a.bf_out[zo + (int64_t)m * a.ld_bf + c] = f32_to_bf16_bits(r);
  }
}
// column n (in the GLU segment, a gate column: n - glu_base mod 32 < 16)
__device__ __forceinline__ void dense_store_glu(const DenseArgs& a, int m, int n, float g,
                                                float u, int64_t zo = 0) {
  const int c = n - (a.n_f32 + a.n_bf16);
  const int col = (c >> 5) * 16 + (c & 15);
  a.glu_out[zo + (int64_t)m * a.ld_glu + col] = f32_to_bf16_bits(silu(g) * u);
}

// physical 16-byte segment of logical segment g (0..7) of staged row r
__device__ __forceinline__ int dn_seg(int r, int g) { return g ^ (r & 7); }

// A BM x BN workgroup tile computed by NW waves, WM of them along M.
template <int BM, int BN, int NW>
struct DnCfg {
  static constexpr int WM = BM >= 64 ? 2 : 1;       // waves along M
  static constexpr int WN = NW / WM;                // waves along N
  static constexpr int TM = BM / WM / 32;           // 32-row MFMA tiles per wave
  static constexpr int TN = BN / WN / 32;           // 32-column MFMA tiles per wave
  static constexpr int kRows = BM + BN;             // staged rows per chunk (A then B)
  static constexpr int kCopies = kRows / 8 / NW;    // DMA instructions per wave and chunk
  static_assert(kCopies * 8 * NW == kRows, "rows shared evenly by the waves");
  static_assert(TM >= 1 && TN >= 1, "at least one MFMA tile per wave");
};

template <int BM, int BN, int NW>
using DnSlot = uint8_t[DnCfg<BM, BN, NW>::kRows * 128];

// The tile of workgroup b: tiles are ordered in groups of G row tiles, all
// columns of a group before the next, and the chip's eight XCDs (workgroup b
// runs on XCD b % 8) each take one contiguous range of that order, so the
// workgroups running together on one XCD share a few A and B tiles in its L2.
__device__ __forceinline__ bool dense_tile(const DenseArgs& a, int* rt, int* ct) {
  const int b = blockIdx.x;
  const int n_tiles = a.n_rt * a.n_ct;
  const int per_xcd = (n_tiles + 7) / 8;
  const int t = (b & 7) * per_xcd + (b >> 3);
  if ((b >> 3) >= per_xcd || t >= n_tiles) return false;
  const int G = a.group_rows;
  const int grp = t / (G * a.n_ct);
  const int w = t - grp * G * a.n_ct;
  const int rows_in = min(G, a.n_rt - grp * G);
  *rt = grp * G + w % rows_in;
  *ct = w / rows_in;
  return true;
}

template <int BM, int BN, int NW, int NS>
__global__ __launch_bounds__(64 * NW, 8 / NW) void dense_gemm_kernel(DenseArgs a) {
  using C = DnCfg<BM, BN, NW>;
  using Slot = DnSlot<BM, BN, NW>;
  __shared__ __attribute__((aligned(16))) Slot s0, s1, s2, s3;
  auto slot = [&](int r) -> Slot& {
    return r == 0 ? s0 : r == 1 ? s1 : r == 2 ? s2 : s3;
  };
  static_assert(NS >= 2 && NS <= 4, "two to four slots");
  int rt, ct;
  if (!dense_tile(a, &rt, &ct)) return;
  const int m0 = rt * BM, n0 = ct * BN;
  // the first product, or (blockIdx.y >= ks1) the second one of a pair
  const bool second = (int)blockIdx.y >= a.ks1;
  const int kz = second ? (int)blockIdx.y - a.ks1 : (int)blockIdx.y;
  const int z = blockIdx.z;
  const int64_t zo = z * a.out_zstride;  // output offset of problem z
  const uint16_t* A = (second ? a.a2 : a.a) + z * a.a_zstride;
  const uint16_t* B = (second ? a.b2 : a.b) + z * a.b_zstride;
  const uint16_t* Bup = a.b_up ? a.b_up + z * a.b_zstride : nullptr;
  const int64_t lda = second ? a.lda2 : a.lda, ldb = second ? a.ldb2 : a.ldb;
  const int K = second ? a.K2 : a.K, k_per = second ? a.k_per2 : a.k_per;
  float* part = second ? a.part2 : a.part;
  const int kb = kz * k_per;                         // first K of this split
  const int nk = min(k_per, K - kb) / kDnBK;         // chunks
  // the wave index in a scalar register: the copies' LDS addresses are then
  // scalar too
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int r32 = lane & 31, hh = lane >> 5;
  const int wm = wave / C::WN, wn = wave % C::WN;

  // this wave's DMA sources: staged rows wave*8*kCopies + 8 i + lane / 8
  const uint16_t* src[C::kCopies];
#pragma unroll
  for (int i = 0; i < C::kCopies; ++i) {
    const int row = (wave * C::kCopies + i) * 8 + (lane >> 3);
    const int g = dn_seg(row, lane & 7);
    const uint16_t* p;
    if (row < BM) {
      p = A + (int64_t)min(m0 + row, a.M - 1) * lda;
    } else {
      const int v = min(n0 + row - BM, a.N - 1);
      if (Bup)  // 16 gate rows, then the 16 up rows of the same outputs
        p = ((v & 16) ? Bup : B) + (int64_t)((v >> 5) * 16 + (v & 15)) * ldb;
      else
        p = B + (int64_t)v * ldb;
    }
    src[i] = p + kb + g * 8;
  }
  auto copy = [&](int c, int buf) {
    const int cc = min(c, nk - 1);
#pragma unroll
    for (int i = 0; i < C::kCopies; ++i)
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(src[i] + cc * kDnBK),
          (__attribute__((address_space(3))) void*)(&slot(buf)[(wave * C::kCopies + i) * 8 * 128]),
          16, 0, 0);
  };

  f32x16_t acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  auto compute = [&](int buf) {
    const uint8_t* sp = slot(buf);
#pragma unroll
    for (int s = 0; s < kDnBK / 16; ++s) {
      bf16x8_t av[C::TM], bv[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        const int row = wm * (BM / C::WM) + i * 32 + r32;
        av[i] = *reinterpret_cast<const bf16x8_t*>(sp + row * 128 + 16 * dn_seg(row, 2 * s + hh));
      }
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        const int row = BM + wn * (BN / C::WN) + j * 32 + r32;
        bv[j] = *reinterpret_cast<const bf16x8_t*>(sp + row * 128 + 16 * dn_seg(row, 2 * s + hh));
      }
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
  };

  // chunk c's copies are complete once only the copies of the NS - 2 later
  // chunks are outstanding
  constexpr int kAhead = (NS - 2) * C::kCopies;
  static_assert(kAhead < 64, "vmcnt field");
  constexpr int kWait = 0x0F70 | (kAhead & 15) | ((kAhead >> 4) << 14);
#pragma unroll
  for (int i = 0; i < NS - 1; ++i) copy(i, i);
  auto group = [&](int cb, bool last) {
#pragma unroll
    for (int r = 0; r < NS; ++r) {
      const int c = cb + r;
      __builtin_amdgcn_s_waitcnt(kWait);
      __builtin_amdgcn_s_barrier();
      copy(c + NS - 1, (r + NS - 1) % NS);
      __builtin_amdgcn_sched_barrier(0);
      if (!last || c < nk) compute(r);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const int full = nk / NS;
  if (full > 0) group(0, false);
  for (int g = 1; g < full; ++g) group(g * NS, false);
  if (nk % NS) group(full * NS, true);
  __builtin_amdgcn_s_waitcnt(0);

  // fully unrolled, so every accumulator index is a constant (registers,
  // not scratch)
#pragma clang loop unroll(full)
  for (int i = 0; i < C::TM; ++i)
#pragma clang loop unroll(full)
    for (int j = 0; j < C::TN; ++j) {
      const int nb = n0 + wn * (BN / C::WN) + j * 32;  // first column of the MFMA tile
      const int n = nb + r32;
      const bool glu = nb >= a.n_f32 + a.n_bf16;          // the same for the whole tile
#pragma clang loop unroll(full)
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * (BM / C::WM) + i * 32 + 8 * (e / 4) + 4 * hh + (e & 3);
        const float v = acc[i][j][e];
        if (part) {
          if (m < a.M && n < a.N) part[((int64_t)kz * a.M + m) * a.N + n] = v;
        } else if (glu) {
          const float u = __shfl_down(v, 16, 64);
          if (r32 < 16 && m < a.M && n < a.N) dense_store_glu(a, m, n, v, u, zo);
        } else if (m < a.M && n < a.N) {
          dense_store(a, m, n, v, 0.f, zo);
        }
      }
    }
}

// Sum of the K-split partial tiles in split order, then the epilogue: one
// thread per output element (a GLU thread takes its gate and up columns).
// ksplit2 > 0: a pair, the second product's sum rounded to bf16 and added.
__global__ __launch_bounds__(256) void dense_finish_kernel(DenseArgs a, int ksplit, int ksplit2) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.M * a.N) return;
  const int m = (int)(i / a.N), n = (int)(i - (int64_t)m * a.N);
  const int gb = a.n_f32 + a.n_bf16;
  if (n >= gb && ((n - gb) & 16)) return;  // up columns: read by their gate column's thread
  float v = 0.f;
  for (int z = 0; z < ksplit; ++z) v += a.part[((int64_t)z * a.M + m) * a.N + n];
  if (n >= gb) {
    float u = 0.f;
    for (int z = 0; z < ksplit; ++z) u += a.part[((int64_t)z * a.M + m) * a.N + n + 16];
    dense_store_glu(a, m, n, v, u);
  } else {
    float extra = 0.f;
    if (ksplit2) {
      for (int z = 0; z < ksplit2; ++z) extra += a.part2[((int64_t)z * a.M + m) * a.N + n];
      extra = bf16_bits_to_f32(f32_to_bf16_bits(extra));
    }
    dense_store(a, m, n, v, extra);
  }
}

// Routed RMSNorm: n = bf16(r * (1 / sqrt(mean(r^2) + eps)) * gamma), one
// workgroup per row, the squares summed in fp32. The row is read once, 16
// bytes per thread and step (L % 8 == 0), and kept in registers for the
// scaling pass (up to kRmsVec vectors per thread: L <= 16384).
constexpr int kRmsVec = 8;
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ r,
                                                      const uint16_t* __restrict__ gamma,
                                                      int L, float eps,
                                                      uint16_t* __restrict__ out) {
  __shared__ float part[4];
  const int row = blockIdx.x;
  const u32x4_t* rr = reinterpret_cast<const u32x4_t*>(r + (int64_t)row * L);
  const int nv = L / 8;
  u32x4_t v[kRmsVec];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kRmsVec; ++j) {
    const int i = threadIdx.x + 256 * j;
    v[j] = i < nv ? rr[i] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float lo = __uint_as_float(v[j][q] << 16), hi = __uint_as_float(v[j][q] & 0xFFFF0000u);
      s += lo * lo + hi * hi;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float inv = 1.f / sqrtf(tot / (float)L + eps);
  const u32x4_t* gv = reinterpret_cast<const u32x4_t*>(gamma);
  u32x4_t* ov = reinterpret_cast<u32x4_t*>(out + (int64_t)row * L);
#pragma unroll
  for (int j = 0; j < kRmsVec; ++j) {
    const int i = threadIdx.x + 256 * j;
    if (i < nv) {
      const u32x4_t g = gv[i];
      u32x4_t o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = __uint_as_float(v[j][q] << 16) * inv * __uint_as_float(g[q] << 16);
        const float hi =
            __uint_as_float(v[j][q] & 0xFFFF0000u) * inv * __uint_as_float(g[q] & 0xFFFF0000u);
        o[q] = (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
      }
      ov[i] = o;
    }
  }
}

DensePlan dense_plan(int M, int N, int K) {
  DensePlan p;
  p.bm = M <= 32 ? 32 : M <= 64 ? 64 : 128;
  p.bn = 128;
#ifndef LMOE_DENSE_BIG
#define LMOE_DENSE_BIG 1
#endif
  // enough rows for several 256-row tiles: 256 x 256 tiles of eight waves,
  // 128 x 64 each (0.75 KB of operand reads per MFMA, against 1 KB at 64 x 64)
  if (LMOE_DENSE_BIG && M >= 512 && N >= 1024) p.bm = p.bn = 256;
  const int n_rt = (M + p.bm - 1) / p.bm, n_ct = (N + p.bn - 1) / p.bn;
  const int tiles = n_rt * n_ct;
  const int nkc = K / kDnBK;
  // Fewer tiles than resident workgroups (two per CU): split K. The split
  // count minimises (rounds of resident workgroups) x (chunks each streams,
  // plus about two chunks of start-up), so the grid fills whole rounds with
  // long-lived workgroups rather than leaving a last round half empty.
  constexpr int kSlots = 512;
  int best = 1;
  if (tiles < kSlots) {
    double best_cost = 1e30;
    for (int ks = 1; ks <= std::min(nkc, 64); ++ks) {
      const int per = (nkc + ks - 1) / ks;
      const int kse = (nkc + per - 1) / per;
      const double rounds = (double)((tiles * kse + kSlots - 1) / kSlots);
      const double cost = rounds * (per + 2) + (kse > 1 ? 1.0 : 0.0);  // + the finishing pass
      if (cost < best_cost - 1e-9) {
        best_cost = cost;
        best = kse;
      }
    }
  }
  const int per = (nkc + best - 1) / best;
  p.ksplit = (nkc + per - 1) / per;
  p.k_per = per * kDnBK;
  p.part_floats = p.ksplit > 1 ? (size_t)p.ksplit * M * N : 0;
  return p;
}

static hipError_t launch_gemm_grid(const DenseArgs& a, int bm, int ky, hipStream_t s) {
  const int n_tiles = a.n_rt * a.n_ct;
  const dim3 grid((unsigned)(8 * ((n_tiles + 7) / 8)), (unsigned)ky);
  if (bm == 32)
    hipLaunchKernelGGL((dense_gemm_kernel<32, 128, 4, 3>), grid, dim3(256), 0, s, a);
  else if (bm == 64)
    hipLaunchKernelGGL((dense_gemm_kernel<64, 128, 4, 3>), grid, dim3(256), 0, s, a);
  else if (bm == 128)
    hipLaunchKernelGGL((dense_gemm_kernel<128, 128, 4, 2>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((dense_gemm_kernel<256, 256, 8, 2>), grid, dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dense(DenseArgs a, const DensePlan& p, float* part, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  a.n_rt = (a.M + p.bm - 1) / p.bm;
  a.n_ct = (a.N + p.bn - 1) / p.bn;
  a.group_rows = 4;
  a.k_per = p.k_per;
  a.ks1 = p.ksplit;  // no second product
  a.part = p.ksplit > 1 ? part : nullptr;
  a.part2 = nullptr;
  hipError_t err = launch_gemm_grid(a, p.bm, p.ksplit, s);
  if (err != hipSuccess || p.ksplit == 1) return err;
  const int64_t n = (int64_t)a.M * a.N;
  hipLaunchKernelGGL(dense_finish_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a,
                     p.ksplit, 0);
  return hipGetLastError();
}

hipError_t launch_dense_batched(DenseArgs a, int nz, hipStream_t s) {
  if (a.M == 0 || nz == 0) return hipSuccess;
  DensePlan p = dense_plan(a.M, a.N, a.K);
  p.ksplit = 1;  // no K split across problems
  p.k_per = a.K;
  a.n_rt = (a.M + p.bm - 1) / p.bm;
  a.n_ct = (a.N + p.bn - 1) / p.bn;
  a.group_rows = 4;
  a.k_per = p.k_per;
  a.ks1 = 1;
  a.part = a.part2 = nullptr;
  const int n_tiles = a.n_rt * a.n_ct;
  const dim3 grid((unsigned)(8 * ((n_tiles + 7) / 8)), 1, (unsigned)nz);
  if (p.bm == 32)
    hipLaunchKernelGGL((dense_gemm_kernel<32, 128, 4, 3>), grid, dim3(256), 0, s, a);
  else if (p.bm == 64)
    hipLaunchKernelGGL((dense_gemm_kernel<64, 128, 4, 3>), grid, dim3(256), 0, s, a);
  else if (p.bm == 128)
    hipLaunchKernelGGL((dense_gemm_kernel<128, 128, 4, 2>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((dense_gemm_kernel<256, 256, 8, 2>), grid, dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dense_pair(DenseArgs a, const DensePlan& p1, const DensePlan& p2, float* part,
                             hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  if (p1.bm != p2.bm || p1.bn != p2.bn || p1.ksplit < 2 || p2.ksplit < 2)
    return hipErrorInvalidValue;
  a.n_rt = (a.M + p1.bm - 1) / p1.bm;
  a.n_ct = (a.N + p1.bn - 1) / p1.bn;
  a.group_rows = 4;
  a.k_per = p1.k_per;
  a.k_per2 = p2.k_per;
  a.ks1 = p1.ksplit;
  a.part = part;
  a.part2 = part + p1.part_floats;
  hipError_t err = launch_gemm_grid(a, p1.bm, p1.ksplit + p2.ksplit, s);
  if (err != hipSuccess) return err;
  const int64_t n = (int64_t)a.M * a.N;
  hipLaunchKernelGGL(dense_finish_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a,
                     p1.ksplit, p2.ksplit);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const uint16_t* r, const uint16_t* gamma, int T, int L, float eps,
                          uint16_t* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)T), dim3(256), 0, s, r, gamma, L, eps, out);
  return hipGetLastError();
}

}  // namespace lmoe
