// Expert kernels: grouped GEMMs over the selected experts with MXFP4 weights
// decoded to bf16 in registers and fed to bf16 MFMA, the shared experts with
// bf16 weights, and the deterministic combine.
//
// Per expert e and route r of token t (dev48.org "Kimi K3 on AMD Instinct GPUs
// with TokenSpeed", section 4; the pages print the activation word garbled,
// SiLU is used):
//     h_r = bf16( silu(x_t Gq_e^T) * (x_t Uq_e^T) )      gate/up + GLU, fused
//     y_r = h_r Dq_e^T                                    down, fp32 partials
//     out_t = bf16( sum_j w_(t,j) y_(t,j) + sum_s ysh_(s,t) )
// Route partials are kept in fp32 and summed in a fixed order (TokenSpeed
// section 4.3 writes route partials and sums them in FP32).
//
// MFMA K-slot mapping. A 16x16x32 bf16 MFMA sums 4 lane groups x 8 K values.
// The sum is over K, so any assignment of K values to (lane group, element)
// works as long as A and B use the same one. Here a lane group always takes
// whole 32-value MX blocks: one 16-byte load of codes plus one scale byte
// feeds four MFMA steps, and no lane ever needs another lane's scale.
#include "lmoe_device.h"
#include "lmoe_internal.h"

namespace lmoe {

struct GemmArgs {
  // Activations (bf16 rows). Row of sorted position p: gather ? gather[p] / gather_div : p.
  const uint16_t* act;
  int64_t act_stride;   // elements between rows
  int64_t act_estride;  // elements between experts (dense mode)
  const int32_t* gather;
  int gather_div;
  // Tiles: routed mode reads (expert, first position, rows) from `tiles`;
  // dense mode (tiles == nullptr) uses expert = blockIdx.z and rows 0..dense_rows-1.
  const int32_t* tiles;
  const int32_t* ntiles;
  int dense_rows;
  // Weights of expert e: MXFP4 codes q + e*q_estride, exponents s + e*s_estride,
  // or bf16 rows b + e*b_estride. Matrix 1 is the up projection of a GLU.
  const uint8_t* q0;
  const uint8_t* s0;
  const uint8_t* q1;
  const uint8_t* s1;
  const uint16_t* b0;
  const uint16_t* b1;
  int64_t q_estride, s_estride, b_estride;
  int N, K;
  // Output row of sorted position p (dense: e*dense_rows + p).
  uint16_t* h_out;  // GLU: bf16 [rows][N]
  float* y_out;     // plain: fp32 [rows][N]
  int64_t out_stride;
  int n_tiles_n;    // column tiles per row tile
};

struct TileInfo {
  int e, p0, cnt;
};

__device__ __forceinline__ bool resolve_tile(const GemmArgs& a, int tile, int rows,
                                             TileInfo* ti) {
  if (a.tiles) {
    if (tile >= *a.ntiles) return false;
    ti->e = a.tiles[3 * tile + 0];
    ti->p0 = a.tiles[3 * tile + 1];
    ti->cnt = a.tiles[3 * tile + 2];
  } else {
    ti->e = blockIdx.z;
    ti->p0 = tile * rows;
    ti->cnt = min(rows, a.dense_rows - ti->p0);
    if (ti->cnt <= 0) return false;
  }
  return true;
}

__device__ __forceinline__ const uint16_t* act_row(const GemmArgs& a, const TileInfo& ti, int r) {
  const int p = ti.p0 + r;
  int64_t row = a.gather ? (int64_t)(a.gather[p] / a.gather_div) : (int64_t)p;
  const uint16_t* base = a.act + (a.tiles ? 0 : (int64_t)ti.e * a.act_estride);
  return base + row * a.act_stride;
}

__device__ __forceinline__ int64_t out_row(const GemmArgs& a, const TileInfo& ti, int r) {
  const int64_t p = ti.p0 + r;
  return a.tiles ? p : (int64_t)ti.e * a.dense_rows + p;
}

// ---------------------------------------------------------------------------
// Small groups (<= 16 rows): one 16-row x 16-column output tile per
// workgroup, K split over the four waves in contiguous quarters. In a wave
// iteration the four lane groups take adjacent runs of U MX blocks, so one
// wave-wide load covers 4*U*16 contiguous bytes of every weight row it touches
// (whole cache lines, nothing fetched twice). The next iteration's weight
// loads are issued before the current iteration's MFMAs. The four waves'
// partial tiles are added in LDS in a fixed order.
// ---------------------------------------------------------------------------
template <bool FP4>
struct SmallOps;

template <>
struct SmallOps<true> {  // two MX blocks of codes and their exponents per matrix
  u32x4_t c0[2], c1[2];
  uint32_t s0[2], s1[2];
};

template <>
struct SmallOps<false> {  // one 32-value block of bf16 weights per matrix
  u32x4_t b0[4], b1[4];
};

template <bool GLU, bool FP4>
__global__ __launch_bounds__(256) void gemm_small_kernel(GemmArgs a) {
  constexpr int U = FP4 ? 2 : 1;   // MX blocks per lane per iteration
  constexpr int SPAN = 4 * U;      // blocks per wave iteration
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int nt = blockIdx.x % a.n_tiles_n;
  const int tile = blockIdx.x / a.n_tiles_n;
  TileInfo ti;
  if (!resolve_tile(a, tile, kSmallRows, &ti)) return;

  const int K = a.K, N = a.N;
  const int n0 = nt * 16;
  const int nblk = K / 32;
  const int bw_lo = (wave * nblk) / 4;
  const int bw_hi = ((wave + 1) * nblk) / 4;
  const int iters = (bw_hi - bw_lo + SPAN - 1) / SPAN;

  const bool mvalid = col < ti.cnt;
  const uint16_t* ap = mvalid ? act_row(a, ti, col) : a.act;
  const int n = n0 + col;
  const bool nvalid = n < N;
  const int nn = nvalid ? n : 0;

  const uint8_t* q0r = nullptr;
  const uint8_t* s0r = nullptr;
  const uint8_t* q1r = nullptr;
  const uint8_t* s1r = nullptr;
  const uint16_t* b0r = nullptr;
  const uint16_t* b1r = nullptr;
  if (FP4) {
    q0r = a.q0 + ti.e * a.q_estride + (int64_t)nn * (K / 2);
    s0r = a.s0 + ti.e * a.s_estride + (int64_t)nn * (K / 32);
    if (GLU) {
      q1r = a.q1 + ti.e * a.q_estride + (int64_t)nn * (K / 2);
      s1r = a.s1 + ti.e * a.s_estride + (int64_t)nn * (K / 32);
    }
  } else {
    b0r = a.b0 + ti.e * a.b_estride + (int64_t)nn * K;
    if (GLU) b1r = a.b1 + ti.e * a.b_estride + (int64_t)nn * K;
  }

  // first block of this lane in iteration it
  auto first_blk = [&](int it) { return bw_lo + it * SPAN + grp * U; };

  auto load_ops = [&](int it, SmallOps<FP4>& o) {
    const int b0 = first_blk(it);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int blk = b0 + u;
      const bool ok = nvalid && it < iters && blk < bw_hi;
      if constexpr (FP4) {
        o.c0[u] = ok ? load16(q0r + blk * 16) : zero16();
        o.s0[u] = ok ? (uint32_t)s0r[blk] : 127u;
        if (GLU) {
          o.c1[u] = ok ? load16(q1r + blk * 16) : zero16();
          o.s1[u] = ok ? (uint32_t)s1r[blk] : 127u;
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          o.b0[q] = ok ? load16(b0r + blk * 32 + q * 8) : zero16();
          if (GLU) o.b1[q] = ok ? load16(b1r + blk * 32 + q * 8) : zero16();
        }
      }
    }
  };

  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f};
  f32x4_t acc1 = {0.f, 0.f, 0.f, 0.f};
  SmallOps<FP4> cur, nxt;
  load_ops(0, cur);
  for (int it = 0; it < iters; ++it) {
    load_ops(it + 1, nxt);
    const int b0 = first_blk(it);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int blk = b0 + u;
      const bool aok = mvalid && blk < bw_hi;
      u32x4_t xv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) xv[q] = aok ? load16(ap + blk * 32 + q * 8) : zero16();
      float sc0 = 1.f, sc1 = 1.f;
      if constexpr (FP4) {
        sc0 = e8m0_to_f32(cur.s0[u]);
        if (GLU) sc1 = e8m0_to_f32(cur.s1[u]);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x8_t bv0, bv1;
        if constexpr (FP4) {
          bv0 = dequant8(cur.c0[u][q], sc0);
          if (GLU) bv1 = dequant8(cur.c1[u][q], sc1);
        } else {
          bv0 = as_bf16x8(cur.b0[q]);
          if (GLU) bv1 = as_bf16x8(cur.b1[q]);
        }
        const bf16x8_t av = as_bf16x8(xv[q]);
        acc0 = mfma16(av, bv0, acc0);
        if (GLU) acc1 = mfma16(av, bv1, acc1);
      }
    }
    cur = nxt;
  }

  __shared__ f32x4_t red[2][4][64];
  red[0][wave][lane] = acc0;
  if (GLU) red[1][wave][lane] = acc1;
  __syncthreads();
  if (wave != 0) return;
  f32x4_t g4 = red[0][0][lane];
  g4 += red[0][1][lane];
  g4 += red[0][2][lane];
  g4 += red[0][3][lane];
  f32x4_t u4 = {0.f, 0.f, 0.f, 0.f};
  if (GLU) {
    u4 = red[1][0][lane];
    u4 += red[1][1][lane];
    u4 += red[1][2][lane];
    u4 += red[1][3][lane];
  }
  if (!nvalid) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = grp * 4 + j;
    if (r < ti.cnt) {
      const int64_t o = out_row(a, ti, r) * a.out_stride + n;
      if (GLU) {
        a.h_out[o] = f32_to_bf16_bits(silu(g4[j]) * u4[j]);
      } else {
        a.y_out[o] = g4[j];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Large groups (<= 128 rows): 128 rows x 128 columns per workgroup; each wave
// owns 32 columns (two 16-wide MFMA tiles, paired gate/up tiles for the GLU)
// over all row tiles. Activations are staged in LDS one 128-wide K chunk at a
// time; in a chunk lane group g takes MX block g, so one 16-byte code load
// and one scale feed the four MFMA steps of that block. The chunk after the
// current one (activations into registers, then LDS; MXFP4 weights into
// registers) is loaded while the current one is multiplied, the LDS chunk is
// double-buffered with one barrier per chunk, and two workgroups share a CU
// (accumulators in AGPRs) so one's loads overlap the other's MFMAs.
// ---------------------------------------------------------------------------
constexpr int kLgCols = 128;
constexpr int kLgKc = 128;
constexpr int kLgPad = kLgKc + 8;  // LDS row length in bf16

template <bool GLU, bool FP4>
__global__ __launch_bounds__(256, 2) void gemm_large_kernel(GemmArgs a) {
  // two K chunks of the tile's activations: the MFMAs read one while the next
  // is written
  __shared__ __attribute__((aligned(16))) uint16_t sx[2][kLargeRows][kLgPad];
  __shared__ const uint16_t* s_arow[kLargeRows];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int nt = blockIdx.x % a.n_tiles_n;
  const int tile = blockIdx.x / a.n_tiles_n;
  TileInfo ti;
  if (!resolve_tile(a, tile, kLargeRows, &ti)) return;
  const int K = a.K, N = a.N;
  const int nblk = K / 32;
  const int nchunks = (nblk + 3) / 4;
  const int n0 = nt * kLgCols + wave * 32;
  const int mtiles = (ti.cnt + 15) / 16;

  // rows past the tile repeat its last row: finite values, never stored
  for (int r = tid; r < kLargeRows; r += 256) s_arow[r] = act_row(a, ti, min(r, ti.cnt - 1));

  int nrow[2];
  bool nvalid[2];
  const uint8_t* q0r[2];
  const uint8_t* s0r[2];
  const uint8_t* q1r[2];
  const uint8_t* s1r[2];
  const uint16_t* b0r[2];
  const uint16_t* b1r[2];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    nrow[w] = n0 + w * 16 + col;
    nvalid[w] = nrow[w] < N;
    const int nn = nvalid[w] ? nrow[w] : 0;  // padding columns read row 0, never stored
    if (FP4) {
      q0r[w] = a.q0 + ti.e * a.q_estride + (int64_t)nn * (K / 2);
      s0r[w] = a.s0 + ti.e * a.s_estride + (int64_t)nn * (K / 32);
      q1r[w] = GLU ? a.q1 + ti.e * a.q_estride + (int64_t)nn * (K / 2) : q0r[w];
      s1r[w] = GLU ? a.s1 + ti.e * a.s_estride + (int64_t)nn * (K / 32) : s0r[w];
      b0r[w] = b1r[w] = nullptr;
    } else {
      b0r[w] = a.b0 + ti.e * a.b_estride + (int64_t)nn * K;
      b1r[w] = GLU ? a.b1 + ti.e * a.b_estride + (int64_t)nn * K : b0r[w];
      q0r[w] = s0r[w] = q1r[w] = s1r[w] = nullptr;
    }
  }

  f32x4_t acc0[8][2], acc1[8][2];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      acc0[m][w] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      acc1[m][w] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

  // Activation staging: thread tid moves row (tid >> 4) + 16 i, values
  // q * 8 .. q * 8 + 7 of the chunk, for the tile's 16-row groups i < mtiles.
  const int srow = tid >> 4, sq = tid & 15;
  u32x4_t xr[8];
  auto load_x = [&](int c) {
    const int kk = c * kLgKc + sq * 8;
    const int kc = min(kk, K - 8);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < mtiles) {
        const u32x4_t v = load16(s_arow[srow + 16 * i] + kc);
        xr[i] = kk < K ? v : zero16();
      }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < mtiles) *reinterpret_cast<u32x4_t*>(&sx[buf][srow + 16 * i][sq * 8]) = xr[i];
  };
  // MXFP4 weights of a chunk: one 32-value block per lane, codes and exponent
  struct Bfp4 {
    u32x4_t c0[2], c1[2];
    uint32_t e0[2], e1[2];
  };
  auto load_b = [&](int c, Bfp4& b) {
    const int blk = min(c * 4 + grp, nblk - 1);
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      b.c0[w] = load16(q0r[w] + blk * 16);
      b.e0[w] = s0r[w][blk];
      if (GLU) {
        b.c1[w] = load16(q1r[w] + blk * 16);
        b.e1[w] = s1r[w][blk];
      }
    }
  };

  auto compute = [&](int c, int buf, const Bfp4& bq) {
    const int blk = c * 4 + grp;
    const bool kv = blk < nblk;  // past-the-end blocks: zero codes
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8_t bv0[2], bv1[2];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        if (FP4) {
          bv0[w] = dequant8(kv ? bq.c0[w][s] : 0u, e8m0_to_f32(kv ? bq.e0[w] : 127u));
          if (GLU) bv1[w] = dequant8(kv ? bq.c1[w][s] : 0u, e8m0_to_f32(kv ? bq.e1[w] : 127u));
        } else {
          const int bb = min(blk, nblk - 1);
          const u32x4_t v0 = load16(b0r[w] + bb * 32 + s * 8);
          bv0[w] = as_bf16x8(kv ? v0 : zero16());
          if (GLU) {
            const u32x4_t v1 = load16(b1r[w] + bb * 32 + s * 8);
            bv1[w] = as_bf16x8(kv ? v1 : zero16());
          }
        }
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if (m < mtiles) {
          const bf16x8_t av =
              *reinterpret_cast<const bf16x8_t*>(&sx[buf][m * 16 + col][grp * 32 + s * 8]);
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            acc0[m][w] = mfma16(av, bv0[w], acc0[m][w]);
            if (GLU) acc1[m][w] = mfma16(av, bv1[w], acc1[m][w]);
          }
        }
      }
    }
  };

  __syncthreads();  // s_arow
  Bfp4 bc, bn;
  load_x(0);
  if (FP4) load_b(0, bc);
  store_x(0);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    // the next chunk's activations and weights are in flight during this one
    // (the last iteration reloads its own chunk: harmless, never stored)
    const int cn = min(c + 1, nchunks - 1);
    load_x(cn);
    if (FP4) load_b(cn, bn);
    compute(c, c & 1, bc);
    store_x((c + 1) & 1);
    __syncthreads();
    if (FP4) bc = bn;
  }

#pragma unroll
  for (int m = 0; m < 8; ++m) {
    if (m >= mtiles) continue;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      if (!nvalid[w]) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = m * 16 + grp * 4 + j;
        if (r < ti.cnt) {
          const int64_t o = out_row(a, ti, r) * a.out_stride + nrow[w];
          if (GLU) {
            a.h_out[o] = f32_to_bf16_bits(silu(acc0[m][w][j]) * acc1[m][w][j]);
          } else {
            a.y_out[o] = acc0[m][w][j];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Combine: out[t] = bf16( sum_j w[t,j] y[inv[t*k+j]] + sum_s ysh[s][t] ),
// j ascending then s ascending, fp32. Four outputs per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const float* __restrict__ ysh,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int T, int k,
                                                      int L, int S, uint16_t* __restrict__ out) {
  const int L4 = L / 4;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)T * L4) return;
  const int t = (int)(id / L4);
  const int l = (int)(id % L4) * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // routes in groups of 8: indices and weights first, then the partial rows,
  // so the loads of a group are in flight together
  for (int j0 = 0; j0 < k; j0 += 8) {
    int pos[8];
    float wj[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u;
      pos[u] = j < k ? inv[t * k + j] : 0;
      wj[u] = j < k ? w[t * k + j] : 0.f;
    }
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = (j0 + u < k) ? *reinterpret_cast<const float4*>(y + (int64_t)pos[u] * L + l)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (j0 + u < k) {
        acc.x = fmaf(wj[u], v[u].x, acc.x);
        acc.y = fmaf(wj[u], v[u].y, acc.y);
        acc.z = fmaf(wj[u], v[u].z, acc.z);
        acc.w = fmaf(wj[u], v[u].w, acc.w);
      }
    }
  }
  for (int s = 0; s < S; ++s) {
    const float4 v = *reinterpret_cast<const float4*>(ysh + ((int64_t)s * T + t) * L + l);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  uint2 o;
  o.x = (uint32_t)f32_to_bf16_bits(acc.x) | ((uint32_t)f32_to_bf16_bits(acc.y) << 16);
  o.y = (uint32_t)f32_to_bf16_bits(acc.z) | ((uint32_t)f32_to_bf16_bits(acc.w) << 16);
  *reinterpret_cast<uint2*>(out + (int64_t)t * L + l) = o;
}

// ---------------------------------------------------------------------------
// Dequantisation test hook: the expert kernels' decode, eight values a thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ q,
                                                      const uint8_t* __restrict__ sc, int rows,
                                                      int K, uint16_t* __restrict__ out) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int per_row = K / 8;
  if (id >= (int64_t)rows * per_row) return;
  const int64_t n = id / per_row;
  const int g = (int)(id % per_row);
  const uint32_t w = *reinterpret_cast<const uint32_t*>(q + n * (K / 2) + g * 4);
  const float s = e8m0_to_f32(sc[n * (K / 32) + g / 4]);
  const bf16x8_t v = dequant8(w, s);
  *reinterpret_cast<bf16x8_t*>(out + n * K + g * 8) = v;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <bool GLU, bool FP4>
static hipError_t launch_gemm(const GemmArgs& a0, bool large, int row_tiles, int z,
                              hipStream_t s) {
  GemmArgs a = a0;
  const int cols = large ? kLgCols : 16;
  a.n_tiles_n = (a.N + cols - 1) / cols;
  dim3 grid((unsigned)(row_tiles * a.n_tiles_n), 1, (unsigned)z);
  if (large)
    hipLaunchKernelGGL((gemm_large_kernel<GLU, FP4>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_small_kernel<GLU, FP4>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_experts(const Plan& p, const uint16_t* x, const lmoe_weights& w,
                          const Workspace& ws, const int32_t* perm, const int32_t* inv,
                          const float* topk_w, uint16_t* out, hipStream_t s,
                          const hipEvent_t* ev) {
  const lmoe_dims& d = p.d;
  const bool large = p.rows_per_tile == kLargeRows;
  hipError_t err;
  {  // routed gate/up + GLU
    GemmArgs a = {};
    a.act = x;
    a.act_stride = d.L;
    a.gather = perm;
    a.gather_div = d.k;
    a.tiles = ws.tiles;
    a.ntiles = ws.ntiles;
    a.q0 = w.gate_q;
    a.s0 = w.gate_s;
    a.q1 = w.up_q;
    a.s1 = w.up_s;
    a.q_estride = (int64_t)d.I * d.L / 2;
    a.s_estride = (int64_t)d.I * d.L / 32;
    a.N = d.I;
    a.K = d.L;
    a.h_out = ws.h;
    a.out_stride = d.I;
    err = launch_gemm<true, true>(a, large, p.max_tiles, 1, s);
    if (err != hipSuccess) return err;
    if ((err = record_stage(ev, LMOE_STAGE_GATEUP, s)) != hipSuccess) return err;
  }
  {  // routed down
    GemmArgs a = {};
    a.act = ws.h;
    a.act_stride = d.I;
    a.tiles = ws.tiles;
    a.ntiles = ws.ntiles;
    a.q0 = w.down_q;
    a.s0 = w.down_s;
    a.q_estride = (int64_t)d.L * d.I / 2;
    a.s_estride = (int64_t)d.L * d.I / 32;
    a.N = d.L;
    a.K = d.I;
    a.y_out = ws.y;
    a.out_stride = d.L;
    err = launch_gemm<false, true>(a, large, p.max_tiles, 1, s);
    if (err != hipSuccess) return err;
    if ((err = record_stage(ev, LMOE_STAGE_DOWN, s)) != hipSuccess) return err;
  }
  if (d.S > 0) {
    const bool sh_large = d.T > 64;
    const int rows = sh_large ? kLargeRows : kSmallRows;
    const int row_tiles = (d.T + rows - 1) / rows;
    {  // shared gate/up + GLU
      GemmArgs a = {};
      a.act = x;
      a.act_stride = d.L;
      a.act_estride = 0;
      a.dense_rows = d.T;
      a.b0 = w.sh_gate;
      a.b1 = w.sh_up;
      a.b_estride = (int64_t)d.Is * d.L;
      a.N = d.Is;
      a.K = d.L;
      a.h_out = ws.h_sh;
      a.out_stride = d.Is;
      err = launch_gemm<true, false>(a, sh_large, row_tiles, d.S, s);
      if (err != hipSuccess) return err;
    }
    if ((err = record_stage(ev, LMOE_STAGE_SHARED_GATEUP, s)) != hipSuccess) return err;
    {  // shared down
      GemmArgs a = {};
      a.act = ws.h_sh;
      a.act_stride = d.Is;
      a.act_estride = (int64_t)d.T * d.Is;
      a.dense_rows = d.T;
      a.b0 = w.sh_down;
      a.b_estride = (int64_t)d.L * d.Is;
      a.N = d.L;
      a.K = d.Is;
      a.y_out = ws.y_sh;
      a.out_stride = d.L;
      err = launch_gemm<false, false>(a, sh_large, row_tiles, d.S, s);
      if (err != hipSuccess) return err;
    }
    if ((err = record_stage(ev, LMOE_STAGE_SHARED_DOWN, s)) != hipSuccess) return err;
  } else {
    if ((err = record_stage(ev, LMOE_STAGE_SHARED_GATEUP, s)) != hipSuccess) return err;
    if ((err = record_stage(ev, LMOE_STAGE_SHARED_DOWN, s)) != hipSuccess) return err;
  }
  {
    const int64_t n = (int64_t)d.T * (d.L / 4);
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(256), 0, s, ws.y, ws.y_sh, inv, topk_w,
                       d.T, d.k, d.L, d.S, out);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    err = record_stage(ev, LMOE_STAGE_COMBINE, s);
  }
  return err;
}

hipError_t launch_dequant(const uint8_t* q, const uint8_t* sc, int rows, int K, uint16_t* out,
                          hipStream_t s) {
  const int64_t n = (int64_t)rows * (K / 8);
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(dequant_kernel, dim3(blocks), dim3(256), 0, s, q, sc, rows, K, out);
  return hipGetLastError();
}

}  // namespace lmoe
