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
    // the same for every lane: kept in scalar registers
    ti->e = __builtin_amdgcn_readfirstlane(a.tiles[3 * tile + 0]);
    ti->p0 = __builtin_amdgcn_readfirstlane(a.tiles[3 * tile + 1]);
    ti->cnt = __builtin_amdgcn_readfirstlane(a.tiles[3 * tile + 2]);
  } else {
    ti->e = blockIdx.z;
    ti->p0 = tile * rows;
    ti->cnt = min(rows, a.dense_rows - ti->p0);
    if (ti->cnt <= 0) return false;
  }
  return true;
}

// The tile of this workgroup. Workgroups are dealt to the chip's eight XCDs
// in turn (workgroup i runs on XCD i % 8, each XCD with its own L2), so the
// column tiles of one row tile go to workgroups of one XCD: the tile's
// activation rows are fetched into that L2 once and read there by all of them.
constexpr int kXcds = 8;
__device__ __forceinline__ void tile_of_block(int n_tiles_n, int* tile, int* nt) {
  const int b = blockIdx.x;
  const int s = b / kXcds;
  *nt = s % n_tiles_n;
  *tile = (s / n_tiles_n) * kXcds + b % kXcds;
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
// Small dense tiles (bf16 weights, <= 16 rows: the shared experts for up to
// 64 tokens): one 16-row x 16-column output tile per workgroup, K split over
// the four waves in contiguous quarters, so the few rows still give a
// workgroup per 16 columns. In a wave iteration lane group g reads values
// 8 g .. 8 g + 7 of each 32-value step, 64 contiguous bytes of every weight
// row per load; the next iteration's weights are loaded before the current
// iteration's MFMAs. The four waves' partial tiles are added in LDS in a
// fixed order. (MXFP4 groups of any size go to the large kernel: for 1-5
// routes per expert it streams the weights faster than these tiles did.)
// ---------------------------------------------------------------------------
struct SmallOps {  // one 32-value block of bf16 weights per matrix
  u32x4_t b0[4], b1[4];
};

template <bool GLU>
__global__ __launch_bounds__(256) void gemm_small_kernel(GemmArgs a) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  // Column tiles in consecutive workgroups, which run on different XCDs: with
  // the few row tiles of these sizes, dealing each row tile to one XCD would
  // leave the other seven idle, and the at most 16 activation rows (a few KB
  // per K range) are cheap to fetch into every L2.
  const int nt = (int)(blockIdx.x % a.n_tiles_n);
  const int tile = (int)(blockIdx.x / a.n_tiles_n);
  TileInfo ti;
  if (!resolve_tile(a, tile, kSmallRows, &ti)) return;

  const int K = a.K, N = a.N;
  const int n0 = nt * 16;
  const int nblk = K / 32;
  const int bw_lo = (wave * nblk) / 4;
  const int bw_hi = ((wave + 1) * nblk) / 4;
  const int iters = (bw_hi - bw_lo + 3) / 4;

  const bool mvalid = col < ti.cnt;
  const uint16_t* ap = mvalid ? act_row(a, ti, col) : a.act;
  const int n = n0 + col;
  const bool nvalid = n < N;
  const int nn = nvalid ? n : 0;
  const uint16_t* b0r = a.b0 + ti.e * a.b_estride + (int64_t)nn * K;
  const uint16_t* b1r = GLU ? a.b1 + ti.e * a.b_estride + (int64_t)nn * K : nullptr;

  // block of this lane in iteration it
  auto blk_of = [&](int it) { return bw_lo + it * 4 + grp; };
  auto load_ops = [&](int it, SmallOps& o) {
    const int blk = blk_of(it);
    const bool ok = nvalid && it < iters && blk < bw_hi;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o.b0[q] = ok ? load16(b0r + blk * 32 + q * 8) : zero16();
      if (GLU) o.b1[q] = ok ? load16(b1r + blk * 32 + q * 8) : zero16();
    }
  };

  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f};
  f32x4_t acc1 = {0.f, 0.f, 0.f, 0.f};
  SmallOps cur, nxt;
  load_ops(0, cur);
  for (int it = 0; it < iters; ++it) {
    load_ops(it + 1, nxt);
    const int blk = blk_of(it);
    const bool aok = mvalid && blk < bw_hi;
    u32x4_t xv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) xv[q] = aok ? load16(ap + blk * 32 + q * 8) : zero16();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x8_t av = as_bf16x8(xv[q]);
      acc0 = mfma16(av, as_bf16x8(cur.b0[q]), acc0);
      if (GLU) acc1 = mfma16(av, as_bf16x8(cur.b1[q]), acc1);
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
// Large groups: up to 96 rows (MXFP4) or 256 rows (bf16, the shared
// experts) x 128 (gate/up) or 256 (down) columns per workgroup with MXFP4
// weights, and the same columns over eight waves with bf16 ones; each
// wave owns two paired gate/up 16-wide MFMA tiles for the GLU, or four tiles
// of the down projection, over all row tiles, so both kinds issue the same
// MFMAs per chunk.
//
// K runs in chunks of 128 values; in a chunk lane group g takes MX block g, so
// one 16-byte code load and one exponent feed four MFMA steps. A chunk of the
// tile's activations (its row groups only) is copied straight into LDS by the
// load unit (16-byte global-to-LDS loads, no registers) while the previous
// chunk is multiplied, with the chunk's weights loaded into registers beside
// it; two LDS buffers and one barrier per chunk. Rows are stored with their
// 16-byte segments XOR-swizzled by the row index, so the MFMA operand reads of
// 16 rows hit distinct banks, and the operands of four row tiles are read
// back to back before their MFMAs. Two MXFP4 workgroups share a CU; 96 rows
// leave LDS room for the exponent rows (the prefill groups of the Kimi-K3
// layer average 73 rows and rarely pass 96).
// ---------------------------------------------------------------------------
constexpr int kLgKc = 128;  // K values per chunk
// Exponent bytes per weight row that the large MXFP4 kernel stages in LDS
// (K <= 3584, the Kimi-K3 latent width).
constexpr int kExRowMax = 112;

// 16-column MFMA tiles per wave: two gate/up pairs or four down tiles; half
// as many for bf16 weights, whose chunk takes four times the registers.
__host__ __device__ constexpr int lg_tiles_per_wave(bool glu, bool fp4) {
  return (glu ? 2 : 4) / (fp4 ? 1 : 2);
}

// One array per buffer, so the compiler can tell a copy into one buffer from
// a read of the other and does not wait for every copy before every read.
template <int ROWS>
using LgChunk = uint16_t[ROWS][kLgKc];

// Routed groups (MXFP4): four waves, up to 96 rows, two workgroups per CU.
// Shared experts (bf16, dense): eight waves and 256 rows, one workgroup per
// CU, so each weight chunk serves twice the rows (every row tile reads all of
// the shared weights) and each activation chunk eight waves.
__host__ __device__ constexpr int lg_waves(bool fp4) { return fp4 ? 4 : 8; }
__host__ __device__ constexpr int lg_rows(bool fp4) { return fp4 ? kLargeRows : kDenseRows; }

template <int N>
struct IntC {
  static constexpr int value = N;
};

template <bool GLU, bool FP4, bool EXW>
__global__ __launch_bounds__(64 * lg_waves(FP4), FP4 ? 2 : 1) void gemm_large_kernel(GemmArgs a) {
  constexpr int WAVES = lg_waves(FP4);
  constexpr int ROWS = lg_rows(FP4);
  constexpr int MTMAX = ROWS / 16;
  __shared__ __attribute__((aligned(16))) LgChunk<ROWS> sx0, sx1;
  __shared__ const uint16_t* s_arow[ROWS];
  // EXW: each wave's exponent rows (its 64 weight rows, whole K range)
  __shared__ __attribute__((aligned(16))) uint8_t s_ex[EXW ? WAVES : 1][EXW ? 64 * kExRowMax : 16];
  auto slot = [&](int r) -> LgChunk<ROWS>& { return r == 0 ? sx0 : sx1; };
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  // Fewer dense row tiles than XCDs (the shared experts below 8 x 256 tokens):
  // column tiles in consecutive workgroups, over every XCD, as the small
  // tiles do; otherwise each row tile on one XCD.
  int tile, nt;
  if (!a.tiles && (a.dense_rows + ROWS - 1) / ROWS < kXcds) {
    nt = (int)(blockIdx.x % a.n_tiles_n);
    tile = (int)(blockIdx.x / a.n_tiles_n);
  } else {
    tile_of_block(a.n_tiles_n, &tile, &nt);
  }
  TileInfo ti;
  if (!resolve_tile(a, tile, ROWS, &ti)) return;
  constexpr int NW = lg_tiles_per_wave(GLU, FP4);  // 16-column tiles per wave
  constexpr int NM = GLU ? 2 : 1;                   // weight matrices per column tile
  const int K = a.K, N = a.N;
  const int nblk = K / 32;
  const int nchunks = (K + kLgKc - 1) / kLgKc;
  const int n0 = nt * (WAVES * 16 * NW) + wave * (16 * NW);
  const int mtiles = (ti.cnt + 15) / 16;

  // rows past the tile repeat its last row: finite values, never stored
  for (int r = tid; r < ROWS; r += 64 * WAVES) s_arow[r] = act_row(a, ti, min(r, ti.cnt - 1));

  int nrow[NW];
  bool nvalid[NW];
  const uint8_t* qr[NW][NM];
  const uint8_t* er[NW][NM];
  const uint16_t* br[NW][NM];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    nrow[w] = n0 + w * 16 + col;
    nvalid[w] = nrow[w] < N;
    const int nn = nvalid[w] ? nrow[w] : 0;  // padding columns read row 0, never stored
#pragma unroll
    for (int mm = 0; mm < NM; ++mm) {
      if (FP4) {
        qr[w][mm] = (mm ? a.q1 : a.q0) + ti.e * a.q_estride + (int64_t)nn * (K / 2);
        er[w][mm] = (mm ? a.s1 : a.s0) + ti.e * a.s_estride + (int64_t)nn * (K / 32);
        br[w][mm] = nullptr;
      } else {
        br[w][mm] = (mm ? a.b1 : a.b0) + ti.e * a.b_estride + (int64_t)nn * K;
        qr[w][mm] = er[w][mm] = nullptr;
      }
    }
  }

  // Exponents, EXW: a wave's 64 weight rows are NM runs of 16 * NW
  // consecutive rows, so their exponents are NM contiguous runs of
  // 16 * NW * nblk bytes. They are copied into LDS once, whole, by 16-byte
  // global-to-LDS loads that read every byte of every line they touch (row r
  // of the wave, r = mm * 16 * NW + w * 16 + col, at byte r * nblk). Copies
  // of part of each row per K window read each line once per window, and the
  // weight stream evicts it in between: for the Kimi-K3 gate/up that fetched
  // eight times the exponent bytes. Each wave reads only its own rows, so no
  // barrier is needed.
  static_assert(!EXW || (FP4 && NW * NM == 4), "64 weight rows per wave");
  if constexpr (EXW) {
    const int bytes = 64 * nblk;  // a multiple of 1024 (nblk % 16 == 0)
#pragma unroll
    for (int i = 0; i < kExRowMax / 16; ++i) {
      if (i * 1024 < bytes) {  // the same for every lane
        const int o = i * 1024 + lane * 16;
        const int r = o / nblk, byte = o - r * nblk;  // 16 bytes inside row r
        const int mm = r / (16 * NW);
        const int n = n0 + r % (16 * NW);
        const uint8_t* src =
            (mm ? a.s1 : a.s0) + ti.e * a.s_estride + (int64_t)(n < N ? n : 0) * nblk + byte;
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(src),
            (__attribute__((address_space(3))) void*)(&s_ex[wave][i * 1024]), 16, 0, 0);
      }
    }
  }
  // the exponents of this lane's blocks in window win (blocks 16 win + 4j +
  // grp, chunks 4 win + j), packed one byte per chunk
  uint32_t exw[NW][NM];
  auto read_ex = [&](int win) {
    if constexpr (EXW) {
      const uint32_t sel = (uint32_t)grp | ((uint32_t)(4 + grp) << 8) | 0x0c0c0000u;
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int mm = 0; mm < NM; ++mm) {
          const int r = mm * 16 * NW + w * 16 + col;
          const u32x4_t d = *reinterpret_cast<const u32x4_t*>(&s_ex[wave][r * nblk + 16 * win]);
          exw[w][mm] = __builtin_amdgcn_perm(d[1], d[0], sel) |
                       (__builtin_amdgcn_perm(d[3], d[2], sel) << 16);
        }
    }
  };

  // The rest runs with MT row tiles known at compile time for MXFP4 weights
  // (one instantiation per count a tile can have), and with the tile's count
  // tested at run time for bf16 ones (sixteen row tiles).
  auto body = [&](auto mt_c) {
    constexpr int MT = decltype(mt_c)::value;
    f32x4_t acc[MT][NW][NM];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int mm = 0; mm < NM; ++mm) acc[m][w][mm] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // copy of chunk c (clamped to the last chunk) into LDS buffer `buf`:
    // instruction j of wave w moves rows w*32 + 4j .. +4, lane l the 16-byte
    // segment at physical slot l % 16 of row l / 16 (logical segment slot ^ row
    // % 16); instructions wholly past the tile's row groups are skipped
    auto copy_x = [&](int c, int buf) {
      const int cc = min(c, nchunks - 1);
#pragma unroll
      for (int j = 0; j < ROWS / WAVES / 4; ++j) {
        const int row0 = wave * (ROWS / WAVES) + j * 4;
        if (row0 < (FP4 ? MT : mtiles) * 16) {
          const int row = row0 + (lane >> 4);
          const int seg = (lane & 15) ^ (row & 15);
          const int k = min(cc * kLgKc + seg * 8, K - 8);  // K % 32 == 0, so k + 8 <= K
          __builtin_amdgcn_global_load_lds(
              reinterpret_cast<const void*>(s_arow[row] + k),
              (__attribute__((address_space(3))) void*)(&slot(buf)[row0][0]), 16, 0, 0);
        }
      }
    };
    // weights of chunk c for this lane: MX block c*4 + grp
    struct Bq {
      u32x4_t q[NW][NM];     // MXFP4: 32 codes
      uint32_t e[NW][NM];    //        their exponent
      u32x4_t h[NW][NM][4];  // bf16: 32 values
    };
    auto load_b = [&](int c, Bq& b) {
      const int blk = min(c * 4 + grp, nblk - 1);
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int mm = 0; mm < NM; ++mm) {
          if (FP4) {
            b.q[w][mm] = load16(qr[w][mm] + blk * 16);
            if (!EXW) b.e[w][mm] = er[w][mm][blk];
          } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) b.h[w][mm][s] = load16(br[w][mm] + blk * 32 + s * 8);
          }
        }
    };
    auto compute = [&](int c, int buf, const Bq& b) {
      const bool kv = c * 4 + grp < nblk;  // past the end: zero weights
      // the lane's block scale per weight tile, once per chunk; zero past the
      // end (E2M1 codes are finite, so a zero scale gives zero weights)
      float scale[NW][NM];
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int mm = 0; mm < NM; ++mm) {
          const uint32_t ex = !FP4 ? 127u : EXW ? (exw[w][mm] >> (8 * (c & 3))) & 0xffu : b.e[w][mm];
          scale[w][mm] = kv ? e8m0_to_f32(ex) : 0.f;
        }
      // FP4: every row tile's operands of step s + 1 are read from LDS while
      // step s multiplies
      bf16x8_t av[2][FP4 ? MT : 1];
      auto read_a = [&](int s, bf16x8_t (&dst)[FP4 ? MT : 1]) {
#pragma unroll
        for (int m = 0; m < (FP4 ? MT : 0); ++m) {
          const int row = m * 16 + col;
          const int phys = (grp * 4 + s) ^ (row & 15);
          dst[m] = *reinterpret_cast<const bf16x8_t*>(&slot(buf)[row][phys * 8]);
        }
      };
      read_a(0, av[0]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s < 3) read_a(s + 1, av[(s + 1) & 1]);
        bf16x8_t bv[NW][NM];
#pragma unroll
        for (int w = 0; w < NW; ++w)
#pragma unroll
          for (int mm = 0; mm < NM; ++mm) {
            if (FP4)
              bv[w][mm] = dequant8(b.q[w][mm][s], scale[w][mm]);
            else
              bv[w][mm] = as_bf16x8(kv ? b.h[w][mm][s] : zero16());
          }
        if constexpr (FP4) {
          // MT is this tile's row-tile count: no branches, so each MFMA
          // block can overlap the next step's operand reads
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int w = 0; w < NW; ++w)
#pragma unroll
              for (int mm = 0; mm < NM; ++mm)
                acc[m][w][mm] = mfma16(av[s & 1][m], bv[w][mm], acc[m][w][mm]);
        } else {
        // the operands of four row tiles are read back to back, then their
        // MFMAs run; the next four only when the tile has them
#pragma unroll
        for (int h = 0; h < MT / 4; ++h) {
          if (h == 0 || mtiles > 4 * h) {
            bf16x8_t a4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int row = (4 * h + i) * 16 + col;
              const int phys = (grp * 4 + s) ^ (row & 15);
              a4[i] = *reinterpret_cast<const bf16x8_t*>(&slot(buf)[row][phys * 8]);
            }
            // keeps the reads ahead of the branches below (the compiler would
            // otherwise sink each into its branch and wait for it alone)
            asm volatile("" ::"v"(a4[0]), "v"(a4[1]), "v"(a4[2]), "v"(a4[3]));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int m = 4 * h + i;
              if (m < mtiles) {
#pragma unroll
                for (int w = 0; w < NW; ++w)
#pragma unroll
                  for (int mm = 0; mm < NM; ++mm)
                    acc[m][w][mm] = mfma16(a4[i], bv[w][mm], acc[m][w][mm]);
              }
            }
          }
        }
        }
      }
    };

    __syncthreads();  // s_arow
    Bq bq[2];
    copy_x(0, 0);
    load_b(0, bq[0]);
    // No chunk load is conditional (a branch around the loads would make the
    // compiler wait for all of them): a chunk past the end multiplies zero
    // weights.
    for (int cb = 0; cb < nchunks; cb += 2) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int c = cb + r;
        // chunk c (loaded during the previous step) has landed for this thread,
        // then for every thread, and every wave is done with the other buffer
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __builtin_amdgcn_s_barrier();
        if (EXW && (c & 3) == 0) read_ex(min(c / 4, nblk / 16 - 1));
        copy_x(c + 1, r ^ 1);
        load_b(c + 1, bq[r ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
        compute(c, r, bq[r]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);

#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (!FP4 && m >= mtiles) continue;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        if (!nvalid[w]) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = m * 16 + grp * 4 + j;
          if (r < ti.cnt) {
            const int64_t o = out_row(a, ti, r) * a.out_stride + nrow[w];
            if constexpr (GLU) {
              a.h_out[o] = f32_to_bf16_bits(silu(acc[m][w][0][j]) * acc[m][w][1][j]);
            } else {
              a.y_out[o] = acc[m][w][0][j];
            }
          }
        }
      }
    }
  };
  if constexpr (FP4) {
    static_assert(MTMAX == 6, "row-tile counts dispatched below");
    switch (mtiles) {
      case 1: body(IntC<1>{}); break;
      case 2: body(IntC<2>{}); break;
      case 3: body(IntC<3>{}); break;
      case 4: body(IntC<4>{}); break;
      case 5: body(IntC<5>{}); break;
      default: body(IntC<6>{}); break;
    }
  } else {
    body(IntC<MTMAX>{});
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
  // so the loads of a group are in flight together. Each partial is read
  // once: non-temporal loads (K3 prefill 214-220 -> 188 us)
  for (int j0 = 0; j0 < k; j0 += 8) {
    int pos[8];
    float wj[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u;
      pos[u] = j < k ? inv[t * k + j] : 0;
      wj[u] = j < k ? w[t * k + j] : 0.f;
    }
    f32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = (j0 + u < k) ? __builtin_nontemporal_load(
                                reinterpret_cast<const f32x4_t*>(y + (int64_t)pos[u] * L + l))
                          : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (j0 + u < k) {
        acc.x = fmaf(wj[u], v[u][0], acc.x);
        acc.y = fmaf(wj[u], v[u][1], acc.y);
        acc.z = fmaf(wj[u], v[u][2], acc.z);
        acc.w = fmaf(wj[u], v[u][3], acc.w);
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
// Measurement hook: the plain HBM read rate the decode kernel is held
// against. Every byte of the buffer is read once with 16-byte loads, four in
// flight per thread, the workgroups striding over the buffer; each workgroup
// folds what it read into one word (so no load is dead).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4_t* __restrict__ p,
                                                          int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t x = 0;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_t a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3];
    x ^= c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
  }
  for (; i < n16; i += stride) {
    const u32x4_t a = p[i];
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x ^= __shfl_xor(x, off, kWave);
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

hipError_t launch_read_stream(const void* p, size_t bytes, uint32_t* sink, int blocks,
                              hipStream_t s) {
  hipLaunchKernelGGL(read_stream_kernel, dim3(blocks), dim3(256), 0, s,
                     static_cast<const u32x4_t*>(p), (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <bool GLU, bool FP4>
static hipError_t launch_gemm(const GemmArgs& a0, bool large, int row_tiles, int z,
                              hipStream_t s) {
  // exponent rows through LDS when they hold whole 16-block windows and fit
  const bool exw = FP4 && (a0.K / 32) % 16 == 0 && a0.K / 32 <= kExRowMax;
  GemmArgs a = a0;
  // large tiles: four waves of lg_tiles_per_wave 16-column MFMA tiles
  const int cols = large ? 16 * lg_waves(FP4) * lg_tiles_per_wave(GLU, FP4) : 16;
  a.n_tiles_n = (a.N + cols - 1) / cols;
  // row tiles dealt to the XCDs (tile_of_block): rounded up to whole rounds
  // of them; spread over the XCDs by column tile (small tiles, and fewer
  // dense row tiles than XCDs): one workgroup per (row tile, column tile)
  const int rounds = (row_tiles + kXcds - 1) / kXcds;
  const bool spread = !large || (!a.tiles && row_tiles < kXcds);
  dim3 grid((unsigned)((spread ? row_tiles : rounds * kXcds) * a.n_tiles_n), 1, (unsigned)z);
  if (large && exw)
    hipLaunchKernelGGL((gemm_large_kernel<GLU, FP4, FP4>), grid, dim3(64 * lg_waves(FP4)), 0, s, a);
  else if (large)
    hipLaunchKernelGGL((gemm_large_kernel<GLU, FP4, false>), grid, dim3(64 * lg_waves(FP4)), 0, s, a);
  else if constexpr (!FP4)
    hipLaunchKernelGGL((gemm_small_kernel<GLU>), grid, dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;  // MXFP4 groups always take the large kernel
  return hipGetLastError();
}

hipError_t launch_routed(const Plan& p, const uint16_t* x, const lmoe_weights& w,
                         const Workspace& ws, const int32_t* perm, hipStream_t s,
                         const hipEvent_t* ev) {
  const lmoe_dims& d = p.d;
  const bool large = true;  // MXFP4 groups of every size (see the small tiles)
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
    err = record_stage(ev, LMOE_STAGE_DOWN, s);
  }
  return err;
}

hipError_t launch_shared(const Plan& p, const uint16_t* x, const lmoe_weights& w,
                         const Workspace& ws, hipStream_t s, const hipEvent_t* ev) {
  const lmoe_dims& d = p.d;
  hipError_t err = hipSuccess;
  if (d.S > 0 && d.T > 64 && d.L % 64 == 0 && d.Is % 64 == 0) {
    // the block's dense GEMMs (dense.hip), one launch for all S experts:
    // gate/up with the GLU over the separate gate and up matrices, then down
    DenseArgs g = {};
    g.a = x;
    g.lda = d.L;
    g.b = w.sh_gate;
    g.b_up = w.sh_up;
    g.ldb = d.L;
    g.b_zstride = (int64_t)d.Is * d.L;
    g.M = d.T;
    g.N = 2 * d.Is;
    g.K = d.L;
    g.glu_out = ws.h_sh;
    g.ld_glu = d.Is;
    g.out_zstride = (int64_t)d.T * d.Is;
    if ((err = launch_dense_batched(g, d.S, s)) != hipSuccess) return err;
    if ((err = record_stage(ev, LMOE_STAGE_SHARED_GATEUP, s)) != hipSuccess) return err;
    DenseArgs dn = {};
    dn.a = ws.h_sh;
    dn.lda = d.Is;
    dn.a_zstride = (int64_t)d.T * d.Is;
    dn.b = w.sh_down;
    dn.ldb = d.Is;
    dn.b_zstride = (int64_t)d.L * d.Is;
    dn.M = d.T;
    dn.N = d.L;
    dn.K = d.Is;
    dn.n_f32 = d.L;
    dn.f32_out = ws.y_sh;
    dn.ld_f32 = d.L;
    dn.out_zstride = (int64_t)d.T * d.L;
    if ((err = launch_dense_batched(dn, d.S, s)) != hipSuccess) return err;
    return record_stage(ev, LMOE_STAGE_SHARED_DOWN, s);
  }
  if (d.S > 0) {
    const bool sh_large = d.T > 64;
    const int rows = sh_large ? kDenseRows : kSmallRows;
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
  return err;
}

hipError_t launch_combine(const Plan& p, const Workspace& ws, const int32_t* inv,
                          const float* topk_w, uint16_t* out, hipStream_t s,
                          const hipEvent_t* ev) {
  const lmoe_dims& d = p.d;
  hipError_t err;
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
