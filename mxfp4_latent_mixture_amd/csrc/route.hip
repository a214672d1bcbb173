// Routing kernels: router logits, top-k selection with softmax weights, and
// the stable grouping of routes by expert.
//
// Router scores over the experts are one projection of the MoE input (dev48.org
// "Kimi K3 on AMD Instinct GPUs with TokenSpeed", section 4.3); here the router
// reads the latent activations. Each token keeps its 16 best of 896 experts
// (infervisor.ai "Bringing up Kimi-K3 on day zero", "The model we hadn't run").
// Routes are then sorted by expert so one loaded weight panel serves every
// route of that expert (TokenSpeed section 4.1).
#include "lmoe_device.h"
#include "lmoe_internal.h"
#include "lmoe_topk.h"

namespace lmoe {

// ---------------------------------------------------------------------------
// Router: part[split][t][e] = sum over the split's K range of x[t][k] W[e][k].
// Tile: TOK tokens (64, or 128 for prefill sizes) x 64 experts per
// 256-thread workgroup; each wave owns TOK/4 tokens (one or two 16-token MFMA
// tiles) and four 16-expert MFMA tiles, so a 128-token tile reads each
// router row once for twice the tokens. K runs in chunks of 128 values (four
// MFMA steps per pair of barriers); the next chunk is loaded into registers
// while the current one is multiplied from LDS. A split's range is whole
// 32-value steps; values past it are loaded as zeros.
// ---------------------------------------------------------------------------
constexpr int kRtExp = 64;
constexpr int kRtKc = 128;             // K values per chunk
constexpr int kRtPad = kRtKc + 8;      // LDS row length in bf16: rows 272 bytes apart
constexpr int kRtPieces = kRtKc / 8;   // 16-byte pieces per chunk row (16)

template <int TOK>
__global__ __launch_bounds__(256) void router_kernel(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ wr,
                                                     float* __restrict__ part, int T, int L,
                                                     int E, int steps_per) {
  constexpr int MT = TOK / 64;              // 16-token MFMA tiles per wave
  constexpr int XTPR = 256 / TOK;           // threads per token row of a chunk
  constexpr int XV = kRtPieces / XTPR;      // their 16-byte pieces each
  constexpr int WV = kRtPieces / 4;         // four threads per router row
  __shared__ __attribute__((aligned(16))) uint16_t sx[TOK][kRtPad];
  __shared__ __attribute__((aligned(16))) uint16_t sw[kRtExp][kRtPad];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int e0 = blockIdx.x * kRtExp;
  const int t0 = blockIdx.y * TOK;
  const int split = blockIdx.z;
  const int nsteps = L / 32;
  const int k0 = split * steps_per * 32;
  const int k1 = min(nsteps, (split + 1) * steps_per) * 32;

  // token row tid / XTPR, pieces tid % XTPR + XTPR i; router row tid / 4,
  // pieces tid % 4 + 4 i
  const int xrow = tid / XTPR, xq = tid % XTPR;
  const int wrow = tid >> 2, wq = tid & 3;
  const int t = t0 + xrow, e = e0 + wrow;
  const uint16_t* xr = x + (size_t)min(t, T - 1) * L;
  const uint16_t* wrr = wr + (size_t)min(e, E - 1) * L;
  u32x4_t vx[XV], vw[WV];
  auto load = [&](int kc) {
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      const int k = kc + (xq + XTPR * i) * 8;
      vx[i] = (k < k1 && t < T) ? load16(xr + k) : zero16();
    }
#pragma unroll
    for (int i = 0; i < WV; ++i) {
      const int k = kc + (wq + 4 * i) * 8;
      vw[i] = (k < k1 && e < E) ? load16(wrr + k) : zero16();
    }
  };

  f32x4_t acc[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[m][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load(k0);
  for (int kc = k0; kc < k1; kc += kRtKc) {
    __syncthreads();  // every wave is done with the previous chunk
#pragma unroll
    for (int i = 0; i < XV; ++i)
      *reinterpret_cast<u32x4_t*>(&sx[xrow][(xq + XTPR * i) * 8]) = vx[i];
#pragma unroll
    for (int i = 0; i < WV; ++i)
      *reinterpret_cast<u32x4_t*>(&sw[wrow][(wq + 4 * i) * 8]) = vw[i];
    __syncthreads();
    load(kc + kRtKc);  // in flight while this chunk is multiplied
#pragma unroll
    for (int s = 0; s < kRtKc / 32; ++s) {
      bf16x8_t a[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m)
        a[m] = *reinterpret_cast<const bf16x8_t*>(&sx[wave * 16 * MT + m * 16 + col][s * 32 + grp * 8]);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(&sw[nt * 16 + col][s * 32 + grp * 8]);
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m][nt] = mfma16(a[m], b, acc[m][nt]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int ee = e0 + nt * 16 + col;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tt = t0 + wave * 16 * MT + m * 16 + grp * 4 + j;
        if (tt < T && ee < E) part[((size_t)split * T + tt) * E + ee] = acc[m][nt][j];
      }
    }
}

// ---------------------------------------------------------------------------
// Top-k. The logits are summed from the router's K-split partials in a fixed
// order (split 0 first); one wave then selects by threshold (lmoe_topk.h; by k
// rounds when the largest keys crowd into fewer lanes than there are
// candidates) and takes the softmax over the selected logits.
//   SPLIT = false (one partial, prefill sizes): one wave per token, four
//     tokens per workgroup; lane l holds experts l + 64 i.
//   SPLIT = true (many partials, small T): one workgroup per token; its 256
//     threads sum the partials of four experts each, eight splits in flight,
//     into LDS, and wave 0 selects.
// ---------------------------------------------------------------------------
constexpr int kTopkWaves = 4;
constexpr int kMaxE = kWave * kTopkKeysPerLane;  // experts (1024)

template <bool SPLIT>
__global__ __launch_bounds__(64 * kTopkWaves) void topk_kernel(
    const float* __restrict__ part, int ks, int T, int E, int k, float* __restrict__ logits_out,
    int32_t* __restrict__ idx, float* __restrict__ wout) {
  __shared__ TopkScratch scr[SPLIT ? 1 : kTopkWaves];
  __shared__ float sl[SPLIT ? kMaxE : 1];
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int t = SPLIT ? blockIdx.x : blockIdx.x * kTopkWaves + wave;
  float lv[kTopkKeysPerLane];
  if constexpr (SPLIT) {
    for (int e = threadIdx.x; e < E; e += 64 * kTopkWaves) {
      float sum = 0.f;
#pragma unroll 8
      for (int q = 0; q < ks; ++q) sum += part[((size_t)q * T + t) * E + e];
      sl[e] = sum;
      if (logits_out) logits_out[(size_t)t * E + e] = sum;
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int i = 0; i < kTopkKeysPerLane; ++i) {
      const int e = lane + kWave * i;
      lv[i] = e < E ? sl[e] : 0.f;
    }
  } else {
    if (t >= T) return;  // the whole wave; no workgroup barrier follows
    const float* pt = part + (size_t)t * E;
#pragma unroll
    for (int i = 0; i < kTopkKeysPerLane; ++i) {
      const int e = lane + kWave * i;
      lv[i] = e < E ? pt[e] : 0.f;
      if (logits_out && e < E) logits_out[(size_t)t * E + e] = lv[i];
    }
  }
  uint64_t key[kTopkKeysPerLane];
#pragma unroll
  for (int i = 0; i < kTopkKeysPerLane; ++i) {
    const int e = lane + kWave * i;
    key[i] = e < E ? order_key(lv[i], e) : 0ull;
  }
  uint64_t mine = 0ull;  // lane j: the j-th largest key
  if (!select_by_threshold(k, key, scr[SPLIT ? 0 : wave], mine)) select_by_rounds(k, key, mine);
  // softmax over the selected logits, relative to the largest (the first)
  const int my_e = (int)(~(uint32_t)mine);
  const float my_l = lane < k ? key_value(mine) : 0.f;
  const float l0 = __shfl(my_l, 0, kWave);
  const float z = (lane < k) ? expf(my_l - l0) : 0.f;
  float s = z;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_down(s, off, kWave);
  s = __shfl(s, 0, kWave);
  if (lane < k) {
    idx[(size_t)t * k + lane] = my_e;
    wout[(size_t)t * k + lane] = z / s;
  }
}

// ---------------------------------------------------------------------------
// Grouping of routes by expert (one 1024-thread workgroup).
// counts by LDS histogram; offsets by an exclusive scan; then positions: a
// token selects each expert at most once, so within expert e the routes are
// ordered by token and pos(t, e) = offsets[e] + #{t' < t selecting e}. Tokens
// are processed 64 at a time with one 64-bit membership mask per expert.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int block_exclusive_scan_1024(int v, int* s_wave, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int w = (lane < 16) ? s_wave[lane] : 0;
    int wi = w;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      int o = __shfl_up(wi, off, kWave);
      if (lane >= off) wi += o;
    }
    if (lane < 16) s_wave[16 + lane] = wi - w;  // exclusive prefix of wave totals
    if (lane == 15) s_wave[32] = wi;
  }
  __syncthreads();
  const int r = s_wave[16 + wave] + incl - v;
  *total = s_wave[32];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(1024) void permute_kernel(const int32_t* __restrict__ idx, int T,
                                                       int k, int E, int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ inv,
                                                       int32_t* __restrict__ tiles,
                                                       int32_t* __restrict__ ntiles, int rows) {
  __shared__ int s_cnt[kMaxE];
  __shared__ int s_run[kMaxE];
  __shared__ unsigned long long s_mask[kMaxE];
  __shared__ int s_wave[48];
  const int tid = threadIdx.x;
  const int R = T * k;
  s_cnt[tid] = 0;
  __syncthreads();
  for (int r = tid; r < R; r += 1024) atomicAdd(&s_cnt[idx[r]], 1);
  __syncthreads();

  const int c = (tid < E) ? s_cnt[tid] : 0;
  int total = 0;
  const int off = block_exclusive_scan_1024(c, s_wave, &total);
  const int nt = (c + rows - 1) / rows;
  int ntot = 0;
  const int tbase = block_exclusive_scan_1024(nt, s_wave, &ntot);
  if (tid < E) {
    counts[tid] = c;
    offsets[tid] = off;
    s_run[tid] = off;
    for (int i = 0; i < nt; ++i) {
      tiles[3 * (tbase + i) + 0] = tid;
      tiles[3 * (tbase + i) + 1] = off + i * rows;
      tiles[3 * (tbase + i) + 2] = min(rows, c - i * rows);
    }
  }
  if (tid == 0) {
    offsets[E] = total;
    *ntiles = ntot;
  }
  __syncthreads();

  for (int tg = 0; tg < T; tg += 64) {
    if (tid < E) s_mask[tid] = 0ull;
    __syncthreads();
    const int r0 = tg * k;
    const int r1 = min(T, tg + 64) * k;
    for (int r = r0 + tid; r < r1; r += 1024) {
      const int t = r / k;
      atomicOr(&s_mask[idx[r]], 1ull << (t - tg));
    }
    __syncthreads();
    for (int r = r0 + tid; r < r1; r += 1024) {
      const int t = r / k;
      const int e = idx[r];
      const unsigned long long below = (1ull << (t - tg)) - 1ull;
      const int pos = s_run[e] + __popcll(s_mask[e] & below);
      perm[pos] = r;
      inv[r] = pos;
    }
    __syncthreads();
    if (tid < E) s_run[tid] += __popcll(s_mask[tid]);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// The same permutation over many workgroups, for large T: tokens in chunks of
// 64 (one bit each in the membership masks above); each chunk's routes to an
// expert are placed after those of all earlier chunks, so the order stays
// by expert, then by route.
// ---------------------------------------------------------------------------
constexpr int kPermChunk = 64;  // tokens per chunk

// cnt[b][e]: routes of chunk b (tokens 64b .. 64b + 63) to expert e
__global__ __launch_bounds__(256) void chunk_count_kernel(const int32_t* __restrict__ idx, int T,
                                                          int k, int E,
                                                          int32_t* __restrict__ cnt) {
  __shared__ int s_cnt[kMaxE];
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) s_cnt[e] = 0;
  __syncthreads();
  const int r0 = b * kPermChunk * k, r1 = min(T, (b + 1) * kPermChunk) * k;
  for (int r = r0 + threadIdx.x; r < r1; r += 256) atomicAdd(&s_cnt[idx[r]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) cnt[(size_t)b * E + e] = s_cnt[e];
}

// counts, offsets and the tile list from the chunk counts, which become each
// chunk's first sorted position per expert (one thread per expert)
__global__ __launch_bounds__(1024) void chunk_scan_kernel(int32_t* __restrict__ cnt, int nb, int E,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ tiles,
                                                         int32_t* __restrict__ ntiles, int rows) {
  __shared__ int s_wave[48];
  const int e = threadIdx.x;
  int c = 0;
  if (e < E) {
#pragma unroll 8
    for (int b = 0; b < nb; ++b) c += cnt[(size_t)b * E + e];
  }
  int total = 0;
  const int off = block_exclusive_scan_1024(c, s_wave, &total);
  const int nt = (c + rows - 1) / rows;
  int ntot = 0;
  const int tbase = block_exclusive_scan_1024(nt, s_wave, &ntot);
  if (e < E) {
    counts[e] = c;
    offsets[e] = off;
    for (int i = 0; i < nt; ++i) {
      tiles[3 * (tbase + i) + 0] = e;
      tiles[3 * (tbase + i) + 1] = off + i * rows;
      tiles[3 * (tbase + i) + 2] = min(rows, c - i * rows);
    }
    int run = off;
    for (int b = 0; b < nb; ++b) {
      const int v = cnt[(size_t)b * E + e];
      cnt[(size_t)b * E + e] = run;
      run += v;
    }
  }
  if (e == 0) {
    offsets[E] = total;
    *ntiles = ntot;
  }
}

// each route's position: its chunk's first position for the expert plus the
// rank of its token among the chunk's tokens routed there (a token routes to
// an expert at most once)
__global__ __launch_bounds__(256) void chunk_scatter_kernel(const int32_t* __restrict__ idx, int T,
                                                            int k, int E,
                                                            const int32_t* __restrict__ base,
                                                            int32_t* __restrict__ perm,
                                                            int32_t* __restrict__ inv) {
  __shared__ unsigned long long s_mask[kMaxE];
  const int b = blockIdx.x, tg = b * kPermChunk;
  for (int e = threadIdx.x; e < E; e += 256) s_mask[e] = 0ull;
  __syncthreads();
  const int r0 = tg * k, r1 = min(T, tg + kPermChunk) * k;
  for (int r = r0 + threadIdx.x; r < r1; r += 256) atomicOr(&s_mask[idx[r]], 1ull << (r / k - tg));
  __syncthreads();
  for (int r = r0 + threadIdx.x; r < r1; r += 256) {
    const int t = r / k;
    const int e = idx[r];
    const int pos = base[(size_t)b * E + e] + __popcll(s_mask[e] & ((1ull << (t - tg)) - 1ull));
    perm[pos] = r;
    inv[r] = pos;
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_router(const Plan& p, const uint16_t* x, const uint16_t* wr, float* part,
                         hipStream_t s) {
  const lmoe_dims& d = p.d;
  const int tok = p.router.tok;
  dim3 grid((d.E + kRtExp - 1) / kRtExp, (d.T + tok - 1) / tok, p.router.ks);
  if (tok == 128)
    hipLaunchKernelGGL(router_kernel<128>, grid, dim3(256), 0, s, x, wr, part, d.T, d.L, d.E,
                       p.router.steps_per);
  else
    hipLaunchKernelGGL(router_kernel<64>, grid, dim3(256), 0, s, x, wr, part, d.T, d.L, d.E,
                       p.router.steps_per);
  return hipGetLastError();
}

hipError_t launch_topk(const Plan& p, const float* part, int ks, float* logits_out,
                       int32_t* idx, float* w, hipStream_t s) {
  const lmoe_dims& d = p.d;
  if (ks == 1)
    hipLaunchKernelGGL(topk_kernel<false>, dim3((d.T + kTopkWaves - 1) / kTopkWaves),
                       dim3(64 * kTopkWaves), 0, s, part, ks, d.T, d.E, d.k, logits_out, idx, w);
  else
    hipLaunchKernelGGL(topk_kernel<true>, dim3(d.T), dim3(64 * kTopkWaves), 0, s, part, ks, d.T,
                       d.E, d.k, logits_out, idx, w);
  return hipGetLastError();
}

hipError_t launch_permute(const Plan& p, const int32_t* idx, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv, int32_t* tiles, int32_t* ntiles,
                          int32_t* chunk_base, hipStream_t s) {
  const lmoe_dims& d = p.d;
  if (d.T <= kPermManyFrom) {
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(1024), 0, s, idx, d.T, d.k, d.E, counts,
                       offsets, perm, inv, tiles, ntiles, p.rows_per_tile);
    return hipGetLastError();
  }
  const int nb = (d.T + kPermChunk - 1) / kPermChunk;
  hipLaunchKernelGGL(chunk_count_kernel, dim3(nb), dim3(256), 0, s, idx, d.T, d.k, d.E,
                     chunk_base);
  hipLaunchKernelGGL(chunk_scan_kernel, dim3(1), dim3(1024), 0, s, chunk_base, nb, d.E, counts,
                     offsets, tiles, ntiles, p.rows_per_tile);
  hipLaunchKernelGGL(chunk_scatter_kernel, dim3(nb), dim3(256), 0, s, idx, d.T, d.k, d.E,
                     chunk_base, perm, inv);
  return hipGetLastError();
}

}  // namespace lmoe
