// Single-token decode of the LatentMoE layer as one persistent kernel.
//
// Batch-1 decode streams the active weights once per token and is bound by
// HBM bandwidth (infervisor.ai "Bringing up Kimi-K3 on day zero", "The
// roofline"): for this layer that is the router, the two bf16 shared experts
// and the 16 selected MXFP4 experts. Launch boundaries between dependent
// steps leave the memory system idle, so the whole layer runs as one launch:
// workgroups draw work items from ticket counters in dependency order and
// resolve dependencies with on-device counters (the pages' decode runtime
// likewise orders work with device counters instead of host launches:
// "One kernel, no host in the loop").
//
// Work items, in ticket order:
//   router      partial logits of a K slice x 128 experts; the last one to
//               finish sums the partials in a fixed order, selects the top-k
//               with softmax weights and publishes them
//   shared g/u  one shared expert, 8 intermediate columns (gate and up in one
//               16-column MFMA tile), h = bf16(silu(g) * u)
//   routed g/u  one selected expert, 16 intermediate columns; waits for the
//               routing
//   shared dn   16 output rows of the shared experts (both experts' K
//               concatenated); waits for all shared g/u items
//   routed dn   one selected expert, 64 output rows; waits for that expert's
//               g/u items
//   combine     done by whichever item completes a 64-row block last:
//               out = bf16(sum_j w_j y_j + ysh), j ascending
// Items are dealt round-robin into eight ticket queues (device-scope atomics
// on one address serialise, at about 12 ns each on MI355X, so one queue for
// ~3800 items would cost ~45 us). A workgroup only ever waits for smaller
// items: the smallest unfinished item is either being processed (all its
// inputs are done) or is the head of its queue, which a resident workgroup of
// that queue will draw next. Workgroups are dispatched in index order and a
// workgroup leaves only when its queue is empty, so each queue with work left
// keeps a resident workgroup and the kernel cannot deadlock.
//
// Cross-workgroup data (partial logits, routing, h, y) is written with
// device-scope stores and read with device-scope loads, which the MI355X
// keeps coherent across its eight L2 partitions; a producer waits for its
// stores to complete before bumping a counter. No L2 writeback or invalidate
// is needed. Counters live in the first bytes of the workspace, must be zero
// when the kernel starts and are zeroed again by the last workgroup to exit.
#include "lmoe_device.h"
#include "lmoe_internal.h"

namespace lmoe {

namespace {

constexpr long kSpinLimit = 1l << 22;

__device__ __forceinline__ int ld_dev(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int add_dev(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_f32(float* p, float v) {
  st_dev(reinterpret_cast<uint32_t*>(p), __float_as_uint(v));
}
__device__ __forceinline__ float ld_dev_f32(const float* p) {
  return __uint_as_float(ld_dev(reinterpret_cast<const uint32_t*>(p)));
}
// 16 bytes written by another workgroup of this launch
__device__ __forceinline__ u32x4_t ld16_dev(const void* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  u32x4_t r = {(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
  return r;
}

// Every thread's device-scope stores have completed; then one bump.
__device__ __forceinline__ int publish(int* ctr) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  __shared__ int s_old;
  if (threadIdx.x == 0) s_old = add_dev(ctr, 1);
  __syncthreads();
  return s_old;
}

// Thread 0 waits until *ctr >= target; a wait that outlives the spin limit
// (a broken producer) is counted in the error slot and abandoned.
__device__ __forceinline__ void wait_geq(const int* ctr, int target, int* err) {
  if (threadIdx.x == 0) {
    long it = 0;
    while (ld_dev(ctr) < target) {
      if (++it > kSpinLimit) {
        add_dev(err, 1);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

// Thread 0 waits until the kQueues spread counters at ctr, ctr + 32, ... sum
// to at least target.
__device__ __forceinline__ void wait_sum_geq(const int* ctr, int target, int* err) {
  if (threadIdx.x == 0) {
    long it = 0;
    for (;;) {
      int s = 0;
#pragma unroll
      for (int q = 0; q < kQueues; ++q) s += ld_dev(ctr + 32 * q);
      if (s >= target) break;
      if (++it > kSpinLimit) {
        add_dev(err, 1);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

__device__ __forceinline__ uint64_t order_key(float f, int e) {
  uint32_t u = __float_as_uint(f);
  if (f == 0.0f) u = 0u;
  const uint32_t k32 = (f != f) ? 0u : ((u & 0x80000000u) ? ~u : (u | 0x80000000u));
  return ((uint64_t)k32 << 32) | (uint64_t)(~(uint32_t)e);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

constexpr int kMaxL = kDecodeMaxWidth;    // largest latent / intermediate width
constexpr int kMaxSIs = kDecodeMaxWidth;  // largest S * Is
constexpr int kMaxKs = 16;                // router K slices

struct Smem {
  uint16_t xs[kMaxL];          // the token, bf16
  uint16_t as[kMaxSIs];        // A row of the current down item: h_j or both shared h
  float red[16][129];          // router phase partials / cross-wave tile sums
  float logit[1024];
  int sel[32];
  int misc[8];
};

}  // namespace

// ---------------------------------------------------------------------------
// Router item: partial logits for rows [r0, r1) x experts [e0, e0 + 128).
// Thread (c, ph): experts e0 + 8c .. +8, rows r0 + ph + 16 i.
// ---------------------------------------------------------------------------
__device__ void router_item(const DecodeArgs& a, int item, Smem& sm) {
  const int tid = threadIdx.x;
  const int c = tid & 15, ph = tid >> 4;
  const int kr = item / a.neg, eg = item % a.neg;
  const int e0 = eg * 128 + c * 8;
  const int r0 = kr * a.rk;
  const int r1 = min(a.L, r0 + a.rk);
  const bool vec = (a.E % 8) == 0 && e0 + 8 <= a.E;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  u32x4_t wv[16];
  float xv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = r0 + ph + 16 * i;
    const bool ok = r < r1;
    xv[i] = ok ? bf16_bits_to_f32(sm.xs[r]) : 0.f;
    if (ok && vec) {
      wv[i] = load16(a.wr + (size_t)r * a.E + e0);
    } else {
      uint32_t p[4] = {0u, 0u, 0u, 0u};
      if (ok) {
        for (int q = 0; q < 8; ++q) {
          const uint32_t v = (e0 + q < a.E) ? a.wr[(size_t)r * a.E + e0 + q] : 0u;
          p[q >> 1] |= v << (16 * (q & 1));
        }
      }
      wv[i] = u32x4_t{p[0], p[1], p[2], p[3]};
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = fmaf(xv[i], __uint_as_float(wv[i][q] << 16), acc[2 * q]);
      acc[2 * q + 1] = fmaf(xv[i], __uint_as_float(wv[i][q] & 0xFFFF0000u), acc[2 * q + 1]);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) sm.red[ph][c * 8 + i] = acc[i];
  __syncthreads();
  if (tid < 128) {
    float s = 0.f;
#pragma unroll
    for (int p = 0; p < 16; ++p) s += sm.red[p][tid];
    const int e = eg * 128 + tid;
    if (e < a.E) st_dev_f32(a.part + (size_t)kr * a.E + e, s);
  }
}

// ---------------------------------------------------------------------------
// Top-k of the summed partial logits, softmax weights, routing outputs; then
// the routing flag is raised.
// ---------------------------------------------------------------------------
__device__ void topk_item(const DecodeArgs& a, Smem& sm) {
  const int tid = threadIdx.x;
  {
    // every partial of this thread's experts in flight at once, then summed
    // in K-slice order
    float v[4][kMaxKs];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = tid + 256 * r;
#pragma unroll
      for (int kr = 0; kr < kMaxKs; ++kr)
        v[r][kr] = (e < a.E && kr < a.nks) ? ld_dev_f32(a.part + (size_t)kr * a.E + e) : 0.f;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = tid + 256 * r;
      float s = 0.f;
#pragma unroll
      for (int kr = 0; kr < kMaxKs; ++kr)
        if (kr < a.nks) s += v[r][kr];
      if (e < a.E) {
        sm.logit[e] = s;
        if (a.logits_out) a.logits_out[e] = s;
      }
    }
  }
  __syncthreads();
  if (tid < kWave) {
    const int lane = tid;
    uint64_t key[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = lane + kWave * i;
      key[i] = (e < a.E) ? order_key(sm.logit[e], e) : 0ull;
    }
    uint64_t best = 0ull;
#pragma unroll
    for (int i = 0; i < 16; ++i) best = key[i] > best ? key[i] : best;
    int my_e = 0;
    float my_l = 0.f;
    for (int j = 0; j < a.k; ++j) {
      const uint64_t b = wave_max_u64(best);
      const int ew = (int)(~(uint32_t)b);
      if (lane == j) {
        my_e = ew;
        my_l = sm.logit[ew];
      }
      if ((ew & (kWave - 1)) == lane) {
        const int slot = ew / kWave;
        best = 0ull;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (i == slot) key[i] = 0ull;
          best = key[i] > best ? key[i] : best;
        }
      }
    }
    const float l0 = __shfl(my_l, 0, kWave);
    const float z = (lane < a.k) ? expf(my_l - l0) : 0.f;
    float s = z;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_down(s, off, kWave);
    s = __shfl(s, 0, kWave);
    if (lane < a.k) {
      st_dev(reinterpret_cast<uint32_t*>(a.idx) + lane, (uint32_t)my_e);
      st_dev_f32(a.w + lane, z / s);
      sm.sel[lane] = my_e;
    }
  }
  __syncthreads();
  // grouping outputs for one token: each route is its own group, in expert order
  for (int e = tid; e < a.E; e += 256) {
    int below = 0, hit = 0;
    for (int j = 0; j < a.k; ++j) {
      below += sm.sel[j] < e;
      hit += sm.sel[j] == e;
    }
    a.counts[e] = hit;
    a.offsets[e] = below;
  }
  if (tid == 0) a.offsets[a.E] = a.k;
  if (tid < a.k) {
    int pos = 0;
    for (int j = 0; j < a.k; ++j) pos += sm.sel[j] < sm.sel[tid];
    a.perm[pos] = tid;
    a.inv[tid] = pos;
  }
  publish(a.ctr + kCtrTopk);
}

// ---------------------------------------------------------------------------
// GEMV core: NT weight tiles of 16 rows each against the token row held in
// LDS. K is split over the four waves in contiguous quarters; in a wave
// iteration the four lane groups take adjacent runs of U MX blocks (full
// cache lines per wave-wide load). Weights are fetched in bursts of CH
// iterations (all loads of a burst in flight together), then consumed. Every
// lane of a lane group reads the same A values (an LDS broadcast), so all 16
// rows of each MFMA result equal the token's row; row 0 is used.
// ---------------------------------------------------------------------------
template <bool FP4>
struct WOps;
template <>
struct WOps<true> {
  u32x4_t c[2];
  uint32_t s[2];
};
template <>
struct WOps<false> {
  u32x4_t b[4];
};

// wrow(t, col, q, sc, b) gives tile t's weight row for this lane (codes and
// exponents, or bf16), nullptr for a padding column.
template <bool FP4, int NT, int CH, typename WRow>
__device__ __forceinline__ void gemv_tiles(const uint16_t* arow_lds, int K, WRow wrow,
                                           f32x4_t (&acc)[NT]) {
  constexpr int U = FP4 ? 2 : 1;
  constexpr int SPAN = 4 * U;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int nblk = K / 32;
  const int bw_lo = (wave * nblk) / 4;
  const int bw_hi = ((wave + 1) * nblk) / 4;
  const int iters = (bw_hi - bw_lo + SPAN - 1) / SPAN;

  const uint8_t* q[NT];
  const uint8_t* sc[NT];
  const uint16_t* bw[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    wrow(t, col, q[t], sc[t], bw[t]);
    acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  for (int it0 = 0; it0 < iters; it0 += CH) {
    WOps<FP4> w[CH][NT];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int b0 = bw_lo + (it0 + c) * SPAN + grp * U;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int blk = b0 + u;
          const bool ok = it0 + c < iters && blk < bw_hi;
          if constexpr (FP4) {
            const bool w_ok = ok && q[t] != nullptr;
            w[c][t].c[u] = w_ok ? load16(q[t] + blk * 16) : zero16();
            w[c][t].s[u] = w_ok ? (uint32_t)sc[t][blk] : 127u;
          } else {
            const bool w_ok = ok && bw[t] != nullptr;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
              w[c][t].b[qq] = w_ok ? load16(bw[t] + blk * 32 + qq * 8) : zero16();
          }
        }
      }
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int b0 = bw_lo + (it0 + c) * SPAN + grp * U;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // past-the-end blocks carry zero weights; their A reads stay inside the row
        const int blk = min(b0 + u, nblk - 1);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const bf16x8_t av =
              *reinterpret_cast<const bf16x8_t*>(arow_lds + blk * 32 + qq * 8);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            bf16x8_t bv;
            if constexpr (FP4)
              bv = dequant8(w[c][t].c[u][qq], e8m0_to_f32(w[c][t].s[u]));
            else
              bv = as_bf16x8(w[c][t].b[qq]);
            acc[t] = mfma16(av, bv, acc[t]);
          }
        }
      }
    }
  }
}

// Sum the 16 row-0 results of every wave's tile(s) into sm.red[tile * 4 + wave][col].
template <int NT>
__device__ __forceinline__ void reduce_row0(const f32x4_t (&acc)[NT], Smem& sm) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane < 16) {
#pragma unroll
    for (int t = 0; t < NT; ++t) sm.red[t * 4 + wave][lane] = acc[t][0];
  }
  __syncthreads();
}

__device__ __forceinline__ float sum_waves(const Smem& sm, int t, int c) {
  float s = sm.red[t * 4 + 0][c];
  s += sm.red[t * 4 + 1][c];
  s += sm.red[t * 4 + 2][c];
  s += sm.red[t * 4 + 3][c];
  return s;
}

// Copy n bf16 values written by other workgroups of this launch into LDS.
__device__ __forceinline__ void stage_dev(uint16_t* dst, const uint16_t* src, int n) {
  for (int i = threadIdx.x * 8; i < n; i += 256 * 8)
    *reinterpret_cast<u32x4_t*>(dst + i) = ld16_dev(src + i);
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Items
// ---------------------------------------------------------------------------
__device__ void shared_gu_item(const DecodeArgs& a, int item, Smem& sm) {
  const int per = (a.Is + 7) / 8;
  const int s = item / per;
  const int i0 = (item % per) * 8;
  f32x4_t acc[1];
  gemv_tiles<false, 1, 4>(sm.xs, a.L,
      [&](int, int col, const uint8_t*& q, const uint8_t*& sc, const uint16_t*& b) {
        q = sc = nullptr;
        const int i = i0 + (col & 7);
        const uint16_t* m = (col < 8) ? a.shg : a.shu;
        b = (i < a.Is) ? m + ((size_t)s * a.Is + i) * a.L : nullptr;
      }, acc);
  reduce_row0<1>(acc, sm);
  const int tid = threadIdx.x;
  if (tid < 8) {
    const float g = sum_waves(sm, 0, tid);
    const float u = sum_waves(sm, 0, tid + 8);
    sm.logit[tid] = __uint_as_float((uint32_t)f32_to_bf16_bits(silu(g) * u));
  }
  __syncthreads();
  if (tid < 4) {
    const int i = i0 + 2 * tid;
    if (i < a.Is) {  // Is % 32 == 0, so i + 1 < Is too
      const uint32_t lo = __float_as_uint(sm.logit[2 * tid]);
      const uint32_t hi = __float_as_uint(sm.logit[2 * tid + 1]);
      st_dev(reinterpret_cast<uint32_t*>(a.hsh + (size_t)s * a.Is + i), lo | (hi << 16));
    }
  }
  publish(a.ctr + kCtrShared + 32 * (item % kQueues));
}

__device__ void routed_gu_item(const DecodeArgs& a, int item, Smem& sm, bool& routed) {
  const int j = item / a.gu_per_route;
  const int i0 = (item % a.gu_per_route) * 16;
  if (!routed) {
    wait_geq(a.ctr + kCtrTopk, 1, a.ctr + kCtrError);
    routed = true;
  }
  if (threadIdx.x == 0) sm.misc[0] = (int)ld_dev(reinterpret_cast<const uint32_t*>(a.idx) + j);
  __syncthreads();
  const int e = min(max(sm.misc[0], 0), a.E - 1);  // in range even after a timed-out wait
  const size_t qoff = (size_t)e * a.I * (a.L / 2);
  const size_t soff = (size_t)e * a.I * (a.L / 32);
  f32x4_t acc[2];
  gemv_tiles<true, 2, 4>(sm.xs, a.L,
      [&](int t, int col, const uint8_t*& q, const uint8_t*& sc, const uint16_t*& b) {
        b = nullptr;
        const int i = i0 + col;
        if (i < a.I) {
          q = (t == 0 ? a.gq : a.uq) + qoff + (size_t)i * (a.L / 2);
          sc = (t == 0 ? a.gs : a.us) + soff + (size_t)i * (a.L / 32);
        } else {
          q = sc = nullptr;
        }
      }, acc);
  reduce_row0<2>(acc, sm);
  const int tid = threadIdx.x;
  if (tid < 16) {
    const float g = sum_waves(sm, 0, tid);
    const float u = sum_waves(sm, 1, tid);
    sm.logit[tid] = __uint_as_float((uint32_t)f32_to_bf16_bits(silu(g) * u));
  }
  __syncthreads();
  if (tid < 8) {
    const int i = i0 + 2 * tid;
    if (i < a.I) {
      const uint32_t lo = __float_as_uint(sm.logit[2 * tid]);
      const uint32_t hi = __float_as_uint(sm.logit[2 * tid + 1]);
      st_dev(reinterpret_cast<uint32_t*>(a.h + (size_t)j * a.I + i), lo | (hi << 16));
    }
  }
  publish(a.ctr + kCtrRoute + 16 * j);
}

__device__ void combine_block(const DecodeArgs& a, int b) {
  const int tid = threadIdx.x;
  const int l = b * 64 + tid;
  if (tid < 64 && l < a.L) {
    float acc = 0.f;
    for (int j = 0; j < a.k; ++j)
      acc = fmaf(ld_dev_f32(a.w + j), ld_dev_f32(a.y + (size_t)j * a.L + l), acc);
    if (a.S > 0) acc += ld_dev_f32(a.ysh + l);
    a.out[l] = f32_to_bf16_bits(acc);
  }
}

__device__ void finish_block_part(const DecodeArgs& a, int b) {
  const int old = publish(a.ctr + kCtrBlock + 16 * b);
  const int nt16 = a.L / 16;
  const int nsub = min(4, nt16 - 4 * b);
  const int target = a.k + (a.S > 0 ? nsub : 0);
  if (old == target - 1) combine_block(a, b);
}

__device__ void shared_dn_item(const DecodeArgs& a, int item, Smem& sm, bool& shared_ready) {
  if (!shared_ready) {
    wait_sum_geq(a.ctr + kCtrShared, a.n_shgu, a.ctr + kCtrError);
    shared_ready = true;
  }
  const int l0 = item * 16;
  const int K = a.S * a.Is;  // both experts' inputs, concatenated: A = [h_0 | h_1 | ...]
  stage_dev(sm.as, a.hsh, K);
  f32x4_t acc[1];
  // tile row l of expert s is at shd[s][l]; the concatenated K is addressed per
  // expert, so the row pointer handed to the core is expert 0's and the core's
  // block index runs on into the next experts' rows (see below)
  if (a.S == 1) {
    gemv_tiles<false, 1, 4>(sm.as, K,
        [&](int, int col, const uint8_t*& q, const uint8_t*& sc, const uint16_t*& b) {
          q = sc = nullptr;
          const int l = l0 + col;
          b = (l < a.L) ? a.shd + (size_t)l * a.Is : nullptr;
        }, acc);
  } else {
    // one pass per shared expert, summed in expert order
    f32x4_t part[1];
    acc[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s2 = 0; s2 < a.S; ++s2) {
      gemv_tiles<false, 1, 4>(sm.as + (size_t)s2 * a.Is, a.Is,
          [&](int, int col, const uint8_t*& q, const uint8_t*& sc, const uint16_t*& b) {
            q = sc = nullptr;
            const int l = l0 + col;
            b = (l < a.L) ? a.shd + ((size_t)s2 * a.L + l) * a.Is : nullptr;
          }, part);
      acc[0] += part[0];
    }
  }
  reduce_row0<1>(acc, sm);
  const int tid = threadIdx.x;
  if (tid < 16 && l0 + tid < a.L) st_dev_f32(a.ysh + l0 + tid, sum_waves(sm, 0, tid));
  finish_block_part(a, item / 4);
}

__device__ void routed_dn_item(const DecodeArgs& a, int item, Smem& sm) {
  const int j = item / a.dn_per_route;
  const int b = item % a.dn_per_route;
  wait_geq(a.ctr + kCtrRoute + 16 * j, a.gu_per_route, a.ctr + kCtrError);
  if (threadIdx.x == 0) sm.misc[0] = (int)ld_dev(reinterpret_cast<const uint32_t*>(a.idx) + j);
  __syncthreads();
  const int e = min(max(sm.misc[0], 0), a.E - 1);  // in range even after a timed-out wait
  const size_t qoff = (size_t)e * a.L * (a.I / 2);
  const size_t soff = (size_t)e * a.L * (a.I / 32);
  stage_dev(sm.as, a.h + (size_t)j * a.I, a.I);
  f32x4_t acc[4];
  gemv_tiles<true, 4, 2>(sm.as, a.I,
      [&](int t, int col, const uint8_t*& q, const uint8_t*& sc, const uint16_t*& bb) {
        bb = nullptr;
        const int l = b * 64 + t * 16 + col;
        if (l < a.L) {
          q = a.dq + qoff + (size_t)l * (a.I / 2);
          sc = a.ds + soff + (size_t)l * (a.I / 32);
        } else {
          q = sc = nullptr;
        }
      }, acc);
  reduce_row0<4>(acc, sm);
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int l = b * 64 + tid;
    if (l < a.L) st_dev_f32(a.y + (size_t)j * a.L + l, sum_waves(sm, tid >> 4, tid & 15));
  }
  finish_block_part(a, b);
}

__global__ __launch_bounds__(256, 2) void decode_kernel(DecodeArgs a) {
  __shared__ Smem sm;
  __shared__ int s_ticket;
  const int tid = threadIdx.x;
  // Items are dealt round-robin into kQueues ticket queues; this workgroup
  // draws from queue blockIdx.x % kQueues. Each queue is in item order, so a
  // workgroup only waits for smaller items; the first kQueues workgroups are
  // dispatched first and each stays until its queue is empty, so every queue
  // with work left always has a resident workgroup.
  const int q = blockIdx.x % kQueues;
  int* ticket = a.ctr + kCtrTicket + 32 * q;
  bool routed = false, shared_ready = false;
  for (int i = tid * 8; i < a.L; i += 256 * 8)
    *reinterpret_cast<u32x4_t*>(sm.xs + i) = load16(a.x + i);
  if (tid == 0) s_ticket = q + kQueues * add_dev(ticket, 1);
  __syncthreads();
  int t = s_ticket;
  while (t < a.t_total) {
    int next = 0;
    if (tid == 0) next = q + kQueues * add_dev(ticket, 1);
    if (t < a.t_shgu) {
      router_item(a, t, sm);
      const int old = publish(a.ctr + kCtrRouter);
      if (old == a.n_router - 1) topk_item(a, sm);
    } else if (t < a.t_gu) {
      shared_gu_item(a, t - a.t_shgu, sm);
    } else if (t < a.t_shd) {
      routed_gu_item(a, t - a.t_gu, sm, routed);
    } else if (t < a.t_dn) {
      shared_dn_item(a, t - a.t_shd, sm, shared_ready);
    } else {
      routed_dn_item(a, t - a.t_dn, sm);
    }
    __syncthreads();
    if (tid == 0) s_ticket = next;
    __syncthreads();
    t = s_ticket;
  }
  // the last workgroup out zeroes the counters for the next launch
  if (tid == 0) {
    const int old = add_dev(a.ctr + kCtrExit, 1);
    s_ticket = (old == (int)gridDim.x - 1);
  }
  __syncthreads();
  if (s_ticket) {
    const int nb = (a.L + 63) / 64;
    for (int i = tid; i < a.k; i += 256) st_dev(a.ctr + kCtrRoute + 16 * i, 0);
    for (int i = tid; i < nb; i += 256) st_dev(a.ctr + kCtrBlock + 16 * i, 0);
    if (tid < kQueues) {
      st_dev(a.ctr + kCtrTicket + 32 * tid, 0);
      st_dev(a.ctr + kCtrShared + 32 * tid, 0);
    }
    if (tid == 0) {
      st_dev(a.ctr + kCtrRouter, 0);
      st_dev(a.ctr + kCtrTopk, 0);
      st_dev(a.ctr + kCtrExit, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static int decode_grid() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] > 0) return cached[dev];
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, decode_kernel, 256, 0) != hipSuccess ||
      per <= 0)
    per = 2;
  cached[dev] = cus * per;
  return cached[dev];
}

void make_decode_args(const Plan& p, DecodeArgs& a) {
  const lmoe_dims& d = p.d;
  a.L = d.L;
  a.E = d.E;
  a.k = d.k;
  a.I = d.I;
  a.S = d.S;
  a.Is = d.Is;
  const int nsteps = d.L / 32;
  int nks = std::min(nsteps, 16);
  int rk = 32 * ((nsteps + nks - 1) / nks);
  if (rk > 256) rk = 256;
  nks = (d.L + rk - 1) / rk;
  a.nks = nks;
  a.rk = rk;
  a.neg = (d.E + 127) / 128;
  a.n_router = nks * a.neg;
  a.n_shgu = d.S > 0 ? d.S * ((d.Is + 7) / 8) : 0;
  a.gu_per_route = (d.I + 15) / 16;
  a.dn_per_route = (d.L + 63) / 64;
  a.n_gu = d.k * a.gu_per_route;
  a.n_shd = d.S > 0 ? d.L / 16 : 0;
  a.n_dn = d.k * a.dn_per_route;
  a.t_shgu = a.n_router;
  a.t_gu = a.t_shgu + a.n_shgu;
  a.t_shd = a.t_gu + a.n_gu;
  a.t_dn = a.t_shd + a.n_shd;
  a.t_total = a.t_dn + a.n_dn;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  // at least one workgroup per ticket queue
  const int grid = std::max(kQueues, std::min(decode_grid(), a.t_total));
  hipLaunchKernelGGL(decode_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lmoe
