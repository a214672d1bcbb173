// Building blocks of the persistent decode kernels: device-scope exchange
// between waves of one launch, and the weight-streaming GEMVs whose items
// multiply up to 16 activation rows (one per MFMA row) by a tile of weight
// rows over the whole K range.
//
// Batch-1 (and few-token) decode streams each active expert's weights once
// and is bound by HBM bandwidth (infervisor.ai "Bringing up Kimi-K3 on day
// zero", "The roofline"); the 16 rows of a 16x16x32 MFMA carry one token each
// (or one token in all of them), so a weight tile read once serves every
// token routed to its expert (dev48.org "Kimi K3 on AMD Instinct GPUs with
// TokenSpeed", section 4.1: each expert's weights reused by all its tokens).
#pragma once

#include "lmoe_device.h"

namespace lmoe {

// ---------------------------------------------------------------------------
// Device-scope exchange. Data passed between waves (logits, h, y) is written
// with device-scope stores and read with device-scope loads, which stay
// coherent across the eight L2 partitions; a producer waits for its stores to
// complete before it bumps a counter.
// ---------------------------------------------------------------------------
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
// 16 bytes written by another wave of this launch
__device__ __forceinline__ u32x4_t ld16_dev(const void* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  u32x4_t r = {(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
  return r;
}

// All of this wave's stores have completed; then lane 0 bumps the counter.
// Returns the previous value (uniform) when `want_old`.
__device__ __forceinline__ int publish(int* ctr, bool want_old) {
  // The data stores above are device-scope (coherent in every L2 partition)
  // and complete before the counter bump once the wait returns. The fence
  // keeps the compiler from moving a store past that point: the waitcnt
  // builtin alone touches no memory in the compiler's model.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  int old = 0;
  if (lane_id() == 0) {
    if (want_old)
      old = add_dev(ctr, 1);
    else
      __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return __builtin_amdgcn_readfirstlane(old);
}

// Waits until the sum of n (<= 64) counters spaced `stride` ints apart reaches
// target. A wait that outlives the spin limit (a broken producer) is counted in
// the error slot and abandoned.
__device__ __forceinline__ void wait_geq(const int* ctr, int target, int* err, int n = 1,
                                         int stride = 0) {
  long it = 0;
  for (;;) {
    int s = 0;
    if (lane_id() < n) s = ld_dev(ctr + stride * lane_id());
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) s += __shfl_xor(s, off, kWave);
    s = __builtin_amdgcn_readfirstlane(s);
    if (s >= target) {
      // the dependent loads that follow stay after the counter was seen
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      break;
    }
    if (++it > kSpinLimit) {
      if (lane_id() == 0) add_dev(err, 1);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// ---------------------------------------------------------------------------
// Weight streaming. Weights are read through buffer resources: an offset past
// the end of the matrix returns zeros, so padding rows and past-the-end blocks
// need no branches around loads, and each burst of loads is issued as a group
// (pinned by scheduling barriers) one burst ahead of the MFMAs that consume
// it.
//
// Lane l supplies A row l % 16 of each MFMA (the A source below says where
// that row lives); D comes back as column l % 16, rows 4 (l / 16) + 0..3.
// When every lane's A row is the same token, all 16 result rows are equal and
// lanes 0..15 of acc[t][0] hold the tile's 16 results.
//
// MXFP4 rows (16 bytes of codes per 32-value block): in iteration it, lane
// group g takes blocks 8 it + 2 g + u (u = 0, 1), so the four groups read 128
// contiguous bytes of every row per iteration. Each 64-block window's 64
// exponent bytes are fetched with dword-aligned loads (the range check of a
// buffer load zeroes a whole dword that reaches past the end), realigned,
// reduced to the 16 bytes the lane uses, and prefetched one window ahead.
//
// bf16 rows: in iteration it, instruction j, lane group g reads values
// 128 it + 32 j + 8 g .. +8, so each instruction reads 64 contiguous bytes of
// every row.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kOob = 0x40000000;  // an offset past the end of every matrix

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4_t bload16(rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t bload4(rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
// A 16-byte load with the cache policy of a device-scope load (sc1): data
// that other waves of this launch wrote with device-scope stores.
__device__ __forceinline__ u32x4_t bload16_dev(rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16));
}

// One tile of 16 weight rows: the lane's row starts at byte `row` of its
// resource(s) (kOob for a padding row).
struct Tile4 {
  rsrc_t codes, scales;
  int code_row, scale_row;
};
struct Tile16 {
  rsrc_t w;
  int row;
};

// A operand sources. get(elem, slot, buf) returns the lane's eight A values
// starting at element `elem` of its row; load(elem, slot, buf) is called for
// the same (elem, slot) one burst ahead.
//
// ALds: the lane's row in LDS (the same row in every lane for one token).
struct ALds {
  const uint16_t* row;
  template <int N>
  struct Buf {};
  template <int N>
  __device__ __forceinline__ void load(int, int, Buf<N>&) const {}
  template <int N>
  __device__ __forceinline__ bf16x8_t get(int elem, int, const Buf<N>&) const {
    return *reinterpret_cast<const bf16x8_t*>(row + elem);
  }
};
// ADev: the lane's row in device memory written earlier in this launch by
// other waves (device-scope loads, kept in the burst ring like the weights);
// `row` is its byte offset in the resource, kOob for a lane without a row
// (it reads zeros and moves no data).
struct ADev {
  rsrc_t r;
  int row;
  template <int N>
  struct Buf {
    u32x4_t v[N];
  };
  template <int N>
  __device__ __forceinline__ void load(int elem, int slot, Buf<N>& b) const {
    b.v[slot] = bload16_dev(r, row + elem * 2);
  }
  template <int N>
  __device__ __forceinline__ bf16x8_t get(int, int slot, const Buf<N>& b) const {
    return as_bf16x8(b.v[slot]);
  }
};

// D bursts are kept in flight ahead of the one being computed, in a ring of
// RING buffers. `pre` runs once the first bursts' weights are in flight and
// before the first A value is loaded or read: a dependency wait (and the
// staging of an LDS row) overlaps those loads.
template <int NT, int IPB, int D, typename ASrc, typename Pre>
__device__ __forceinline__ void gemv_fp4(const ASrc& asrc, int nblk, const Tile4 (&tl)[NT],
                                         f32x4_t (&acc)[NT], Pre&& pre) {
  constexpr int BPW = 8 / IPB;  // bursts per 64-block window
  constexpr int RING = D == 1 ? 2 : 4;
  constexpr int NA = IPB * 8;   // A loads per burst: (iteration, u, quarter)
  static_assert(8 % IPB == 0 && BPW % RING == 0 && D < RING, "the ring must tile a window");
  const int grp = lane_id() >> 4;
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nwin = (nblk + 63) / 64;

  // raw exponent window: 17 dwords from the dword at or below the window start
  struct Raw {
    u32x4_t q[4];
    uint32_t tail;
  };
  Raw raw[NT];
  uint32_t ex[NT][4];  // the lane's 16 exponent bytes of the current window
  uint32_t shift[NT];
  auto load_exps = [&](int w) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int off = 64 * w < nblk ? tl[t].scale_row + 64 * w : kOob;
      const int sh = off & 3;
      const int a0 = off - sh;
#pragma unroll
      for (int j = 0; j < 4; ++j) raw[t].q[j] = bload16(tl[t].scales, a0 + 16 * j);
      raw[t].tail = bload4(tl[t].scales, sh ? a0 + 64 : kOob);
      shift[t] = (uint32_t)sh;
    }
  };
  // exponent of block 8 p + 2 g + u of the window is byte 2 p + u of ex:
  // the lane's two bytes of iteration p are halfword g of window bytes 8p..8p+7
  auto take_exps = [&]() {
    const uint32_t gs = 16u * (uint32_t)grp;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      uint32_t d[17];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) d[4 * j + c] = raw[t].q[j][c];
      d[16] = raw[t].tail;
#pragma unroll
      for (int i = 0; i < 16; ++i) d[i] = __builtin_amdgcn_alignbyte(d[i + 1], d[i], shift[t]);
      uint32_t hw[8];
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const uint64_t v = ((uint64_t)d[2 * p + 1] << 32) | d[2 * p];
        hw[p] = (uint32_t)(v >> gs) & 0xFFFFu;
      }
#pragma unroll
      for (int p = 0; p < 8; p += 2) ex[t][p >> 1] = hw[p] | (hw[p + 1] << 16);
    }
  };
  struct Buf {
    u32x4_t c[IPB][NT][2];
    typename ASrc::template Buf<NA> a;
  };
  // element of the lane's A row that step (iteration it, u, quarter qq) reads:
  // past-the-end blocks carry zero codes and exponent 2^0 (never NaN) and
  // read A inside the row
  auto a_elem = [&](int it, int u, int qq) {
    const int blk = 8 * it + 2 * grp + u;
    return (blk < nblk ? blk : nblk - 1) * 32 + qq * 8;
  };
  // bp is a compile-time constant at every call
  auto load_w = [&](int w, const int bp, Buf& b) {
#pragma unroll
    for (int c = 0; c < IPB; ++c) {
      const int it = w * 8 + bp * IPB + c;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int blk = 8 * it + 2 * grp + u;
#pragma unroll
        for (int t = 0; t < NT; ++t)
          b.c[c][t][u] = bload16(tl[t].codes, blk < nblk ? tl[t].code_row + blk * 16 : kOob);
      }
    }
  };
  auto load_a = [&](int w, const int bp, Buf& b) {
#pragma unroll
    for (int c = 0; c < IPB; ++c) {
      const int it = w * 8 + bp * IPB + c;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) asrc.load(a_elem(it, u, qq), (c * 2 + u) * 4 + qq, b.a);
    }
  };
  auto compute = [&](int w, const int bp, const Buf& b) {
#pragma unroll
    for (int c = 0; c < IPB; ++c) {
      const int p = bp * IPB + c;  // iteration within the window
      const int it = w * 8 + p;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int blk = 8 * it + 2 * grp + u;
        const bool ok = blk < nblk;
        float scale[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint32_t e8 = (ex[t][p >> 1] >> (8 * (2 * (p & 1) + u))) & 0xFFu;
          scale[t] = e8m0_to_f32(ok ? e8 : 127u);
        }
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const bf16x8_t av = asrc.get(a_elem(it, u, qq), (c * 2 + u) * 4 + qq, b.a);
#pragma unroll
          for (int t = 0; t < NT; ++t)
            acc[t] = mfma16(av, dequant8(b.c[c][t][u][qq], scale[t]), acc[t]);
        }
      }
    }
  };
  Buf buf[RING];
  load_exps(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int b = 0; b < D; ++b) load_w(0, b, buf[b]);
  __builtin_amdgcn_sched_barrier(0);
  pre();
#pragma unroll
  for (int b = 0; b < D; ++b) load_a(0, b, buf[b]);
  take_exps();
  for (int w = 0; w < nwin; ++w) {
#pragma unroll
    for (int bp = 0; bp < BPW; ++bp) {
      // the burst D ahead (in the next window near the end of this one)
      if (bp + D < BPW) {
        load_w(w, bp + D, buf[(bp + D) % RING]);
        load_a(w, bp + D, buf[(bp + D) % RING]);
      } else {
        load_w(w + 1, bp + D - BPW, buf[(bp + D) % RING]);
        load_a(w + 1, bp + D - BPW, buf[(bp + D) % RING]);
      }
      if (bp == 0) load_exps(w + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(w, bp, buf[bp % RING]);
      __builtin_amdgcn_sched_barrier(0);
    }
    take_exps();
  }
}

template <int NT, int IPB, int D, typename ASrc, typename Pre>
__device__ __forceinline__ void gemv_bf16(const ASrc& asrc, int nblk, const Tile16 (&tl)[NT],
                                          f32x4_t (&acc)[NT], Pre&& pre) {
  constexpr int RING = D == 1 ? 2 : 4;
  constexpr int NA = IPB * 4;  // A loads per burst: (iteration, instruction)
  static_assert(D < RING, "the ring holds the bursts in flight");
  const int grp = lane_id() >> 4;
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int iters = (nblk + 3) / 4;  // 4 blocks of 32 values per iteration
  const int bursts = (iters + IPB - 1) / IPB;
  struct Buf {
    u32x4_t b[IPB][NT][4];
    typename ASrc::template Buf<NA> a;
  };
  auto a_elem = [&](int it, int j) { return min(4 * it + j, nblk - 1) * 32 + grp * 8; };
  auto load_w = [&](int burst, Buf& w) {
#pragma unroll
    for (int c = 0; c < IPB; ++c) {
      const int it = burst * IPB + c;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int blk = 4 * it + j;
#pragma unroll
        for (int t = 0; t < NT; ++t)
          w.b[c][t][j] = bload16(tl[t].w, blk < nblk ? tl[t].row + blk * 64 + grp * 16 : kOob);
      }
    }
  };
  auto load_a = [&](int burst, Buf& w) {
#pragma unroll
    for (int c = 0; c < IPB; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) asrc.load(a_elem(burst * IPB + c, j), c * 4 + j, w.a);
  };
  auto compute = [&](int burst, const Buf& w) {
#pragma unroll
    for (int c = 0; c < IPB; ++c) {
      const int it = burst * IPB + c;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8_t av = asrc.get(a_elem(it, j), c * 4 + j, w.a);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = mfma16(av, as_bf16x8(w.b[c][t][j]), acc[t]);
      }
    }
  };
  // no load is conditional: bursts past the end read out of bounds (zeros)
  Buf buf[RING];
#pragma unroll
  for (int b = 0; b < D; ++b) load_w(b, buf[b]);
  __builtin_amdgcn_sched_barrier(0);
  pre();
#pragma unroll
  for (int b = 0; b < D; ++b) load_a(b, buf[b]);
  for (int b = 0; b < bursts; b += RING) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      load_w(b + r + D, buf[(r + D) % RING]);
      load_a(b + r + D, buf[(r + D) % RING]);
      __builtin_amdgcn_sched_barrier(0);
      compute(b + r, buf[r]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

}  // namespace lmoe
