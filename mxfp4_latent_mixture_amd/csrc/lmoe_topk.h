// Top-k selection shared by the routing kernels: one wave selects the k
// largest of up to 1024 logits held 16 per lane.
//
// Order (the routing rule of the layer: ties go to the lower expert index):
// larger logit first, equal logits by lower expert index, NaN after every
// number, -0 == +0. Encoded as one distinct 64-bit key per expert, the high
// word an order-preserving image of the float and the low word ~expert, so
// larger keys come first and a key of 0 never beats a real one.
#ifndef LMOE_TOPK_H_
#define LMOE_TOPK_H_

#include "lmoe_device.h"

namespace lmoe {

constexpr int kTopkMaxK = 32;         // routes per token
constexpr int kTopkKeysPerLane = 16;  // E <= 1024 logits, 16 per lane

__device__ __forceinline__ uint64_t order_key(float f, int e) {
  uint32_t u = __float_as_uint(f);
  if (f == 0.0f) u = 0u;
  const uint32_t k32 = (f != f) ? 0u : ((u & 0x80000000u) ? ~u : (u | 0x80000000u));
  return ((uint64_t)k32 << 32) | (uint64_t)(~(uint32_t)e);
}

// The logit a key was made from (-0 reads back as +0, NaN as a NaN).
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t k32 = (uint32_t)(key >> 32);
  return __uint_as_float((k32 & 0x80000000u) ? (k32 & 0x7fffffffu) : ~k32);
}

// Wave-wide maximum of a 32-bit value with DPP row shifts and row broadcasts;
// the result is returned to every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
// lanes without a source (and rows outside the mask) read 0, the identity of
// the maximum, which lets the move fold into one v_max_u32 with DPP
#define LMOE_DPP_MAX32(ctrl, rmask)                                                        \
  {                                                                                        \
    const uint32_t t = __builtin_amdgcn_update_dpp(0u, v, ctrl, rmask, 0xf, false);        \
    v = t > v ? t : v;                                                                     \
  }
  LMOE_DPP_MAX32(0x111, 0xf)  // row_shr:1
  LMOE_DPP_MAX32(0x112, 0xf)  // row_shr:2
  LMOE_DPP_MAX32(0x114, 0xf)  // row_shr:4
  LMOE_DPP_MAX32(0x118, 0xf)  // row_shr:8: lane 15 of each row holds the row max
  LMOE_DPP_MAX32(0x142, 0xa)  // row_bcast:15 into rows 1 and 3
  LMOE_DPP_MAX32(0x143, 0xc)  // row_bcast:31 into rows 2 and 3: lane 63 holds the max
#undef LMOE_DPP_MAX32
  return __builtin_amdgcn_readlane(v, 63);
}

// LDS working space of one selecting wave.
struct TopkScratch {
  uint64_t cand[kWave];        // candidates
  uint64_t sorted[kTopkMaxK];  // selected keys, largest first
};

// Orders a wave's LDS accesses before and after this point (a wave's LDS
// operations complete in issue order; this keeps the compiler from moving
// them across lanes' exchanges).
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Selection of the k largest of the wave's keys (kTopkKeysPerLane per lane,
// distinct, valid ones nonzero, at least k valid and at least min(E, 64)
// lanes holding one) without k serial rounds. The k-th largest of the lanes'
// own maxima is a threshold that at least k keys reach; the keys that reach
// it are gathered in LDS and each is ranked by counting the larger ones.
// Returns false, leaving the selection to the caller, when more keys reach
// the threshold than the wave has lanes (possible only when the largest keys
// crowd into a few lanes).
__device__ inline bool select_by_threshold(int k, const uint64_t* key, TopkScratch& tk,
                                           uint64_t& mine) {
  const int lane = lane_id();
  uint64_t m = 0ull;
#pragma unroll
  for (int i = 0; i < kTopkKeysPerLane; ++i) m = key[i] > m ? key[i] : m;
  tk.cand[lane] = m;
  wave_lds_sync();
  // all 64 maxima are read before the first comparison: one LDS latency
  uint64_t v[kWave];
#pragma unroll
  for (int j = 0; j < kWave; ++j) v[j] = tk.cand[j];
  int rank = 0;
#pragma unroll
  for (int j = 0; j < kWave; ++j) rank += v[j] > m ? 1 : 0;
  // nonzero maxima are distinct, so exactly one lane has rank k - 1
  const uint64_t at = __builtin_amdgcn_ballot_w64(rank == k - 1);
  const int tl = __builtin_ctzll(at);
  // (the builtin returns a signed int: widen each word without extension)
  const uint64_t tau = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((uint32_t)(m >> 32), tl) << 32) |
                       (uint64_t)(uint32_t)__builtin_amdgcn_readlane((uint32_t)m, tl);
  wave_lds_sync();
  int n = 0;
#pragma unroll
  for (int i = 0; i < kTopkKeysPerLane; ++i) {
    const bool p = key[i] >= tau;
    const uint64_t bits = __builtin_amdgcn_ballot_w64(p);
    const int pos = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bits >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0u));
    if (p && pos < kWave) tk.cand[pos] = key[i];
    n += __builtin_popcountll(bits);
  }
  if (n > kWave) return false;
  wave_lds_sync();
  const uint64_t c = lane < n ? tk.cand[lane] : 0ull;
  int r = 0;
  for (int j0 = 0; j0 < n; j0 += 16) {  // 16 candidates per LDS latency
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = tk.cand[j0 + q];
#pragma unroll
    for (int q = 0; q < 16; ++q) r += (j0 + q < n && v[q] > c) ? 1 : 0;
  }
  if (lane < n && r < k) tk.sorted[r] = c;
  wave_lds_sync();
  mine = lane < k ? tk.sorted[lane] : 0ull;
  return true;
}

// The same selection by k serial rounds, for any spread of the keys over the
// lanes: each round takes a wave-wide maximum over each lane's best remaining
// key. A lane keeps its best two keys, so a win usually costs a register move;
// a lane that wins a third time rescans its keys below the last one it gave.
__device__ inline void select_by_rounds(int k, const uint64_t* key, uint64_t& mine) {
  const int lane = lane_id();
  uint64_t b1 = 0ull, b2 = 0ull;
#pragma unroll
  for (int i = 0; i < kTopkKeysPerLane; ++i) {
    const uint64_t kk = key[i];
    b2 = kk > b1 ? b1 : (kk > b2 ? kk : b2);
    b1 = kk > b1 ? kk : b1;
  }
  bool have2 = true, need = false;
  uint64_t last = ~0ull;
  for (int j = 0; j < k; ++j) {
    const uint32_t hi = (uint32_t)(b1 >> 32), lo = (uint32_t)b1;
    const uint32_t mhi = wave_max_u32(hi);
    // the low word decides only between lanes holding the same high word
    const uint64_t at_max = __builtin_amdgcn_ballot_w64(hi == mhi);
    uint32_t mlo;
    if (__builtin_popcountll(at_max) == 1)
      mlo = __builtin_amdgcn_readlane(lo, __builtin_ctzll(at_max));
    else
      mlo = wave_max_u32(hi == mhi ? lo : 0u);
    const uint64_t won = ((uint64_t)mhi << 32) | mlo;
    if (lane == j) mine = won;
    if (b1 == won) {  // keys are distinct: exactly one lane wins
      last = won;
      if (have2) {
        b1 = b2;
        have2 = false;
      } else {
        need = true;
      }
    }
    if (__builtin_amdgcn_ballot_w64(need)) {
      if (need) {
        b1 = 0ull;
#pragma unroll
        for (int i = 0; i < kTopkKeysPerLane; ++i)
          b1 = (key[i] < last && key[i] > b1) ? key[i] : b1;
        need = false;
      }
    }
  }
}

}  // namespace lmoe

#endif  // LMOE_TOPK_H_
