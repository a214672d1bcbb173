// Decode of 2 to 16 tokens as one persistent kernel: the single-token
// kernel's work-item scheme with one token in each MFMA row.
//
// A few decode tokens still leave the layer bound by HBM: their selected
// experts' weights are streamed once per step (infervisor.ai "Bringing up
// Kimi-K3 on day zero", "The roofline"). With T tokens of k routes, an expert
// chosen by several tokens is streamed once for all of them: the routes are
// grouped by expert inside the launch, and a weight tile read once multiplies
// the rows of every token in its group (dev48.org "Kimi K3 on AMD Instinct
// GPUs with TokenSpeed", section 4.1: small batches walk each token's routes
// directly, and an expert's weights are reused by all its tokens). A 16x16x32
// MFMA has 16 rows: lane l supplies row l % 16, so up to 16 tokens (or the
// tokens of one group) ride in one tile and the weight stream is the same as
// for one token.
//
// Work items, in ticket order (sizes for the Kimi-K3 layer):
//   router      one expert's logits for all T tokens: its 7 KB router row
//               against the T token rows in LDS; each logit is published as
//               a flagged 64-bit word
//   top-k       one token: waits for its E logits, selects k, writes its
//               routes and softmax weights, publishes a count
//   shared g/u  one shared expert, 8 intermediate columns (gate and up in one
//               16-column tile) for all T tokens                 (115 KB)
//   routed g/u  one expert group (an expert and the tokens that chose it),
//               16 intermediate columns                           (61 KB)
//   shared dn   16 output rows of one shared expert for all T tokens (64 KB)
//   routed dn   one expert group, 32 output rows                  (35 KB)
//   combine     for token t and 64-row block b, done by whichever item
//               completes that block's inputs last:
//               out_t = bf16(sum_j w_tj y_tj + sum_s ysh_ts), in that order
// The number of groups (distinct experts) is known only once the routing is;
// the tickets cover min(E, T k) group slots, and the items of slots past the
// last group return at once. Every workgroup builds the grouping in LDS from
// the published routes (a deterministic function of them, so all copies
// agree): routes ordered by expert, then token, which is also the stable
// permutation the layer reports.
//
// Ordering, memory model and the absence of deadlock are those of the
// single-token kernel: a wave only ever waits for items with smaller tickets,
// data passed between waves goes through device-scope stores and loads, and a
// producer's stores complete before it bumps a counter. The routed and shared
// down items read their A rows (h) straight from device memory with
// device-scope loads, kept one burst ahead with the weights; the tokens stay
// in LDS for the router and gate/up items. Counters and flagged logits live
// in the workspace's counter block: zero at launch, zero again at exit (a
// top-k item clears its token's logits, a combine its block's count, the last
// wave out the rest).
#include <atomic>
#include <mutex>

#include "lmoe_internal.h"
#include "lmoe_stream.h"
#include "lmoe_topk.h"

namespace lmoe {

namespace {

constexpr int kMaxT = kMultiMaxT;
constexpr int kMaxR = kMultiMaxRoutes;
constexpr int kMaxK = kTopkMaxK;
constexpr int kKeysPerLane = kTopkKeysPerLane;
constexpr int kMaxShared = 8;
constexpr int kMaxE = 1024;
constexpr int kDepth = 1;  // bursts of weights in flight ahead of the MFMAs
constexpr int kWgPerCu = 1;
constexpr int kWavesPerWg = 4;

// The expert grouping of all T * k routes, built once per workgroup.
struct GroupLds {
  int state;          // 0 not started, 1 being built, 2 ready
  int D;              // groups (distinct experts)
  int cnt[kMaxE];     // routes of expert e
  int base[kMaxE];    // first sorted position of expert e's routes
  int gexp[kMaxR];    // expert of group g
  int gstart[kMaxR];  // first sorted position of group g
  int gcnt[kMaxR];    // routes (one per token) of group g
  int rs[kMaxR];      // route t * k + j at sorted position p
  float w[kMaxR];     // weight of route t * k + j
};

__device__ __forceinline__ uint64_t* logit_word(const DecodeArgs& a, int t, int e) {
  return reinterpret_cast<uint64_t*>(a.ctr + kMcLogit) + (size_t)t * a.E + e;
}
__device__ __forceinline__ int* part_ctr(const DecodeArgs& a, int t, int b) {
  return a.ctr + kMcPart + 16 * (64 * t + b);
}

}  // namespace

// ---------------------------------------------------------------------------
// Router: expert e's logit for every token, fp32 dot products of bf16 pairs.
// With given logits, item e publishes entries 64 e .. 64 e + 63 of the
// [T][E] logits instead.
// ---------------------------------------------------------------------------
__device__ void router_m(const DecodeArgs& a, int e, const uint16_t* xs) {
  const int lane = lane_id();
  if (a.logits_in) {
    const int g = e * kWave + lane;
    if (g < a.T * a.E)
      __hip_atomic_store(logit_word(a, g / a.E, g % a.E),
                         (1ull << 32) | __float_as_uint(a.logits_in[g]), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const rsrc_t r = make_rsrc(a.wr, (uint32_t)a.E * a.L * 2);
  const int row = e * a.L * 2;
  constexpr int kMaxChunks = kDecodeMaxWidth * 2 / 1024;
  u32x4_t v[kMaxChunks];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int off = c * 1024 + lane * 16;
    v[c] = bload16(r, off < a.L * 2 ? row + off : kOob);
  }
  float acc[kMaxT];
#pragma unroll
  for (int t = 0; t < kMaxT; ++t) acc[t] = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int l0 = c * 512 + lane * 8;
    if (l0 < a.L) {
#pragma unroll
      for (int t = 0; t < kMaxT; ++t) {
        if (t < a.T) {
          const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xs + t * a.xstride + l0);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            // the words are copied out first: a bit cast of a vector element
            // in place reads element 0 whatever the index (hipcc 7.2)
            const uint32_t xw = xv[q], ww = v[c][q];
            acc[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xw),
                                                     __builtin_bit_cast(bf16x2_t, ww), acc[t],
                                                     false);
          }
        }
      }
    }
  }
  // Reduce-scatter over the lanes: each exchange halves the tokens a lane
  // carries, until lane l holds the whole sum of token (l >> 2) & 15.
  float v8[8], v4[4], v2[2];
  {
    const bool hi = lane & 32;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float send = hi ? acc[i] : acc[8 + i], keep = hi ? acc[8 + i] : acc[i];
      v8[i] = keep + __shfl_xor(send, 32, kWave);
    }
  }
  {
    const bool hi = lane & 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float send = hi ? v8[i] : v8[4 + i], keep = hi ? v8[4 + i] : v8[i];
      v4[i] = keep + __shfl_xor(send, 16, kWave);
    }
  }
  {
    const bool hi = lane & 8;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float send = hi ? v4[i] : v4[2 + i], keep = hi ? v4[2 + i] : v4[i];
      v2[i] = keep + __shfl_xor(send, 8, kWave);
    }
  }
  float s;
  {
    const bool hi = lane & 4;
    const float send = hi ? v2[0] : v2[1], keep = hi ? v2[1] : v2[0];
    s = keep + __shfl_xor(send, 4, kWave);
  }
  s += __shfl_xor(s, 2, kWave);
  s += __shfl_xor(s, 1, kWave);
  const int t = (lane >> 2) & 15;
  if ((lane & 3) == 0 && t < a.T) {
    if (a.logits_out) a.logits_out[(size_t)t * a.E + e] = s;
    __hip_atomic_store(logit_word(a, t, e), (1ull << 32) | __float_as_uint(s), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------
// Top-k of token t once its E logits are published: selection (ties to the
// lower expert index), softmax over the selected logits, routes out.
// ---------------------------------------------------------------------------
__device__ void topk_m(const DecodeArgs& a, int t, TopkScratch& scr) {
  const int lane = lane_id();
  float lv[kKeysPerLane];
  for (long it = 0;; ++it) {
    uint64_t w[kKeysPerLane];
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i)
      w[i] = __hip_atomic_load(logit_word(a, t, min(lane + kWave * i, a.E - 1)),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool in = true;
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i) {
      in = in && (w[i] >> 32) != 0;
      lv[i] = __uint_as_float((uint32_t)w[i]);
    }
    if (__builtin_amdgcn_ballot_w64(!in) == 0) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      break;
    }
    if (it > kSpinLimit) {  // a broken producer: counted, and the wait abandoned
      if (lane == 0) add_dev(a.ctr + kCtrError, 1);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  uint64_t key[kKeysPerLane];
#pragma unroll
  for (int i = 0; i < kKeysPerLane; ++i) {
    const int e = lane + kWave * i;
    key[i] = (e < a.E) ? order_key(lv[i], e) : 0ull;
  }
  uint64_t mine = 0ull;  // lane j: the j-th largest key
  if (!select_by_threshold(a.k, key, scr, mine)) select_by_rounds(a.k, key, mine);
  const int my_e = (int)(~(uint32_t)mine);
  const float my_l = lane < a.k ? key_value(mine) : 0.f;
  // softmax over the selected logits, relative to the largest
  const float l0 = __shfl(my_l, 0, kWave);
  const float z = (lane < a.k) ? expf(my_l - l0) : 0.f;
  float sum = z;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_down(sum, off, kWave);
  sum = __shfl(sum, 0, kWave);
  if (lane < a.k) {
    st_dev(a.idx + t * a.k + lane, my_e);
    st_dev_f32(a.w + t * a.k + lane, z / sum);
  }
  // this token's logits have no other reader: back to zero
  for (int e = lane; e < a.E; e += kWave)
    __hip_atomic_store(logit_word(a, t, e), 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  publish(a.ctr + kMcTopk, false);
}

// ---------------------------------------------------------------------------
// The grouping, once every token's routes are published: routes counted per
// expert in token order (so a group lists its tokens in ascending order),
// experts scanned in index order. Out-of-range values (possible only after
// an abandoned wait) are clamped so no index leaves its array.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void build_groups(const DecodeArgs& a, GroupLds& gl) {
  const int lane = lane_id();
  const int R = a.T * a.k;
  wait_geq(a.ctr + kMcTopk, a.T, a.ctr + kCtrError);
  int ev[kMaxT];  // lane j < k: expert of route (t, j)
#pragma unroll
  for (int t = 0; t < kMaxT; ++t)
    ev[t] = (t < a.T && lane < a.k) ? min(max(ld_dev(a.idx + t * a.k + lane), 0), a.E - 1) : 0;
#pragma unroll
  for (int i = 0; i < kMaxR / kWave; ++i) {
    const int r = lane + kWave * i;
    if (r < R) {
      gl.w[r] = ld_dev_f32(a.w + r);
      gl.rs[r] = 0;
    }
  }
  for (int e = lane; e < a.E; e += kWave) gl.cnt[e] = 0;
  wave_lds_sync();
  // a token's experts are distinct, so the lanes of one step update
  // different counts
  int slot[kMaxT];
#pragma unroll
  for (int t = 0; t < kMaxT; ++t) {
    slot[t] = 0;
    if (t < a.T) {
      if (lane < a.k) {
        const int c = gl.cnt[ev[t]];
        gl.cnt[ev[t]] = c + 1;
        slot[t] = c;
      }
      wave_lds_sync();
    }
  }
  // lane l scans experts span * l .. span * (l + 1) - 1
  const int span = (a.E + kWave - 1) / kWave;
  const int e0 = lane * span;
  int nd = 0, nr = 0;
  for (int i = 0; i < span; ++i) {
    const int e = e0 + i;
    if (e < a.E) {
      const int c = gl.cnt[e];
      nd += c > 0 ? 1 : 0;
      nr += c;
    }
  }
  int sd = nd, sr = nr;  // inclusive prefix over lanes
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int td = __shfl_up(sd, off, kWave), tr = __shfl_up(sr, off, kWave);
    if (lane >= off) {
      sd += td;
      sr += tr;
    }
  }
  int gd = sd - nd, gr = sr - nr;
  for (int i = 0; i < span; ++i) {
    const int e = e0 + i;
    if (e < a.E) {
      const int c = gl.cnt[e];
      gl.base[e] = gr;
      if (c > 0 && gd < kMaxR) {
        gl.gexp[gd] = e;
        gl.gstart[gd] = min(gr, R - 1);
        gl.gcnt[gd] = c;
        ++gd;
      }
      gr += c;
    }
  }
  if (lane == kWave - 1) gl.D = min(sd, kMaxR);
  wave_lds_sync();
#pragma unroll
  for (int t = 0; t < kMaxT; ++t)
    if (t < a.T && lane < a.k) gl.rs[min(gl.base[ev[t]] + slot[t], R - 1)] = t * a.k + lane;
  wave_lds_sync();
  __hip_atomic_store(&gl.state, 2, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// The grouping of this workgroup: built by the first wave that needs it;
// other waves wait for it in LDS. (Called from the kernel body only, so that
// it inlines and the arguments stay in registers.)
__device__ __forceinline__ void ensure_groups(const DecodeArgs& a, GroupLds& gl) {
  if (__hip_atomic_load(&gl.state, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 2) return;
  int claim = 0;
  if (lane_id() == 0) {
    int expected = 0;
    claim = __hip_atomic_compare_exchange_strong(&gl.state, &expected, 1, __ATOMIC_ACQ_REL,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  if (__builtin_amdgcn_readfirstlane(claim)) {
    build_groups(a, gl);
    return;
  }
  while (__hip_atomic_load(&gl.state, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != 2)
    __builtin_amdgcn_s_sleep(1);
}

// Routing outputs: counts, offsets and the permutation (the top-k items
// wrote the routes and weights).
__device__ void write_routing_m(const DecodeArgs& a, const GroupLds& gl) {
  const int lane = lane_id();
  const int R = a.T * a.k;
  for (int e = lane; e < a.E; e += kWave) {
    a.counts[e] = gl.cnt[e];
    a.offsets[e] = gl.base[e];
  }
  if (lane == 0) a.offsets[a.E] = R;
  for (int p = lane; p < R; p += kWave) {
    const int rt = gl.rs[p];
    a.perm[p] = rt;
    a.inv[rt] = p;
  }
}

// ---------------------------------------------------------------------------
// Combine of token t's 64-row block b, and the count of its inputs.
// ---------------------------------------------------------------------------
__device__ void combine_m(const DecodeArgs& a, const GroupLds& gl, int t, int b) {
  // every load is issued before the first is used (indices clamped in range)
  const int l = min(b * 64 + lane_id(), a.L - 1);
  float yv[kMaxK], sv[kMaxShared];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    yv[j] = ld_dev_f32(a.y + (size_t)(t * a.k + min(j, a.k - 1)) * a.L + l);
#pragma unroll
  for (int s = 0; s < kMaxShared; ++s)
    sv[s] = a.S > 0 ? ld_dev_f32(a.ysh + ((size_t)min(s, a.S - 1) * a.T + t) * a.L + l) : 0.f;
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < a.k) acc = fmaf(gl.w[t * a.k + j], yv[j], acc);
#pragma unroll
  for (int s = 0; s < kMaxShared; ++s)
    if (s < a.S) acc += sv[s];
  if (b * 64 + lane_id() < a.L) a.out[(size_t)t * a.L + l] = f32_to_bf16_bits(acc);
  // every input of the block is in: the count goes back to zero
  if (lane_id() == 0) st_dev(part_ctr(a, t, b), 0);
}

// This wave's outputs for block b are stored; lanes holding a token (tok >= 0,
// distinct) count one more input of that token's block, and the wave combines
// every block it completed (the grouping, which holds the weights, is ready).
__device__ void parts_done(const DecodeArgs& a, const GroupLds& gl, int b, int tok) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  const int nparts = min(2, a.dn_per_route - 2 * b);    // 32-row routed items in the block
  const int ntiles = min(4, a.shd_per_expert - 4 * b);  // 16-row shared items in the block
  const int target = a.k * nparts + a.S * ntiles;
  int old = -1;
  if (tok >= 0) old = add_dev(part_ctr(a, tok, b), 1);
  uint64_t done = __builtin_amdgcn_ballot_w64(tok >= 0 && old == target - 1);
  if (done == 0) return;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  while (done) {
    const int ln = __builtin_ctzll(done);
    done &= done - 1;
    combine_m(a, gl, __builtin_amdgcn_readlane(tok, ln), b);
  }
}

// ---------------------------------------------------------------------------
// Expert items
// ---------------------------------------------------------------------------
__device__ void shared_gu_m(const DecodeArgs& a, int item, const uint16_t* xs) {
  const int s = item / a.shgu_per_expert;
  const int i0 = (item % a.shgu_per_expert) * 8;
  const int lane = lane_id();
  const int c = lane & 15, q = lane >> 4;
  const int i = i0 + (c & 7);
  Tile16 tl[1];
  tl[0].w = make_rsrc((c < 8 ? a.shg : a.shu) + (size_t)s * a.Is * a.L, (uint32_t)a.Is * a.L * 2);
  tl[0].row = i < a.Is ? i * a.L * 2 : kOob;
  f32x4_t acc[1];
  gemv_bf16<1, 2, kDepth>(ALds{xs + min(c, a.T - 1) * a.xstride}, a.L / 32, tl, acc, [] {});
  // row 4 q + ii of the tile is token 4 q + ii: g in columns 0..7, u in 8..15
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int row = 4 * q + ii;
    const float u = __shfl(acc[0][ii], (lane + 8) & 63, kWave);
    const uint32_t h = f32_to_bf16_bits(silu(acc[0][ii]) * u);
    const uint32_t h_next = __shfl_down(h, 1, kWave);
    if (c < 8 && (c & 1) == 0 && row < a.T && i0 + c < a.Is)
      st_dev(reinterpret_cast<uint32_t*>(a.hsh + ((size_t)s * a.T + row) * a.Is + i0 + c),
             h | (h_next << 16));
  }
  publish(a.ctr + kMcShared + 16 * s, false);
}

__device__ void routed_gu_m(const DecodeArgs& a, int item, const uint16_t* xs,
                            const GroupLds& gl) {
  const int g = item / a.gu_per_route;
  const int i0 = (item % a.gu_per_route) * 16;
  if (g >= __builtin_amdgcn_readfirstlane(gl.D)) return;
  const int R = a.T * a.k;
  const int e = min(max(__builtin_amdgcn_readfirstlane(gl.gexp[g]), 0), a.E - 1);
  const int m = __builtin_amdgcn_readfirstlane(gl.gcnt[g]);
  const int p0 = __builtin_amdgcn_readfirstlane(gl.gstart[g]);
  const int lane = lane_id();
  const int c = lane & 15, q = lane >> 4;
  // A row c: the token of the group's route c (rows past the group repeat its
  // first token; their results are not stored)
  const int tok = gl.rs[min(p0 + (c < m ? c : 0), R - 1)] / a.k;
  const int i = i0 + c;
  const size_t qoff = (size_t)e * a.I * (a.L / 2);
  const size_t soff = (size_t)e * a.I * (a.L / 32);
  const uint32_t qbytes = (uint32_t)a.I * (a.L / 2), sbytes = (uint32_t)a.I * (a.L / 32);
  Tile4 tl[2];
  tl[0].codes = make_rsrc(a.gq + qoff, qbytes);
  tl[0].scales = make_rsrc(a.gs + soff, sbytes);
  tl[1].codes = make_rsrc(a.uq + qoff, qbytes);
  tl[1].scales = make_rsrc(a.us + soff, sbytes);
  tl[0].code_row = tl[1].code_row = i < a.I ? i * (a.L / 2) : kOob;
  tl[0].scale_row = tl[1].scale_row = i < a.I ? i * (a.L / 32) : kOob;
  f32x4_t acc[2];
  gemv_fp4<2, 2, kDepth>(ALds{xs + tok * a.xstride}, a.L / 32, tl, acc, [] {});
  // element ii of lane (c, q): route 4 q + ii of the group, column i0 + c
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int row = 4 * q + ii;
    const uint32_t h = f32_to_bf16_bits(silu(acc[0][ii]) * acc[1][ii]);
    const uint32_t h_next = __shfl_down(h, 1, kWave);
    if ((c & 1) == 0 && row < m && i < a.I) {
      const int rt = gl.rs[min(p0 + row, R - 1)];
      st_dev(reinterpret_cast<uint32_t*>(a.h + (size_t)rt * a.I + i), h | (h_next << 16));
    }
  }
  publish(a.ctr + kMcGroup + 16 * g, false);
}

__device__ void shared_dn_m(const DecodeArgs& a, int item, const GroupLds& gl) {
  // item = (expert, tile): 16 output rows of shared expert s over its whole K
  const int s = item / a.shd_per_expert;
  const int tile = item % a.shd_per_expert;
  const int l0 = tile * 16;
  const int lane = lane_id();
  const int c = lane & 15, q = lane >> 4;
  Tile16 tl[1];
  tl[0].w = make_rsrc(a.shd + (size_t)s * a.L * a.Is, (uint32_t)a.L * a.Is * 2);
  tl[0].row = l0 + c < a.L ? (l0 + c) * a.Is * 2 : kOob;
  const ADev src{make_rsrc(a.hsh + (size_t)s * a.T * a.Is, (uint32_t)a.T * a.Is * 2),
                 c < a.T ? c * a.Is * 2 : kOob};
  f32x4_t acc[1];
  gemv_bf16<1, 2, kDepth>(src, a.Is / 32, tl, acc, [&] {
    wait_geq(a.ctr + kMcShared + 16 * s, a.shgu_per_expert, a.ctr + kCtrError);
  });
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int t = 4 * q + ii;
    if (t < a.T && l0 + c < a.L)
      st_dev_f32(a.ysh + ((size_t)s * a.T + t) * a.L + l0 + c, acc[0][ii]);
  }
  parts_done(a, gl, tile / 4, lane < a.T ? lane : -1);
}

__device__ void routed_dn_m(const DecodeArgs& a, int item, const GroupLds& gl) {
  const int g = item / a.dn_per_route;
  const int p = item % a.dn_per_route;  // 32-row part of the output
  if (g >= __builtin_amdgcn_readfirstlane(gl.D)) return;
  const int R = a.T * a.k;
  const int e = min(max(__builtin_amdgcn_readfirstlane(gl.gexp[g]), 0), a.E - 1);
  const int m = __builtin_amdgcn_readfirstlane(gl.gcnt[g]);
  const int p0 = __builtin_amdgcn_readfirstlane(gl.gstart[g]);
  const int lane = lane_id();
  const int c = lane & 15, q = lane >> 4;
  // A row c: h of the group's route c
  const int rt_c = gl.rs[min(p0 + (c < m ? c : 0), R - 1)];
  const ADev src{make_rsrc(a.h, (uint32_t)R * a.I * 2), c < m ? rt_c * a.I * 2 : kOob};
  const size_t qoff = (size_t)e * a.L * (a.I / 2);
  const size_t soff = (size_t)e * a.L * (a.I / 32);
  const uint32_t qbytes = (uint32_t)a.L * (a.I / 2), sbytes = (uint32_t)a.L * (a.I / 32);
  Tile4 tl[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int l = p * 32 + t * 16 + c;
    tl[t].codes = make_rsrc(a.dq + qoff, qbytes);
    tl[t].scales = make_rsrc(a.ds + soff, sbytes);
    tl[t].code_row = l < a.L ? l * (a.I / 2) : kOob;
    tl[t].scale_row = l < a.L ? l * (a.I / 32) : kOob;
  }
  f32x4_t acc[2];
  gemv_fp4<2, 2, kDepth>(src, a.I / 32, tl, acc, [&] {
    wait_geq(a.ctr + kMcGroup + 16 * g, a.gu_per_route, a.ctr + kCtrError);
  });
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int row = 4 * q + ii;
    if (row < m) {
      const int rt = gl.rs[min(p0 + row, R - 1)];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int l = p * 32 + t * 16 + c;
        if (l < a.L) st_dev_f32(a.y + (size_t)rt * a.L + l, acc[t][ii]);
      }
    }
  }
  parts_done(a, gl, p / 2, (lane < 16 && lane < m) ? rt_c / a.k : -1);
}

// ---------------------------------------------------------------------------
// The kernel: four independent waves per workgroup sharing the tokens and the
// grouping in LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 1) void decode_multi_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];  // [T][xstride]
  __shared__ GroupLds gl;
  __shared__ TopkScratch scr[kWavesPerWg];
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x * 8; i < a.T * a.L; i += 256 * 8) {
    const int t = i / a.L, l = i - t * a.L;
    *reinterpret_cast<u32x4_t*>(xs + t * a.xstride + l) = load16(a.x + i);
  }
  if (threadIdx.x == 0) gl.state = 0;
  __syncthreads();

  const int gw = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerWg + wave);
  const int q = gw % kQueues;
  int* ticket = a.ctr + kCtrTicket + 16 * q;
  // the drawn ticket stays in lane 0's register until the next item starts
  auto draw = [&]() {
    int v = 0;
    if (lane_id() == 0) v = add_dev(ticket, 1);
    return v;
  };
  auto ticket_of = [&](int v) { return q + kQueues * __builtin_amdgcn_readfirstlane(v); };
  int t = ticket_of(draw());
  while (t < a.t_total) {
    const int next = draw();  // in flight while this item runs
    // the routed items and every item that may complete a token's block
    // need the grouping
    if (t >= a.t_gu) ensure_groups(a, gl);
    if (t < a.t_topk)
      router_m(a, t, xs);
    else if (t < a.t_shgu)
      topk_m(a, t - a.t_topk, scr[wave]);
    else if (t < a.t_gu)
      shared_gu_m(a, t - a.t_shgu, xs);
    else if (t < a.t_shd)
      routed_gu_m(a, t - a.t_gu, xs, gl);
    else if (t < a.t_dn)
      shared_dn_m(a, t - a.t_shd, gl);
    else
      routed_dn_m(a, t - a.t_dn, gl);
    t = ticket_of(next);
  }
  if (blockIdx.x == 0 && wave == 0) {
    ensure_groups(a, gl);
    write_routing_m(a, gl);
  }
  // the last wave out zeroes the counters for the next launch
  int last = 0;
  if (lane_id() == 0) {
    __builtin_amdgcn_s_waitcnt(0);
    last = add_dev(a.ctr + kCtrExit, 1) == (int)gridDim.x * kWavesPerWg - 1;
  }
  if (__builtin_amdgcn_readfirstlane(last)) {
    const int lane = lane_id();
    if (lane < kQueues) st_dev(a.ctr + kCtrTicket + 16 * lane, 0);
    if (lane == 0) st_dev(a.ctr + kMcTopk, 0);
    if (lane < a.S) st_dev(a.ctr + kMcShared + 16 * lane, 0);
    for (int g = lane; g < a.n_groups; g += kWave) st_dev(a.ctr + kMcGroup + 16 * g, 0);
    // after an abandoned wait the per-token counts and logits may be left set
    if (__builtin_amdgcn_readfirstlane(ld_dev(a.ctr + kCtrError)) != 0) {
      const int nb = (a.L + 63) / 64;
      for (int i = lane; i < a.T * nb; i += kWave) st_dev(part_ctr(a, i / nb, i % nb), 0);
      for (int i = lane; i < a.T * a.E; i += kWave)
        __hip_atomic_store(logit_word(a, i / a.E, i % a.E), 0ull, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    if (lane == 0) st_dev(a.ctr + kCtrExit, 0);
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
size_t decode_multi_lds_bytes(const lmoe_dims& d) {
  return (size_t)d.T * (d.L + 8) * 2 + sizeof(GroupLds) + kWavesPerWg * sizeof(TopkScratch);
}

void make_decode_multi_args(const Plan& p, DecodeArgs& a, bool logits_given) {
  const lmoe_dims& d = p.d;
  a.T = d.T;
  a.L = d.L;
  a.E = d.E;
  a.k = d.k;
  a.I = d.I;
  a.S = d.S;
  a.Is = d.Is;
  const int R = d.T * d.k;
  a.n_groups = std::min(d.E, R);
  a.n_router = logits_given ? (d.T * d.E + kWave - 1) / kWave : d.E;
  a.shgu_per_expert = d.S > 0 ? (d.Is + 7) / 8 : 0;
  a.n_shgu = d.S * a.shgu_per_expert;
  a.gu_per_route = (d.I + 15) / 16;
  a.n_gu = a.n_groups * a.gu_per_route;
  a.shd_per_expert = d.L / 16;
  a.n_shd = d.S * a.shd_per_expert;
  a.dn_per_route = (d.L + 31) / 32;
  a.n_dn = a.n_groups * a.dn_per_route;
  a.t_topk = a.n_router;
  a.t_shgu = a.t_topk + d.T;
  a.t_gu = a.t_shgu + a.n_shgu;
  a.t_shd = a.t_gu + a.n_gu;
  a.t_dn = a.t_shd + a.n_shd;
  a.t_total = a.t_dn + a.n_dn;
  a.xstride = d.L + 8;  // rows 16 bytes apart in the banks: no conflicts
  a.a_region = 0;
  a.lds_bytes = (size_t)d.T * a.xstride * 2;
}

static int decode_multi_grid(size_t lds_bytes) {
  static std::atomic<uint64_t> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  const uint64_t c = cached[dev].load(std::memory_order_relaxed);
  if ((uint32_t)c > 0 && (c >> 32) == lds_bytes) return (int)(uint32_t)c;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_multi_kernel, 256,
                                                   lds_bytes) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  const int grid = cus * std::min(per_cu, kWgPerCu);
  cached[dev].store(((uint64_t)lds_bytes << 32) | (uint32_t)grid, std::memory_order_relaxed);
  return grid;
}

hipError_t launch_decode_multi(const DecodeArgs& a, hipStream_t s, const hipEvent_t* ev) {
  hipError_t e = record_stage(ev, LMOE_STAGE_BEGIN, s);
  if (e != hipSuccess) return e;
  // dynamic LDS beyond 64 KiB must be allowed for the kernel first
  static std::once_flag once;
  static hipError_t attr = hipSuccess;
  std::call_once(once, [] {
    attr = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_multi_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)((size_t)kMultiMaxT * (kDecodeMaxWidth + 8) * 2));
  });
  if (attr != hipSuccess) return attr;
  // at least one wave per ticket queue
  const int grid =
      std::max((kQueues + kWavesPerWg - 1) / kWavesPerWg, decode_multi_grid(a.lds_bytes));
  hipLaunchKernelGGL(decode_multi_kernel, dim3(grid), dim3(256), a.lds_bytes, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // one kernel holds every stage
  for (int i = LMOE_STAGE_ROUTER; i < LMOE_NUM_STAGE_EVENTS; ++i)
    if ((e = record_stage(ev, i, s)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace lmoe
