// Single-token decode of the LatentMoE layer as one persistent kernel.
//
// Batch-1 decode streams the active weights once per token and is bound by
// HBM bandwidth (infervisor.ai "Bringing up Kimi-K3 on day zero", "The
// roofline"): the router, the two bf16 shared experts and the 16 selected
// MXFP4 experts. Launch boundaries between dependent steps leave the memory
// system idle, so the whole layer is one launch in which every wave draws work
// items from ticket queues in dependency order and resolves dependencies with
// on-device counters (the pages' decode runtime likewise orders work with
// device counters rather than host launches: "One kernel, no host in the
// loop").
//
// Waves work independently: an item covers the whole K range of its rows, so
// no item needs a workgroup barrier or a cross-wave reduction, and a wave keeps
// its next burst of weights in flight while it computes the current one.
//
// Work items, in ticket order (sizes for the Kimi-K3 layer):
//   router      the logit of one expert: its 7 KB router row against the
//               token; published as one 64-bit word that carries a flag
//   shared g/u  one shared expert, 8 intermediate columns, gate and up in one
//               16-column MFMA tile: h = bf16(silu(g) * u)          (115 KB)
//   routed g/u  one selected expert, 16 intermediate columns         (61 KB)
//   shared dn   16 output rows of one shared expert                  (64 KB)
//   routed dn   one selected expert, 32 output rows                  (35 KB)
//   combine     done by whichever item completes a 64-row block last:
//               out = bf16(sum_j w_j y_j + sum_s ysh_s), in that order
// The routing decision is not broadcast: every workgroup that needs it waits
// for all logits to be published and selects the top-k itself into LDS (a
// deterministic function of the published logits, so all copies agree), which
// saves the round trips of a single selecting wave writing and every consumer
// reading back the choice. Workgroup 0 writes the routing outputs.
//
// Tickets: items are dealt round-robin into 32 queues (device-scope atomics
// on one address serialise, about 12 ns each on MI355X). A wave only
// ever waits for smaller items. The smallest unfinished item is either being
// processed (its inputs are all done) or heads its queue, and a resident wave
// of that queue will draw it: waves are dispatched in index order and a wave
// leaves only when its queue is empty. So the kernel cannot deadlock.
//
// Memory ordering: data passed between waves (logits, h, y) is written with
// device-scope stores and read with device-scope loads, which stay coherent
// across the eight L2 partitions; a producer waits for its stores to complete
// before it bumps a counter. A logit needs no counter: its flag and value are
// one aligned 64-bit word, so a reader that sees the flag sees the value,
// which saves the selecting wave one round trip. No L2 writeback or
// invalidate is issued. Counters and flagged logits sit in the workspace's
// counter block, are zero when a launch starts and are zeroed again by its
// last wave to leave.
#include <atomic>

#include "lmoe_internal.h"
#include "lmoe_stream.h"
#include "lmoe_topk.h"

namespace lmoe {

namespace {

constexpr int kMaxK = kTopkMaxK;  // routes per token on this path
constexpr int kKeysPerLane = kTopkKeysPerLane;
constexpr int kMaxShared = 8;     // shared experts
constexpr int kDepth = 1;         // bursts of weights in flight ahead of the MFMAs
// Workgroups per compute unit. Four streaming waves per CU keep enough bytes
// in flight; more concurrent items only lengthen each item and the tail.
constexpr int kWgPerCu = 1;

// Per-wave state kept across items.
struct WaveState {
  int staged;  // what the wave's LDS A row holds: -1 none, route j, or 1000 + shared expert
};

// Per-workgroup routing decision in LDS.
struct TopkLds {
  int state;  // 0 not started, 1 being computed, 2 ready
  int sel[kMaxK];
  float w[kMaxK];
  TopkScratch scr;  // the selecting wave's working space
};

}  // namespace

// Copy n (<= kDecodeMaxWidth, a multiple of 8) bf16 values written by other
// waves of this launch into the wave's LDS row. Every load is issued before
// the first store (indices clamped in range).
__device__ __forceinline__ void stage_row(uint16_t* dst, const uint16_t* src, int n) {
  constexpr int kChunks = kDecodeMaxWidth / (kWave * 8);
  u32x4_t v[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) v[c] = ld16_dev(src + min(c * kWave * 8 + lane_id() * 8, n - 8));
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int i = c * kWave * 8 + lane_id() * 8;
    if (i < n) *reinterpret_cast<u32x4_t*>(dst + i) = v[c];
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
}

// h = bf16(silu(g) * u) for n consecutive intermediate columns held as g in
// lanes 0..n-1 and u in lanes un..un+n-1 of `u_src`; stored in pairs with
// device-scope stores (columns below `limit` only).
__device__ __forceinline__ void store_glu(uint16_t* dst, float g, float u_src, int n, int un,
                                          int limit) {
  const int lane = lane_id();
  const float u = __shfl(u_src, (lane + un) & 63, kWave);
  const uint32_t h = f32_to_bf16_bits(silu(g) * u);
  const uint32_t h_next = __shfl_down(h, 1, kWave);
  if (lane < n && (lane & 1) == 0 && lane < limit)
    st_dev(reinterpret_cast<uint32_t*>(dst + lane), h | (h_next << 16));
}

// ---------------------------------------------------------------------------
// Router: the logit of expert e, fp32 sum of x[l] W[e][l] over the row. With
// given logits, item e publishes logits 64 e .. 64 e + 63 instead.
// ---------------------------------------------------------------------------
__device__ void router_item(const DecodeArgs& a, int e, const uint16_t* xs) {
  const int lane = lane_id();
  if (a.logits_in) {
    const int g = e * kWave + lane;
    if (g < a.E)
      __hip_atomic_store(reinterpret_cast<uint64_t*>(a.ctr + kCtrLogit) + g,
                         (1ull << 32) | __float_as_uint(a.logits_in[g]), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const uint32_t bytes = (uint32_t)a.E * a.L * 2;
  const rsrc_t r = make_rsrc(a.wr, bytes);
  const int row = e * a.L * 2;
  // the row in 1 KB chunks, 16 bytes (8 values) per lane and chunk
  constexpr int kMaxChunks = kDecodeMaxWidth * 2 / 1024;
  u32x4_t v[kMaxChunks];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int off = c * 1024 + lane * 16;
    v[c] = bload16(r, off < a.L * 2 ? row + off : kOob);
  }
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int l0 = c * 512 + lane * 8;
    if (l0 < a.L) {
      const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xs + l0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc = fmaf(__uint_as_float(xv[q] << 16), __uint_as_float(v[c][q] << 16), acc);
        acc = fmaf(__uint_as_float(xv[q] & 0xFFFF0000u), __uint_as_float(v[c][q] & 0xFFFF0000u),
                   acc);
      }
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) acc += __shfl_xor(acc, off, kWave);
  if (lane == 0) {
    if (a.logits_out) a.logits_out[e] = acc;
    __hip_atomic_store(reinterpret_cast<uint64_t*>(a.ctr + kCtrLogit) + e,
                       (1ull << 32) | __float_as_uint(acc), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ void compute_topk(const DecodeArgs& a, TopkLds& tk);
__device__ void finish_topk(const DecodeArgs& a, TopkLds& tk, uint64_t mine);

// The routing decision of this workgroup: computed by the first wave that
// needs it once every logit is published; other waves wait for it in LDS.
__device__ void ensure_topk(const DecodeArgs& a, TopkLds& tk) {
  if (__hip_atomic_load(&tk.state, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 2) return;
  int claim = 0;
  if (lane_id() == 0) {
    int expected = 0;
    claim = __hip_atomic_compare_exchange_strong(&tk.state, &expected, 1, __ATOMIC_ACQ_REL,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  if (__builtin_amdgcn_readfirstlane(claim)) {
    compute_topk(a, tk);
    return;
  }
  while (__hip_atomic_load(&tk.state, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != 2)
    __builtin_amdgcn_s_sleep(1);
}

// Computed once every logit is published: selection, then softmax weights.
__device__ void compute_topk(const DecodeArgs& a, TopkLds& tk) {
  const int lane = lane_id();
  // every logit with its flag, all loads issued before the first is used
  // (indices clamped in range), until every flag is set
  const uint64_t* pub = reinterpret_cast<const uint64_t*>(a.ctr + kCtrLogit);
  float lv[kKeysPerLane];
  for (long it = 0;; ++it) {
    uint64_t w[kKeysPerLane];
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i)
      w[i] = __hip_atomic_load(pub + min(lane + kWave * i, a.E - 1), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
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
  if (!select_by_threshold(a.k, key, tk.scr, mine)) select_by_rounds(a.k, key, mine);
  finish_topk(a, tk, mine);
}

// Softmax weights of the selected keys (lane j holds the j-th largest) and
// the release of the decision to the workgroup.
__device__ void finish_topk(const DecodeArgs& a, TopkLds& tk, uint64_t mine) {
  const int lane = lane_id();
  const int my_e = (int)(~(uint32_t)mine);
  const float my_l = lane < a.k ? key_value(mine) : 0.f;
  // softmax over the selected logits, relative to the largest
  const float l0 = __shfl(my_l, 0, kWave);
  const float z = (lane < a.k) ? expf(my_l - l0) : 0.f;
  float s = z;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_down(s, off, kWave);
  s = __shfl(s, 0, kWave);
  if (lane < a.k) {
    tk.sel[lane] = my_e;
    tk.w[lane] = z / s;
  }
  __hip_atomic_store(&tk.state, 2, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Routing outputs for one token: the selection, its weights, and the grouping
// (each route is its own group, in expert order).
__device__ void write_routing(const DecodeArgs& a, const TopkLds& tk) {
  const int lane = lane_id();
  const int my_e = lane < a.k ? tk.sel[lane] : 0x7fffffff;
  if (lane < a.k) {
    a.idx[lane] = my_e;
    a.w[lane] = tk.w[lane];
  }
  for (int e = lane; e < a.E; e += kWave) {
    int below = 0, hit = 0;
    for (int j = 0; j < a.k; ++j) {
      const int sj = tk.sel[j];
      below += sj < e;
      hit += sj == e;
    }
    a.counts[e] = hit;
    a.offsets[e] = below;
  }
  if (lane == 0) a.offsets[a.E] = a.k;
  if (lane < a.k) {
    int pos = 0;
    for (int j = 0; j < a.k; ++j) pos += tk.sel[j] < my_e;
    a.perm[pos] = lane;
    a.inv[lane] = pos;
  }
}

// ---------------------------------------------------------------------------
// Expert items
// ---------------------------------------------------------------------------
__device__ void shared_gu_item(const DecodeArgs& a, int item, const uint16_t* xs) {
  const int s = item / a.shgu_per_expert;
  const int i0 = (item % a.shgu_per_expert) * 8;
  const int col = lane_id() & 15;
  const int i = i0 + (col & 7);
  const uint32_t mbytes = (uint32_t)a.Is * a.L * 2;
  Tile16 tl[1];
  tl[0].w = make_rsrc((col < 8 ? a.shg : a.shu) + (size_t)s * a.Is * a.L, mbytes);
  tl[0].row = i < a.Is ? i * a.L * 2 : kOob;
  f32x4_t acc[1];
  gemv_bf16<1, 2, kDepth>(ALds{xs}, a.L / 32, tl, acc, [] {});
  // g in lanes 0..7, u in lanes 8..15
  store_glu(a.hsh + (size_t)s * a.Is + i0, acc[0][0], acc[0][0], 8, 8, a.Is - i0);
  publish(a.ctr + kCtrShared + 16 * s, false);
}

__device__ void routed_gu_item(const DecodeArgs& a, int item, const uint16_t* xs,
                               TopkLds& tk) {
  const int j = item / a.gu_per_route;
  const int i0 = (item % a.gu_per_route) * 16;
  ensure_topk(a, tk);
  const int e = min(max(__builtin_amdgcn_readfirstlane(tk.sel[j]), 0), a.E - 1);
  const int i = i0 + (lane_id() & 15);
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
  gemv_fp4<2, 2, kDepth>(ALds{xs}, a.L / 32, tl, acc, [] {});
  // g in lanes 0..15 of tile 0, u in lanes 0..15 of tile 1
  store_glu(a.h + (size_t)j * a.I + i0, acc[0][0], acc[1][0], 16, 0, a.I - i0);
  publish(a.ctr + kCtrRoute + 16 * j, false);
}

__device__ void combine_block(const DecodeArgs& a, int b, const TopkLds& tk) {
  // every load is issued before the first is used (indices clamped in range)
  const int l = min(b * 64 + lane_id(), a.L - 1);
  float yv[kMaxK], sv[kMaxShared];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) yv[j] = ld_dev_f32(a.y + (size_t)min(j, a.k - 1) * a.L + l);
#pragma unroll
  for (int s = 0; s < kMaxShared; ++s)
    sv[s] = a.S > 0 ? ld_dev_f32(a.ysh + (size_t)min(s, a.S - 1) * a.L + l) : 0.f;
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < a.k) acc = fmaf(tk.w[j], yv[j], acc);
#pragma unroll
  for (int s = 0; s < kMaxShared; ++s)
    if (s < a.S) acc += sv[s];
  if (b * 64 + lane_id() < a.L) a.out[l] = f32_to_bf16_bits(acc);
}

// One more input of 64-row block b is ready; the last one combines the block.
__device__ void finish_block_part(const DecodeArgs& a, int b, TopkLds& tk) {
  const int old = publish(a.ctr + kCtrBlock + 16 * b, true);
  const int nparts = min(2, a.dn_per_route - 2 * b);    // 32-row routed items in the block
  const int ntiles = min(4, a.shd_per_expert - 4 * b);  // 16-row shared items in the block
  const int target = a.k * nparts + a.S * ntiles;
  if (old != target - 1) return;
  ensure_topk(a, tk);
  combine_block(a, b, tk);
}

__device__ void shared_dn_item(const DecodeArgs& a, int item, uint16_t* arow, WaveState& st,
                               TopkLds& tk) {
  // item = (expert, tile): 16 output rows of shared expert s over its whole K
  const int s = item / a.shd_per_expert;
  const int tile = item % a.shd_per_expert;
  const int l0 = tile * 16;
  const int l = l0 + (lane_id() & 15);
  Tile16 tl[1];
  tl[0].w = make_rsrc(a.shd + (size_t)s * a.L * a.Is, (uint32_t)a.L * a.Is * 2);
  tl[0].row = l < a.L ? l * a.Is * 2 : kOob;
  f32x4_t acc[1];
  gemv_bf16<1, 2, kDepth>(ALds{arow}, a.Is / 32, tl, acc, [&] {
    if (st.staged != 1000 + s) {
      wait_geq(a.ctr + kCtrShared + 16 * s, a.shgu_per_expert, a.ctr + kCtrError);
      stage_row(arow, a.hsh + (size_t)s * a.Is, a.Is);
      st.staged = 1000 + s;
    }
  });
  const int lane = lane_id();
  if (lane < 16 && l0 + lane < a.L) st_dev_f32(a.ysh + (size_t)s * a.L + l0 + lane, acc[0][0]);
  finish_block_part(a, tile / 4, tk);
}

__device__ void routed_dn_item(const DecodeArgs& a, int item, uint16_t* arow, WaveState& st,
                               TopkLds& tk) {
  const int j = item / a.dn_per_route;
  const int p = item % a.dn_per_route;  // 32-row part of the output
  ensure_topk(a, tk);
  const int e = min(max(__builtin_amdgcn_readfirstlane(tk.sel[j]), 0), a.E - 1);
  const size_t qoff = (size_t)e * a.L * (a.I / 2);
  const size_t soff = (size_t)e * a.L * (a.I / 32);
  const uint32_t qbytes = (uint32_t)a.L * (a.I / 2), sbytes = (uint32_t)a.L * (a.I / 32);
  Tile4 tl[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int l = p * 32 + t * 16 + (lane_id() & 15);
    tl[t].codes = make_rsrc(a.dq + qoff, qbytes);
    tl[t].scales = make_rsrc(a.ds + soff, sbytes);
    tl[t].code_row = l < a.L ? l * (a.I / 2) : kOob;
    tl[t].scale_row = l < a.L ? l * (a.I / 32) : kOob;
  }
  f32x4_t acc[2];
  gemv_fp4<2, 2, kDepth>(ALds{arow}, a.I / 32, tl, acc, [&] {
    if (st.staged != j) {
      wait_geq(a.ctr + kCtrRoute + 16 * j, a.gu_per_route, a.ctr + kCtrError);
      stage_row(arow, a.h + (size_t)j * a.I, a.I);
      st.staged = j;
    }
  });
  const int lane = lane_id();
  if (lane < 16) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int l = p * 32 + t * 16 + lane;
      if (l < a.L) st_dev_f32(a.y + (size_t)j * a.L + l, acc[t][0]);
    }
  }
  finish_block_part(a, p / 2, tk);
}

// ---------------------------------------------------------------------------
// The kernel: four independent waves per workgroup sharing the token and the
// routing decision in LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 1) void decode_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  __shared__ TopkLds tk;
  uint16_t* xs = lds;
  const int wave = threadIdx.x >> 6;
  uint16_t* arow = lds + ((a.L + 7) & ~7) + wave * a.a_region;
  for (int i = threadIdx.x * 8; i < a.L; i += 256 * 8)
    *reinterpret_cast<u32x4_t*>(xs + i) = load16(a.x + i);
  if (threadIdx.x == 0) tk.state = 0;
  __syncthreads();

  const int gw = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + wave);
  const int q = gw % kQueues;
  int* ticket = a.ctr + kCtrTicket + 16 * q;
  WaveState st{-1};
  // The drawn ticket stays in lane 0's register until the next item starts:
  // reading it into a scalar at once would wait out the atomic's round trip
  // before every item.
  auto draw = [&]() {
    int v = 0;
    if (lane_id() == 0) v = add_dev(ticket, 1);
    return v;
  };
  auto ticket_of = [&](int v) { return q + kQueues * __builtin_amdgcn_readfirstlane(v); };
  int t = ticket_of(draw());
  while (t < a.t_total) {
    const int next = draw();  // in flight while this item runs
    if (t < a.t_shgu) {
      router_item(a, t, xs);
    }
    else if (t < a.t_gu)
      shared_gu_item(a, t - a.t_shgu, xs);
    else if (t < a.t_shd)
      routed_gu_item(a, t - a.t_gu, xs, tk);
    else if (t < a.t_dn)
      shared_dn_item(a, t - a.t_shd, arow, st, tk);
    else
      routed_dn_item(a, t - a.t_dn, arow, st, tk);
    t = ticket_of(next);
  }
  if (blockIdx.x == 0 && wave == 0) {
    ensure_topk(a, tk);
    write_routing(a, tk);
  }
  // the last wave out zeroes the counters for the next launch
  int last = 0;
  if (lane_id() == 0) {
    __builtin_amdgcn_s_waitcnt(0);
    last = add_dev(a.ctr + kCtrExit, 1) == (int)gridDim.x * 4 - 1;
  }
  if (__builtin_amdgcn_readfirstlane(last)) {
    const int lane = lane_id();
    const int nb = (a.L + 63) / 64;
    for (int i = lane; i < a.k; i += kWave) st_dev(a.ctr + kCtrRoute + 16 * i, 0);
    for (int i = lane; i < nb; i += kWave) st_dev(a.ctr + kCtrBlock + 16 * i, 0);
    for (int i = lane; i < a.S; i += kWave) st_dev(a.ctr + kCtrShared + 16 * i, 0);
    if (lane < kQueues) st_dev(a.ctr + kCtrTicket + 16 * lane, 0);
    uint64_t* pub = reinterpret_cast<uint64_t*>(a.ctr + kCtrLogit);
    for (int i = lane; i < a.E; i += kWave)
      __hip_atomic_store(pub + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (lane == 0) st_dev(a.ctr + kCtrExit, 0);
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static int decode_grid(size_t lds_bytes) {
  // per device: the grid in the low half, the LDS size it was computed for in
  // the high half, so concurrent callers see a consistent pair
  static std::atomic<uint64_t> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  const uint64_t c = cached[dev].load(std::memory_order_relaxed);
  if ((uint32_t)c > 0 && (c >> 32) == lds_bytes) return (int)(uint32_t)c;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel, 256, lds_bytes) !=
          hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  const int grid = cus * std::min(per_cu, kWgPerCu);
  cached[dev].store(((uint64_t)lds_bytes << 32) | (uint32_t)grid, std::memory_order_relaxed);
  return grid;
}

void make_decode_args(const Plan& p, DecodeArgs& a, bool logits_given) {
  const lmoe_dims& d = p.d;
  a.T = 1;
  a.L = d.L;
  a.E = d.E;
  a.k = d.k;
  a.I = d.I;
  a.S = d.S;
  a.Is = d.Is;
  a.n_router = logits_given ? (d.E + kWave - 1) / kWave : d.E;
  a.n_groups = d.k;
  a.xstride = d.L;
  a.shgu_per_expert = d.S > 0 ? (d.Is + 7) / 8 : 0;
  a.n_shgu = d.S * a.shgu_per_expert;
  a.gu_per_route = (d.I + 15) / 16;
  a.n_gu = d.k * a.gu_per_route;
  a.shd_per_expert = d.L / 16;
  a.n_shd = d.S * a.shd_per_expert;
  a.dn_per_route = (d.L + 31) / 32;
  a.n_dn = d.k * a.dn_per_route;
  a.t_topk = a.t_shgu = a.n_router;
  a.t_gu = a.t_shgu + a.n_shgu;
  a.t_shd = a.t_gu + a.n_gu;
  a.t_dn = a.t_shd + a.n_shd;
  a.t_total = a.t_dn + a.n_dn;
  // per-wave A row: h of one route or of one shared expert
  a.a_region = std::max(d.I, d.S > 0 ? d.Is : 0);
  a.lds_bytes = (size_t)(((d.L + 7) & ~7) + 4 * a.a_region) * 2;
}

__global__ __launch_bounds__(64) void read_errors_kernel(int32_t* ctr, int32_t* count) {
  if (threadIdx.x == 0)
    *count = __hip_atomic_exchange(ctr + kCtrError, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_read_errors(int32_t* ctr, int32_t* count, hipStream_t s) {
  hipLaunchKernelGGL(read_errors_kernel, dim3(1), dim3(64), 0, s, ctr, count);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s, const hipEvent_t* ev) {
  hipError_t e = record_stage(ev, LMOE_STAGE_BEGIN, s);
  if (e != hipSuccess) return e;
  // at least one wave per ticket queue
  const int grid = std::max((kQueues + 3) / 4, decode_grid(a.lds_bytes));
  hipLaunchKernelGGL(decode_kernel, dim3(grid), dim3(256), a.lds_bytes, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // one kernel holds every stage
  for (int i = LMOE_STAGE_ROUTER; i < LMOE_NUM_STAGE_EVENTS; ++i)
    if ((e = record_stage(ev, i, s)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace lmoe
