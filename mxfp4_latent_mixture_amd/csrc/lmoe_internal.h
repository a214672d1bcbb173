// Host-side internals: launch plans, workspace layout and kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/lmoe.h"

namespace lmoe {

// Rows (routes) per tile of the grouped expert GEMMs.
constexpr int kSmallRows = 16;   // one 16-row MFMA tile: shared-expert tiles up to 64 tokens
constexpr int kLargeRows = 96;   // six 16-row MFMA tiles: prefill-sized groups
constexpr int kDenseRows = 256;  // sixteen: the shared experts' tokens, in one group

// Router: K steps of 32, split over ks partial sums when T is small so the
// 6.4 MB weight stream is spread over enough workgroups.
struct RouterPlan {
  int ks;          // number of K splits (partial sums)
  int steps_per;   // 32-wide K steps per split
  int tok;         // tokens per router tile (64, or 128 beyond 512 tokens)
};

// Counter block at the start of every workspace (int32 slots, each counter on
// its own 64-byte line; device-scope atomics on one address serialise, so
// heavily bumped counts are spread over several slots). Only the persistent
// decode kernels use it; it must be zero when one starts and is left zeroed
// when it ends. Slots common to both decode kernels:
constexpr int kQueues = 32;         // ticket queues: item i is in queue i % kQueues
constexpr int kCtrTicket = 0;       // + 16 * queue
constexpr int kCtrExit = 1024;      // waves that have left
constexpr int kCtrError = 1040;     // dependency waits abandoned at the spin limit
// single token:
constexpr int kCtrRoute = 1056;     // + 16 * route (< 32): gate/up items done
constexpr int kCtrBlock = 1568;     // + 16 * block (< 64): parts of a 64-row output block done
constexpr int kCtrShared = 2592;    // + 16 * shared expert (< 8): gate/up items done
// Published logits, one 64-bit word per expert (E <= 1024): the float's bits
// in the low half and 1 in the high half once written, so a reader sees
// every logit and whether it is in with one load, without a done count.
constexpr int kCtrLogit = 4096;
// 2..16 tokens:
constexpr int kMcTopk = 1056;       // tokens whose top-k is published
constexpr int kMcShared = 1072;     // + 16 * shared expert (< 8): gate/up items done
constexpr int kMcGroup = 2048;      // + 16 * expert group (< 256): gate/up items done
constexpr int kMcPart = 8192;       // + 16 * (64 * token + block): inputs of a 64-row block done
constexpr int kMcLogit = 32768;     // 64-bit flagged logits [token][expert], E <= 1024
constexpr size_t kCtrBytes = LMOE_COUNTER_BYTES;
static_assert((size_t)kMcLogit * 4 + 16 * 1024 * 8 <= kCtrBytes, "counter block");
static_assert((size_t)kCtrLogit * 4 + 1024 * 8 <= kCtrBytes, "counter block");
// The single-token decode kernel keeps the token and one A row in LDS.
constexpr int kDecodeMaxWidth = 4096;

// The multi-token decode kernel: one token per MFMA row, the routes of all
// tokens grouped by expert inside the launch.
constexpr int kMultiMaxT = 16;
constexpr int kMultiMaxRoutes = 256;  // T * k
constexpr size_t kLdsBytes = 160 * 1024;  // LDS of one workgroup on gfx950

struct Plan {
  lmoe_dims d;
  bool fused_decode;  // T == 1: the whole layer in one persistent kernel
  bool fused_multi;   // 2 <= T <= kMultiMaxT: likewise, one token per MFMA row
  bool multi_ok;      // the fused multi-token kernel could run this shape
  int R;              // T * k routes
  RouterPlan router;
  int rows_per_tile;  // routed group tiles: kLargeRows
  int max_tiles;      // upper bound on routed tiles
};

struct Workspace {
  int32_t* ctr;       // counter block (kCtrBytes)
  float* part;        // [ks][T][E] router partial sums
  int32_t* idx;       // [R]
  float* w;           // [R]
  int32_t* counts;    // [E]
  int32_t* offsets;   // [E+1]
  int32_t* perm;      // [R]
  int32_t* inv;       // [R]
  int32_t* tiles;     // [max_tiles][3]: expert, first sorted position, rows
  int32_t* ntiles;    // [1]
  int32_t* chunk_base;  // [ceil(T/64)][E] permutation chunk counts, then first positions
  uint16_t* h;        // [R][I] bf16, sorted route order
  uint16_t* h_sh;     // [S][T][Is] bf16
  float* y;           // [R][L] fp32 route partials, sorted route order
  float* y_sh;        // [S][T][L] fp32
  // quantised activations of the packed path (LMOE_ACT_E4M3 / _E2M1 only;
  // sized for E4M3, one byte a value): x [T][L] and h [R][I], exponents
  // [T][L/32] and [R][I/32]
  uint8_t *xq, *xq_s, *hq, *hq_s;
  // fused decode (one launch per token)
  size_t bytes;       // total bytes needed
};

struct DecodeArgs {
  const uint16_t* x;   // [T][L] bf16
  const uint16_t* wr;  // [E][L] bf16
  const uint8_t *gq, *gs, *uq, *us, *dq, *ds;
  const uint16_t *shg, *shu, *shd;
  int T, L, E, k, I, S, Is;
  float* logits_out;   // optional [T][E]
  const float* logits_in;  // given logits [T][E] (router items publish them), or null
  int32_t* idx;
  float* w;
  int32_t *counts, *offsets, *perm, *inv;
  uint16_t* out;
  int32_t* ctr;
  uint16_t* h;         // [T * k][I] bf16, by route t * k + j
  uint16_t* hsh;       // [S][T][Is] bf16
  float* y;            // [T * k][L] routed down outputs
  float* ysh;          // [S][T][L] shared down outputs
  // work items by kind, in ticket order, and where each kind starts (the
  // single-token kernel has no top-k items: t_topk == t_shgu)
  int n_router, n_shgu, n_gu, n_shd, n_dn;
  int t_topk, t_shgu, t_gu, t_shd, t_dn, t_total;
  int n_groups;        // multi-token: expert group slots, min(E, T * k)
  int xstride;         // multi-token: LDS row stride of the tokens, bf16 elements
  int shgu_per_expert, gu_per_route, dn_per_route, shd_per_expert;
  int a_region;        // per-wave LDS A row, bf16 elements
  size_t lds_bytes;    // dynamic LDS per workgroup
};

// Tile-packed routed weights (lmoe_pack_weights).
struct PackedWeights {
  const uint8_t *gu_q, *gu_s, *down_q, *down_s;
};
struct PackedSizes {
  size_t gu_q, gu_s, down_q, down_s;
};
// Routes per row tile of the packed GEMMs (three 32-row MFMA tiles).
constexpr int kPackedRows = 96;

Plan make_plan(const lmoe_dims& d);
// The plan of the packed path: 128-route row tiles.
Plan make_packed_plan(const lmoe_dims& d);
// with_q: room for the quantised activations (every public workspace size
// includes it; the no-alloc entry point, bf16 only, does not)
Workspace carve_workspace(const Plan& p, void* base, bool with_q = true);

// ---- kernel launchers (route.hip) ----
hipError_t launch_router(const Plan& p, const uint16_t* x, const uint16_t* wr, float* part,
                         hipStream_t s);
hipError_t launch_topk(const Plan& p, const float* part, int ks, float* logits_out,
                       int32_t* idx, float* w, hipStream_t s);
// Up to kPermManyFrom tokens one workgroup builds the permutation; beyond,
// chunks of 64 tokens are counted, scanned and placed by separate kernels
// (chunk_base: [ceil(T/64)][E] int32 of workspace).
constexpr int kPermManyFrom = 512;
hipError_t launch_permute(const Plan& p, const int32_t* idx, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv, int32_t* tiles, int32_t* ntiles,
                          int32_t* chunk_base, hipStream_t s);

// ---- kernel launchers (experts.hip) ----
// ev: optional stage events (LMOE_NUM_STAGE_EVENTS entries), recorded after
// each stage.
// its three parts: routed gate/up and down; the shared experts (they read
// only x, so they may run beside the routing); the combine, which needs both
hipError_t launch_routed(const Plan& p, const uint16_t* x, const lmoe_weights& w,
                         const Workspace& ws, const int32_t* perm, hipStream_t s,
                         const hipEvent_t* ev);
hipError_t launch_shared(const Plan& p, const uint16_t* x, const lmoe_weights& w,
                         const Workspace& ws, hipStream_t s, const hipEvent_t* ev);
hipError_t launch_combine(const Plan& p, const Workspace& ws, const int32_t* inv,
                          const float* topk_w, uint16_t* out, hipStream_t s,
                          const hipEvent_t* ev);

inline hipError_t record_stage(const hipEvent_t* ev, int stage, hipStream_t s) {
  return ev ? hipEventRecord(ev[stage], s) : hipSuccess;
}
// ---- tile-packed experts (packed.hip) ----
PackedSizes packed_sizes(const lmoe_dims& d);
hipError_t launch_pack(const lmoe_dims& d, const lmoe_weights& w, uint8_t* gu_q, uint8_t* gu_s,
                       uint8_t* dn_q, uint8_t* dn_s, hipStream_t s);
// act: LMOE_ACT_BF16, or quantised activations (E4M3 / E2M1 with E8M0
// scales per 32, quantised into the workspace first)
hipError_t launch_routed_packed(const Plan& p, const uint16_t* x, const PackedWeights& w,
                                const Workspace& ws, const int32_t* perm, hipStream_t s,
                                const hipEvent_t* ev, int act);
hipError_t launch_quantize_act(const uint16_t* src, int64_t rows, int K, bool fp8, uint8_t* codes,
                               uint8_t* exps, hipStream_t s);

// ---- single-token decode (decode.hip) ----
// logits_given: the router items publish given logits, 64 per item
void make_decode_args(const Plan& p, DecodeArgs& a, bool logits_given = false);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s, const hipEvent_t* ev);
// ---- 2..16-token decode (decode_multi.hip) ----
void make_decode_multi_args(const Plan& p, DecodeArgs& a, bool logits_given = false);
// LDS bytes the multi-token kernel needs (tokens and grouping tables)
size_t decode_multi_lds_bytes(const lmoe_dims& d);
hipError_t launch_decode_multi(const DecodeArgs& a, hipStream_t s, const hipEvent_t* ev);
// copies the abandoned-wait count of a workspace's counter block to *count
// and resets it
hipError_t launch_read_errors(int32_t* ctr, int32_t* count, hipStream_t s);

// ---- dense bf16 GEMMs of the MoE block (dense.hip) ----
// C = A B^T, A bf16 [M][K] (row stride lda), B bf16 [N][K] (ldb), K a
// multiple of 64. Output columns fall in three consecutive segments:
// [0, n_f32) stored as fp32 (f32_out, ld_f32); [n_f32, n_f32 + n_bf16)
// stored as bf16 after adding the optional bf16 addends add0, add1 (same
// column numbering, ld_add); the rest GLU pairs: in each 32 columns the first
// 16 are gate and the next 16 up values of 16 consecutive outputs,
// bf16(silu(g) * u) to glu_out (ld_glu). Segment starts are multiples of 32.
struct DenseArgs {
  const uint16_t* a;
  int64_t lda;
  const uint16_t* b;
  int64_t ldb;
  int M, N, K;
  int n_f32, n_bf16;
  float* f32_out;
  int64_t ld_f32;
  uint16_t* bf_out;
  int64_t ld_bf;
  uint16_t* glu_out;
  int64_t ld_glu;
  const uint16_t* add0;
  const uint16_t* add1;
  int64_t ld_add;
  // A second product of the same shape [M][N] with its own A, B and K
  // (launch_dense_pair): its K-split partial sums are summed, rounded to bf16
  // and added before add0 / add1, as the tail's shared partial is.
  const uint16_t* a2;
  int64_t lda2;
  const uint16_t* b2;
  int64_t ldb2;
  int K2;
  // b_up: a GLU over two matrices: the B rows of each 32-column group are
  // 16 rows of b (gate) then the same 16 rows of b_up (up), output columns
  // numbering the 2N' virtual rows (N = 2N'). Null: B is b.
  const uint16_t* b_up;
  // independent problems along blockIdx.z (e.g. the shared experts): each
  // pointer advances by its stride per z (without K splits)
  int64_t a_zstride, b_zstride, out_zstride;
  // set by the launchers
  int n_rt, n_ct, group_rows, k_per, k_per2;
  int ks1;      // K splits of the first product (blockIdx.y >= ks1: the second)
  float* part;  // K-split partial tiles [ksplit][M][N] (split launches only)
  float* part2; // the second product's [ksplit2][M][N]
};
struct DensePlan {
  int bm, bn;          // workgroup tile: 32, 64, 128 x 128 rows, or 256 x 256
  int ksplit, k_per;   // K splits and K per split
  size_t part_floats;  // workspace for the partial tiles
};
DensePlan dense_plan(int M, int N, int K);
hipError_t launch_dense(DenseArgs a, const DensePlan& p, float* part, hipStream_t s);
// nz independent problems of one shape in one launch (blockIdx.z), no K
// split; pointers advance by the DenseArgs z strides.
hipError_t launch_dense_batched(DenseArgs a, int nz, hipStream_t s);
// Two products of the same [M][N] shape in one launch, both K-split
// (p1.ksplit > 1 and p2.ksplit > 1, the same tile rows): out = epilogue of
// (A B^T + bf16(A2 B2^T)). part: p1.part_floats + p2.part_floats floats.
hipError_t launch_dense_pair(DenseArgs a, const DensePlan& p1, const DensePlan& p2, float* part,
                             hipStream_t s);
hipError_t launch_rmsnorm(const uint16_t* r, const uint16_t* gamma, int T, int L, float eps,
                          uint16_t* out, hipStream_t s);

hipError_t launch_read_stream(const void* p, size_t bytes, uint32_t* sink, int blocks,
                              hipStream_t s);
hipError_t launch_dequant(const uint8_t* q, const uint8_t* sc, int rows, int K, uint16_t* out,
                          hipStream_t s);

}  // namespace lmoe
