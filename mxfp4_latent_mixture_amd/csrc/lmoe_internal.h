// Host-side internals: launch plans, workspace layout and kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/lmoe.h"

namespace lmoe {

// Rows (routes) per tile of the grouped expert GEMMs.
constexpr int kSmallRows = 16;   // one 16-row MFMA tile: decode-sized groups
constexpr int kLargeRows = 128;  // eight 16-row MFMA tiles: prefill-sized groups

// Router: K steps of 32, split over ks partial sums when T is small so the
// 6.4 MB weight stream is spread over enough workgroups.
struct RouterPlan {
  int ks;          // number of K splits (partial sums)
  int steps_per;   // 32-wide K steps per split
};

struct Plan {
  lmoe_dims d;
  int R;              // T * k routes
  RouterPlan router;
  int rows_per_tile;  // kSmallRows or kLargeRows
  int max_tiles;      // upper bound on routed tiles
};

struct Workspace {
  float* part;        // [ks][T][E] router partial sums
  int32_t* idx;       // [R]
  float* w;           // [R]
  int32_t* counts;    // [E]
  int32_t* offsets;   // [E+1]
  int32_t* perm;      // [R]
  int32_t* inv;       // [R]
  int32_t* tiles;     // [max_tiles][3]: expert, first sorted position, rows
  int32_t* ntiles;    // [1]
  uint16_t* h;        // [R][I] bf16, sorted route order
  uint16_t* h_sh;     // [S][T][Is] bf16
  float* y;           // [R][L] fp32 route partials, sorted route order
  float* y_sh;        // [S][T][L] fp32
  size_t bytes;       // total bytes needed
};

Plan make_plan(const lmoe_dims& d);
Workspace carve_workspace(const Plan& p, void* base);

// ---- kernel launchers (route.hip) ----
hipError_t launch_router(const Plan& p, const uint16_t* x, const uint16_t* wr, float* part,
                         hipStream_t s);
hipError_t launch_topk(const Plan& p, const float* part, int ks, float* logits_out,
                       int32_t* idx, float* w, hipStream_t s);
hipError_t launch_permute(const Plan& p, const int32_t* idx, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv, int32_t* tiles, int32_t* ntiles,
                          hipStream_t s);

// ---- kernel launchers (experts.hip) ----
hipError_t launch_experts(const Plan& p, const uint16_t* x, const lmoe_weights& w,
                          const Workspace& ws, const int32_t* perm, const int32_t* inv,
                          const float* topk_w, uint16_t* out, hipStream_t s);
hipError_t launch_dequant(const uint8_t* q, const uint8_t* sc, int rows, int K, uint16_t* out,
                          hipStream_t s);

}  // namespace lmoe
