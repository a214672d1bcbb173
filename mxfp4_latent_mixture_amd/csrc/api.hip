// C ABI of the LatentMoE layer: argument validation, workspace layout and the
// launch sequence (router -> top-k -> grouping -> experts -> combine).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <mutex>

#include "lmoe_internal.h"

namespace lmoe {

// measure.hip
hipError_t launch_mfma_rate(int iters, uint32_t* sink, int blocks, hipStream_t s);

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

static bool dims_ok(const lmoe_dims& d) {
  if (d.T < 0 || d.T > (1 << 20)) return false;
  if (d.L < 32 || d.L > 16384 || d.L % 32) return false;
  if (d.E < 1 || d.E > 1024) return false;
  if (d.k < 1 || d.k > 32 || d.k > d.E) return false;
  if (d.I < 32 || d.I > 16384 || d.I % 32) return false;
  if (d.S < 0 || d.S > 8) return false;
  if (d.S > 0 && (d.Is < 32 || d.Is > 16384 || d.Is % 32)) return false;
  return true;
}

Plan make_plan(const lmoe_dims& d) {
  Plan p;
  p.d = d;
  if (p.d.S == 0) p.d.Is = 0;
  p.R = d.T * d.k;
  // Router: enough (tile x split) workgroups to spread the weight stream;
  // 128-token tiles beyond 512 tokens (each router row read once per 128
  // tokens), and no K split once they alone fill the chip.
  const int nsteps = d.L / 32;
  p.router.tok = d.T > 512 ? 128 : 64;
  const int tiles = ((d.E + 63) / 64) * ((d.T + p.router.tok - 1) / p.router.tok);
  const int target = p.router.tok == 128 ? 256 : 512;
  int ks = std::max(1, std::min(nsteps, (target + tiles - 1) / std::max(1, tiles)));
  int per = (nsteps + ks - 1) / ks;
  ks = (nsteps + per - 1) / per;
  p.router.ks = ks;
  p.router.steps_per = per;
  // Routed groups are cut into tiles of up to 96 rows whatever their size:
  // measured on the Kimi-K3 layer, the 96-row kernel (one to six 16-row MFMA
  // tiles) streams the weights faster than 16-row tiles even at 1-5 routes
  // per expert (T = 2 .. 384).
  p.rows_per_tile = kLargeRows;
  p.max_tiles = std::min(d.E, p.R) + p.R / p.rows_per_tile;
  // One token, when every row a decode wave stages (h of one route or one
  // shared expert) and the token itself fit its fixed-size staging.
  const bool widths_ok =
      d.L <= kDecodeMaxWidth && d.I <= kDecodeMaxWidth && p.d.Is <= kDecodeMaxWidth;
  p.fused_decode = d.T == 1 && widths_ok;
  // 2..16 tokens: one per MFMA row, when the routes fit the grouping tables
  // and the tokens fit the LDS; taken while the weight stream is small
  // enough that the grouped path's fixed costs outweigh its faster stream.
  p.multi_ok = d.T >= 2 && d.T <= kMultiMaxT && d.T * d.k <= kMultiMaxRoutes && widths_ok &&
               decode_multi_lds_bytes(d) <= kLdsBytes;
  const double fp4_row = 17.0 / 32.0;
  const double stream = (double)std::min(d.E, d.T * d.k) * 3.0 * d.L * d.I * fp4_row +
                        (double)p.d.S * 3.0 * d.L * p.d.Is * 2.0 + 2.0 * d.L * d.E;
  p.fused_multi = p.multi_ok && stream <= (double)LMOE_FUSED_MULTI_BYTES;
  return p;
}

Plan make_packed_plan(const lmoe_dims& d) {
  Plan p = make_plan(d);
  p.rows_per_tile = kPackedRows;
  p.max_tiles = std::min(d.E, p.R) + p.R / p.rows_per_tile;
  p.fused_decode = false;
  p.fused_multi = false;
  p.multi_ok = false;
  return p;
}

// From 512 tokens the router's scores come from the dense GEMM kernel of the
// block (dense.hip: 32x32x16 MFMA tiles, both operands staged through LDS),
// K-split with a finishing pass that writes the fp32 scores; below, the
// router kernel (route.hip). At the Kimi-K3 prefill chunk (4096 tokens, 896
// experts) the router stage measured 70-72 us this way against 82-88 us with
// the router kernel on the same box.
static bool dense_router(const lmoe_dims& d) {
  return d.T >= 512 && d.L % 64 == 0 && d.E % 32 == 0;
}

// floats of the router's workspace: the router kernel's K-split partial
// scores, or the dense kernel's partial tiles and then the final scores
static size_t router_floats(const Plan& p) {
  const lmoe_dims& d = p.d;
  size_t n = (size_t)p.router.ks * d.T * d.E;
  if (dense_router(d)) {
    const DensePlan rp = dense_plan(d.T, d.E, d.L);
    n = std::max(n, rp.part_floats + (size_t)d.T * d.E);
  }
  return n;
}

Workspace carve_workspace(const Plan& p, void* base, bool with_q) {
  const lmoe_dims& d = p.d;
  Workspace w = {};
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t bytes) -> char* {
    char* r = b ? b + off : nullptr;
    off = align_up(off + bytes, 256);
    return r;
  };
  const size_t T = d.T, E = d.E, R = p.R, L = d.L, I = d.I, S = d.S, Is = d.Is;
  w.ctr = reinterpret_cast<int32_t*>(take(kCtrBytes));
  w.part = reinterpret_cast<float*>(take(router_floats(p) * 4));
  w.idx = reinterpret_cast<int32_t*>(take(R * 4));
  w.w = reinterpret_cast<float*>(take(R * 4));
  w.counts = reinterpret_cast<int32_t*>(take(E * 4));
  w.offsets = reinterpret_cast<int32_t*>(take((E + 1) * 4));
  w.perm = reinterpret_cast<int32_t*>(take(R * 4));
  w.inv = reinterpret_cast<int32_t*>(take(R * 4));
  w.tiles = reinterpret_cast<int32_t*>(take((size_t)p.max_tiles * 3 * 4));
  w.ntiles = reinterpret_cast<int32_t*>(take(4));
  w.chunk_base = reinterpret_cast<int32_t*>(take(((T + 63) / 64) * E * 4));
  w.h = reinterpret_cast<uint16_t*>(take(R * I * 2));
  w.h_sh = reinterpret_cast<uint16_t*>(take(S * T * Is * 2));
  w.y = reinterpret_cast<float*>(take(R * L * 4));
  w.y_sh = reinterpret_cast<float*>(take(S * T * L * 4));
  if (with_q) {  // last, so the layout before does not depend on it
    w.xq = reinterpret_cast<uint8_t*>(take(T * L));
    w.xq_s = reinterpret_cast<uint8_t*>(take(T * L / 32));
    w.hq = reinterpret_cast<uint8_t*>(take(R * I));
    w.hq_s = reinterpret_cast<uint8_t*>(take(R * I / 32));
  }
  w.bytes = off;
  return w;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static int check_opt_ptr(const void* p) {
  if (p && !aligned16(p)) return LMOE_ERR_ALIGN;
  return LMOE_OK;
}

// Validate and run steps router -> top-k -> grouping. Fills the resolved
// routing buffers (user's when given, workspace otherwise).
struct Routing {
  int32_t* idx;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv;
};

static int run_route(const Plan& p, const Workspace& ws, const uint16_t* x, const uint16_t* wr,
                     int logits_given, const lmoe_routing* r, Routing* out, hipStream_t s,
                     const hipEvent_t* ev) {
  Routing rt;
  rt.idx = (r && r->topk_idx) ? r->topk_idx : ws.idx;
  rt.w = (r && r->topk_w) ? r->topk_w : ws.w;
  rt.counts = (r && r->counts) ? r->counts : ws.counts;
  rt.offsets = (r && r->offsets) ? r->offsets : ws.offsets;
  rt.perm = (r && r->perm) ? r->perm : ws.perm;
  rt.inv = (r && r->inv_perm) ? r->inv_perm : ws.inv;
  hipError_t e = record_stage(ev, LMOE_STAGE_BEGIN, s);
  if (e != hipSuccess) return LMOE_ERR_HIP;
  const float* part;
  int ks;
  float* logits_out = nullptr;
  if (logits_given) {
    part = r->logits;
    ks = 1;
  } else if (dense_router(p.d)) {
    // the scores straight into the caller's logits when asked for, else the
    // workspace after the partial tiles; top-k then reads them whole
    const lmoe_dims& d = p.d;
    const DensePlan rp = dense_plan(d.T, d.E, d.L);
    float* scores = (r && r->logits) ? r->logits : ws.part + rp.part_floats;
    DenseArgs a = {};
    a.a = x;
    a.lda = d.L;
    a.b = wr;
    a.ldb = d.L;
    a.M = d.T;
    a.N = d.E;
    a.K = d.L;
    a.n_f32 = d.E;
    a.f32_out = scores;
    a.ld_f32 = d.E;
    e = launch_dense(a, rp, ws.part, s);
    if (e != hipSuccess) return LMOE_ERR_HIP;
    part = scores;
    ks = 1;
  } else {
    e = launch_router(p, x, wr, ws.part, s);
    if (e != hipSuccess) return LMOE_ERR_HIP;
    part = ws.part;
    ks = p.router.ks;
    logits_out = r ? r->logits : nullptr;
  }
  if (record_stage(ev, LMOE_STAGE_ROUTER, s) != hipSuccess) return LMOE_ERR_HIP;
  e = launch_topk(p, part, ks, logits_out, rt.idx, rt.w, s);
  if (e != hipSuccess || record_stage(ev, LMOE_STAGE_TOPK, s) != hipSuccess) return LMOE_ERR_HIP;
  e = launch_permute(p, rt.idx, rt.counts, rt.offsets, rt.perm, rt.inv, ws.tiles, ws.ntiles,
                     ws.chunk_base, s);
  if (e != hipSuccess || record_stage(ev, LMOE_STAGE_PERMUTE, s) != hipSuccess)
    return LMOE_ERR_HIP;
  *out = rt;
  return LMOE_OK;
}

// T == 1, or 2..16 tokens: the whole layer as one persistent kernel. Stage
// events: the kernel's time lands on the router stage. With given logits
// (r->logits) the router items publish them instead of computing them.
static int run_fused_decode(const Plan& p, const Workspace& ws, const uint16_t* x,
                            const lmoe_weights& w, const lmoe_routing* r, uint16_t* out,
                            hipStream_t s, const hipEvent_t* ev, bool logits_given) {
  DecodeArgs a;
  if (p.fused_multi)
    make_decode_multi_args(p, a, logits_given);
  else
    make_decode_args(p, a, logits_given);
  a.x = x;
  a.wr = w.router_w;
  a.gq = w.gate_q;
  a.gs = w.gate_s;
  a.uq = w.up_q;
  a.us = w.up_s;
  a.dq = w.down_q;
  a.ds = w.down_s;
  a.shg = w.sh_gate;
  a.shu = w.sh_up;
  a.shd = w.sh_down;
  int32_t* idx = (r && r->topk_idx) ? r->topk_idx : ws.idx;
  float* wt = (r && r->topk_w) ? r->topk_w : ws.w;
  int32_t* counts = (r && r->counts) ? r->counts : ws.counts;
  int32_t* offsets = (r && r->offsets) ? r->offsets : ws.offsets;
  int32_t* perm = (r && r->perm) ? r->perm : ws.perm;
  int32_t* inv = (r && r->inv_perm) ? r->inv_perm : ws.inv;
  a.ctr = ws.ctr;
  a.h = ws.h;
  a.hsh = ws.h_sh;
  a.y = ws.y;
  a.ysh = ws.y_sh;
  a.out = out;
  a.logits_out = (r && !logits_given) ? r->logits : nullptr;
  a.logits_in = logits_given ? r->logits : nullptr;
  a.idx = idx;
  a.w = wt;
  a.counts = counts;
  a.offsets = offsets;
  a.perm = perm;
  a.inv = inv;
  const hipError_t e = p.fused_multi ? launch_decode_multi(a, s, ev) : launch_decode(a, s, ev);
  return e == hipSuccess ? LMOE_OK : LMOE_ERR_HIP;
}

static int check_routing(const lmoe_routing* r, int logits_given) {
  if (logits_given && (!r || !r->logits)) return LMOE_ERR_NULL;
  if (!r) return LMOE_OK;
  const void* ps[] = {r->logits, r->topk_idx, r->topk_w, r->counts,
                      r->offsets, r->perm, r->inv_perm};
  for (const void* q : ps) {
    int st = check_opt_ptr(q);
    if (st) return st;
  }
  return LMOE_OK;
}

}  // namespace lmoe

using namespace lmoe;

extern "C" size_t lmoe_workspace_bytes(const lmoe_dims* dims) {
  if (!dims || !dims_ok(*dims)) return 0;
  Plan p = make_plan(*dims);
  return carve_workspace(p, nullptr).bytes;
}

extern "C" const char* lmoe_status_string(int status) {
  switch (status) {
    case LMOE_OK: return "ok";
    case LMOE_ERR_NULL: return "required pointer is NULL";
    case LMOE_ERR_SHAPE: return "dimensions violate the layer constraints";
    case LMOE_ERR_ALIGN: return "device pointer is not 16-byte aligned";
    case LMOE_ERR_WORKSPACE: return "workspace smaller than lmoe_workspace_bytes()";
    case LMOE_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

extern "C" int lmoe_route(const lmoe_dims* dims, const uint16_t* x, const uint16_t* router_w,
                          int logits_given, const lmoe_routing* r, void* ws, size_t ws_bytes,
                          void* stream) {
  if (!dims) return LMOE_ERR_NULL;
  if (!dims_ok(*dims)) return LMOE_ERR_SHAPE;
  int st = check_routing(r, logits_given);
  if (st) return st;
  if (dims->T == 0) return LMOE_OK;
  if (!logits_given && (!x || !router_w)) return LMOE_ERR_NULL;
  if (!ws) return LMOE_ERR_NULL;
  if (check_opt_ptr(x) || check_opt_ptr(router_w) || !aligned16(ws)) return LMOE_ERR_ALIGN;
  Plan p = make_plan(*dims);
  Workspace w = carve_workspace(p, ws);
  if (ws_bytes < w.bytes) return LMOE_ERR_WORKSPACE;
  Routing rt;
  return run_route(p, w, x, router_w, logits_given, r, &rt, static_cast<hipStream_t>(stream),
                   nullptr);
}

// A second stream per device, with a fork and a join event, on which the
// shared experts run beside the routing and the routed GEMMs (they depend
// only on x). Created on a device's first grouped call; if creation fails,
// calls stay on the caller's stream. The mutex makes each call's fork, side
// launches and join one unit, so concurrent callers cannot interleave their
// event records; calls from different caller streams queue on the one side
// stream.
struct SideStream {
  std::mutex mu;
  bool tried = false;
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

static SideStream* side_stream() {
  static SideStream sides[64];
  static std::mutex create_mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  SideStream& st = sides[dev];
  std::lock_guard<std::mutex> g(create_mu);
  if (!st.tried) {
    st.tried = true;
    // default priority, like every stream here
    if (hipStreamCreateWithFlags(&st.s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&st.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&st.join, hipEventDisableTiming) != hipSuccess)
      st.s = nullptr;
  }
  return st.s ? &st : nullptr;
}

// Where one call runs its shared experts: the caller's stream (s == nullptr),
// the library's per-device second stream (under its mutex), or the caller's
// stream and events (lmoe_forward_ex).
struct SideExec {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex* mu = nullptr;
};

enum class SideMode { kLibrary, kCaller };

// pk: the tile-packed routed weights (lmoe_forward_packed), whose gate/up
// and down pointers replace wts' (which then carries router and shared ones).
static int forward_impl(const lmoe_dims* dims, const uint16_t* x, const lmoe_weights* wts,
                        int logits_given, const lmoe_routing* r, uint16_t* out, void* ws,
                        size_t ws_bytes, void* stream, const hipEvent_t* ev, SideMode mode,
                        const lmoe_exec* exec, const PackedWeights* pk = nullptr,
                        bool ws_with_q = true) {
  if (!dims || !wts) return LMOE_ERR_NULL;
  if (!dims_ok(*dims)) return LMOE_ERR_SHAPE;
  int st = check_routing(r, logits_given);
  if (st) return st;
  hipEvent_t exec_ev[LMOE_NUM_STAGE_EVENTS];
  if (mode == SideMode::kCaller && exec && exec->stage_events) {
    if (ev) return LMOE_ERR_NULL;
    for (int i = 0; i < LMOE_NUM_STAGE_EVENTS; ++i) {
      if (!exec->stage_events[i]) return LMOE_ERR_NULL;
      exec_ev[i] = static_cast<hipEvent_t>(exec->stage_events[i]);
    }
    ev = exec_ev;
  } else if (mode == SideMode::kCaller && exec && exec->side_stream &&
             (!exec->fork_event || !exec->join_event)) {
    return LMOE_ERR_NULL;
  }
  if (dims->T == 0) return LMOE_OK;
  const lmoe_weights& w = *wts;
  if (!x || !out || !ws) return LMOE_ERR_NULL;
  if (!logits_given && !w.router_w) return LMOE_ERR_NULL;
  if (pk) {
    if (!pk->gu_q || !pk->gu_s || !pk->down_q || !pk->down_s) return LMOE_ERR_NULL;
    const void* pp[] = {pk->gu_q, pk->gu_s, pk->down_q, pk->down_s};
    for (const void* q : pp)
      if (check_opt_ptr(q)) return LMOE_ERR_ALIGN;
  } else if (!w.gate_q || !w.gate_s || !w.up_q || !w.up_s || !w.down_q || !w.down_s) {
    return LMOE_ERR_NULL;
  }
  if (dims->S > 0 && (!w.sh_gate || !w.sh_up || !w.sh_down)) return LMOE_ERR_NULL;
  const void* ptrs[] = {x, out, ws, w.router_w, w.gate_q, w.gate_s, w.up_q,
                        w.up_s, w.down_q, w.down_s, w.sh_gate, w.sh_up, w.sh_down};
  for (const void* q : ptrs)
    if (check_opt_ptr(q)) return LMOE_ERR_ALIGN;
  // the packed GEMMs address activation rows with 32-bit byte offsets
  if (pk && ((int64_t)dims->T * dims->L >= (int64_t(1) << 31) ||
             (int64_t)dims->T * dims->k * dims->I >= (int64_t(1) << 31)))
    return LMOE_ERR_SHAPE;
  // quantised activations: tile-packed experts only, K multiples of 128
  const int act = (mode == SideMode::kCaller && exec) ? exec->act_format : LMOE_ACT_BF16;
  if (act != LMOE_ACT_BF16 &&
      (act != LMOE_ACT_E4M3 && act != LMOE_ACT_E2M1 || !pk || dims->L % 128 || dims->I % 128))
    return LMOE_ERR_SHAPE;
  Plan p = pk ? make_packed_plan(*dims) : make_plan(*dims);
  if (mode == SideMode::kCaller && exec) {
    if (exec->path == LMOE_PATH_GROUPED) {
      p.fused_decode = p.fused_multi = false;
    } else if (exec->path == LMOE_PATH_FUSED) {
      p.fused_multi = p.multi_ok;
    } else if (exec->path != LMOE_PATH_AUTO) {
      return LMOE_ERR_SHAPE;
    }
  }
  // the workspace is the one lmoe_workspace_bytes sizes (the no-alloc
  // scratch, bf16 only, leaves out the quantised activations)
  Workspace wsp = carve_workspace(p, ws, ws_with_q);
  if (ws_bytes < wsp.bytes) return LMOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.fused_decode || p.fused_multi)
    return run_fused_decode(p, wsp, x, w, r, out, s, ev, logits_given != 0);
  Routing rt;
  // Traced calls keep every stage on the caller's stream, in order, so each
  // stage's events time it alone.
  SideExec side;
  if (!ev && p.d.S > 0) {
    if (mode == SideMode::kLibrary) {
      if (SideStream* lib = side_stream()) {
        side.s = lib->s;
        side.fork = lib->fork;
        side.join = lib->join;
        side.mu = &lib->mu;
      }
    } else if (exec && exec->side_stream) {
      side.s = static_cast<hipStream_t>(exec->side_stream);
      side.fork = static_cast<hipEvent_t>(exec->fork_event);
      side.join = static_cast<hipEvent_t>(exec->join_event);
    }
  }
  auto routed = [&](hipStream_t rs, const hipEvent_t* rev) {
    return pk ? launch_routed_packed(p, x, *pk, wsp, rt.perm, rs, rev, act)
              : launch_routed(p, x, w, wsp, rt.perm, rs, rev);
  };
  if (!side.s) {
    st = run_route(p, wsp, x, w.router_w, logits_given, r, &rt, s, ev);
    if (st) return st;
    hipError_t e = routed(s, ev);
    if (e == hipSuccess) e = launch_shared(p, x, w, wsp, s, ev);
    if (e == hipSuccess) e = launch_combine(p, wsp, rt.inv, rt.w, out, s, ev);
    return e == hipSuccess ? LMOE_OK : LMOE_ERR_HIP;
  }
  std::unique_lock<std::mutex> g;
  if (side.mu) g = std::unique_lock<std::mutex>(*side.mu);
  if (hipEventRecord(side.fork, s) != hipSuccess ||
      hipStreamWaitEvent(side.s, side.fork, 0) != hipSuccess ||
      launch_shared(p, x, w, wsp, side.s, nullptr) != hipSuccess ||
      hipEventRecord(side.join, side.s) != hipSuccess)
    return LMOE_ERR_HIP;
  st = run_route(p, wsp, x, w.router_w, logits_given, r, &rt, s, nullptr);
  hipError_t e = st ? hipSuccess : routed(s, nullptr);
  // the join is waited for on every path, so no later call on s can reuse
  // the workspace before the shared experts are done with it
  if (hipStreamWaitEvent(s, side.join, 0) != hipSuccess) return LMOE_ERR_HIP;
  if (st) return st;
  if (e == hipSuccess) e = launch_combine(p, wsp, rt.inv, rt.w, out, s, nullptr);
  return e == hipSuccess ? LMOE_OK : LMOE_ERR_HIP;
}

extern "C" int lmoe_forward(const lmoe_dims* dims, const uint16_t* x, const lmoe_weights* wts,
                            int logits_given, const lmoe_routing* r, uint16_t* out, void* ws,
                            size_t ws_bytes, void* stream) {
  return forward_impl(dims, x, wts, logits_given, r, out, ws, ws_bytes, stream, nullptr,
                      SideMode::kLibrary, nullptr);
}

extern "C" int lmoe_forward_ex(const lmoe_dims* dims, const uint16_t* x, const lmoe_weights* wts,
                               int logits_given, const lmoe_routing* r, uint16_t* out, void* ws,
                               size_t ws_bytes, void* stream, const lmoe_exec* exec) {
  return forward_impl(dims, x, wts, logits_given, r, out, ws, ws_bytes, stream, nullptr,
                      SideMode::kCaller, exec);
}

namespace {

// ---------------------------------------------------------------------------
// Scratch of lmoe_forward_noalloc: one array per GPU (each device holds its
// own copy at its own address). In host code `scratch` names a host-side
// stand-in, never the device memory: its device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[LMOE_NOALLOC_SCRATCH_BYTES];

__global__ __launch_bounds__(256) void zero_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

struct ScratchSlot {
  std::once_flag once;
  hipError_t err = hipErrorNotInitialized;
  void* ptr = nullptr;
};

// The device address of this device's scratch (nullptr on failure).
static void* scratch_ptr(int dev) {
  static ScratchSlot slots[64];
  if (dev < 0 || dev >= 64) return nullptr;
  ScratchSlot& sl = slots[dev];
  std::call_once(sl.once, [&] {
    void* p = nullptr;
    sl.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    sl.ptr = sl.err == hipSuccess ? p : nullptr;
  });
  return sl.ptr;
}

// True from the second time it is asked for a device on: the first caller
// clears the counter block.
static bool scratch_cleared_once(int dev) {
  static std::atomic<bool> cleared[64];
  return cleared[dev].exchange(true);
}

}  // namespace

extern "C" int lmoe_forward_noalloc(const lmoe_dims* dims, const uint16_t* x,
                                    const lmoe_weights* wts, int logits_given,
                                    const lmoe_routing* r, uint16_t* out, void* stream) {
  if (!dims || !wts) return LMOE_ERR_NULL;
  if (!dims_ok(*dims)) return LMOE_ERR_SHAPE;
  const size_t need = carve_workspace(make_plan(*dims), nullptr, false).bytes;
  if (need > LMOE_NOALLOC_SCRATCH_BYTES) return LMOE_ERR_WORKSPACE;
  if (dims->T == 0) return forward_impl(dims, x, wts, logits_given, r, out, nullptr, 0, stream,
                                        nullptr, SideMode::kCaller, nullptr);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LMOE_ERR_HIP;
  void* ws = scratch_ptr(dev);
  if (!ws) return LMOE_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!scratch_cleared_once(dev)) {
    // the counter block must be zero before the first call; every call
    // leaves it zero (a fill kernel, not a memset, so capture is safe)
    const int n = (int)(kCtrBytes / 4);
    hipLaunchKernelGGL(zero_kernel, dim3((n + 255) / 256), dim3(256), 0, s,
                       static_cast<uint32_t*>(ws), n);
    if (hipGetLastError() != hipSuccess) return LMOE_ERR_HIP;
  }
  return forward_impl(dims, x, wts, logits_given, r, out, ws, LMOE_NOALLOC_SCRATCH_BYTES, stream,
                      nullptr, SideMode::kCaller, nullptr, nullptr, false);
}

extern "C" int lmoe_wait_errors(void* ws, size_t ws_bytes, int32_t* count, void* stream) {
  if (!ws || !count) return LMOE_ERR_NULL;
  if (!aligned16(ws) || (reinterpret_cast<uintptr_t>(count) & 3u)) return LMOE_ERR_ALIGN;
  if (ws_bytes < kCtrBytes) return LMOE_ERR_WORKSPACE;
  hipError_t e = launch_read_errors(static_cast<int32_t*>(ws), count,
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LMOE_OK : LMOE_ERR_HIP;
}

extern "C" int lmoe_packed_sizes_of(const lmoe_dims* dims, lmoe_packed_sizes* sizes) {
  if (!dims || !sizes) return LMOE_ERR_NULL;
  if (!dims_ok(*dims)) return LMOE_ERR_SHAPE;
  const PackedSizes z = packed_sizes(*dims);
  sizes->gu_q = z.gu_q;
  sizes->gu_s = z.gu_s;
  sizes->down_q = z.down_q;
  sizes->down_s = z.down_s;
  return LMOE_OK;
}

extern "C" int lmoe_pack_weights(const lmoe_dims* dims, const lmoe_weights* w, uint8_t* gu_q,
                                 uint8_t* gu_s, uint8_t* down_q, uint8_t* down_s, void* stream) {
  if (!dims || !w) return LMOE_ERR_NULL;
  if (!dims_ok(*dims)) return LMOE_ERR_SHAPE;
  if (!w->gate_q || !w->gate_s || !w->up_q || !w->up_s || !w->down_q || !w->down_s || !gu_q ||
      !gu_s || !down_q || !down_s)
    return LMOE_ERR_NULL;
  const void* ptrs[] = {w->gate_q, w->gate_s, w->up_q, w->up_s, w->down_q, w->down_s,
                        gu_q,      gu_s,      down_q,  down_s};
  for (const void* q : ptrs)
    if (!aligned16(q)) return LMOE_ERR_ALIGN;
  hipError_t e = launch_pack(*dims, *w, gu_q, gu_s, down_q, down_s,
                             static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LMOE_OK : LMOE_ERR_HIP;
}

extern "C" int lmoe_forward_packed(const lmoe_dims* dims, const uint16_t* x,
                                   const lmoe_packed_weights* w, int logits_given,
                                   const lmoe_routing* r, uint16_t* out, void* ws,
                                   size_t ws_bytes, void* stream, const lmoe_exec* exec) {
  if (!w) return LMOE_ERR_NULL;
  lmoe_weights cw = {};
  cw.router_w = w->router_w;
  cw.sh_gate = w->sh_gate;
  cw.sh_up = w->sh_up;
  cw.sh_down = w->sh_down;
  PackedWeights pk = {w->gu_q, w->gu_s, w->down_q, w->down_s};
  return forward_impl(dims, x, &cw, logits_given, r, out, ws, ws_bytes, stream, nullptr,
                      SideMode::kCaller, exec, &pk);
}

extern "C" int lmoe_forward_traced(const lmoe_dims* dims, const uint16_t* x,
                                   const lmoe_weights* wts, int logits_given,
                                   const lmoe_routing* r, uint16_t* out, void* ws,
                                   size_t ws_bytes, void* stream, void* const* events) {
  if (!events) return LMOE_ERR_NULL;
  hipEvent_t ev[LMOE_NUM_STAGE_EVENTS];
  for (int i = 0; i < LMOE_NUM_STAGE_EVENTS; ++i) {
    if (!events[i]) return LMOE_ERR_NULL;
    ev[i] = static_cast<hipEvent_t>(events[i]);
  }
  return forward_impl(dims, x, wts, logits_given, r, out, ws, ws_bytes, stream, ev,
                      SideMode::kLibrary, nullptr);
}

extern "C" const char* lmoe_path_name(const lmoe_dims* dims, int logits_given) {
  if (!dims || !dims_ok(*dims)) return "invalid";
  Plan p = make_plan(*dims);
  (void)logits_given;  // given logits take the same paths (published, not computed)
  if (p.fused_decode) return "fused_decode";
  if (p.fused_multi) return "fused_multi";
  return "grouped";
}

extern "C" const char* lmoe_stage_name(int stage) {
  static const char* names[LMOE_NUM_STAGE_EVENTS] = {
      "begin", "router", "topk", "permute", "gate_up", "down", "shared_gate_up",
      "shared_down", "combine"};
  return (stage >= 0 && stage < LMOE_NUM_STAGE_EVENTS) ? names[stage] : "?";
}

extern "C" int lmoe_debug_read_stream(const void* p, size_t bytes, uint32_t* sink,
                                     int32_t blocks, void* stream) {
  if (!p || !sink) return LMOE_ERR_NULL;
  if (bytes % 16 || blocks < 1 || blocks > 65536) return LMOE_ERR_SHAPE;
  if (!aligned16(p) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return LMOE_ERR_ALIGN;
  if (bytes == 0) return LMOE_OK;
  hipError_t e = launch_read_stream(p, bytes, sink, blocks, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LMOE_OK : LMOE_ERR_HIP;
}

extern "C" int lmoe_debug_mfma_rate(int32_t iters, uint32_t* sink, int32_t blocks, void* stream) {
  if (!sink) return LMOE_ERR_NULL;
  if (iters < 0 || blocks < 1 || blocks > 65536) return LMOE_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(sink) & 3u) return LMOE_ERR_ALIGN;
  hipError_t e = launch_mfma_rate(iters, sink, blocks, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LMOE_OK : LMOE_ERR_HIP;
}

extern "C" int lmoe_debug_quantize_act(const uint16_t* src, int32_t rows, int32_t K,
                                       int32_t act_format, uint8_t* codes, uint8_t* exps,
                                       void* stream) {
  if (rows < 0 || K <= 0 || K % 32) return LMOE_ERR_SHAPE;
  if (act_format != LMOE_ACT_E4M3 && act_format != LMOE_ACT_E2M1) return LMOE_ERR_SHAPE;
  if (rows == 0) return LMOE_OK;
  if (!src || !codes || !exps) return LMOE_ERR_NULL;
  if (!aligned16(src) || !aligned16(codes)) return LMOE_ERR_ALIGN;
  hipError_t e = launch_quantize_act(src, rows, K, act_format == LMOE_ACT_E4M3, codes, exps,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LMOE_OK : LMOE_ERR_HIP;
}

extern "C" int lmoe_debug_dequant_mxfp4(const uint8_t* q, const uint8_t* s, int32_t rows,
                                        int32_t K, uint16_t* out, void* stream) {
  if (rows < 0 || K <= 0 || K % 32) return LMOE_ERR_SHAPE;
  if (rows == 0) return LMOE_OK;
  if (!q || !s || !out) return LMOE_ERR_NULL;
  if (!aligned16(q) || !aligned16(out)) return LMOE_ERR_ALIGN;
  hipError_t e = launch_dequant(q, s, rows, K, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LMOE_OK : LMOE_ERR_HIP;
}

// ---------------------------------------------------------------------------
// The MoE block around the layer: input step, layer, tail (dense.hip).
// ---------------------------------------------------------------------------
namespace {

bool block_dims_ok(const lmoe_block_dims& b) {
  const lmoe_dims d = {b.T, b.L, b.E, b.k, b.I, 0, 0};
  if (!dims_ok(d)) return false;
  if (b.H < 64 || b.H > 16384 || b.H % 64) return false;
  if (b.L % 64 || b.E % 32) return false;
  if (b.S < 0 || b.S > 8) return false;
  if (b.S > 0 && (b.Is < 32 || b.Is > 16384 || b.Is % 32 || (b.S * b.Is) % 64)) return false;
  return true;
}

lmoe_dims layer_dims(const lmoe_block_dims& b) { return {b.T, b.L, b.E, b.k, b.I, 0, 0}; }

int block_shared(const lmoe_block_dims& b) { return b.S > 0 ? b.S * b.Is : 0; }

// Workspace of the block: the layer's own workspace first, then the block's
// buffers, then the K-split partial tiles (sized for the largest GEMM).
struct BlockWs {
  void* layer;
  size_t layer_bytes;
  float* logits;    // [T][E]
  uint16_t* x;      // [T][L]
  uint16_t* h_sh;   // [T][S*Is]
  uint16_t* routed; // [T][L]
  uint16_t* n;      // [T][L]
  uint16_t* sh;     // [T][H]
  float* part;
  size_t bytes;
};

BlockWs carve_block(const lmoe_block_dims& b, void* base) {
  BlockWs w = {};
  const lmoe_dims ld = layer_dims(b);
  w.layer_bytes = carve_workspace(make_plan(ld), nullptr).bytes;
  size_t off = 0;
  char* p = static_cast<char*>(base);
  auto take = [&](size_t bytes) -> char* {
    char* r = p ? p + off : nullptr;
    off = align_up(off + bytes, 256);
    return r;
  };
  const size_t T = b.T, SI = block_shared(b);
  w.layer = take(w.layer_bytes);
  w.logits = reinterpret_cast<float*>(take(T * b.E * 4));
  w.x = reinterpret_cast<uint16_t*>(take(T * b.L * 2));
  w.h_sh = reinterpret_cast<uint16_t*>(take(T * SI * 2));
  w.routed = reinterpret_cast<uint16_t*>(take(T * b.L * 2));
  w.n = reinterpret_cast<uint16_t*>(take(T * b.L * 2));
  w.sh = reinterpret_cast<uint16_t*>(take(T * (size_t)b.H * 2));
  // the input GEMM's partials, or the tail's two products' (in one launch)
  const size_t parts =
      std::max(dense_plan(b.T, b.E + b.L + 2 * (int)SI, b.H).part_floats,
               (SI ? dense_plan(b.T, b.H, (int)SI).part_floats : (size_t)0) +
                   dense_plan(b.T, b.H, b.L).part_floats);
  w.part = reinterpret_cast<float*>(take(std::max(parts, (size_t)1) * 4));
  w.bytes = off;
  return w;
}

int run_moe_input(const lmoe_block_dims& b, const uint16_t* u, const uint16_t* w_in,
                  float* logits, uint16_t* x, uint16_t* h_sh, const BlockWs& ws, hipStream_t s) {
  const int SI = block_shared(b);
  DenseArgs a = {};
  a.a = u;
  a.lda = b.H;
  a.b = w_in;
  a.ldb = b.H;
  a.M = b.T;
  a.N = b.E + b.L + 2 * SI;
  a.K = b.H;
  a.n_f32 = b.E;
  a.n_bf16 = b.L;
  a.f32_out = logits;
  a.ld_f32 = b.E;
  a.bf_out = x;
  a.ld_bf = b.L;
  a.glu_out = h_sh;
  a.ld_glu = SI;
  return launch_dense(a, dense_plan(a.M, a.N, a.K), ws.part, s) == hipSuccess ? LMOE_OK
                                                                              : LMOE_ERR_HIP;
}

int run_moe_tail(const lmoe_block_dims& b, const uint16_t* routed, const uint16_t* h_sh,
                 const uint16_t* norm_w, const uint16_t* w_up, const uint16_t* w_sd,
                 const uint16_t* residual, uint16_t* out, const BlockWs& ws, hipStream_t s) {
  const int SI = block_shared(b);
  if (launch_rmsnorm(routed, norm_w, b.T, b.L, 1e-6f, ws.n, s) != hipSuccess) return LMOE_ERR_HIP;
  const DensePlan pu = dense_plan(b.T, b.H, b.L);
  const DensePlan ps = SI ? dense_plan(b.T, b.H, SI) : pu;
  if (SI && pu.ksplit > 1 && ps.ksplit > 1) {
    // few tokens: both products K-split in one launch, one finishing pass
    // adds bf16(h_sh w_sd^T) and the residual to n w_up^T
    DenseArgs a = {};
    a.a = ws.n;
    a.lda = b.L;
    a.b = w_up;
    a.ldb = b.L;
    a.K = b.L;
    a.a2 = h_sh;
    a.lda2 = SI;
    a.b2 = w_sd;
    a.ldb2 = SI;
    a.K2 = SI;
    a.M = b.T;
    a.N = b.H;
    a.n_bf16 = b.H;
    a.bf_out = out;
    a.ld_bf = b.H;
    a.add1 = residual;
    a.ld_add = b.H;
    return launch_dense_pair(a, pu, ps, ws.part, s) == hipSuccess ? LMOE_OK : LMOE_ERR_HIP;
  }
  if (SI) {  // sh = bf16(h_sh w_sd^T)
    DenseArgs a = {};
    a.a = h_sh;
    a.lda = SI;
    a.b = w_sd;
    a.ldb = SI;
    a.M = b.T;
    a.N = b.H;
    a.K = SI;
    a.n_bf16 = b.H;
    a.bf_out = ws.sh;
    a.ld_bf = b.H;
    if (launch_dense(a, ps, ws.part, s) != hipSuccess) return LMOE_ERR_HIP;
  }
  DenseArgs a = {};  // out = bf16(n w_up^T + sh + residual)
  a.a = ws.n;
  a.lda = b.L;
  a.b = w_up;
  a.ldb = b.L;
  a.M = b.T;
  a.N = b.H;
  a.K = b.L;
  a.n_bf16 = b.H;
  a.bf_out = out;
  a.ld_bf = b.H;
  a.add0 = SI ? ws.sh : nullptr;
  a.add1 = residual;
  a.ld_add = b.H;
  return launch_dense(a, pu, ws.part, s) == hipSuccess ? LMOE_OK : LMOE_ERR_HIP;
}

}  // namespace

extern "C" size_t lmoe_block_workspace_bytes(const lmoe_block_dims* dims) {
  if (!dims || !block_dims_ok(*dims)) return 0;
  return carve_block(*dims, nullptr).bytes;
}

extern "C" int lmoe_moe_input(const lmoe_block_dims* dims, const uint16_t* u,
                              const uint16_t* w_in, float* logits, uint16_t* x, uint16_t* h_sh,
                              void* ws, size_t ws_bytes, void* stream) {
  if (!dims) return LMOE_ERR_NULL;
  if (!block_dims_ok(*dims)) return LMOE_ERR_SHAPE;
  if (dims->T == 0) return LMOE_OK;
  if (!u || !w_in || !logits || !x || !ws || (dims->S > 0 && !h_sh)) return LMOE_ERR_NULL;
  const void* ptrs[] = {u, w_in, logits, x, h_sh, ws};
  for (const void* q : ptrs)
    if (check_opt_ptr(q)) return LMOE_ERR_ALIGN;
  BlockWs w = carve_block(*dims, ws);
  if (ws_bytes < w.bytes) return LMOE_ERR_WORKSPACE;
  return run_moe_input(*dims, u, w_in, logits, x, h_sh, w, static_cast<hipStream_t>(stream));
}

extern "C" int lmoe_moe_tail(const lmoe_block_dims* dims, const uint16_t* routed,
                             const uint16_t* h_sh, const uint16_t* norm_w, const uint16_t* w_up,
                             const uint16_t* w_sd, const uint16_t* residual, uint16_t* out,
                             void* ws, size_t ws_bytes, void* stream) {
  if (!dims) return LMOE_ERR_NULL;
  if (!block_dims_ok(*dims)) return LMOE_ERR_SHAPE;
  if (dims->T == 0) return LMOE_OK;
  if (!routed || !norm_w || !w_up || !residual || !out || !ws) return LMOE_ERR_NULL;
  if (dims->S > 0 && (!h_sh || !w_sd)) return LMOE_ERR_NULL;
  const void* ptrs[] = {routed, h_sh, norm_w, w_up, w_sd, residual, out, ws};
  for (const void* q : ptrs)
    if (check_opt_ptr(q)) return LMOE_ERR_ALIGN;
  BlockWs w = carve_block(*dims, ws);
  if (ws_bytes < w.bytes) return LMOE_ERR_WORKSPACE;
  return run_moe_tail(*dims, routed, h_sh, norm_w, w_up, w_sd, residual, out, w,
                      static_cast<hipStream_t>(stream));
}

extern "C" int lmoe_block_forward(const lmoe_block_dims* dims, const uint16_t* u,
                                  const uint16_t* residual, const lmoe_block_weights* bw,
                                  const lmoe_weights* experts, const lmoe_routing* r,
                                  uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  if (!dims || !bw || !experts) return LMOE_ERR_NULL;
  if (!block_dims_ok(*dims)) return LMOE_ERR_SHAPE;
  if (dims->T == 0) return LMOE_OK;
  if (!u || !residual || !out || !ws || !bw->w_in || !bw->norm_w || !bw->w_up)
    return LMOE_ERR_NULL;
  if (dims->S > 0 && !bw->w_sd) return LMOE_ERR_NULL;
  const void* ptrs[] = {u, residual, out, ws, bw->w_in, bw->norm_w, bw->w_up, bw->w_sd};
  for (const void* q : ptrs)
    if (check_opt_ptr(q)) return LMOE_ERR_ALIGN;
  BlockWs w = carve_block(*dims, ws);
  if (ws_bytes < w.bytes) return LMOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the routing outputs the caller asked for; the logits are the input
  // step's, given to the layer
  lmoe_routing rr = {};
  if (r) rr = *r;
  if (!rr.logits) rr.logits = w.logits;
  int st = run_moe_input(*dims, u, bw->w_in, rr.logits, w.x, w.h_sh, w, s);
  if (st) return st;
  lmoe_weights lw = *experts;
  lw.router_w = nullptr;
  lw.sh_gate = lw.sh_up = lw.sh_down = nullptr;
  const lmoe_dims ld = layer_dims(*dims);
  st = forward_impl(&ld, w.x, &lw, 1, &rr, w.routed, w.layer, w.layer_bytes, stream, nullptr,
                    SideMode::kCaller, nullptr);
  if (st) return st;
  return run_moe_tail(*dims, w.routed, w.h_sh, bw->norm_w, bw->w_up, bw->w_sd, residual, out, w,
                      s);
}
