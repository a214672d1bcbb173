/*
 * lmoe.h — C ABI of the LatentMoE MXFP4 (w4a16) routed-expert layer on MI355X.
 *
 * The layer (dev48.org "Kimi K3 on AMD Instinct GPUs with TokenSpeed",
 * section 4 "Latent MoE"; infervisor.ai "Bringing up Kimi-K3 on day zero",
 * section "The model we hadn't run"): every token of a bf16 activation block
 * in the latent width L is scored by a router over E experts, sent to its k
 * best experts plus S always-on shared experts, and each expert applies a GLU
 * feed-forward network
 *     h = bf16( silu(x Gq^T) * (x Uq^T) ),   y = h Dq^T
 * whose routed weights are MXFP4: 4-bit E2M1 codes with one E8M0 exponent
 * (bias 127) per 32 consecutive values of a row. The output is
 *     out[t] = bf16( sum_j w[t,j] y_(t,j) + sum_s ysh_s[t] ).
 *
 * Conventions for every call:
 *  - Pointers marked "device" are HIP device pointers owned by the caller and
 *    must be 16-byte aligned; "host" pointers are read during the call only.
 *  - The library never allocates device memory, frees or synchronises.
 *    Temporary storage comes from the caller's workspace (see
 *    lmoe_workspace_bytes).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    default stream). Arguments are validated on the host before anything is
 *    enqueued: a non-zero status means nothing was launched.
 *  - lmoe_forward on the grouped path (lmoe_path_name) with shared experts runs the
 *    shared experts on a second stream of the current device, which the
 *    library creates with two events on its first such call: forked from
 *    `stream` by an event at the start and joined back to it before the
 *    combine, so the call is complete when `stream` has reached its end, as
 *    if all of it ran there. That stream is shared by every call on the
 *    device, so calls from different streams can wait on each other's
 *    shared-expert work (never on anything else). A call under stream
 *    capture pulls the second stream into the capture; calls on the device
 *    must not overlap one being captured. lmoe_forward_traced keeps every
 *    stage on `stream`.
 *  - Calls are re-entrant provided concurrent calls use distinct workspaces
 *    and outputs.
 *  - Results are deterministic: the same inputs give bit-identical outputs
 *    (no floating-point atomics anywhere).
 */
#ifndef LMOE_H_
#define LMOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  LMOE_OK = 0,
  LMOE_ERR_NULL = 1,      /* a required pointer is NULL */
  LMOE_ERR_SHAPE = 2,     /* dimensions violate the constraints below */
  LMOE_ERR_ALIGN = 3,     /* a device pointer is not 16-byte aligned */
  LMOE_ERR_WORKSPACE = 4, /* workspace smaller than lmoe_workspace_bytes() */
  LMOE_ERR_HIP = 5        /* a kernel launch failed */
};

/* Layer dimensions.
 *   T  tokens (T >= 0; T == 0 is a no-op)
 *   L  latent width: input of gate/up, output of down (L % 32 == 0, 32..16384)
 *   E  routed experts (1..1024)
 *   k  experts selected per token (1 <= k <= min(E, 32))
 *   I  routed-expert intermediate width (I % 32 == 0, 32..16384)
 *   S  shared experts (0..8)
 *   Is shared-expert intermediate width (Is % 32 == 0 when S > 0)
 * The Kimi-K3 LatentMoE has L = 3584, E = 896, k = 16, S = 2 (pages above).
 */
typedef struct lmoe_dims {
  int32_t T, L, E, k, I, S, Is;
} lmoe_dims;

/* Weights, all device pointers, row-major.
 *   router_w  bf16 [E][L]      router projection of the latent, one row per expert
 *   gate_q    uint8 [E][I][L/2]   E2M1 codes of the gate rows; element 2m of a
 *                                 row is the low nibble of byte m
 *   gate_s    uint8 [E][I][L/32]  E8M0 exponent of elements 32j..32j+31 of a
 *                                 row; value = E2M1(code) * 2^(byte - 127),
 *                                 byte 255 is NaN
 *   up_q, up_s      same layout as gate
 *   down_q    uint8 [E][L][I/2], down_s uint8 [E][L][I/32]
 *   sh_gate, sh_up  bf16 [S][Is][L];  sh_down bf16 [S][L][Is]
 * The per-32 exponent along the input dimension is the checkpoint format
 * described in huggingface.co "Notes from an NVFP4 port of Kimi K3.1 Pro"
 * (introduction). router_w may be NULL when logits are given. The shared
 * pointers may be NULL when S == 0.
 */
typedef struct lmoe_weights {
  const uint16_t* router_w;
  const uint8_t* gate_q;
  const uint8_t* gate_s;
  const uint8_t* up_q;
  const uint8_t* up_s;
  const uint8_t* down_q;
  const uint8_t* down_s;
  const uint16_t* sh_gate;
  const uint16_t* sh_up;
  const uint16_t* sh_down;
} lmoe_weights;

/* Routing results, all device pointers; any member may be NULL, in which case
 * the value lives only in the workspace.
 *   logits    float [T][E]  router logits. INPUT when logits_given != 0 (then
 *                           required), otherwise written if non-NULL.
 *   topk_idx  int32 [T][k]  selected experts of each token, ordered by
 *                           descending logit, equal logits by ascending expert
 *                           index (NaN ranks below -inf, -0 equals +0)
 *   topk_w    float [T][k]  softmax over the selected logits
 *   counts    int32 [E]     routes per expert
 *   offsets   int32 [E+1]   exclusive prefix sum of counts (offsets[E] = T*k)
 *   perm      int32 [T*k]   perm[pos] = route r = t*k + j, routes grouped by
 *                           expert and stable in r
 *   inv_perm  int32 [T*k]   inv_perm[r] = pos
 * Selection is the exact top-k of the fp32 logits (the tie rule mirrors the
 * boundary rule of huggingface.co "Notes from an NVFP4 port of Kimi K3.1 Pro",
 * "Details that silently change the answer" (4)); grouping routes by expert so
 * that one weight panel serves several routes follows TokenSpeed section 4.1.
 */
typedef struct lmoe_routing {
  float* logits;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv_perm;
} lmoe_routing;

/* Size of the counter block at the start of every workspace: the dependency
 * counters of the persistent decode kernels (1 to 16 tokens). */
#define LMOE_COUNTER_BYTES ((size_t)256 << 10)

/* Largest weight stream (bytes of min(E, T k) routed experts plus the shared
 * experts and router) for which lmoe_forward takes the fused multi-token
 * kernel; measured on the Kimi-K3 layer, the fused kernel is faster at
 * T = 2 (374 MB) and even at T = 4 (836 MB), slower from T = 8. */
#define LMOE_FUSED_MULTI_BYTES ((size_t)800 << 20)

/* Bytes of device workspace lmoe_route / lmoe_forward need for these
 * dimensions (the same value serves every entry point and option, the
 * quantised activations of lmoe_exec.act_format included). Returns 0 for
 * invalid dims.
 * The workspace must be zero-filled before its first use; every call leaves
 * its first LMOE_COUNTER_BYTES (the decode kernels' dependency counters)
 * zeroed again, so a workspace can be reused across calls and dimensions.
 * After lmoe_wait_errors reports an abandoned wait, zero that block again. */
size_t lmoe_workspace_bytes(const lmoe_dims* dims);

/* Routing only: router logits (unless logits_given), top-k selection with
 * softmax weights, and the expert grouping (counts, offsets, perm, inv_perm).
 * The router scores every expert from the MoE input in one projection
 * (dev48.org "Kimi K3 on AMD Instinct GPUs with TokenSpeed", section 4.3; here
 * from the latent x), each token keeps its k best of E (k = 16 of 896 in
 * infervisor.ai "Bringing up Kimi-K3 on day zero", "The model we hadn't run"),
 * and routes are grouped by expert, stable in route order, so that one weight
 * panel serves every route of an expert (TokenSpeed section 4.1).
 *   dims      host; x bf16 [T][L] device (may be NULL if logits_given)
 *   router_w  bf16 [E][L] device (ignored if logits_given)
 *   r         host struct of device pointers (may be NULL: nothing returned)
 *   ws        device workspace of ws_bytes >= lmoe_workspace_bytes(dims)
 * Errors: LMOE_ERR_NULL, _SHAPE, _ALIGN, _WORKSPACE, _HIP. */
int lmoe_route(const lmoe_dims* dims, const uint16_t* x, const uint16_t* router_w,
               int logits_given, const lmoe_routing* r, void* ws, size_t ws_bytes,
               void* stream);

/* The whole layer: routing, routed experts, shared experts and combine: the
 * Latent MoE of dev48.org "Kimi K3 on AMD Instinct GPUs with TokenSpeed",
 * section 4 (k of E routed MXFP4 experts plus S always-on shared experts in
 * the latent width), with route partials kept and summed in FP32 (section
 * 4.3) and the MXFP4 format of infervisor.ai "Bringing up Kimi-K3 on day
 * zero", "The model we hadn't run".
 *   x    bf16 [T][L] device;  w  host struct of device weight pointers
 *   r    optional routing outputs (see lmoe_routing); when logits_given,
 *        r->logits is the input logits and r must not be NULL
 *   out  bf16 [T][L] device, written with the combined output
 *   ws   device workspace of ws_bytes >= lmoe_workspace_bytes(dims)
 * On the grouped path with S > 0 the shared experts run on the library's
 * per-device second stream (see the conventions above); lmoe_forward_ex lets
 * the caller choose.
 * Errors: LMOE_ERR_NULL, _SHAPE, _ALIGN, _WORKSPACE, _HIP. */
int lmoe_forward(const lmoe_dims* dims, const uint16_t* x, const lmoe_weights* w,
                 int logits_given, const lmoe_routing* r, uint16_t* out, void* ws,
                 size_t ws_bytes, void* stream);

/* Where lmoe_forward_ex runs the shared experts. They read only x, so on the
 * grouped path they can run beside the routing and the routed GEMMs.
 *   side_stream  hipStream_t for the shared experts, or NULL: every stage on
 *                the call's stream
 *   fork_event   hipEvent_t (created by the caller, timing may be disabled):
 *                recorded on the call's stream at the start; side_stream waits
 *                for it before the shared experts
 *   join_event   hipEvent_t: recorded on side_stream after the shared
 *                experts; the call's stream waits for it before the combine
 * The events are re-recorded by every call that names them: calls sharing
 * them must not be enqueued concurrently from different host threads. The
 * call is complete when its own stream has reached its end. */
typedef struct lmoe_exec {
  void* side_stream;
  void* fork_event;
  void* join_event;
  /* NULL, or LMOE_NUM_STAGE_EVENTS caller-created hipEvent_t recorded at the
   * stage boundaries as lmoe_forward_traced does; every stage then runs on
   * the call's stream and side_stream is not used */
  void* const* stage_events;
  /* LMOE_PATH_AUTO (0): the implementation lmoe_path_name reports;
   * LMOE_PATH_GROUPED: the grouped kernels whatever T;
   * LMOE_PATH_FUSED: a fused decode kernel wherever its limits allow one
   * (lmoe_path_name's conditions without the byte threshold), else grouped;
   * any other value is LMOE_ERR_SHAPE */
  int32_t path;
  /* The routed experts' activation precision. LMOE_ACT_BF16 (0): bf16
   * activations (w4a16, the layer's reference numerics). LMOE_ACT_E4M3 and
   * LMOE_ACT_E2M1: the routed GEMMs' inputs (each token's row for gate/up, h
   * after its bf16 rounding for down) quantised to FP8 E4M3 or FP4 E2M1
   * elements with one E8M0 scale per 32 values along K, and multiplied with
   * the MXFP4 weights on gfx950's scaled MFMA. dev48.org "Kimi K3 on AMD
   * Instinct GPUs with TokenSpeed", precision table, row "Routed-expert
   * GEMMs": FP8/MXFP4 for small decode, MXFP4/MXFP4 for prefill; the pages
   * give no activation scale granularity, the weights' MX scheme is taken:
   * scale exponent floor(log2 max|v|) - emax (8 for E4M3, 2 for E2M1),
   * elements rounded to nearest, ties to the even code, saturating at 448 /
   * 6. The shared experts and the router stay bf16. Only with
   * lmoe_forward_packed and L, I multiples of 128 (else LMOE_ERR_SHAPE). */
  int32_t act_format;
} lmoe_exec;

enum { LMOE_PATH_AUTO = 0, LMOE_PATH_GROUPED = 1, LMOE_PATH_FUSED = 2 };
enum { LMOE_ACT_BF16 = 0, LMOE_ACT_E4M3 = 1, LMOE_ACT_E2M1 = 2 };

/* lmoe_forward with the shared experts' stream chosen by the caller instead
 * of the library's per-device second stream: exec NULL (or its side_stream
 * NULL) runs every stage on `stream`, and the library then creates no stream
 * or event of its own. The decode paths (lmoe_path_name "fused_decode"
 * and "fused_multi") are one kernel on `stream` whatever exec says. Same
 * arguments, results and errors as lmoe_forward, plus LMOE_ERR_NULL when
 * exec->side_stream is set and an event is missing. */
int lmoe_forward_ex(const lmoe_dims* dims, const uint16_t* x, const lmoe_weights* w,
                    int logits_given, const lmoe_routing* r, uint16_t* out, void* ws,
                    size_t ws_bytes, void* stream, const lmoe_exec* exec);

/* The decode kernels (1 to 16 tokens) resolve their dependencies with bounded
 * waits on device counters in the workspace; a wait that outlives its bound
 * (about a quarter of a second: a producer that never ran) is abandoned and
 * counted in the workspace, and that call's output is then not valid. This
 * enqueues on
 * `stream` a copy of that count into *count (int32 device, 4-byte aligned)
 * and resets it to zero, with no host synchronisation: a caller that reads 0
 * after its calls knows no wait was abandoned in them. The count accumulates
 * over calls on one workspace until read.
 *   ws  the workspace of those calls (ws_bytes >= LMOE_COUNTER_BYTES)
 * Errors: LMOE_ERR_NULL, _ALIGN, _WORKSPACE, _HIP. */
int lmoe_wait_errors(void* ws, size_t ws_bytes, int32_t* count, void* stream);

/* ---------------------------------------------------------------------------
 * Tile-packed routed experts. The checkpoint's MXFP4 matrices, repacked once
 * (as the MXFP4 experts are repacked at load time in huggingface.co "Notes
 * from an NVFP4 port of Kimi K3.1 Pro", introduction) into the order the
 * grouped 32x32x16-MFMA GEMMs read: every 64-lane load instruction then reads
 * 1 KB contiguous. Codes and exponents are the same bytes, reordered, so the
 * layer's results are the same as from the row-major layout.
 *
 * A packed matrix of N rows and K values per row (K % 32 == 0) has
 * N32 = ceil(N/32) tiles of 32 rows, K128 = ceil(K/128) chunks and
 * K512 = ceil(K/512) exponent windows; per expert, in that order:
 *   codes      [N32][K128][2][64][16] bytes: the 16 bytes of lane l, half j
 *              of chunk c of tile n are the codes of row 32n + l%32, MX block
 *              4c + 2(l/32) + j (32 values, element 2m in the low nibble of
 *              byte m)
 *   exponents  [N32][K512][64][8] bytes: byte b of lane l in window w of tile
 *              n is the E8M0 exponent of row 32n + l%32, block
 *              4(4w + b/2) + 2(l/32) + b%2
 * Rows and blocks past the matrix hold code 0 and exponent 127.
 * gu: the gate and up matrices of an expert as one matrix of N = 2I rows and
 *     K = L: tile n holds gate rows 16n .. 16n+15, then up rows 16n .. 16n+15.
 * down: the down matrix, N = L, K = I.
 * --------------------------------------------------------------------------- */
typedef struct lmoe_packed_sizes {
  size_t gu_q, gu_s, down_q, down_s;  /* bytes over all E experts */
} lmoe_packed_sizes;

/* Bytes of each packed array for these dims (host).
 * Errors: LMOE_ERR_NULL, _SHAPE. */
int lmoe_packed_sizes_of(const lmoe_dims* dims, lmoe_packed_sizes* sizes);

/* Repack the routed experts of w (row-major, as lmoe_weights; router and
 * shared pointers are not read) into the caller's device arrays gu_q, gu_s,
 * down_q, down_s of lmoe_packed_sizes_of bytes. Asynchronous on `stream`;
 * the sources must stay valid until it completes.
 * Errors: LMOE_ERR_NULL, _SHAPE, _ALIGN, _HIP. */
int lmoe_pack_weights(const lmoe_dims* dims, const lmoe_weights* w, uint8_t* gu_q,
                      uint8_t* gu_s, uint8_t* down_q, uint8_t* down_s, void* stream);

/* The layer's weights with the routed experts tile-packed. */
typedef struct lmoe_packed_weights {
  const uint16_t* router_w;  /* bf16 [E][L], as lmoe_weights */
  const uint8_t* gu_q;       /* packed gate/up codes and exponents */
  const uint8_t* gu_s;
  const uint8_t* down_q;     /* packed down codes and exponents */
  const uint8_t* down_s;
  const uint16_t* sh_gate;   /* as lmoe_weights */
  const uint16_t* sh_up;
  const uint16_t* sh_down;
} lmoe_packed_weights;

/* lmoe_forward_ex on tile-packed routed experts: the same layer and results
 * (up to the order of fp32 sums), with the routed GEMMs on 32x32x16 bf16
 * MFMA over expert groups of up to 128 routes. Every token count runs the
 * grouped path (routing kernels, grouped GEMMs, combine). exec as in
 * lmoe_forward_ex (NULL: every stage on `stream`). The workspace is the one
 * lmoe_workspace_bytes gives. T * L and T * k * I must stay below 2^31
 * (LMOE_ERR_SHAPE otherwise; 65536 tokens at the Kimi-K3 widths).
 * Errors: as lmoe_forward_ex. */
int lmoe_forward_packed(const lmoe_dims* dims, const uint16_t* x, const lmoe_packed_weights* w,
                        int logits_given, const lmoe_routing* r, uint16_t* out, void* ws,
                        size_t ws_bytes, void* stream, const lmoe_exec* exec);

/* ---- The MoE block around the layer ----
 * In Kimi-K3 the layer sits inside a block (dev48.org "Kimi K3 on AMD
 * Instinct GPUs with TokenSpeed", sections 4.2-4.4 and 6): one packed
 * projection of the normalised hidden input u gives the router scores, the
 * routed experts' latent input and the shared experts' gate/up values, the
 * shared activation applied in its epilogue (section 4.3); the routed layer
 * runs in the latent; the tail RMS-normalises the routed result, projects it
 * up to the hidden width and adds the shared experts' output and the running
 * residual (sections 4.2, 4.3 and 6). Here the shared experts read u and
 * write the hidden width, as in K3; the layer inside has none of its own.
 *
 * Block dimensions: T, L, E, k, I as lmoe_dims, and
 *   H   hidden width (H % 64 == 0, 64..16384)
 *   S   shared experts (0..8), Is their intermediate width (Is % 32 == 0 and
 *       S * Is % 64 == 0 when S > 0)
 * with also L % 64 == 0 and E % 32 == 0. Kimi-K3: H = 7168. */
typedef struct lmoe_block_dims {
  int32_t T, H, L, E, k, I, S, Is;
} lmoe_block_dims;

/* The block's own weights, bf16 device pointers, row-major:
 *   w_in    [E + L + 2*S*Is][H]  the three input projections one after another
 *           (section 4.3): E router rows, L rows of the hidden -> latent
 *           projection, then for each shared expert s its gate and up rows
 *           interleaved in groups of 16: row E + L + 2*Is*s + 32*j + c is
 *           gate row 16*j + c for c < 16 and up row 16*j + c - 16 otherwise
 *   norm_w  [L]        weight of the routed RMSNorm
 *   w_up    [H][L]     latent -> hidden up-projection
 *   w_sd    [H][S*Is]  the shared experts' down projections side by side
 *                      along the input dimension (NULL when S == 0) */
typedef struct lmoe_block_weights {
  const uint16_t* w_in;
  const uint16_t* norm_w;
  const uint16_t* w_up;
  const uint16_t* w_sd;
} lmoe_block_weights;

/* Workspace bytes for lmoe_moe_input, lmoe_moe_tail and lmoe_block_forward
 * (0 for invalid dims). It must be zero-filled before its first use, as the
 * layer's (it contains one). */
size_t lmoe_block_workspace_bytes(const lmoe_block_dims* dims);

/* The MoE input step (TokenSpeed section 4.3): z = u W_in^T in one GEMM,
 * accumulated in fp32, with
 *   logits float [T][E]     = z's router columns
 *   x      bf16 [T][L]      = bf16(z's latent columns)
 *   h_sh   bf16 [T][S*Is]   = bf16(silu(g) * v) for each shared expert's
 *                             gate and up columns g, v (NULL when S == 0)
 * u bf16 [T][H]. All device pointers. Errors: LMOE_ERR_NULL, _SHAPE, _ALIGN,
 * _WORKSPACE, _HIP. */
int lmoe_moe_input(const lmoe_block_dims* dims, const uint16_t* u, const uint16_t* w_in,
                   float* logits, uint16_t* x, uint16_t* h_sh, void* ws, size_t ws_bytes,
                   void* stream);

/* The MoE tail (sections 4.2, 4.3 and 6): with the routed result routed
 * bf16 [T][L], the shared activations h_sh bf16 [T][S*Is] and the residual
 * bf16 [T][H],
 *   n   = bf16(routed * (1 / sqrt(mean(routed^2) + 1e-6)) * norm_w), fp32 inside
 *   sh  = bf16(h_sh w_sd^T)                    (zero when S == 0)
 *   out = bf16(n w_up^T + sh + residual)       bf16 [T][H]
 * All device pointers. Errors: as lmoe_moe_input. */
int lmoe_moe_tail(const lmoe_block_dims* dims, const uint16_t* routed, const uint16_t* h_sh,
                  const uint16_t* norm_w, const uint16_t* w_up, const uint16_t* w_sd,
                  const uint16_t* residual, uint16_t* out, void* ws, size_t ws_bytes,
                  void* stream);

/* The whole block: lmoe_moe_input, then the layer (lmoe_forward with the
 * input step's logits given, no shared experts of its own) on the latent
 * rows with the routed experts of `experts` (lmoe_weights' layout; its
 * router and shared members are ignored), then lmoe_moe_tail; out bf16
 * [T][H]. r: optional routing outputs as lmoe_forward's; here r->logits,
 * when non-NULL, receives the input step's router scores. Every kernel runs
 * on `stream`. Errors: as lmoe_moe_input. */
int lmoe_block_forward(const lmoe_block_dims* dims, const uint16_t* u, const uint16_t* residual,
                       const lmoe_block_weights* bw, const lmoe_weights* experts,
                       const lmoe_routing* r, uint16_t* out, void* ws, size_t ws_bytes,
                       void* stream);

/* Size of the device scratch lmoe_forward_noalloc uses: one static array per
 * GPU, held from the library's first such call on that GPU until the process
 * ends. */
#define LMOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* lmoe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same layer and results, with the workspace taken from a static device array
 * of LMOE_NOALLOC_SCRATCH_BYTES on the current GPU instead of a caller
 * buffer. The call allocates nothing (no hipMalloc, hipFree, stream or event
 * creation; every stage runs on `stream`); its first call on a GPU looks up
 * that GPU's array and clears the part that must start at zero.
 * Every call on one GPU shares that array, which keeps the last call's
 * contents: calls that overlap on one GPU (different streams or threads)
 * race and must be serialised by the caller.
 * Arguments, results and errors as lmoe_forward, plus LMOE_ERR_WORKSPACE when
 * lmoe_workspace_bytes(dims) exceeds LMOE_NOALLOC_SCRATCH_BYTES (at the
 * Kimi-K3 widths: up to about 150 tokens). */
int lmoe_forward_noalloc(const lmoe_dims* dims, const uint16_t* x, const lmoe_weights* w,
                         int logits_given, const lmoe_routing* r, uint16_t* out, void* stream);

/* Stage boundaries recorded by lmoe_forward_traced. Event i is recorded on
 * the stream right after stage i has been enqueued (event 0 before the first
 * one); a stage that does not run for these arguments (the router when logits
 * are given, the shared experts when S == 0) records its event right after the
 * previous one. Stage i's time is the elapsed time between events i-1 and i.
 * When one kernel runs several stages (the single-token decode path, see
 * lmoe_path_name), all their events are recorded after it, so its whole time
 * is attributed to the first of them.
 * Per-stage attribution follows the per-opcode rate attribution of
 * infervisor.ai "Bringing up Kimi-K3 on day zero", "The 28.9 ms, taken apart". */
enum {
  LMOE_STAGE_BEGIN = 0,
  LMOE_STAGE_ROUTER = 1,
  LMOE_STAGE_TOPK = 2,
  LMOE_STAGE_PERMUTE = 3,
  LMOE_STAGE_GATEUP = 4,
  LMOE_STAGE_DOWN = 5,
  LMOE_STAGE_SHARED_GATEUP = 6,
  LMOE_STAGE_SHARED_DOWN = 7,
  LMOE_STAGE_COMBINE = 8,
  LMOE_NUM_STAGE_EVENTS = 9
};

/* lmoe_forward, additionally recording the LMOE_NUM_STAGE_EVENTS events
 * (hipEvent_t handles created by the caller, host array `events`) at the stage
 * boundaries above. Same arguments, results and errors as lmoe_forward, plus
 * LMOE_ERR_NULL when events or any of its entries is NULL. */
int lmoe_forward_traced(const lmoe_dims* dims, const uint16_t* x, const lmoe_weights* w,
                        int logits_given, const lmoe_routing* r, uint16_t* out, void* ws,
                        size_t ws_bytes, void* stream, void* const* events);

/* Short name of stage i (0 <= i < LMOE_NUM_STAGE_EVENTS), else "?". */
const char* lmoe_stage_name(int stage);

/* Which implementation lmoe_forward uses for these dimensions (static
 * string): "fused_decode" (T == 1 with computed logits and L, I, Is at
 * most 4096: the whole layer in one persistent kernel), "fused_multi"
 * (2 <= T <= 16 with computed logits, T * k <= 256, the same widths, and at
 * most LMOE_FUSED_MULTI_BYTES of weights for min(E, T k) experts plus the
 * shared ones: one persistent kernel with one token per MFMA row, each
 * selected expert streamed once for all the tokens that chose it; beyond
 * that size the grouped kernels stream the weights faster), "grouped"
 * (routing kernels, then grouped GEMMs over expert groups of up to 96 rows,
 * then the combine), "invalid" for bad dims. Decode streams the active weights once
 * per step (infervisor.ai "Bringing up Kimi-K3 on day zero", "The
 * roofline"); small batches walk their tokens' routes directly and the
 * grouped form follows the expert-sorted tiling of dev48.org "Kimi K3 on AMD
 * Instinct GPUs with TokenSpeed", section 4.1. lmoe_forward_packed always
 * takes the grouped form. */
const char* lmoe_path_name(const lmoe_dims* dims, int logits_given);

/* Test hook: dequantise an MXFP4 matrix with the same device routine the
 * expert kernels use.
 *   q    uint8 [rows][K/2] device codes;  s  uint8 [rows][K/32] device exponents
 *   out  bf16 [rows][K] device
 * K % 32 == 0, rows >= 0. Errors: LMOE_ERR_NULL, _SHAPE, _ALIGN, _HIP. */
int lmoe_debug_dequant_mxfp4(const uint8_t* q, const uint8_t* s, int32_t rows, int32_t K,
                             uint16_t* out, void* stream);

/* Test hook: quantise a bf16 matrix with the device routine the quantised
 * activation path uses (lmoe_exec.act_format).
 *   src    bf16 [rows][K] device;  act_format LMOE_ACT_E4M3 or LMOE_ACT_E2M1
 *   codes  E4M3: u8 [rows][K]; E2M1: u8 [rows][K/2], element 2m in the low
 *          nibble of byte m (device)
 *   exps   u8 [rows][K/32] E8M0 (device)
 * K % 32 == 0, rows >= 0. Errors: LMOE_ERR_NULL, _SHAPE, _ALIGN, _HIP. */
int lmoe_debug_quantize_act(const uint16_t* src, int32_t rows, int32_t K, int32_t act_format,
                            uint8_t* codes, uint8_t* exps, void* stream);

/* Measurement hook: read every byte of p (device, 16-byte aligned, bytes a
 * multiple of 16) once with 16-byte loads from `blocks` workgroups of 256
 * threads striding over it, and write one word per workgroup to sink
 * (uint32 [blocks] device). The plain HBM read rate this reaches is the
 * ceiling the HBM-bound decode kernel is measured against (infervisor.ai
 * "Bringing up Kimi-K3 on day zero", "The roofline": batch-1 decode is bound
 * by weight bytes). Errors: LMOE_ERR_NULL, _SHAPE (blocks outside 1..65536),
 * _ALIGN, _HIP. */
int lmoe_debug_read_stream(const void* p, size_t bytes, uint32_t* sink, int32_t blocks,
                           void* stream);

/* Measurement hook: `blocks` workgroups of four waves each run `iters`
 * rounds of eight independent 32x32x16 bf16 MFMAs (32768 flops each) on
 * register operands and write one word per workgroup to sink (uint32
 * [blocks] device). blocks * 4 * iters * 8 * 32768 flops over the launch's
 * duration is the bf16 MFMA rate this GPU sustains under full load: the
 * practical ceiling the prefill GEMMs are measured against next to the
 * 2.5 PFLOP/s figure (dev48.org "Kimi K3 on AMD Instinct GPUs with
 * TokenSpeed", section 4.4: at prefill sizes the layer is bound by the
 * matrix cores). Errors: LMOE_ERR_NULL, _SHAPE (iters < 0, blocks outside
 * 1..65536), _ALIGN, _HIP. */
int lmoe_debug_mfma_rate(int32_t iters, uint32_t* sink, int32_t blocks, void* stream);

/* Human-readable name of a status code (static string). */
const char* lmoe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* LMOE_H_ */
