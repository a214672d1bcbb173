// Tile-packed MXFP4 experts: a one-time repack of the checkpoint's MXFP4
// matrices into the order in which the grouped GEMMs read them, and those
// GEMMs on 32x32x16 bf16 MFMA.
//
// The checkpoint keeps each expert matrix row-major with the E8M0 exponent
// running along K (huggingface.co "Notes from an NVFP4 port of Kimi K3.1 Pro",
// introduction, which likewise repacks the experts once at load time). A wave
// of the GEMMs multiplies a 32-row weight tile: lane l supplies row l % 32 and
// the K values 8 (l / 32) .. +7 of each MFMA step. Read from the row-major
// layout, one 16-byte load per lane then touches 32 rows per instruction;
// packed, every load instruction reads 1 KB contiguous and every exponent
// load 512 bytes contiguous. The values are untouched: the same E2M1 codes
// and E8M0 bytes, reordered (layout in include/lmoe.h, lmoe_pack_weights).
//
// Gate and up are interleaved in one packed matrix GU of 2I rows: packed
// tile n holds gate rows 16n .. 16n+15 then up rows 16n .. 16n+15, so one
// MFMA output tile carries g and u of the same 16 intermediate columns (with
// the weights as operand A, in slots i and i + 8 of the same lane).
//
// Per expert e and route r of token t (dev48.org "Kimi K3 on AMD Instinct GPUs
// with TokenSpeed", section 4): h_r = bf16(silu(x_t Gq_e^T) * (x_t Uq_e^T)),
// y_r = h_r Dq_e^T in fp32 (route partials summed in FP32, section 4.3).
#include "lmoe_device.h"
#include "lmoe_internal.h"

namespace lmoe {

// ---------------------------------------------------------------------------
// Pack kernels
// ---------------------------------------------------------------------------
struct PackSrc {
  const uint8_t* q0;  // matrix rows [N0][K/2]; GU: gate
  const uint8_t* s0;  //             [N0][K/32]
  const uint8_t* q1;  // GU: up (nullptr for a plain matrix)
  const uint8_t* s1;
  int64_t q_estride, s_estride;  // bytes per expert of q0 / s0 (and q1 / s1)
  int N;                         // packed rows (GU: 2 I)
  int K;
  bool gu;
};

// Source row of packed row p: plain p; GU tile n = p / 32 holds gate rows
// 16 n .. 16 n + 15, then up rows 16 n .. 16 n + 15.
__device__ __forceinline__ void packed_source(const PackSrc& a, int e, int p, const uint8_t** q,
                                              const uint8_t** s) {
  int row = p, m = 0;
  if (a.gu) {
    const int n = p >> 5, r = p & 31;
    m = r >> 4;
    row = 16 * n + (r & 15);
  }
  const int64_t qrow = (int64_t)row * (a.K / 2), srow = (int64_t)row * (a.K / 32);
  *q = (m ? a.q1 : a.q0) + e * a.q_estride + qrow;
  *s = (m ? a.s1 : a.s0) + e * a.s_estride + srow;
}

// One thread per 16 bytes of packed codes: expert e, tile n, chunk c, half j,
// lane l <- codes of packed row 32 n + l % 32, MX block 4 c + 2 (l / 32) + j.
__global__ __launch_bounds__(256) void pack_codes_kernel(PackSrc a, int E, uint8_t* __restrict__ dst) {
  const int N32 = (a.N + 31) / 32, K128 = (a.K + 127) / 128, nblk = a.K / 32;
  const int64_t units = (int64_t)E * N32 * K128 * 128;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const int l = (int)(u & 63);
  const int j = (int)((u >> 6) & 1);
  int64_t rest = u >> 7;
  const int c = (int)(rest % K128);
  rest /= K128;
  const int n = (int)(rest % N32);
  const int e = (int)(rest / N32);
  const int p = 32 * n + (l & 31);
  const int blk = 4 * c + 2 * (l >> 5) + j;
  u32x4_t v = zero16();
  if (p < a.N && blk < nblk) {
    const uint8_t *q, *s;
    packed_source(a, e, p, &q, &s);
    v = load16(q + blk * 16);
  }
  *reinterpret_cast<u32x4_t*>(dst + u * 16) = v;
}

// One thread per 8 bytes of packed exponents: expert e, tile n, window w of
// four chunks, lane l <- byte b = exponent of packed row 32 n + l % 32, block
// 4 (4 w + b / 2) + 2 (l / 32) + b % 2; 127 (a scale of 1) past the end.
__global__ __launch_bounds__(256) void pack_scales_kernel(PackSrc a, int E, uint8_t* __restrict__ dst) {
  const int N32 = (a.N + 31) / 32, K512 = (a.K + 511) / 512, nblk = a.K / 32;
  const int64_t units = (int64_t)E * N32 * K512 * 64;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const int l = (int)(u & 63);
  int64_t rest = u >> 6;
  const int w = (int)(rest % K512);
  rest /= K512;
  const int n = (int)(rest % N32);
  const int e = (int)(rest / N32);
  const int p = 32 * n + (l & 31);
  uint32_t lo = 0, hi = 0;
  const uint8_t *q = nullptr, *s = nullptr;
  if (p < a.N) packed_source(a, e, p, &q, &s);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int blk = 4 * (4 * w + b / 2) + 2 * (l >> 5) + (b & 1);
    const uint32_t v = (p < a.N && blk < nblk) ? s[blk] : 127u;
    if (b < 4)
      lo |= v << (8 * b);
    else
      hi |= v << (8 * (b - 4));
  }
  *reinterpret_cast<uint2*>(dst + u * 8) = make_uint2(lo, hi);
}

PackedSizes packed_sizes(const lmoe_dims& d) {
  PackedSizes z;
  const int64_t gu32 = (2 * (int64_t)d.I + 31) / 32, dn32 = ((int64_t)d.L + 31) / 32;
  z.gu_q = (size_t)d.E * gu32 * ((d.L + 127) / 128) * 2048;
  z.gu_s = (size_t)d.E * gu32 * ((d.L + 511) / 512) * 512;
  z.down_q = (size_t)d.E * dn32 * ((d.I + 127) / 128) * 2048;
  z.down_s = (size_t)d.E * dn32 * ((d.I + 511) / 512) * 512;
  return z;
}

hipError_t launch_pack(const lmoe_dims& d, const lmoe_weights& w, uint8_t* gu_q, uint8_t* gu_s,
                       uint8_t* dn_q, uint8_t* dn_s, hipStream_t st) {
  PackSrc g = {};
  g.q0 = w.gate_q;
  g.s0 = w.gate_s;
  g.q1 = w.up_q;
  g.s1 = w.up_s;
  g.q_estride = (int64_t)d.I * d.L / 2;
  g.s_estride = (int64_t)d.I * d.L / 32;
  g.N = 2 * d.I;
  g.K = d.L;
  g.gu = true;
  PackSrc dn = {};
  dn.q0 = w.down_q;
  dn.s0 = w.down_s;
  dn.q_estride = (int64_t)d.L * d.I / 2;
  dn.s_estride = (int64_t)d.L * d.I / 32;
  dn.N = d.L;
  dn.K = d.I;
  dn.gu = false;
  const PackSrc* srcs[2] = {&g, &dn};
  uint8_t* qd[2] = {gu_q, dn_q};
  uint8_t* sd[2] = {gu_s, dn_s};
  for (int i = 0; i < 2; ++i) {
    const PackSrc& a = *srcs[i];
    const int64_t N32 = (a.N + 31) / 32;
    const int64_t cu = (int64_t)d.E * N32 * ((a.K + 127) / 128) * 128;
    hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)((cu + 255) / 256)), dim3(256), 0, st, a,
                       d.E, qd[i]);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t su = (int64_t)d.E * N32 * ((a.K + 511) / 512) * 64;
    hipLaunchKernelGGL(pack_scales_kernel, dim3((unsigned)((su + 255) / 256)), dim3(256), 0, st,
                       a, d.E, sd[i]);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Grouped GEMM over packed weights: 32x32x16 bf16 MFMA.
//
// A workgroup covers one row tile of up to 96 routes of one expert (three
// 32-row MFMA tiles) and eight packed 32-row weight tiles: gate/up 128
// intermediate columns, down 256 output columns. Each of its four waves owns
// two weight tiles over every row tile. K runs in chunks of 128 values: the
// chunk's activation rows are copied into LDS by 16-byte global-to-LDS loads
// (no registers), segments XOR-swizzled by row so the MFMA operand reads of
// 16 rows hit distinct banks; the chunk's weights (two 1 KB loads per tile)
// are loaded into registers two chunks ahead; three LDS buffers and one
// barrier per chunk. Lane (r, h) = (l % 32, l / 32) takes, in chunk c, MX
// blocks 4c + 2h and 4c + 2h + 1 (the packed order), so the activation
// operand of MFMA step (j, m) is segment 8h + 4j + m of the chunk row. The
// operand layouts of A and B are alike (lane l: row or column l % 32, K
// 8 (l / 32) .. + 7 of the step), so either side can take the weights: the
// down GEMM puts the routes in A (each lane stores two whole 128-byte lines
// of fp32 y per instruction), the gate/up GEMM the weights in A (each lane
// holds one route's gates and ups). Exponents come one 4-byte load per tile
// per chunk.
// ---------------------------------------------------------------------------
struct PkArgs {
  const uint16_t* act;  // bf16 rows; row of sorted position p: gather ? gather[p] / div : p
  int64_t act_stride;
  const int32_t* gather;
  int gather_div;
  const int32_t* tiles;  // (expert, first sorted position, rows)
  const int32_t* ntiles;
  const uint8_t* q;      // packed codes / exponents of expert 0
  const uint8_t* s;
  int64_t q_estride, s_estride;
  int N32;               // packed weight tiles per expert
  int K, K128, K512;
  int N;                 // output columns: GLU I, plain N rows
  uint16_t* h_out;       // GLU: bf16 [rows][N]
  float* y_out;          // plain: fp32 [rows][N]
  int64_t out_stride;
  int n_tiles_n;         // column workgroups per row tile
  // quantised activations (gemm_packed_q_kernel): row r's codes at
  // aq + r * aq_stride, its exponents at as + r * K / 32
  const uint8_t* aq;
  const uint8_t* as;
  int64_t aq_stride;
  // quantised gate/up: h quantised in the epilogue, the down GEMM's input
  // (codes at hq_out + row * hq_stride, exponents at hqs_out + row * N / 32)
  uint8_t* hq_out;
  uint8_t* hqs_out;
  int64_t hq_stride;
};

// Weight tiles are read once. A workgroup of one 32-row tile (batched
// decode: a few routes per expert) streams them with the non-temporal hint,
// measured faster there (gate/up 773 -> 734 us at K3 T=64 with MXFP4
// activations); with more row tiles (prefill) the plain load measured faster.
template <int MT>
__device__ __forceinline__ u32x4_t load_w(const uint8_t* p) {
  if constexpr (MT == 1)
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  else
    return load16(p);
}

constexpr int kPkRows = 96;    // routes per row tile (three 32-row MFMA tiles)
constexpr int kPkKc = 128;     // K values per chunk
constexpr int kPkWaves = 4;    // waves per workgroup (two workgroups per CU)
constexpr int kPkThreads = 64 * kPkWaves;
constexpr int kPkNB = 2;       // weight tiles per wave

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// One array per LDS buffer: the compiler then tells a global-to-LDS copy into
// one buffer from the MFMA operand reads of the other, and does not wait for
// the copy before every read.
template <int R>
using PkChunk = uint16_t[R][kPkKc];

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// KA: K is a multiple of the 128-value chunk, so no copy needs clamping and
// each copy's row offset is fixed: computed once, a chunk only adds a
// uniform base (the compiler then issues the copies with a scalar base and
// a 32-bit offset, no per-chunk address arithmetic).
template <bool GLU, int MT, bool KA>
__device__ __forceinline__ void pk_body(const PkArgs& a, int e, int p0, int cnt, int nt,
                                        PkChunk<kPkRows>& sx0, PkChunk<kPkRows>& sx1,
                                        PkChunk<kPkRows>& sx2, const uint32_t* s_arow) {
  auto slot = [&](int r) -> PkChunk<kPkRows>& { return r == 0 ? sx0 : r == 1 ? sx1 : sx2; };
  const int tid = threadIdx.x;
  // the wave index in a scalar register: the copies' LDS addresses are then
  // scalar too
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int r32 = lane & 31, hh = lane >> 5;
  // this wave's weight tiles (clamped: tiles past the matrix read the last
  // one, their columns are never stored)
  int bt[kPkNB];
  const uint8_t* qb[kPkNB];
  const uint8_t* sb[kPkNB];
#pragma unroll
  for (int t = 0; t < kPkNB; ++t) {
    bt[t] = (nt * kPkWaves + wave) * kPkNB + t;
    const int btc = min(bt[t], a.N32 - 1);
    qb[t] = a.q + e * a.q_estride + (int64_t)btc * a.K128 * 2048 + lane * 16;
    sb[t] = a.s + e * a.s_estride + (int64_t)btc * a.K512 * 512 + lane * 8;
  }
  f32x16_t acc[MT][kPkNB];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < kPkNB; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][t][i] = 0.f;

  constexpr int kCopies = MT * 32 / 4 / kPkWaves;  // copy instructions per wave and chunk
  static_assert(kCopies * 4 * kPkWaves == MT * 32, "rows shared evenly by the waves");
  // activation chunk c (clamped to the last) into LDS buffer `buf`: the
  // MT * 32 rows are shared by the waves, four rows per instruction (every
  // wave issues the same number, so the waits below count the same loads in
  // every wave); lane l moves the 16-byte segment at physical slot l % 16 of
  // row l / 16, which holds logical segment (l % 16) ^ (row % 16)
  // KA: byte offset of each copy's 16-byte segment in chunk 0
  uint32_t xoff[KA ? kCopies : 1];
  if constexpr (KA) {
    __syncthreads();  // s_arow
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
      const int row = wave * kCopies * 4 + i * 4 + (lane >> 4);
      const int seg = (lane & 15) ^ (row & 15);
      xoff[i] = (s_arow[row] + seg * 8) * 2;  // < 2^32: checked on the host
    }
  }
  auto copy_x = [&](int c, int buf) {
    const int cc = min(c, a.K128 - 1);
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
      const int row0 = wave * kCopies * 4 + i * 4;
      const void* src;
      if constexpr (KA) {
        src = reinterpret_cast<const uint8_t*>(a.act) + (size_t)cc * kPkKc * 2 + xoff[i];
      } else {
        const int row = row0 + (lane >> 4);
        const int seg = (lane & 15) ^ (row & 15);
        const int k = min(cc * kPkKc + seg * 8, a.K - 8);
        src = a.act + s_arow[row] + k;
      }
      __builtin_amdgcn_global_load_lds(
          src, (__attribute__((address_space(3))) void*)(&slot(buf)[row0][0]), 16, 0, 0);
    }
  };
  // a chunk's weight codes and the exponent word that covers it: the dword
  // of its window (four chunks), bytes 2 (c % 2) + j
  struct Bq {
    u32x4_t q[kPkNB][2];
    uint32_t ex[kPkNB];
  };
  auto load_b = [&](int c, Bq& b) {
    const int cc = min(c, a.K128 - 1);
#pragma unroll
    for (int t = 0; t < kPkNB; ++t)
#pragma unroll
      for (int j = 0; j < 2; ++j) b.q[t][j] = load_w<MT>(qb[t] + (int64_t)cc * 2048 + j * 1024);
#pragma unroll
    for (int t = 0; t < kPkNB; ++t)
      b.ex[t] =
          *reinterpret_cast<const uint32_t*>(sb[t] + (cc / 4) * 512 + 4 * ((cc >> 1) & 1));
  };
  auto compute = [&](int c, int buf, const Bq& b) {
    // blocks past K are packed as zero codes with exponent 127: zeros
    float scale[kPkNB][2];
#pragma unroll
    for (int t = 0; t < kPkNB; ++t)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        scale[t][j] = e8m0_to_f32((b.ex[t] >> (8 * (2 * (c & 1) + j))) & 0xffu);
    // step st = 4 j + m of the chunk; the operands of step st + 1 (LDS
    // reads and dequantisation) are prepared while step st multiplies
    bf16x8_t av[2][MT], bv[2][kPkNB];
    auto prep = [&](int st, bf16x8_t (&a_)[MT], bf16x8_t (&b_)[kPkNB]) {
      const int j = st >> 2, m = st & 3;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = mt * 32 + r32;
        const int phys = (8 * hh + 4 * j + m) ^ (row & 15);
        a_[mt] = *reinterpret_cast<const bf16x8_t*>(&slot(buf)[row][phys * 8]);
      }
#pragma unroll
      for (int t = 0; t < kPkNB; ++t) b_[t] = dequant8(b.q[t][j][m], scale[t][j]);
    };
    // Each step's MFMAs are issued first; the next step's reads and
    // conversions follow in their shadow (the scheduling barriers keep the
    // compiler from moving each read next to its first use, which exposed
    // the LDS latency).
    prep(0, av[0], bv[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < kPkNB; ++t)
          acc[mt][t] = GLU ? mfma32(bv[st & 1][t], av[st & 1][mt], acc[mt][t])
                           : mfma32(av[st & 1][mt], bv[st & 1][t], acc[mt][t]);
      if (st < 7) prep(st + 1, av[(st + 1) & 1], bv[(st + 1) & 1]);
      // interleave: after each of the first MT MFMAs one operand read of the
      // next step, after each of the others a share of its conversions
#pragma unroll
      for (int i = 0; i < MT * kPkNB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if (i < MT)
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        else
          __builtin_amdgcn_sched_group_barrier(0x002, (8 * kPkNB / 2 + MT - 1) / MT, 0);  // VALU
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Activations (in a ring of three LDS buffers) and weights with their
  // exponents (in a ring of three register buffers) stay two chunks ahead:
  // in chunk c the loads of chunk c + 2 are issued, so at the top of chunk
  // c + 1, waiting until at most those are outstanding (vector memory loads
  // complete in issue order) leaves everything chunk c + 1 needs landed
  // while the next chunk's loads stay in flight across the barrier.
  // Groups of three chunks are unrolled so ring slots are fixed registers and
  // buffers; the first group runs before the loop (both edges into the loop
  // then carry the same loads in flight, which keeps the compiler's waits
  // exact) and a last, partial group after it.
  constexpr int U = 3;
  constexpr int kAhead = kCopies + 3 * kPkNB;        // loads of chunk c + 2
  constexpr int kWaitAhead = 0x0F70 | kAhead;        // vmcnt(kAhead)
  static_assert(kAhead < 16, "vmcnt field");
  __syncthreads();  // s_arow
  Bq bq[U];
  copy_x(0, 0);
  load_b(0, bq[0]);
  copy_x(1, 1);
  load_b(1, bq[1]);
  auto group = [&](int cb, bool last) {
#pragma unroll
    for (int r = 0; r < U; ++r) {
      const int c = cb + r;
      __builtin_amdgcn_s_waitcnt(kWaitAhead);
      __builtin_amdgcn_s_barrier();
      copy_x(c + 2, (r + 2) % U);
      load_b(c + 2, bq[(r + 2) % U]);
      __builtin_amdgcn_sched_barrier(0);
      if (!last || c < a.K128) compute(c, r, bq[r]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const int full = a.K128 / U;  // whole groups
  if (full > 0) group(0, false);
  for (int g = 1; g < full; ++g) group(g * U, false);
  if (a.K128 % U) group(full * U, true);
  __builtin_amdgcn_s_waitcnt(0);

  if constexpr (GLU) {
    // The MFMAs took the weight tile as operand A and the routes as operand
    // B: slot i of lane l is weight row 8 (i / 4) + 4 (l / 32) + i % 4 of
    // packed tile bt (rows 0..15 the gates of intermediate columns
    // 16 bt .. 16 bt + 15, rows 16..31 their ups) for route mt * 32 + l % 32.
    // Slots 0..3 (gates of columns 4 (l / 32) + 0..3) pair with slots 8..11,
    // slots 4..7 (columns 8 + 4 (l / 32) + 0..3) with 12..15: each lane
    // finishes eight h values of its route in place and stores them as two
    // runs of four.
#pragma unroll
    for (int t = 0; t < kPkNB; ++t) {
      if (bt[t] >= a.N32) continue;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = mt * 32 + r32;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t w[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const float h0 = silu(acc[mt][t][4 * h + 2 * k]) * acc[mt][t][8 + 4 * h + 2 * k];
            const float h1 =
                silu(acc[mt][t][4 * h + 2 * k + 1]) * acc[mt][t][8 + 4 * h + 2 * k + 1];
            w[k] = (uint32_t)f32_to_bf16_bits(h0) | ((uint32_t)f32_to_bf16_bits(h1) << 16);
          }
          const int col = bt[t] * 16 + 8 * h + 4 * hh;  // I is a multiple of 32
          if (row < cnt && col < a.N)
            *reinterpret_cast<u32x2_t*>(a.h_out + (int64_t)(p0 + row) * a.out_stride + col) =
                u32x2_t{w[0], w[1]};
        }
      }
    }
  } else {
    // output slot i of lane l: row 8 (i / 4) + 4 (l / 32) + i % 4 of the MFMA
    // tile, column l % 32
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < kPkNB; ++t) {
        if (bt[t] >= a.N32) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = mt * 32 + 8 * (i / 4) + 4 * hh + (i & 3);
          const int col = bt[t] * 32 + r32;
          if (row < cnt && col < a.N)
            a.y_out[(int64_t)(p0 + row) * a.out_stride + col] = acc[mt][t][i];
        }
      }
  }
}

template <bool GLU, bool KA>
__global__ __launch_bounds__(kPkThreads, 8 / kPkWaves) void gemm_packed_kernel(PkArgs a) {
  __shared__ __attribute__((aligned(16))) PkChunk<kPkRows> sx0, sx1, sx2;
  __shared__ uint32_t s_arow[kPkRows];  // element offset of each row in act
  // XCD-aware order: workgroup i runs on XCD i % 8; the column workgroups of
  // one row tile go to one XCD, so its activation rows are fetched into that
  // L2 once
  const int b = blockIdx.x;
  const int s = b / 8;
  const int nt = s % a.n_tiles_n;
  const int tile = (s / a.n_tiles_n) * 8 + b % 8;
  if (tile >= *a.ntiles) return;
  const int e = __builtin_amdgcn_readfirstlane(a.tiles[3 * tile + 0]);
  const int p0 = __builtin_amdgcn_readfirstlane(a.tiles[3 * tile + 1]);
  const int cnt = __builtin_amdgcn_readfirstlane(a.tiles[3 * tile + 2]);
  // rows past the tile repeat its last row: finite values, never stored
  for (int r = threadIdx.x; r < kPkRows; r += kPkThreads) {
    const int p = p0 + min(r, cnt - 1);
    const int64_t row = a.gather ? (int64_t)(a.gather[p] / a.gather_div) : (int64_t)p;
    s_arow[r] = (uint32_t)(row * a.act_stride);  // < 2^32: checked on the host
  }
  switch ((cnt + 31) / 32) {
    case 1: pk_body<GLU, 1, KA>(a, e, p0, cnt, nt, sx0, sx1, sx2, s_arow); break;
    case 2: pk_body<GLU, 2, KA>(a, e, p0, cnt, nt, sx0, sx1, sx2, s_arow); break;
    default: pk_body<GLU, 3, KA>(a, e, p0, cnt, nt, sx0, sx1, sx2, s_arow); break;
  }
}

// ---------------------------------------------------------------------------
// Quantised activations: FP8 E4M3 or FP4 E2M1 elements with one E8M0 scale
// per 32 values along K (the routed-expert precisions of dev48.org "Kimi K3
// on AMD Instinct GPUs with TokenSpeed", precision table, row "Routed-expert
// GEMMs"; the MX scheme of the weights for the scale). A block's scale
// exponent is floor(log2 max|v|) minus the element format's largest exponent
// (8 for E4M3 = 1.75 * 2^8, 2 for E2M1 = 1.5 * 2^2), clamped to the E8M0
// range, 2^0 for a block of zeros; each element is v / 2^X (exact: a power of
// two) rounded to nearest with ties to the even code, saturating at 448 / 6.
// Codes: E4M3 one byte per value, E2M1 two per byte (element 2m in the low
// nibble of byte m); exponents one byte per block.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_code(float q) {
  const float a = fabsf(q);
  uint32_t code;
  if (a >= 448.f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {  // below 2^-6: multiples of 2^-9, exact scaling
    code = (uint32_t)rintf(a * 512.f);
  } else {
    const uint32_t bits = __float_as_uint(a);
    const uint32_t e = (bits >> 23) - 120u;  // biased by 7
    const uint32_t m = bits & 0x7FFFFFu;
    const uint32_t r = m + 0x7FFFFu + ((m >> 20) & 1u);  // nearest, ties to even
    code = min((e << 3) + (r >> 20), 0x7Eu);             // a carry moves to e
  }
  return code | ((__float_as_uint(q) >> 24) & 0x80u);
}

__device__ __forceinline__ uint32_t e2m1_code(float q) {
  const float a = fabsf(q);
  // midpoints of 0, .5, 1, 1.5, 2, 3, 4, 6; a tie goes to the even code
  const uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                     (a >= 3.5f) + (a > 5.0f);
  return c | ((__float_as_uint(q) >> 28) & 0x8u);
}

// floor(log2 a) of a finite a > 0 (fp32 subnormals included)
__device__ __forceinline__ int ilog2f(float a) {
  const uint32_t bits = __float_as_uint(a);
  const int e = (int)(bits >> 23);
  if (e) return e - 127;
  return (31 - __clz(bits & 0x7FFFFFu)) - 149;
}

// One thread per 32-value block of a bf16 [rows][K] matrix.
template <bool FP8>
__global__ __launch_bounds__(256) void quantize_act_kernel(const uint16_t* __restrict__ src,
                                                           int64_t blocks, int K,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ exps) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= blocks) return;
  const int nb = K / 32;
  const int64_t row = b / nb;
  const int blk = (int)(b - row * nb);
  const uint16_t* p = src + row * K + blk * 32;
  u32x4_t v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = load16(p + 8 * i);
  float f[32];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[8 * i + 2 * j] = __uint_as_float(v[i][j] << 16);
      f[8 * i + 2 * j + 1] = __uint_as_float(v[i][j] & 0xFFFF0000u);
    }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(f[i]));
  const int emax = FP8 ? 8 : 2;
  const int X = amax > 0.f ? min(max(ilog2f(amax) - emax, -127), 127) : 0;
  exps[b] = (uint8_t)(X + 127);
  if constexpr (FP8) {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      w[i] = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[i] |= e4m3_code(ldexpf(f[4 * i + j], -X)) << (8 * j);
    }
    u32x4_t* d = reinterpret_cast<u32x4_t*>(codes + row * K + blk * 32);
    d[0] = u32x4_t{w[0], w[1], w[2], w[3]};
    d[1] = u32x4_t{w[4], w[5], w[6], w[7]};
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[i] = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) w[i] |= e2m1_code(ldexpf(f[8 * i + j], -X)) << (4 * j);
    }
    *reinterpret_cast<u32x4_t*>(codes + row * (K / 2) + blk * 16) =
        u32x4_t{w[0], w[1], w[2], w[3]};
  }
}

hipError_t launch_quantize_act(const uint16_t* src, int64_t rows, int K, bool fp8, uint8_t* codes,
                               uint8_t* exps, hipStream_t s) {
  const int64_t blocks = rows * (K / 32);
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)((blocks + 255) / 256));
  if (fp8)
    hipLaunchKernelGGL(quantize_act_kernel<true>, grid, dim3(256), 0, s, src, blocks, K, codes,
                       exps);
  else
    hipLaunchKernelGGL(quantize_act_kernel<false>, grid, dim3(256), 0, s, src, blocks, K, codes,
                       exps);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grouped GEMM of quantised activations and packed MXFP4 weights on the
// scaled MFMA, v_mfma_scale_f32_32x32x64_f8f6f4 (32 rows x 32 columns x 64 K,
// an E8M0 scale per 32 K of each row and column). Its operand layouts, as
// measured on gfx950 with an in-bounds probe: lane l = (row r = l % 32,
// half h = l / 32); an FP4 operand holds K 32h .. 32h+31 (element e in nibble
// e, low nibble first), an FP8 operand K 16h .. 16h+15 in bytes 0..15 and
// K 32+16h .. 32+16h+15 in bytes 16..31; in both the lane's scale register
// scales K 32h .. 32h+31 of its row.
//
// Same tiling as gemm_packed_kernel. In chunk c (128 K), step s (0, 1) takes
// MX blocks 4c + s (K half 0) and 4c + 2 + s (K half 1): for the weights
// that is packed block 4c + 2h + s of lane (r, h), as loaded; for the
// activations the same blocks of the row from LDS. The chunk's activation
// codes (64 or 128 bytes a row) and exponents (4 bytes a row) are copied to
// LDS by global-to-LDS loads, each wave 32 of 128 row slots (rows past the
// tile repeat its last row), segments XOR-swizzled by row so that the 16
// rows an LDS read serves hit distinct banks. K must be a multiple of 128.
// ---------------------------------------------------------------------------
// ring slots of the quantised GEMM's pipeline (chunks in flight + 1)
#ifndef LMOE_QRING
#define LMOE_QRING 4
#endif
constexpr int kQRing = LMOE_QRING;
static_assert(kQRing >= 3 && kQRing <= 5, "ring of three to five slots");

template <bool FP8>
struct QCfg {
  static constexpr int kRowB = FP8 ? 128 : 64;  // code bytes of a row per chunk
  static constexpr int kRowsPerCopy = 1024 / kRowB;
  static constexpr int kCopies = 32 / kRowsPerCopy;  // code copies per wave and chunk
  // physical 16-byte segment of logical segment g in row r
  static __device__ __forceinline__ int seg(int r, int g) {
    return FP8 ? g ^ ((r >> 1) & 7) : g ^ ((r >> 2) & 3);
  }
};

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));

template <bool FP8>
using QChunk = uint8_t[128 * QCfg<FP8>::kRowB];
using QExp = uint32_t[256];  // wave w's 32 rows at 64 w .. 64 w + 31

// The quantised GEMMs' epilogue: GLU writes h quantised for the down GEMM,
// plain writes the fp32 route partials.
template <bool GLU, bool FP8, int MT>
__device__ __forceinline__ void pkq_store(const PkArgs& a, const f32x16_t (&acc)[MT][kPkNB],
                                          const int (&bt)[kPkNB], int p0, int cnt) {
  const int lane = threadIdx.x & 63;
  const int r32 = lane & 31, hh = lane >> 5;
  if constexpr (GLU) {
    // h = bf16(silu(g) u), then quantised as the down GEMM's input with the
    // activation quantiser's arithmetic (quantize_act_kernel), so h is never
    // written in bf16. The MFMAs took the weight tile as operand A: slot i
    // of lane l is weight row 8 (i / 4) + 4 (l / 32) + i % 4 of packed tile
    // bt (rows 0..15 gates of intermediate columns 16 bt .. 16 bt + 15, rows
    // 16..31 their ups) for route mt * 32 + l % 32; slots 0..3 pair with
    // 8..11 and 4..7 with 12..15. The wave's two tiles (bt even) cover the 32
    // columns of one MX block: lane l holds columns 4 (l / 32) + 0..3 and
    // 8 + 4 (l / 32) + 0..3 of each tile, lane l ^ 32 the others, so the
    // block's maximum takes one exchange.
    constexpr int emax = FP8 ? 8 : 2;
    const int blk = bt[0] >> 1;  // the wave's MX block of h columns
    const bool live = bt[0] < a.N32 && 32 * blk < a.N;  // I is a multiple of 32
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = mt * 32 + r32;
      float f[16];  // local column 16 t + 8 h + 4 hh + k of the block is f[8 t + 4 h + k]
#pragma unroll
      for (int t = 0; t < kPkNB; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float g = acc[mt][t][4 * h + k], u = acc[mt][t][8 + 4 * h + k];
            f[8 * t + 4 * h + k] = bf16_bits_to_f32(f32_to_bf16_bits(silu(g) * u));
          }
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
      amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
      const int X = amax > 0.f ? min(max(ilog2f(amax) - emax, -127), 127) : 0;
      const int64_t r = (int64_t)(p0 + row);
      const bool ok = live && row < cnt;
      if constexpr (FP8) {
        // byte c of the block's 32 is column c: this lane's four runs of four
        // at bytes 16 t + 8 h + 4 hh; lane hh = 0 gathers its partner's and
        // writes the 32 bytes
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          w[q] = 0;
#pragma unroll
          for (int k = 0; k < 4; ++k) w[q] |= e4m3_code(ldexpf(f[4 * q + k], -X)) << (8 * k);
        }
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = __shfl_xor(w[q], 32, kWave);
        if (hh == 0 && ok) {
          u32x4_t* d = reinterpret_cast<u32x4_t*>(a.hq_out + r * a.hq_stride + 32 * blk);
          d[0] = u32x4_t{w[0], o[0], w[1], o[1]};
          d[1] = u32x4_t{w[2], o[2], w[3], o[3]};
        }
      } else {
        // element c in nibble c % 2 of byte c / 2: this lane's four runs of
        // four values are two bytes each, at bytes 8 t + 4 h + 2 hh
        uint32_t w[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          uint32_t lo = 0, hi = 0;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            lo |= e2m1_code(ldexpf(f[8 * q + k], -X)) << (4 * k);
            hi |= e2m1_code(ldexpf(f[8 * q + 4 + k], -X)) << (4 * k);
          }
          w[q] = lo | (hi << 16);  // runs (t = q, h = 0) and (t = q, h = 1)
        }
        uint32_t o[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) o[q] = __shfl_xor(w[q], 32, kWave);
        if (hh == 0 && ok)
          *reinterpret_cast<u32x4_t*>(a.hq_out + r * a.hq_stride + 16 * blk) =
              u32x4_t{(w[0] & 0xFFFFu) | (o[0] << 16), (w[0] >> 16) | (o[0] & 0xFFFF0000u),
                      (w[1] & 0xFFFFu) | (o[1] << 16), (w[1] >> 16) | (o[1] & 0xFFFF0000u)};
      }
      if (hh == 1 && ok) a.hqs_out[r * (a.N / 32) + blk] = (uint8_t)(X + 127);
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < kPkNB; ++t) {
        if (bt[t] >= a.N32) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = mt * 32 + 8 * (i / 4) + 4 * hh + (i & 3);
          const int col = bt[t] * 32 + r32;
          // the partials are read once, by the combine: streamed past the
          // caches (down with MXFP4 activations 824 -> 795 us at K3 prefill;
          // the bf16 kernel measured no difference)
          if (row < cnt && col < a.N)
            __builtin_nontemporal_store(acc[mt][t][i],
                                        &a.y_out[(int64_t)(p0 + row) * a.out_stride + col]);
        }
      }
  }
}

template <bool GLU, bool FP8, int MT>
__device__ __forceinline__ void pkq_body(const PkArgs& a, int e, int p0, int cnt, int nt,
                                         QChunk<FP8>& sq0, QChunk<FP8>& sq1, QChunk<FP8>& sq2,
                                         QChunk<FP8>& sq3, QChunk<FP8>& sq4, QExp& se0,
                                         QExp& se1, QExp& se2, QExp& se3, QExp& se4,
                                         const uint32_t* s_row) {
  using C = QCfg<FP8>;
  // one LDS array per ring slot: a read of one slot then never waits for the
  // copy into another
  auto qslot = [&](int r) -> QChunk<FP8>& {
    return r == 0 ? sq0 : r == 1 ? sq1 : r == 2 ? sq2 : r == 3 ? sq3 : sq4;
  };
  auto eslot = [&](int r) -> QExp& {
    return r == 0 ? se0 : r == 1 ? se1 : r == 2 ? se2 : r == 3 ? se3 : se4;
  };
  const int tid = threadIdx.x;
  // the wave index in a scalar register: the copies' LDS addresses are then
  // scalar too
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int r32 = lane & 31, hh = lane >> 5;
  int bt[kPkNB];
  const uint8_t* qb[kPkNB];
  const uint8_t* sb[kPkNB];
#pragma unroll
  for (int t = 0; t < kPkNB; ++t) {
    bt[t] = (nt * kPkWaves + wave) * kPkNB + t;
    const int btc = min(bt[t], a.N32 - 1);
    qb[t] = a.q + e * a.q_estride + (int64_t)btc * a.K128 * 2048 + lane * 16;
    sb[t] = a.s + e * a.s_estride + (int64_t)btc * a.K512 * 512 + lane * 8;
  }
  f32x16_t acc[MT][kPkNB];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < kPkNB; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][t][i] = 0.f;

  const int kb = a.K / 32;  // exponent bytes of an activation row
  // byte offsets, in chunk 0, of this wave's copies (K is a multiple of the
  // chunk, so a chunk only adds a uniform base): codes, then exponents
  __syncthreads();  // s_row
  uint32_t qoff[C::kCopies], eoff;
#pragma unroll
  for (int i = 0; i < C::kCopies; ++i) {
    const int row = wave * 32 + i * C::kRowsPerCopy + lane / (C::kRowB / 16);
    const int g = C::seg(row, lane % (C::kRowB / 16));
    qoff[i] = s_row[row] * (uint32_t)a.aq_stride + g * 16;  // < 2^32: checked on the host
  }
  // lane l < 32: the exponents of row 32 w + l; lanes 32..63 repeat them
  // into the wave's spare slots
  eoff = s_row[wave * 32 + (lane & 31)] * (uint32_t)kb;
  // this wave's 32 row slots of chunk c into LDS buffer `buf`
  auto copy_a = [&](int c, int buf) {
    const int cc = min(c, a.K128 - 1);
#pragma unroll
    for (int i = 0; i < C::kCopies; ++i) {
      const int row0 = wave * 32 + i * C::kRowsPerCopy;
      __builtin_amdgcn_global_load_lds(
          a.aq + (size_t)cc * C::kRowB + qoff[i],
          (__attribute__((address_space(3))) void*)(&qslot(buf)[row0 * C::kRowB]), 16, 0, 0);
    }
    __builtin_amdgcn_global_load_lds(
        a.as + (size_t)cc * 4 + eoff,
        (__attribute__((address_space(3))) void*)(&eslot(buf)[wave * 64]), 4, 0, 0);
  };
  // a chunk's weight codes and the exponent word that covers it
  struct Bq {
    u32x4_t q[kPkNB][2];
    uint32_t ex[kPkNB];
  };
  auto load_b = [&](int c, Bq& b) {
    const int cc = min(c, a.K128 - 1);
#pragma unroll
    for (int t = 0; t < kPkNB; ++t)
#pragma unroll
      for (int j = 0; j < 2; ++j) b.q[t][j] = load_w<MT>(qb[t] + (int64_t)cc * 2048 + j * 1024);
#pragma unroll
    for (int t = 0; t < kPkNB; ++t)
      b.ex[t] =
          *reinterpret_cast<const uint32_t*>(sb[t] + (cc / 4) * 512 + 4 * ((cc >> 1) & 1));
  };
  auto compute = [&](int c, int buf, const Bq& b) {
    const uint8_t* sq = qslot(buf);
    const QExp& se = eslot(buf);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      i32x8_t av[MT];
      int sa[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = mt * 32 + r32;
        const uint8_t* rp = sq + row * C::kRowB;
        if constexpr (FP8) {
          const u32x4_t lo =
              *reinterpret_cast<const u32x4_t*>(rp + 16 * C::seg(row, 2 * s + hh));
          const u32x4_t hi =
              *reinterpret_cast<const u32x4_t*>(rp + 16 * C::seg(row, 4 + 2 * s + hh));
          av[mt] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                           (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        } else {
          const u32x4_t v =
              *reinterpret_cast<const u32x4_t*>(rp + 16 * C::seg(row, 2 * hh + s));
          av[mt] = i32x8_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        }
        sa[mt] = (int)((se[mt * 64 + r32] >> (8 * (2 * hh + s))) & 0xFFu);
      }
#pragma unroll
      for (int t = 0; t < kPkNB; ++t) {
        const u32x4_t w = b.q[t][s];
        const i32x8_t bv = i32x8_t{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
        const int sbv = (int)((b.ex[t] >> (8 * (2 * (c & 1) + s))) & 0xFFu);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt][t] =
              GLU ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        bv, av[mt], acc[mt][t], 4, FP8 ? 0 : 4, 0, sbv, 0, sa[mt])
                  : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        av[mt], bv, acc[mt][t], FP8 ? 0 : 4, 4, 0, sa[mt], 0, sbv);
      }
    }
  };

  // A ring of U chunks (LDS for the activations, registers for the weights
  // and their exponents), loaded U - 1 chunks ahead; chunk c's loads are
  // complete once only the loads of the U - 2 later chunks are outstanding.
  // Groups of U chunks, the first peeled so both loop edges carry the same
  // loads.
  constexpr int U = kQRing;
  constexpr int kPerChunk = C::kCopies + 1 + 3 * kPkNB;  // loads issued per chunk
  constexpr int kAhead = (U - 2) * kPerChunk;
  static_assert(kAhead < 64, "vmcnt field");
  constexpr int kWaitAhead = 0x0F70 | (kAhead & 15) | ((kAhead >> 4) << 14);
  Bq bq[U];
#pragma unroll
  for (int i = 0; i < U - 1; ++i) {
    copy_a(i, i);
    load_b(i, bq[i]);
  }
  auto group = [&](int cb, bool last) {
#pragma unroll
    for (int r = 0; r < U; ++r) {
      const int c = cb + r;
      __builtin_amdgcn_s_waitcnt(kWaitAhead);
      __builtin_amdgcn_s_barrier();
      copy_a(c + U - 1, (r + U - 1) % U);
      load_b(c + U - 1, bq[(r + U - 1) % U]);
      __builtin_amdgcn_sched_barrier(0);
      if (!last || c < a.K128) compute(c, r, bq[r]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const int full = a.K128 / U;
  if (full > 0) group(0, false);
  for (int g = 1; g < full; ++g) group(g * U, false);
  if (a.K128 % U) group(full * U, true);
  __builtin_amdgcn_s_waitcnt(0);

  pkq_store<GLU, FP8, MT>(a, acc, bt, p0, cnt);
}

template <bool GLU, bool FP8>
__global__ __launch_bounds__(kPkThreads, 8 / kPkWaves) void gemm_packed_q_kernel(PkArgs a) {
  // kQRing of the five slots are used
  __shared__ __attribute__((aligned(16))) QChunk<FP8> sq0, sq1, sq2, sq3, sq4;
  __shared__ __attribute__((aligned(16))) QExp se0, se1, se2, se3, se4;
  __shared__ uint32_t s_row[128];  // activation row of each row slot
  const int b = blockIdx.x;
  const int s = b / 8;
  const int nt = s % a.n_tiles_n;
  const int tile = (s / a.n_tiles_n) * 8 + b % 8;
  if (tile >= *a.ntiles) return;
  const int e = __builtin_amdgcn_readfirstlane(a.tiles[3 * tile + 0]);
  const int p0 = __builtin_amdgcn_readfirstlane(a.tiles[3 * tile + 1]);
  const int cnt = __builtin_amdgcn_readfirstlane(a.tiles[3 * tile + 2]);
  for (int r = threadIdx.x; r < 128; r += kPkThreads) {
    const int p = p0 + min(r, cnt - 1);
    s_row[r] = (uint32_t)(a.gather ? a.gather[p] / a.gather_div : p);
  }
#define LMOE_PKQ(MT)                                                                      \
  pkq_body<GLU, FP8, MT>(a, e, p0, cnt, nt, sq0, sq1, sq2, sq3, sq4, se0, se1, se2, se3, se4, \
                         s_row)
  switch ((cnt + 31) / 32) {
    case 1: LMOE_PKQ(1); break;
    case 2: LMOE_PKQ(2); break;
    default: LMOE_PKQ(3); break;
  }
#undef LMOE_PKQ
}

// ---------------------------------------------------------------------------
// The MXFP4-activation GEMM when K is a multiple of 256 and at most 4096
// (the K3 layer: 3584 and 2048). A row's codes for one 128-K chunk are 64
// bytes, half a cache line, and its exponents for the chunk one 4-byte word:
// copied chunk by chunk from gathered rows, each row's line is requested
// twice and each exponent word costs a line of its own. Here the tile's
// exponents (96 rows x K / 32 bytes) are copied into an LDS table once, at
// the start, and the codes of two chunks travel together as whole 128-byte
// lines into one of two double slots, laid out and swizzled like the FP8
// rows. Otherwise the tiling, the weight ring (three chunks ahead) and the
// epilogue are those of gemm_packed_q_kernel.
// ---------------------------------------------------------------------------
constexpr int kA4MaxK = 4096;
constexpr int kA4TabW = kA4MaxK / 128 + 1;  // words a row (one of padding, so rows fall on odd strides)
constexpr int kA4TabLoads = (kPkRows * kA4TabW + 4 * 64 - 1) / (4 * 64);  // per wave, at most
using A4Tab = uint32_t[kA4TabLoads * 4 * 64];

template <bool GLU, int MT>
__device__ __forceinline__ void pka4_body(const PkArgs& a, int e, int p0, int cnt, int nt,
                                          QChunk<true>& d0, QChunk<true>& d1, A4Tab& tab,
                                          const uint32_t* s_row) {
  using C = QCfg<true>;  // 128-byte rows: the codes of a chunk pair
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int r32 = lane & 31, hh = lane >> 5;
  int bt[kPkNB];
  const uint8_t* qb[kPkNB];
  const uint8_t* sb[kPkNB];
#pragma unroll
  for (int t = 0; t < kPkNB; ++t) {
    bt[t] = (nt * kPkWaves + wave) * kPkNB + t;
    const int btc = min(bt[t], a.N32 - 1);
    qb[t] = a.q + e * a.q_estride + (int64_t)btc * a.K128 * 2048 + lane * 16;
    sb[t] = a.s + e * a.s_estride + (int64_t)btc * a.K512 * 512 + lane * 8;
  }
  f32x16_t acc[MT][kPkNB];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < kPkNB; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][t][i] = 0.f;

  const int kw = a.K128;    // exponent words of a row (one per chunk)
  const int tw = kw + 1;    // table stride in words (K128 is even: odd)
  const int kb = a.K / 32;  // exponent bytes of an activation row
  __syncthreads();          // s_row
  // the exponent table: word q of the table is word q % tw of row q / tw
  // (the padding word and positions past the MT * 32 rows load a harmless
  // word)
  {
    const int loads = (MT * 32 * tw + 4 * 64 - 1) / (4 * 64);
    for (int j = 0; j < loads; ++j) {
      const int q = (wave * loads + j) * 64 + lane;
      const int row = q / tw, d = q - row * tw;
      const bool live = row < MT * 32 && d < kw;
      const uint8_t* src = a.as + (size_t)s_row[live ? row : 0] * kb + (live ? d : 0) * 4;
      __builtin_amdgcn_global_load_lds(
          src, (__attribute__((address_space(3))) void*)(&tab[(wave * loads + j) * 64]), 4, 0,
          0);
    }
  }
  int trow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) trow[mt] = (mt * 32 + r32) * tw;
  // the MT * 32 rows are shared by the waves: MT copies of 8 rows of 128
  // bytes each (every wave issues the same number, so the waits below count
  // the same loads in every wave); byte offsets in chunk pair 0
  constexpr int kCopies = MT;
  static_assert(kCopies * C::kRowsPerCopy * kPkWaves == MT * 32, "rows shared evenly");
  uint32_t qoff[kCopies];
#pragma unroll
  for (int i = 0; i < kCopies; ++i) {
    const int row = (wave * kCopies + i) * C::kRowsPerCopy + lane / 8;
    qoff[i] = s_row[row] * (uint32_t)a.aq_stride + C::seg(row, lane % 8) * 16;
  }
  // the codes of chunks 2 cp and 2 cp + 1 into a double slot
  auto copy_pair = [&](int cp, QChunk<true>& dst) {
    const int cc = min(cp, a.K128 / 2 - 1);
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
      const int row0 = (wave * kCopies + i) * C::kRowsPerCopy;
      __builtin_amdgcn_global_load_lds(
          a.aq + (size_t)cc * C::kRowB + qoff[i],
          (__attribute__((address_space(3))) void*)(&dst[row0 * C::kRowB]), 16, 0, 0);
    }
  };
  struct Bq {
    u32x4_t q[kPkNB][2];
    uint32_t ex[kPkNB];
  };
  auto load_b = [&](int c, Bq& b) {
    const int cc = min(c, a.K128 - 1);
#pragma unroll
    for (int t = 0; t < kPkNB; ++t)
#pragma unroll
      for (int j = 0; j < 2; ++j) b.q[t][j] = load_w<MT>(qb[t] + (int64_t)cc * 2048 + j * 1024);
#pragma unroll
    for (int t = 0; t < kPkNB; ++t)
      b.ex[t] =
          *reinterpret_cast<const uint32_t*>(sb[t] + (cc / 4) * 512 + 4 * ((cc >> 1) & 1));
  };
  // chunk c (half `half` of its double slot)
  auto compute = [&](int c, int half, const QChunk<true>& sq, const Bq& b) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      i32x8_t av[MT];
      int sa[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = mt * 32 + r32;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(
            sq + row * C::kRowB + 16 * C::seg(row, 4 * half + 2 * hh + s));
        av[mt] = i32x8_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        sa[mt] = (int)((tab[trow[mt] + c] >> (8 * (2 * hh + s))) & 0xFFu);
      }
#pragma unroll
      for (int t = 0; t < kPkNB; ++t) {
        const u32x4_t w = b.q[t][s];
        const i32x8_t bv = i32x8_t{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
        const int sbv = (int)((b.ex[t] >> (8 * (2 * (c & 1) + s))) & 0xFFu);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt][t] = GLU ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                 bv, av[mt], acc[mt][t], 4, 4, 0, sbv, 0, sa[mt])
                           : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                 av[mt], bv, acc[mt][t], 4, 4, 0, sa[mt], 0, sbv);
      }
    }
  };

  // Weights in a ring of four register buffers, three chunks ahead; codes
  // in double slots D0 (chunks 4g, 4g + 1) and D1 (4g + 2, 4g + 3), each
  // pair copied at the even chunk two before it. Before chunk c, the loads
  // issued after its last one are: c even (its codes, copied at c - 2,
  // were last): the weights of c + 1 and c + 2; c odd (its weights, loaded
  // at c - 3, were last): the weights of c + 1, the next pair, the weights
  // of c + 2. The table went out before everything.
  constexpr int kW = 3 * kPkNB;  // weight loads a chunk
  constexpr int kEven = 2 * kW, kOdd = 2 * kW + kCopies;
  static_assert(kOdd < 64, "vmcnt field");
  constexpr int kWaitEven = 0x0F70 | (kEven & 15) | ((kEven >> 4) << 14);
  constexpr int kWaitOdd = 0x0F70 | (kOdd & 15) | ((kOdd >> 4) << 14);
  Bq bq[4];
  copy_pair(0, d0);
#pragma unroll
  for (int i = 0; i < 3; ++i) load_b(i, bq[i]);
  auto group = [&](int cb, bool last) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = cb + r;
      if (r & 1)
        __builtin_amdgcn_s_waitcnt(kWaitOdd);
      else
        __builtin_amdgcn_s_waitcnt(kWaitEven);
      __builtin_amdgcn_s_barrier();
      if (r == 0) copy_pair(c / 2 + 1, d1);
      if (r == 2) copy_pair(c / 2 + 1, d0);
      load_b(c + 3, bq[(r + 3) & 3]);
      __builtin_amdgcn_sched_barrier(0);
      if (!last || c < a.K128) compute(c, r & 1, r < 2 ? d0 : d1, bq[r]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const int full = a.K128 / 4;
  for (int g = 0; g < full; ++g) group(g * 4, false);
  if (a.K128 % 4) group(full * 4, true);
  __builtin_amdgcn_s_waitcnt(0);

  pkq_store<GLU, false, MT>(a, acc, bt, p0, cnt);
}

template <bool GLU>
__global__ __launch_bounds__(kPkThreads, 8 / kPkWaves) void gemm_packed_a4_kernel(PkArgs a) {
  __shared__ __attribute__((aligned(16))) QChunk<true> d0, d1;
  __shared__ __attribute__((aligned(16))) A4Tab tab;
  __shared__ uint32_t s_row[128];  // activation row of each row slot
  const int b = blockIdx.x;
  const int s = b / 8;
  const int nt = s % a.n_tiles_n;
  const int tile = (s / a.n_tiles_n) * 8 + b % 8;
  if (tile >= *a.ntiles) return;
  const int e = __builtin_amdgcn_readfirstlane(a.tiles[3 * tile + 0]);
  const int p0 = __builtin_amdgcn_readfirstlane(a.tiles[3 * tile + 1]);
  const int cnt = __builtin_amdgcn_readfirstlane(a.tiles[3 * tile + 2]);
  for (int r = threadIdx.x; r < 128; r += kPkThreads) {
    const int p = p0 + min(r, cnt - 1);
    s_row[r] = (uint32_t)(a.gather ? a.gather[p] / a.gather_div : p);
  }
  switch ((cnt + 31) / 32) {
    case 1: pka4_body<GLU, 1>(a, e, p0, cnt, nt, d0, d1, tab, s_row); break;
    case 2: pka4_body<GLU, 2>(a, e, p0, cnt, nt, d0, d1, tab, s_row); break;
    default: pka4_body<GLU, 3>(a, e, p0, cnt, nt, d0, d1, tab, s_row); break;
  }
}

hipError_t launch_routed_packed(const Plan& p, const uint16_t* x, const PackedWeights& w,
                                const Workspace& ws, const int32_t* perm, hipStream_t s,
                                const hipEvent_t* ev, int act) {
  const lmoe_dims& d = p.d;
  const int rounds = (p.max_tiles + 7) / 8;
  const bool q = act != LMOE_ACT_BF16, fp8 = act == LMOE_ACT_E4M3;
  hipError_t err;
  auto launch = [&](bool glu, const PkArgs& a) {
    const dim3 grid((unsigned)(rounds * 8 * a.n_tiles_n));
    const bool ka = a.K % kPkKc == 0;
    if (!q && glu) {
      if (ka)
        hipLaunchKernelGGL((gemm_packed_kernel<true, true>), grid, dim3(kPkThreads), 0, s, a);
      else
        hipLaunchKernelGGL((gemm_packed_kernel<true, false>), grid, dim3(kPkThreads), 0, s, a);
    } else if (!q) {
      if (ka)
        hipLaunchKernelGGL((gemm_packed_kernel<false, true>), grid, dim3(kPkThreads), 0, s, a);
      else
        hipLaunchKernelGGL((gemm_packed_kernel<false, false>), grid, dim3(kPkThreads), 0, s, a);
    } else if (!fp8 && a.K % 256 == 0 && a.K <= kA4MaxK) {
      if (glu)
        hipLaunchKernelGGL((gemm_packed_a4_kernel<true>), grid, dim3(kPkThreads), 0, s, a);
      else
        hipLaunchKernelGGL((gemm_packed_a4_kernel<false>), grid, dim3(kPkThreads), 0, s, a);
    } else if (glu && fp8)
      hipLaunchKernelGGL((gemm_packed_q_kernel<true, true>), grid, dim3(kPkThreads), 0, s, a);
    else if (glu)
      hipLaunchKernelGGL((gemm_packed_q_kernel<true, false>), grid, dim3(kPkThreads), 0, s, a);
    else if (fp8)
      hipLaunchKernelGGL((gemm_packed_q_kernel<false, true>), grid, dim3(kPkThreads), 0, s, a);
    else
      hipLaunchKernelGGL((gemm_packed_q_kernel<false, false>), grid, dim3(kPkThreads), 0, s, a);
    return hipGetLastError();
  };
  {  // gate/up + GLU
    if (q && (err = launch_quantize_act(x, d.T, d.L, fp8, ws.xq, ws.xq_s, s)) != hipSuccess)
      return err;
    PkArgs a = {};
    a.act = x;
    a.act_stride = d.L;
    a.aq = ws.xq;
    a.as = ws.xq_s;
    a.aq_stride = fp8 ? d.L : d.L / 2;
    a.gather = perm;
    a.gather_div = d.k;
    a.tiles = ws.tiles;
    a.ntiles = ws.ntiles;
    a.q = w.gu_q;
    a.s = w.gu_s;
    a.N32 = (2 * d.I + 31) / 32;
    a.K = d.L;
    a.K128 = (d.L + 127) / 128;
    a.K512 = (d.L + 511) / 512;
    a.q_estride = (int64_t)a.N32 * a.K128 * 2048;
    a.s_estride = (int64_t)a.N32 * a.K512 * 512;
    a.N = d.I;
    a.h_out = ws.h;
    a.out_stride = d.I;
    a.hq_out = ws.hq;
    a.hqs_out = ws.hq_s;
    a.hq_stride = fp8 ? d.I : d.I / 2;
    a.n_tiles_n = (a.N32 + kPkWaves * kPkNB - 1) / (kPkWaves * kPkNB);
    if ((err = launch(true, a)) != hipSuccess) return err;
    if ((err = record_stage(ev, LMOE_STAGE_GATEUP, s)) != hipSuccess) return err;
  }
  {  // down
    // (the quantised gate/up kernel wrote h quantised already)
    PkArgs a = {};
    a.act = ws.h;
    a.act_stride = d.I;
    a.aq = ws.hq;
    a.as = ws.hq_s;
    a.aq_stride = fp8 ? d.I : d.I / 2;
    a.tiles = ws.tiles;
    a.ntiles = ws.ntiles;
    a.q = w.down_q;
    a.s = w.down_s;
    a.N32 = (d.L + 31) / 32;
    a.K = d.I;
    a.K128 = (d.I + 127) / 128;
    a.K512 = (d.I + 511) / 512;
    a.q_estride = (int64_t)a.N32 * a.K128 * 2048;
    a.s_estride = (int64_t)a.N32 * a.K512 * 512;
    a.N = d.L;
    a.y_out = ws.y;
    a.out_stride = d.L;
    a.n_tiles_n = (a.N32 + kPkWaves * kPkNB - 1) / (kPkWaves * kPkNB);
    if ((err = launch(false, a)) != hipSuccess) return err;
    err = record_stage(ev, LMOE_STAGE_DOWN, s);
  }
  return err;
}

}  // namespace lmoe
