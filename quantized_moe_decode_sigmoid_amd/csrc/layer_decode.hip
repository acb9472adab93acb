// The MoE layer for one decode token (T = 1) in two launches.
//
// Same arithmetic contract as the multi-kernel path (router_math.h; exact
// IQ4_NL weights on v_mfma_f32_16x16x32_bf16, see ffn_exact.hip), organised
// for latency.  Routing is bit-identical to it; the FFN sums are split over
// 8 wavefronts per row tile instead of 4, so outputs agree to fp32 rounding:
//
//   k_decode_scores   one wavefront (workgroup) per router row: fp32 logit and
//                     sigmoid score (row E: the shared expert's gate, when
//                     the shared expert is sigmoid-gated); the chained form
//                     (k_decode_scores_chained, 256 threads per row) first
//                     forms the layer's input from the previous layer's.
//                     It also writes the "not ready" pattern into the words
//                     through which the next kernel hands data between its
//                     workgroups; the previous token's second kernel has
//                     finished, so nobody reads them now.
//   k_decode_experts  roles by block index:
//     [routed]  gate/up + SiLU*up of routed slot k, one 16-row tile of F;
//     [shared]  gate/up + SiLU*up of the shared expert, one 16-row tile of F,
//               then (the shared expert's h complete) its down rows of up to
//               4 row tiles of H;
//     [down]    32 rows of H: down projection of the routed slots, then the
//               slot-order combine of those rows with the shared expert's.
//   Every workgroup that needs the routing ranks the E scores itself, so
//   there is no hand-off for it.  The down workgroups request their weight
//   tiles as soon as they know the experts, then read the h words of the
//   gate/up workgroups, repeating a read while it still shows the "not ready"
//   pattern (a finite value never has it).  Each word is written once with
//   one device-scope store, so a word that is not "not ready" is complete: no
//   counter, atomic or fence is involved.
//
// Every global load of a role is issued before its result is first used and
// none sits behind a runtime branch (indices are clamped, unused values
// discarded), so a wavefront has its HBM requests in flight together.
// Operands shared by all wavefronts of a workgroup (x, block scales, h) are
// staged once in LDS with coalesced loads.  Every wait is bounded: one that
// exceeds the bound sets an error word and gives up, so a launch always ends.
#include <atomic>

#include "device.h"
#include "launch.h"
#include "router_math.h"

namespace qmoe {

constexpr int kDecThreads = 1024;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kGuSplit = kDecWaves / 2;  // waves per matrix in gate/up: each takes 1/kGuSplit of H
// Down: two 16-row tiles of H per workgroup; wave w takes row tile w & 1 and
// packed tile kg = w >> 1 of the F/128 tiles of a row.
constexpr int kDnWavesPerRowTile = kDecWaves / 2;
static_assert(kMaxDecodeFfn / 128 <= kDnWavesPerRowTile, "one packed tile per wave in down");
static_assert(kDecWaves == 16, "the LDS DMA staging assigns its loads to 16 wavefronts");
constexpr int kGuMaxKg = (kMaxDecodeHidden / 128 + kGuSplit - 1) / kGuSplit;  // gate/up tiles per wave

constexpr int kDnSlots = kMaxDecodeK + 1;             // routed slots + shared
constexpr uint32_t kNotReady = 0xffffffffu;           // an h word before it is written
constexpr uint32_t kPollLimit = 1u << 20;

// ---------------------------------------------------------------- device-scope access

constexpr int kDeviceScope = 16;  // cache-policy bit: device coherence

// 16 bytes at byte offset off of a buffer, read through to device scope.
__device__ __forceinline__ uint4 ld_dev_x4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kDeviceScope));
}

__device__ __forceinline__ uint32_t ld_dev(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kDeviceScope);
}

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

__device__ __forceinline__ void st_dev_x4(__amdgpu_buffer_rsrc_t r, int off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, off, 0, kDeviceScope);
}

__device__ __forceinline__ void st_dev(__amdgpu_buffer_rsrc_t r, int off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kDeviceScope);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

__device__ __forceinline__ bool ready(uint4 v) {
  return v.x != kNotReady && v.y != kNotReady && v.z != kNotReady && v.w != kNotReady;
}

// A bounded wait gives up when it has re-read kPollLimit times, or, checked
// every 64 re-reads, when another wait of the launch has already given up
// (so that one failure does not make every later wait run to its bound).
__device__ __forceinline__ bool give_up(const uint32_t* err, uint32_t it) {
  return it > kPollLimit || ((it & 63u) == 0u && ld_dev(buffer_of(err), 0) != 0u);
}

// ---------------------------------------------------------------- LDS

constexpr int kScaleWords = 32;  // 64 fp16 scales of a tile

struct RouteLds {
  uint32_t key[256];  // selection-order keys (sel_order_bits of s + bias)
  float score[256];
  float sval[kMaxDecodeK];
  float w[kMaxDecodeK];
  int32_t ids[kMaxDecodeK];
};

constexpr int kGuMaxRowTiles = 1;  // row tiles of F per gate/up workgroup

struct GateUpLds {
  uint16_t x[kMaxDecodeHidden];                                                // the token's activations
  uint32_t scales[kGuMaxRowTiles][2][kMaxDecodeHidden / 128][kScaleWords];  // [row tile][gate/up][kg]
  f32x4 red[kGuMaxRowTiles][kDecWaves][4];                                  // column 0 of each wave's acc
};

struct DownLds {
  uint32_t scales[kDnSlots][2][kMaxDecodeFfn / 128][kScaleWords];  // [slot][row tile][kg]
  uint16_t hh[kDnSlots][kMaxDecodeFfn];                            // bf16(h)
  uint16_t hl[kDnSlots][kMaxDecodeFfn];                            // bf16(h - bf16(h))
  float part[kDecWaves][kDnSlots][16];                             // column 0 + 1 of each wave's partial
  float y[kDnSlots][32];
};

// The table comes last: every LDS DMA destination (x, scales, a router row)
// then lies in the first 64 KB.
struct ExpertsLds {
  RouteLds route;
  union {
    GateUpLds g;
    DownLds d;
  } u;
  __attribute__((aligned(256))) uint32_t tbl[kPairTableWords];
};
static_assert(offsetof(ExpertsLds, tbl) <= 65536, "LDS DMA destinations in the first 64 KB");

// ---------------------------------------------------------------- kernel 1: scores

template <int MMAX>
__global__ __launch_bounds__(64) void k_decode_scores(DecodeArgs a) {
  const int lane = threadIdx.x;
  const int e = blockIdx.x;
  // reset the h hand-off words of k_decode_experts
  const int n_words = hw_words(a.K, a.F, a.H);
  for (int i = blockIdx.x * 64 + threadIdx.x; i < n_words; i += gridDim.x * 64) a.hw[i] = kNotReady;
  if (e == 0) {
    if (a.zero_err && lane == 0) a.err[0] = 0u;
    if (a.x_copy)
      for (int i = lane; i < (a.H >> 3); i += 64)
        *reinterpret_cast<uint4*>(a.x_copy + 8 * i) = *reinterpret_cast<const uint4*>(a.x + 8 * i);
  }
  if (e < a.E + a.gated) {  // row E: the shared expert's gate
    float4 w[MMAX];
    load_router_row<MMAX>(a.wg + (size_t)e * a.H, a.H, lane, w);
    const float p = router_logit<MMAX>(a.x, a.H, lane, w);
    if (lane == 0) a.scores[e] = sigmoid_fixed(p);
  }
}

// The chained form (x_prev non-null): 256 threads per router row.  The
// layer's input x = bf16(h * r), h = fp32(x_prev) + out_prev,
// r = 1 / sqrt(mean(h^2) + eps), with exactly the operations and order of
// k_residual_rmsnorm (chain.hip): thread v sums h_i^2 over i = v, v + 256, ...
// with fused multiply-adds, each wavefront's 64 sums meet in an xor butterfly,
// the 4 wavefront sums are added in order; every thread forms x of its
// elements into LDS (workgroup 0 also writes x for the experts kernel and the
// caller), then wavefront 0 makes the logit from LDS and its router row in
// registers, in router_logit's order.
template <int MMAX>
__global__ __launch_bounds__(256) void k_decode_scores_chained(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[256 * MMAX];
  __shared__ float nred[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = blockIdx.x;
  const int H = a.H, M = H >> 8;
  const int n_words = hw_words(a.K, a.F, a.H);
  for (int i = blockIdx.x * 256 + tid; i < n_words; i += gridDim.x * 256) a.hw[i] = kNotReady;
  if (e >= a.E + a.gated) return;  // (uniform over the workgroup)
  float4 w[MMAX];
  if (wave == 0) load_router_row<MMAX>(a.wg + (size_t)e * H, H, lane, w);
  float h[MMAX];
#pragma unroll
  for (int n = 0; n < MMAX; n++) {
    const int i = tid + 256 * (n < M ? n : M - 1);
    h[n] = bf16_bits_to_f32(a.x_prev[i]) + a.out_prev[i];
  }
  float ss = 0.0f;
#pragma unroll
  for (int n = 0; n < MMAX; n++)
    if (n < M) ss = __builtin_fmaf(h[n], h[n], ss);
  ss = wave_xor_sum(ss);
  if (lane == 0) nred[wave] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; q++) tot += nred[q];
  const float r = 1.0f / __builtin_sqrtf(tot / (float)H + a.eps);
  uint16_t* xo = const_cast<uint16_t*>(a.x);
#pragma unroll
  for (int n = 0; n < MMAX; n++) {
    if (n < M) {
      const uint16_t y = (uint16_t)f32_to_bf16_rne(h[n] * r);
      xs[tid + 256 * n] = y;
      if (e == 0) xo[tid + 256 * n] = y;  // the layer's input, for the second kernel and the caller
    }
  }
  __syncthreads();
  if (wave == 0) {
    const float p = router_logit<MMAX>(xs, H, lane, w);
    if (lane == 0) a.scores[e] = sigmoid_fixed(p);
  }
}

// ---------------------------------------------------------------- routing in each workgroup

// Top-K of the E scores into r (ids, unbiased scores, weights), by rank: expert
// e takes slot rank(e) when rank(e) < K, rank = number of experts before it in
// the (selection score, index) order.
//
// route_fetch only issues the loads of a thread's score and bias (clamped
// index, no branch), so that a caller can put them ahead of its weight
// loads: a wait for them then does not wait for those.
struct RouteIn {
  float s, b;
};

__device__ __forceinline__ RouteIn route_fetch(const DecodeArgs& a) {
  const int e = min((int)threadIdx.x, a.E - 1);
  RouteIn v;
  v.s = a.scores[e];
  v.b = a.bias ? a.bias[e] : 0.0f;
  return v;
}

// The token's routing (every thread of the workgroup calls it; thread e < E
// brings expert e's score and bias), in two forms with the same result: the
// K largest selection scores s + bias (ties: the lower expert index), their
// scores, and the weights scale * s_k / (((s_0 + s_1) + ...)) in slot order.
// Both compare the scores' order keys (sel_order_bits) with the index as the
// tie-break: a total order whatever the scores hold, so that a NaN score (from
// a NaN input) still leaves K distinct experts in the K slots, the same in
// every workgroup, and no slot's expert id is left unset.
//
// route_rank_lds: every expert's rank among all E counted by its own thread
// from LDS, three barriers (≈2.3 µs at E = 64).  The decode kernel's down
// workgroups use it: they only need the routing to request their routed
// tiles, and requesting those later leaves the routed gate/up tiles more of
// the memory system (measured: 17.57 against 17.64 µs per call with
// route_rank_wave there, and 18.6 against 19.9 µs before the shared expert's
// down rows moved to its own workgroups).
__device__ void route_rank_lds(const DecodeArgs& a, RouteLds& r, RouteIn v) {
  const int e = threadIdx.x;
  if (e < a.E) {
    r.score[e] = v.s;
    r.key[e] = sel_order_bits(a.bias ? v.s + v.b : v.s);
  }
  __syncthreads();
  if (e < a.E) {
    const uint32_t ke = r.key[e];
    int rank = 0;
#pragma unroll 8
    for (int q = 0; q < a.E; q++) {
      const uint32_t kq = r.key[q];
      rank += kq > ke || (kq == ke && q < e);
    }
    if (rank < a.K) {
      r.ids[rank] = e;
      r.sval[rank] = r.score[e];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma clang fp contract(off)
    float S = 0.0f;
    for (int k = 0; k < a.K; k++) S = S + r.sval[k];
    for (int k = 0; k < a.K; k++) r.w[k] = (r.sval[k] / S) * a.scale;
  }
  __syncthreads();
}

// route_rank_wave: wavefront 0 takes the K in K rounds of topk_take, from
// registers when E <= 64, else through LDS, one barrier (≈0.9 µs at E = 64):
// the routed gate/up workgroups' form.
__device__ void route_rank_wave(const DecodeArgs& a, RouteLds& r, RouteIn v) {
#pragma clang fp contract(off)
  const int e = threadIdx.x;
  if (a.E > 64) {  // experts past wavefront 0 meet in LDS
    if (e < a.E) {
      r.score[e] = v.s;
      r.key[e] = sel_order_bits(a.bias ? v.s + v.b : v.s);
    }
    __syncthreads();
  }
  if (e < 64) {
    float S = 0.0f;
    if (a.E <= 64) {
      const bool avail = e < a.E;
      const float s[1] = {avail ? v.s : 0.0f};
      uint32_t key[1] = {avail ? sel_order_bits(a.bias ? v.s + v.b : v.s) : 0u};
      for (int k = 0; k < a.K; k++) {
        float sk;
        const int id = topk_take<1>(key, s, e, sk);
        if (e == 0) {
          r.ids[k] = id;
          r.sval[k] = sk;
        }
        S = S + sk;
      }
    } else {
      float s[4];
      uint32_t key[4];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int x = e + 64 * q;
        const bool avail = x < a.E;
        s[q] = avail ? r.score[x] : 0.0f;
        key[q] = avail ? r.key[x] : 0u;
      }
      for (int k = 0; k < a.K; k++) {
        float sk;
        const int id = topk_take<4>(key, s, e, sk);
        if (e == 0) {
          r.ids[k] = id;
          r.sval[k] = sk;
        }
        S = S + sk;
      }
    }
    if (e == 0)
      for (int k = 0; k < a.K; k++) r.w[k] = (r.sval[k] / S) * a.scale;
  }
  __syncthreads();
}

__device__ __forceinline__ void route_local(const DecodeArgs& a, RouteLds& r) { route_rank_wave(a, r, route_fetch(a)); }

// ---------------------------------------------------------------- gate / up role

// waves 0-3: W_gate over quarters of the blocks of H; waves 4-7: W_up.
// h of (row 16rt + 4G + i) is written to hw[slot][...] as bf16 hi | lo << 16.
//
// 1. the row tiles' scales (16-byte piece p = 64 j + lane of [matrix][kg][8]
//    of row tile t, for j = 0..7) and, with dma_x, x (piece p of the row) by
//    LDS DMA, one wave load each, pieces past the matrix repeating a valid
//    one (never read); then this wave's nibble words.
template <int NRT>
__device__ __forceinline__ void gate_up_dma(const DecodeArgs& a, const uint8_t* ex, int rt0, ExpertsLds& sh,
                                            bool dma_x) {
  static_assert(NRT >= 1 && NRT <= kGuMaxRowTiles, "row tiles per workgroup");
  GateUpLds& g = sh.u.g;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t mat_bytes = a.expert_bytes / 3;
  const int nkg = a.H >> 7;
  const int64_t rt_bytes = (int64_t)nkg * kTileBytes;
  const uint8_t* rowtiles = ex + rt0 * rt_bytes;  // gate of row tile rt0; up is mat_bytes further
  const int n_dma = 8 * NRT + (dma_x ? 8 : 0);
  for (int j = wave; j < n_dma; j += kDecWaves) {
    if (j < 8 * NRT) {
      const int t = j >> 3, p = 64 * (j & 7) + lane, m = p >> 8, kg = min((p >> 3) & 31, nkg - 1);
      dma16_stream(rowtiles + t * rt_bytes + m * mat_bytes + (int64_t)kg * kTileBytes + kTileNibbleBytes + 16 * (p & 7),
                   &g.scales[t][0][0][0] + 256 * (j & 7));
    } else {
      const int p = 64 * (j - 8 * NRT) + lane;
      dma16(a.x + 8 * min(p, (a.H >> 3) - 1), &g.x[512 * (j - 8 * NRT)]);
    }
  }
  asm volatile("" ::: "memory");  // keep later loads after the DMA
}

template <int NRT>
__device__ __forceinline__ void gate_up_words(const DecodeArgs& a, const uint8_t* ex, int rt0,
                                              u32x4 (&nib)[NRT][kGuMaxKg]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t mat_bytes = a.expert_bytes / 3;
  const int nkg = a.H >> 7;
  const int q = wave % kGuSplit, mat = wave / kGuSplit;
  const int kg0 = q * nkg / kGuSplit;
  const int64_t rt_bytes = (int64_t)nkg * kTileBytes;
  const uint8_t* rowtiles = ex + rt0 * rt_bytes;
#pragma unroll
  for (int t = 0; t < NRT; t++)
#pragma unroll
    for (int i = 0; i < kGuMaxKg; i++) {
      const int kg = min(kg0 + i, nkg - 1);
      nib[t][i] = ld16(rowtiles + t * rt_bytes + mat * mat_bytes + (int64_t)kg * kTileBytes + 16 * lane);
    }
}

// 1. the row tiles' scales (16-byte piece p = 64 j + lane of [matrix][kg][8]
//    of row tile t, for j = 0..7) and, with dma_x, x (piece p of the row) by
//    LDS DMA, one wave load each, pieces past the matrix repeating a valid
//    one (never read); then this wave's nibble words.
template <int NRT>
__device__ __forceinline__ void gate_up_issue(const DecodeArgs& a, const uint8_t* ex, int rt0, ExpertsLds& sh,
                                              bool dma_x, u32x4 (&nib)[NRT][kGuMaxKg]) {
  gate_up_dma<NRT>(a, ex, rt0, sh, dma_x);
  gate_up_words<NRT>(a, ex, rt0, nib);
}

// 2. MFMAs: every column carries the token (a broadcast operand), column 0
//    is kept; acc[t][i] (row 4G+i of row tile t) += d * (levels . x).
//    Tiles past this wave's range are skipped (a branch uniform over the
//    wavefront).  3. wave t, column 0: g and u of row tile t summed in wave
//    order, h = silu(g) * u, stored with one device-scope store per 4 rows.
//    Needs the table, the scales and x in LDS.
template <int NRT>
__device__ __forceinline__ void gate_up_compute(const DecodeArgs& a, int slot, int rt0, ExpertsLds& sh,
                                                const u32x4 (&nib)[NRT][kGuMaxKg]) {
  GateUpLds& g = sh.u.g;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, G = lane >> 4;
  const int nkg = a.H >> 7;
  const int q = wave % kGuSplit, mat = wave / kGuSplit;
  const int kg0 = q * nkg / kGuSplit, nk = (q + 1) * nkg / kGuSplit - kg0;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[NRT];
#pragma unroll
  for (int t = 0; t < NRT; t++) acc[t] = zero;
#pragma unroll
  for (int i = 0; i < kGuMaxKg; i++) {
    if (i >= nk) continue;
    const int kg = min(kg0 + i, nkg - 1);
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const bf16x8 xb = *reinterpret_cast<const bf16x8*>(&g.x[32 * (4 * kg + b) + 8 * G]);
#pragma unroll
      for (int t = 0; t < NRT; t++) {
        const bf16x8 wa = decode_word(sh.tbl, uword(nib[t][i], b), lane & 31);
        const uint32_t s01 = g.scales[t][mat][kg][8 * G + 2 * b];
        const uint32_t s23 = g.scales[t][mat][kg][8 * G + 2 * b + 1];
        const f32x4 cc = mfma16x16x32(wa, xb, zero);
        acc[t][0] = __builtin_fmaf(half_bits_to_float(s01), cc[0], acc[t][0]);
        acc[t][1] = __builtin_fmaf(half_bits_to_float(s01 >> 16), cc[1], acc[t][1]);
        acc[t][2] = __builtin_fmaf(half_bits_to_float(s23), cc[2], acc[t][2]);
        acc[t][3] = __builtin_fmaf(half_bits_to_float(s23 >> 16), cc[3], acc[t][3]);
      }
    }
  }
  if (c == 0)
#pragma unroll
    for (int t = 0; t < NRT; t++) g.red[t][wave][G] = acc[t];
  __syncthreads();
  if (wave < NRT && c == 0) {
    const int t = wave;
    f32x4 gs = g.red[t][0][G], us = g.red[t][kGuSplit][G];
    for (int w = 1; w < kGuSplit; w++) {
      gs += g.red[t][w][G];
      us += g.red[t][kGuSplit + w][G];
    }
    uint32_t hw4[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float gv = gs[i];
      const float h = gv / (1.0f + expf(-gv)) * us[i];
      const uint32_t hb = f32_to_bf16_rne(h);
      const uint32_t lb = f32_to_bf16_rne(h - bf16_bits_to_f32(hb));
      hw4[i] = hb | (lb << 16);
    }
    const int off = (int)(((int64_t)slot * a.F + 16 * (rt0 + t) + 4 * G) * 4);
    st_dev_x4(buffer_of(a.hw), off, make_uint4(hw4[0], hw4[1], hw4[2], hw4[3]));
  }
}

// The whole role: only the DMA is waited for before the MFMAs (each tile's
// MFMAs start when its words have landed).
template <int NRT>
__device__ void gate_up_role(const DecodeArgs& a, const uint8_t* ex, int slot, int rt0, ExpertsLds& sh) {
  u32x4 nib[NRT][kGuMaxKg];
  gate_up_issue<NRT>(a, ex, rt0, sh, true, nib);
  build_pair_table(sh.tbl);
  wait_dma_before<NRT * kGuMaxKg>();
  __syncthreads();
  gate_up_compute<NRT>(a, slot, rt0, sh, nib);
}

// ---------------------------------------------------------------- down role

// this wave's down tile (row tile rt, tile kg) of routed slot S (S >= K
// repeats slot 0; those values are not used)
template <int S>
__device__ __forceinline__ void load_routed_slots(const DecodeArgs& a, const RouteLds& r, u32x4 (&nib)[kDnSlots], int rt,
                                                  int kg, int nkg) {
  if constexpr (S < kMaxDecodeK) {
    const int64_t mat_bytes = a.expert_bytes / 3;
    const uint8_t* down = a.arena + (int64_t)r.ids[S < a.K ? S : 0] * a.expert_bytes + 2 * mat_bytes;
    nib[S] = ld16(down + ((int64_t)rt * nkg + kg) * kTileBytes + 16 * (threadIdx.x & 63));
    load_routed_slots<S + 1>(a, r, nib, rt, kg, nkg);
  }
}

// The scale pieces of one expert's two row tiles (2 x 8 kg x 8 pieces of 16
// bytes) into d.scales[slot] by LDS DMA, half per wavefront (half = 0, 1).
// Pieces of kg >= nkg repeat a valid one and are never read.
__device__ __forceinline__ void dma_slot_scales(DownLds& d, const uint8_t* down_rows, int nkg, int slot, int half) {
  const int p = 64 * half + (threadIdx.x & 63);
  const int rtl = p >> 6, kg = min((p >> 3) & 7, nkg - 1);
  dma16_stream(down_rows + ((int64_t)rtl * nkg + kg) * kTileBytes + kTileNibbleBytes + 16 * (p & 7),
               &d.scales[slot][0][0][0] + 256 * half);
}

// MFMAs of slot S over this wave's tile.  Column 0 of the B operand carries
// bf16(h), column 1 bf16(h - bf16(h)) (the other columns repeat column 0 and
// are not used): one MFMA per block gives both products, each lane
// accumulates d * C of its column, and column 0 + column 1 of the C rows is
// this wave's partial, written to d.part.
template <int S>
__device__ __forceinline__ void down_slot(ExpertsLds& sh, const u32x4 (&nib)[kDnSlots], int rtl, int kg) {
  DownLds& d = sh.u.d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, G = lane >> 4;
  const uint16_t* hp = c == 1 ? d.hl[S] : d.hh[S];
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int b = 0; b < 4; b++) {
    const bf16x8 bop = *reinterpret_cast<const bf16x8*>(hp + 32 * (4 * kg + b) + 8 * G);
    const bf16x8 wa = decode_word(sh.tbl, uword(nib[S], b), lane & 31);
    const uint32_t s01 = d.scales[S][rtl][kg][8 * G + 2 * b];
    const uint32_t s23 = d.scales[S][rtl][kg][8 * G + 2 * b + 1];
    const f32x4 cc = mfma16x16x32(wa, bop, zero);
    acc[0] = __builtin_fmaf(half_bits_to_float(s01), cc[0], acc[0]);
    acc[1] = __builtin_fmaf(half_bits_to_float(s01 >> 16), cc[1], acc[1]);
    acc[2] = __builtin_fmaf(half_bits_to_float(s23), cc[2], acc[2]);
    acc[3] = __builtin_fmaf(half_bits_to_float(s23 >> 16), cc[3], acc[3]);
  }
#pragma unroll
  for (int j = 0; j < 4; j++) acc[j] += lane_next_in_row(acc[j]);
  if (c == 0) *reinterpret_cast<f32x4*>(&d.part[wave][S][4 * G]) = acc;
}

// Routed slots S.. in order (slots >= K are skipped).
template <int S>
__device__ __forceinline__ void down_routed_slots(const DecodeArgs& a, ExpertsLds& sh, const u32x4 (&nib)[kDnSlots],
                                                  int rtl, int kg) {
  if constexpr (S < kMaxDecodeK) {
    if (S < a.K) down_slot<S>(sh, nib, rtl, kg);
    down_routed_slots<S + 1>(a, sh, nib, rtl, kg);
  }
}

// Rows first .. first+n-1 of the h words (row r = slot r; row K = the shared
// expert, kept in LDS slot kMaxDecodeK), read until complete -- each thread
// one 16-byte piece, all requested together, re-read while one shows the
// "not ready" pattern -- and split into the two bf16 planes.
__device__ __forceinline__ void poll_h_rows(const DecodeArgs& a, DownLds& d, int first, int n) {
  const __amdgpu_buffer_rsrc_t rh = buffer_of(a.hw);
  const int row_pieces = a.F >> 2;
  const int p = threadIdx.x;
  if (p >= n * row_pieces) return;
  const int row = first + p / row_pieces, e0 = 4 * (p % row_pieces);
  const int off = (row * a.F + e0) * 4;
  uint4 v = ld_dev_x4(rh, off);
  uint32_t it = 0;
  while (!ready(v)) {
    if (give_up(a.err, ++it)) {
      st_dev(buffer_of(a.err), 0, 1u);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    v = ld_dev_x4(rh, off);
  }
  const int slot = row < a.K ? row : kMaxDecodeK;
  *reinterpret_cast<uint2*>(&d.hh[slot][e0]) =
      make_uint2((v.x & 0xffffu) | (v.y << 16), (v.z & 0xffffu) | (v.w << 16));
  *reinterpret_cast<uint2*>(&d.hl[slot][e0]) =
      make_uint2((v.x >> 16) | (v.y & 0xffff0000u), (v.z >> 16) | (v.w & 0xffff0000u));
}

// The shared expert's down rows y_s[H] (fp32 bits) follow the h words of the
// K + 1 slots in the same hand-off buffer.
__device__ __forceinline__ uint32_t* shared_y(const DecodeArgs& a) { return a.hw + (a.K + 1) * a.F; }

// Word i of a hand-off array, re-read until it no longer shows the "not
// ready" pattern (bounded, like every wait).
__device__ __forceinline__ uint32_t poll_word(const DecodeArgs& a, const uint32_t* base, int i) {
  const __amdgpu_buffer_rsrc_t rb = buffer_of(base);
  uint32_t v = ld_dev(rb, 4 * i);
  uint32_t it = 0;
  while (v == kNotReady) {
    if (give_up(a.err, ++it)) {
      st_dev(buffer_of(a.err), 0, 1u);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    v = ld_dev(rb, 4 * i);
  }
  return v;
}

// The shared expert's down projection, spread over the shared workgroups
// after their gate/up row tile (so that the down workgroups only wait for the
// routed slots): workgroup blk takes q = ceil((H/16) / (F/16)) <= 4 row tiles
// of H from tile q * blk.  Item i = wave + 16 j is (row tile i / nkg, packed
// tile kg = i % nkg).  It waits for the shared expert's whole h, then
// publishes its rows of y_s with device-scope stores, in the arithmetic of the
// down role's slots: each item's 4 blocks in order (scale times MFMA result,
// fused), the two B columns added, the items of a row added in kg order.
constexpr int kShDnMaxTiles = 4;
constexpr int kShDnItems = kShDnMaxTiles * (kMaxDecodeFfn / 128) / kDecWaves;
static_assert(kShDnMaxTiles <= 2 * kDnSlots, "row tile t's scale pieces in d.scales[t / 2][t % 2]");
static_assert(kShDnMaxTiles * (kMaxDecodeFfn / 128) * 16 <= kDecWaves * kDnSlots * 16, "the parts fit in d.part");
static_assert(kShDnMaxTiles * (kMaxDecodeFfn / 128) <= kShDnItems * kDecWaves, "the items fit the waves");

__device__ void shared_down_part(const DecodeArgs& a, int blk, ExpertsLds& sh) {
  DownLds& d = sh.u.d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, G = lane >> 4;
  const int nkg = a.F >> 7;
  const int n_rt = a.H >> 4;
  const int q = (n_rt + a.n_shared_wg - 1) / a.n_shared_wg;
  const int t0 = blk * q, nt = max(0, min(q, n_rt - t0));
  const int n_items = nt * nkg;
  const uint8_t* down = a.shared + 2 * (a.expert_bytes / 3);
  // row tile t's scale pieces in d.scales[t / 2][t % 2], its items' parts in
  // part[t][kg][16] (a view of d.part)
  float(*part)[kMaxDecodeFfn / 128][16] = reinterpret_cast<float(*)[kMaxDecodeFfn / 128][16]>(&d.part[0][0][0]);
  u32x4 nib[kShDnItems];
#pragma unroll
  for (int j = 0; j < kShDnItems; j++) {
    const int i = wave + kDecWaves * j;
    if (i < n_items) nib[j] = ld16(down + ((int64_t)(t0 + i / nkg) * nkg + i % nkg) * kTileBytes + 16 * lane);
  }
  if (wave < nt) dma_slot_scales(d, down + (int64_t)(t0 + (wave & ~1)) * nkg * kTileBytes, nkg, wave >> 1, wave & 1);
  poll_h_rows(a, d, a.K, 1);
  wait_loads();
  __syncthreads();
  const uint16_t* hp = c == 1 ? d.hl[kMaxDecodeK] : d.hh[kMaxDecodeK];
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kShDnItems; j++) {
    const int i = wave + kDecWaves * j;
    if (i < n_items) {
      const int t = i / nkg, kg = i % nkg;
      f32x4 acc = zero;
#pragma unroll
      for (int b = 0; b < 4; b++) {
        const bf16x8 bop = *reinterpret_cast<const bf16x8*>(hp + 32 * (4 * kg + b) + 8 * G);
        const bf16x8 wa = decode_word(sh.tbl, uword(nib[j], b), lane & 31);
        const uint32_t s01 = d.scales[t >> 1][t & 1][kg][8 * G + 2 * b];
        const uint32_t s23 = d.scales[t >> 1][t & 1][kg][8 * G + 2 * b + 1];
        const f32x4 cc = mfma16x16x32(wa, bop, zero);
        acc[0] = __builtin_fmaf(half_bits_to_float(s01), cc[0], acc[0]);
        acc[1] = __builtin_fmaf(half_bits_to_float(s01 >> 16), cc[1], acc[1]);
        acc[2] = __builtin_fmaf(half_bits_to_float(s23), cc[2], acc[2]);
        acc[3] = __builtin_fmaf(half_bits_to_float(s23 >> 16), cc[3], acc[3]);
      }
#pragma unroll
      for (int k = 0; k < 4; k++) acc[k] += lane_next_in_row(acc[k]);
      if (c == 0) *reinterpret_cast<f32x4*>(&part[t][kg][4 * G]) = acc;
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < nt * 16) {
    const int t = threadIdx.x >> 4, r16 = threadIdx.x & 15;
    float y = 0.0f;
    for (int kg = 0; kg < nkg; kg++) y += part[t][kg][r16];
    st_dev(buffer_of(shared_y(a)), 4 * (16 * (t0 + t) + r16), __float_as_uint(y));
  }
}

// Down of 32 rows of H over the routed slots, then the slot-order combine
// with the shared expert's rows, which come finished from the shared
// workgroups (shared_down_part) and are waited for.
__device__ void down_role(const DecodeArgs& a, int blk, ExpertsLds& sh) {
  DownLds& d = sh.u.d;
  RouteLds& r = sh.route;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rtl = wave & 1, kg = wave >> 1;
  const int rt = 2 * blk + rtl;  // this wave's 16 rows of H
  const int nkg = a.F >> 7;
  const bool has_tile = kg < nkg;
  const int kgc = has_tile ? kg : nkg - 1;
  const int64_t mat_bytes = a.expert_bytes / 3;

  auto down_tiles = [&](const uint8_t* ex, int rtile) {
    return ex + 2 * mat_bytes + (int64_t)rtile * nkg * kTileBytes;
  };
  u32x4 nib[kDnSlots];
  // 1. the router scores (and the shared expert's gate), routing, then the
  //    routed experts' tiles
  const RouteIn rin = route_fetch(a);
  const float gate = a.gated ? a.scores[a.E] : 1.0f;
  build_pair_table(sh.tbl);
  route_rank_lds(a, r, rin);
  load_routed_slots<0>(a, r, nib, rt, kgc, nkg);
  if (wave >= 2 && wave < 2 + 2 * a.K) {
    const int slot = (wave - 2) >> 1;
    dma_slot_scales(d, down_tiles(a.arena + (int64_t)r.ids[slot] * a.expert_bytes, 2 * blk), nkg, slot, wave & 1);
  }
  // 2. h of the routed slots and their MFMAs
  static_assert(kMaxDecodeK * (kMaxDecodeFfn / 4) <= kDecThreads, "one h piece per thread");
  poll_h_rows(a, d, 0, a.K);
  wait_loads();
  __syncthreads();
  if (has_tile) down_routed_slots<0>(a, sh, nib, rtl, kg);
  __syncthreads();
  // 3. the wave parts of each (row tile, slot) added in order
  for (int i = threadIdx.x; i < kMaxDecodeK * 32; i += kDecThreads) {
    const int s2 = i >> 5, row = i & 31, rt2 = row >> 4, r16 = row & 15;
    if (s2 < a.K) {
      float t = 0.0f;
      for (int q = 0; q < nkg; q++) t += d.part[rt2 + 2 * q][s2][r16];
      d.y[s2][row] = t;
    }
  }
  __syncthreads();
  // 4. slot-order combine of these 32 rows, the shared expert's row last
  if (threadIdx.x < 32) {
    const int row = threadIdx.x;
    float acc = 0.0f;
    for (int k = 0; k < a.K; k++) acc = __builtin_fmaf(r.w[k], d.y[k][row], acc);
    if (a.n_shared) {
      const float ys = __uint_as_float(poll_word(a, shared_y(a), 32 * blk + row));
      acc = a.gated ? __builtin_fmaf(gate, ys, acc) : acc + ys;
    }
    a.out[32 * blk + row] = acc;
  }
  // the routing outputs, written once (w[K]: the shared expert's gate)
  if (blk == 0 && (int)threadIdx.x < a.K) {
    a.ids[threadIdx.x] = r.ids[threadIdx.x];
    a.w[threadIdx.x] = r.w[threadIdx.x];
  }
  if (blk == 0 && a.gated && (int)threadIdx.x == a.K) a.w[a.K] = gate;
}

// ---------------------------------------------------------------- kernel 2: experts

__global__ __launch_bounds__(kDecThreads, 8) void k_decode_experts(DecodeArgs a) {
  __shared__ ExpertsLds sh;
  int blk = blockIdx.x;
  const int n_rt_f = a.F >> 4;
  // Block order: routed gate/up, shared gate/up (then the shared expert's
  // down rows, which wait for the h of every shared workgroup), down.  The
  // waits cross workgroups both ways, so the whole grid must be resident at
  // once (the plan checks it).
  // Workgroups are placed in block order, one per CU first: the routed ones,
  // whose first request is the router scores, get a CU of their own, so that
  // request does not queue behind another workgroup's weight tiles.
  if (blk < a.n_routed_wg) {
    const int slot = blk / n_rt_f, rt = blk % n_rt_f;
    route_local(a, sh.route);
    gate_up_role<1>(a, a.arena + (int64_t)sh.route.ids[slot] * a.expert_bytes, slot, rt, sh);
  } else if ((blk -= a.n_routed_wg) < a.n_shared_wg) {
    // The shared expert's gate/up, then its down rows, is one of the two
    // longest chains of the call, and each of these workgroups shares a CU
    // with a routed one: its waves issue first while their tiles stream.
    // Raising the whole branch (the polling of h as well) starves the
    // routed partner and is slower.
    __builtin_amdgcn_s_setprio(3);
    gate_up_role<1>(a, a.shared, a.K, blk, sh);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();  // the gate/up LDS is reused
    shared_down_part(a, blk, sh);
  } else {
    down_role(a, blk - a.n_shared_wg, sh);
  }
}

namespace {

int decode_grid_size(int F, int K, int H, int n_shared) { return (n_shared ? F / 16 : 0) + K * (F / 16) + H / 32; }

}  // namespace

// Workgroups of k_decode_experts that one device holds at once (0 if unknown),
// cached per device: the kernel's resources do not depend on the shape.
static std::atomic<int> g_decode_capacity[64];

bool decode_grid_coresident(int F, int K, int H, int n_shared) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    clear_last_error();
    return false;
  }
  int cap = g_decode_capacity[dev].load(std::memory_order_relaxed);
  if (cap == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k_decode_experts),
                                                     kDecThreads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      clear_last_error();
      return false;
    }
    cap = per_cu * cus > 0 ? per_cu * cus : -1;  // -1: known not to fit anything
    g_decode_capacity[dev].store(cap, std::memory_order_relaxed);
  }
  return cap > 0 && decode_grid_size(F, K, H, n_shared) <= cap;
}

hipError_t launch_layer_decode(DecodeArgs a, hipStream_t stream) {
  a.n_router = a.E + a.gated;  // one wavefront per router row
  a.n_shared_wg = a.n_shared ? a.F / 16 : 0;
  a.n_routed_wg = a.K * (a.F / 16);
  a.n_down_wg = a.H / 32;
  clear_last_error();
  if (a.x_prev)
    hipLaunchKernelGGL(k_decode_scores_chained<kMaxDecodeHidden / 256>, dim3(a.n_router), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(k_decode_scores<kMaxDecodeHidden / 256>, dim3(a.n_router), dim3(64), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  clear_last_error();
  hipLaunchKernelGGL(k_decode_experts, dim3(a.n_shared_wg + a.n_routed_wg + a.n_down_wg), dim3(kDecThreads), 0,
                     stream, a);
  return hipGetLastError();
}

__global__ void k_fill_u32(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

__global__ void k_copy_u32(const uint32_t* src, uint32_t* dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

hipError_t launch_copy_words(const uint32_t* src, uint32_t* dst, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  clear_last_error();
  hipLaunchKernelGGL(k_copy_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, src, dst, n);
  return hipGetLastError();
}

hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  clear_last_error();
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace qmoe
