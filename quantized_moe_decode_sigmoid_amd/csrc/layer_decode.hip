// The MoE layer for one decode token (T = 1) in two launches.
//
// Same arithmetic as the multi-kernel path (router_math.h; exact IQ4_NL
// weights on v_mfma_f32_16x16x32_bf16, see ffn_exact.hip) -- the outputs are
// bit-identical to it -- organised for latency:
//
//   k_decode_scores   one wavefront (workgroup) per expert: fp32 logit and
//                     sigmoid score.
//                     It also writes the "not ready" pattern into the words
//                     through which the next kernel hands h from its gate/up
//                     workgroups to its down workgroups; the previous token's
//                     second kernel has finished, so nobody reads them now.
//   k_decode_experts  roles by block index:
//     [shared]  gate/up + SiLU*up of the shared expert, one 16-row tile of F;
//     [routed]  gate/up + SiLU*up of routed slot k, one 16-row tile of F;
//     [down]    32 rows of H: down projection of every slot and of the shared
//               expert, then the slot-order combine of those rows.
//   Every workgroup that needs the routing ranks the E scores itself (top-K
//   in LDS), so there is no hand-off for it.  The down workgroups request
//   their weight tiles as soon as they know the experts, then read the h
//   words of the gate/up workgroups, repeating a read while it still shows
//   the "not ready" pattern (a finite h never has it).  Each h word is written
//   once with one device-scope store, so a word that is not "not ready" is
//   complete: no counter, atomic or fence is involved.
//
// Every global load of a role is issued before its result is first used and
// none sits behind a runtime branch (indices are clamped, unused values
// discarded), so a wavefront has its HBM requests in flight together.
// Operands shared by all wavefronts of a workgroup (x, block scales, h) are
// staged once in LDS with coalesced loads.  Every wait is bounded: one that
// exceeds the bound sets an error word and gives up, so a launch always ends.
#include "device.h"
#include "launch.h"
#include "router_math.h"

namespace qmoe {

constexpr int kDecThreads = 512;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kGuMaxKg = kMaxDecodeHidden / 128 / 4;  // gate/up tiles per wave (8)
constexpr int kDnMaxKg = kMaxDecodeFfn / 128 / 4;     // down tiles per wave and expert (2)
constexpr int kDnSlots = kMaxDecodeK + 1;             // routed slots + shared
constexpr uint32_t kNotReady = 0xffffffffu;           // an h word before it is written
constexpr uint32_t kPollLimit = 1u << 20;

// ---------------------------------------------------------------- device-scope access

// 16 bytes at byte offset off of a buffer, read through to device scope.
__device__ __forceinline__ uint4 ld_dev_x4(__amdgpu_buffer_rsrc_t r, int off) {
  constexpr int kDeviceScope = 16;  // cache-policy bit: device coherence
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kDeviceScope));
}

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

__device__ __forceinline__ void st_dev_x4(__amdgpu_buffer_rsrc_t r, int off, uint4 v) {
  constexpr int kDeviceScope = 16;
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, off, 0, kDeviceScope);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

__device__ __forceinline__ bool ready(uint4 v) {
  return v.x != kNotReady && v.y != kNotReady && v.z != kNotReady && v.w != kNotReady;
}

// ---------------------------------------------------------------- LDS

constexpr int kScaleWords = 32;  // 64 fp16 scales of a tile

struct RouteLds {
  float sel[256];
  float score[256];
  float sval[kMaxDecodeK];
  float w[kMaxDecodeK];
  int32_t ids[kMaxDecodeK];
};

struct GateUpLds {
  uint16_t x[kMaxDecodeHidden];                             // the token's activations
  uint32_t scales[2][kMaxDecodeHidden / 128][kScaleWords];  // [gate/up][kg] of this row tile
  f32x4 red[kDecWaves][64];
};

struct DownLds {
  uint32_t h[kDnSlots][kMaxDecodeFfn];                             // bf16 hi | lo << 16 per element
  uint32_t scales[kDnSlots][2][kMaxDecodeFfn / 128][kScaleWords];  // [slot][rtl][kg]
  float part[kDecWaves][kDnSlots][16];                             // column 0 of each wave's partial
  float y[kDnSlots][32];
};

struct ExpertsLds {
  uint32_t tbl[kPairTableWords];
  RouteLds route;
  union {
    GateUpLds g;
    DownLds d;
  } u;
};

// ---------------------------------------------------------------- kernel 1: scores

template <int MMAX>
__global__ __launch_bounds__(64) void k_decode_scores(DecodeArgs a) {
  const int lane = threadIdx.x;
  const int e = blockIdx.x;
  // reset the h hand-off words of k_decode_experts
  const int n_words = (a.K + 1) * a.F;
  for (int i = blockIdx.x * 64 + threadIdx.x; i < n_words; i += gridDim.x * 64) a.hw[i] = kNotReady;
  if (e < a.E) {
    float4 w[MMAX];
    load_router_row<MMAX>(a.wg + (size_t)e * a.H, a.H, lane, w);
    const float p = router_logit<MMAX>(a.x, a.H, lane, w);
    if (lane == 0) a.scores[e] = sigmoid_fixed(p);
  }
}

// ---------------------------------------------------------------- routing in each workgroup

// Top-K of the E scores into r (ids, unbiased scores, weights), by rank: expert
// e takes slot rank(e) when rank(e) < K, rank = number of experts before it in
// the (selection score, index) order.
__device__ void route_local(const DecodeArgs& a, RouteLds& r) {
  const int e = threadIdx.x;
  if (e < a.E) {
    const float s = a.scores[e];
    r.score[e] = s;
    r.sel[e] = a.bias ? s + a.bias[e] : s;
  }
  __syncthreads();
  if (e < a.E) {
    const float se = r.sel[e];
    int rank = 0;
#pragma unroll 8
    for (int q = 0; q < a.E; q++) rank += sel_before(r.sel[q], q, se, e);
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

// ---------------------------------------------------------------- gate / up role

// waves 0-3: W_gate over quarters of the blocks of H; waves 4-7: W_up.
// h of (row 16rt + 4G + i) is written to hw[slot][...] as bf16 hi | lo << 16.
__device__ void gate_up_role(const DecodeArgs& a, const uint8_t* ex, int slot, int rt, ExpertsLds& sh) {
  GateUpLds& g = sh.u.g;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, G = lane >> 4;
  const int64_t mat_bytes = a.expert_bytes / 3;
  const int nkg = a.H >> 7;
  const int q = wave & 3, mat = wave >> 2;
  const int kg0 = (q * nkg) >> 2, nk = (((q + 1) * nkg) >> 2) - kg0;
  const uint8_t* rowtiles = ex + (int64_t)rt * nkg * kTileBytes;  // gate; up is mat_bytes further

  // 1. this wave's nibble words, the row tile's scales, the activations: all requested now
  u32x4 nib[kGuMaxKg];
#pragma unroll
  for (int i = 0; i < kGuMaxKg; i++) {
    const int kg = min(kg0 + i, nkg - 1);
    nib[i] = ld16(rowtiles + mat * mat_bytes + (int64_t)kg * kTileBytes + 16 * lane);
  }
  const int n_scale = 2 * nkg * 8;
  const int sp = (int)threadIdx.x < n_scale ? (int)threadIdx.x : 0;
  const int sp_m = sp / (nkg * 8), sp_kg = (sp >> 3) % nkg, sp_part = sp & 7;
  const u32x4 sv = ld16(rowtiles + sp_m * mat_bytes + (int64_t)sp_kg * kTileBytes + kTileNibbleBytes + 16 * sp_part);
  const int xp = (int)threadIdx.x < (a.H >> 3) ? (int)threadIdx.x : 0;
  const u32x4 xv = ld16(a.x + 8 * xp);
  build_pair_table(sh.tbl);
  if ((int)threadIdx.x < n_scale) *reinterpret_cast<u32x4*>(&g.scales[sp_m][sp_kg][4 * sp_part]) = sv;
  if ((int)threadIdx.x < (a.H >> 3)) *reinterpret_cast<u32x4*>(&g.x[8 * xp]) = xv;
  __syncthreads();

  // 2. MFMAs: every column carries the token (a broadcast operand), column 0
  //    is kept; acc[i] (row 4G+i) += d * (levels . x).  Tiles past this
  //    wave's range are computed and dropped by a select (no branch).
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc = zero;
#pragma unroll
  for (int i = 0; i < kGuMaxKg; i++) {
    const bool take = i < nk;
    const int kg = min(kg0 + i, nkg - 1);
    bf16x8 xb[4], wa[4];
    uint32_t s01[4], s23[4];
#pragma unroll
    for (int b = 0; b < 4; b++) {
      xb[b] = *reinterpret_cast<const bf16x8*>(&g.x[32 * (4 * kg + b) + 8 * G]);
      wa[b] = decode_word(sh.tbl, uword(nib[i], b), lane & 31);
      s01[b] = g.scales[mat][kg][8 * G + 2 * b];
      s23[b] = g.scales[mat][kg][8 * G + 2 * b + 1];
    }
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const f32x4 cc = mfma16x16x32(wa[b], xb[b], zero);
      f32x4 nx;
      nx[0] = __builtin_fmaf(half_bits_to_float(s01[b]), cc[0], acc[0]);
      nx[1] = __builtin_fmaf(half_bits_to_float(s01[b] >> 16), cc[1], acc[1]);
      nx[2] = __builtin_fmaf(half_bits_to_float(s23[b]), cc[2], acc[2]);
      nx[3] = __builtin_fmaf(half_bits_to_float(s23[b] >> 16), cc[3], acc[3]);
      acc = take ? nx : acc;
    }
  }
  g.red[wave][lane] = acc;
  __syncthreads();
  // 3. wave 0, column 0: g and u summed in wave order, h = silu(g) * u
  if (wave == 0 && c == 0) {
    f32x4 gs = g.red[0][lane], us = g.red[4][lane];
    for (int w = 1; w < 4; w++) {
      gs += g.red[w][lane];
      us += g.red[4 + w][lane];
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
    const int off = (int)(((int64_t)slot * a.F + 16 * rt + 4 * G) * 4);
    st_dev_x4(buffer_of(a.hw), off, make_uint4(hw4[0], hw4[1], hw4[2], hw4[3]));
  }
}

// ---------------------------------------------------------------- down role

// the down tiles of routed slot S (S >= K repeats slot 0; those values are not used)
template <int S>
__device__ __forceinline__ void load_routed_slots(const DecodeArgs& a, const RouteLds& r, u32x4 (&nib)[kDnSlots][kDnMaxKg],
                                                  u32x4 (&scv)[kDnSlots], int rt, int rt_scale, int kg0, int nkg,
                                                  int sp_kg, int sp_part) {
  if constexpr (S < kMaxDecodeK) {
    const int64_t mat_bytes = a.expert_bytes / 3;
    const uint8_t* down = a.arena + (int64_t)r.ids[S < a.K ? S : 0] * a.expert_bytes + 2 * mat_bytes;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < kDnMaxKg; i++)
      nib[S][i] = ld16(down + ((int64_t)rt * nkg + min(kg0 + i, nkg - 1)) * kTileBytes + 16 * lane);
    scv[S] = ld16(down + ((int64_t)rt_scale * nkg + sp_kg) * kTileBytes + kTileNibbleBytes + 16 * sp_part);
    load_routed_slots<S + 1>(a, r, nib, scv, rt, rt_scale, kg0, nkg, sp_kg, sp_part);
  }
}

// the scale pieces of every slot into LDS (static slot indices keep scv in registers)
template <int S>
__device__ __forceinline__ void store_slot_scales(DownLds& d, const u32x4 (&scv)[kDnSlots], int rtl, int kg, int part) {
  if constexpr (S < kDnSlots) {
    *reinterpret_cast<u32x4*>(&d.scales[S][rtl][kg][4 * part]) = scv[S];
    store_slot_scales<S + 1>(d, scv, rtl, kg, part);
  }
}

// MFMAs of slot S for this wave's quarter of F (column 0 kept; every column
// carries the same broadcast h operand); the partial goes to d.part.
template <int S>
__device__ __forceinline__ void down_slots(const DecodeArgs& a, ExpertsLds& sh, const u32x4 (&nib)[kDnSlots][kDnMaxKg],
                                           int kg0, int nk, int nkg) {
  if constexpr (S < kDnSlots) {
    DownLds& d = sh.u.d;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane & 15, G = lane >> 4, rtl = wave & 1;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc = zero;
#pragma unroll
    for (int i = 0; i < kDnMaxKg; i++) {
      const bool take = i < nk;
      const int kg = min(kg0 + i, nkg - 1);
      bf16x8 bh[4], bl[4], wa[4];
      uint32_t s01[4], s23[4];
#pragma unroll
      for (int b = 0; b < 4; b++) {
        const int b32 = 4 * kg + b;
        // elements 32 b32 + 8G .. + 7 as (hi, lo) bf16 pairs
        const u32x4 p0 = *reinterpret_cast<const u32x4*>(&d.h[S][32 * b32 + 8 * G]);
        const u32x4 p1 = *reinterpret_cast<const u32x4*>(&d.h[S][32 * b32 + 8 * G + 4]);
        union {
          uint32_t u[4];
          bf16x8 v;
        } oh, ol;
        oh.u[0] = (p0[0] & 0xffffu) | (p0[1] << 16);
        oh.u[1] = (p0[2] & 0xffffu) | (p0[3] << 16);
        oh.u[2] = (p1[0] & 0xffffu) | (p1[1] << 16);
        oh.u[3] = (p1[2] & 0xffffu) | (p1[3] << 16);
        ol.u[0] = (p0[0] >> 16) | (p0[1] & 0xffff0000u);
        ol.u[1] = (p0[2] >> 16) | (p0[3] & 0xffff0000u);
        ol.u[2] = (p1[0] >> 16) | (p1[1] & 0xffff0000u);
        ol.u[3] = (p1[2] >> 16) | (p1[3] & 0xffff0000u);
        bh[b] = oh.v;
        bl[b] = ol.v;
        wa[b] = decode_word(sh.tbl, uword(nib[S][i], b), lane & 31);
        s01[b] = d.scales[S][rtl][kg][8 * G + 2 * b];
        s23[b] = d.scales[S][rtl][kg][8 * G + 2 * b + 1];
      }
#pragma unroll
      for (int b = 0; b < 4; b++) {
        f32x4 cc = mfma16x16x32(wa[b], bh[b], zero);
        cc = mfma16x16x32(wa[b], bl[b], cc);
        f32x4 nx;
        nx[0] = __builtin_fmaf(half_bits_to_float(s01[b]), cc[0], acc[0]);
        nx[1] = __builtin_fmaf(half_bits_to_float(s01[b] >> 16), cc[1], acc[1]);
        nx[2] = __builtin_fmaf(half_bits_to_float(s23[b]), cc[2], acc[2]);
        nx[3] = __builtin_fmaf(half_bits_to_float(s23[b] >> 16), cc[3], acc[3]);
        acc = take ? nx : acc;
      }
    }
    if (c == 0) *reinterpret_cast<f32x4*>(&d.part[wave][S][4 * G]) = acc;
    down_slots<S + 1>(a, sh, nib, kg0, nk, nkg);
  }
}

__device__ void down_role(const DecodeArgs& a, int blk, ExpertsLds& sh) {
  DownLds& d = sh.u.d;
  RouteLds& r = sh.route;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, G = lane >> 4;
  const int rtl = wave & 1, q = wave >> 1;
  const int rt = 2 * blk + rtl;
  (void)rtl;
  const int nkg = a.F >> 7;
  const int kg0 = (q * nkg) >> 2, nk = (((q + 1) * nkg) >> 2) - kg0;
  const int64_t mat_bytes = a.expert_bytes / 3;
  const int n_rows = a.K + a.n_shared;  // h rows: routed slots 0..K-1, then the shared expert at K
  const int n_pieces = 2 * nkg * 8;     // 16-byte scale pieces of this workgroup's tiles of one expert
  const int sp = (int)threadIdx.x < n_pieces ? (int)threadIdx.x : 0;
  const int sp_rtl = sp / (nkg * 8), sp_kg = (sp >> 3) % nkg, sp_part = sp & 7;

  auto down_tiles = [&](const uint8_t* ex, int rtile) {
    return ex + 2 * mat_bytes + (int64_t)rtile * nkg * kTileBytes;
  };
  u32x4 nib[kDnSlots][kDnMaxKg];
  u32x4 scv[kDnSlots];
  // 1. the shared expert's tiles need no routing: request them first
  const uint8_t* shx = a.n_shared ? a.shared : a.arena;
#pragma unroll
  for (int i = 0; i < kDnMaxKg; i++)
    nib[kMaxDecodeK][i] = ld16(down_tiles(shx, rt) + (int64_t)min(kg0 + i, nkg - 1) * kTileBytes + 16 * lane);
  scv[kMaxDecodeK] = ld16(down_tiles(shx, 2 * blk + sp_rtl) + (int64_t)sp_kg * kTileBytes + kTileNibbleBytes + 16 * sp_part);
  build_pair_table(sh.tbl);
  // 2. routing, then the routed experts' tiles
  route_local(a, r);
  load_routed_slots<0>(a, r, nib, scv, rt, 2 * blk + sp_rtl, kg0, nkg, sp_kg, sp_part);
  if ((int)threadIdx.x < n_pieces) store_slot_scales<0>(d, scv, sp_rtl, sp_kg, sp_part);
  // 3. h of every slot, read until complete: each thread requests all its
  //    pieces, then re-reads the ones still "not ready"
  {
    const __amdgpu_buffer_rsrc_t rh = buffer_of(a.hw);
    const int row_pieces = a.F >> 2;  // 16-byte pieces per row
    const int n_total = n_rows * row_pieces;
    constexpr int kMaxPieces = (kDnSlots * kMaxDecodeFfn / 4 + kDecThreads - 1) / kDecThreads;
    uint4 v[kMaxPieces];
    int boff[kMaxPieces];
#pragma unroll
    for (int j = 0; j < kMaxPieces; j++) {
      const int p = min((int)threadIdx.x + j * kDecThreads, n_total - 1);
      boff[j] = (p / row_pieces * a.F + 4 * (p % row_pieces)) * 4;
      v[j] = ld_dev_x4(rh, boff[j]);
    }
    uint32_t it = 0;
    bool all = false;
    while (!all) {
      all = true;
#pragma unroll
      for (int j = 0; j < kMaxPieces; j++) all = all && ready(v[j]);
      if (all) break;
      if (++it > kPollLimit) {
        a.err[0] = 1u;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int j = 0; j < kMaxPieces; j++)
        if (!ready(v[j])) v[j] = ld_dev_x4(rh, boff[j]);
    }
#pragma unroll
    for (int j = 0; j < kMaxPieces; j++) {
      const int p = (int)threadIdx.x + j * kDecThreads;
      if (p < n_total) {
        const int row = p / row_pieces;
        *reinterpret_cast<uint4*>(&d.h[row < a.K ? row : kMaxDecodeK][4 * (p % row_pieces)]) = v[j];
      }
    }
  }
  __syncthreads();
  // 4. every slot's MFMAs, then the four quarters of each (row tile, slot)
  //    added in order
  {
    down_slots<0>(a, sh, nib, kg0, nk, nkg);
    __syncthreads();
    for (int i = threadIdx.x; i < kDnSlots * 32; i += kDecThreads) {
      const int s2 = i >> 5, row = i & 31, rt2 = row >> 4, r16 = row & 15;
      float t = d.part[rt2][s2][r16];
      for (int qq = 1; qq < 4; qq++) t += d.part[rt2 + 2 * qq][s2][r16];
      d.y[s2][row] = t;
    }
    __syncthreads();
  }
  // 5. slot-order combine of these 32 rows
  if (threadIdx.x < 32) {
    const int row = threadIdx.x;
    float acc = 0.0f;
    for (int k = 0; k < a.K; k++) acc = __builtin_fmaf(r.w[k], d.y[k][row], acc);
    if (a.n_shared) acc += d.y[kMaxDecodeK][row];
    a.out[32 * blk + row] = acc;
  }
  // the routing outputs, written once
  if (blk == 0 && (int)threadIdx.x < a.K) {
    a.ids[threadIdx.x] = r.ids[threadIdx.x];
    a.w[threadIdx.x] = r.w[threadIdx.x];
  }
}

// ---------------------------------------------------------------- kernel 2: experts

__global__ __launch_bounds__(kDecThreads) void k_decode_experts(DecodeArgs a) {
  __shared__ ExpertsLds sh;
  int blk = blockIdx.x;
  const int n_rt_f = a.F >> 4;
  if (blk < a.n_shared_wg) {
    gate_up_role(a, a.shared, a.K, blk, sh);
  } else if ((blk -= a.n_shared_wg) < a.n_routed_wg) {
    const int slot = blk / n_rt_f, rt = blk % n_rt_f;
    route_local(a, sh.route);
    gate_up_role(a, a.arena + (int64_t)sh.route.ids[slot] * a.expert_bytes, slot, rt, sh);
  } else {
    down_role(a, blk - a.n_routed_wg, sh);
  }
}

hipError_t launch_layer_decode(DecodeArgs a, hipStream_t stream) {
  a.n_router = a.E;  // one wavefront per expert
  a.n_shared_wg = a.n_shared ? a.F / 16 : 0;
  a.n_routed_wg = a.K * (a.F / 16);
  a.n_down_wg = a.H / 32;
  clear_last_error();
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

hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  clear_last_error();
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace qmoe
