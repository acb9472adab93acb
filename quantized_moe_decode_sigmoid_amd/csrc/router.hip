// Router: fp32 gate GEMV, sigmoid, top-K by wavefront shuffles, normalised
// weights times routed_scale.
//
// Model card xing4_0-29b-IQ4_NL_EPQ, "Model and routing" table: sigmoid
// gating with the selection bias ffn_exp_probs_b (noaux_tc), weights
// normalised over the selected experts and scaled by 2.0; the whole-layer
// NumPy check recomputes exactly this (sigmoid + bias + top-4 + sum
// normalisation + routed_scaling_factor).  The research log's profile shows
// the fp32 router GEMVs as their own hot item, so the router is its own kernel.
//
// Bit-reproducibility: the logit of (token, expert) is the fp32 dot product in
// one fixed order -- lane j of a wavefront owns elements 256m + 4j + c and
// accumulates them with fused multiply-adds in (m, c) order, then the 64 lane
// sums are combined by p_j + p_{j xor s} for s = 32, 16, ..., 1 -- and the
// sigmoid is evaluated in double by a fixed sequence of IEEE operations
// (router_math.h).
#include "device.h"
#include "launch.h"
#include "router_math.h"

namespace qmoe {

// One wavefront per (expert, run of tokens).  The expert's router row stays
// in registers (lane j holds its 4*M elements) while the wave walks its tokens.
template <int MMAX>
__global__ __launch_bounds__(256) void k_router_scores(const uint16_t* __restrict__ x, const float* __restrict__ wg,
                                                       int T, int H, int E, int tokens_per_wave,
                                                       float* __restrict__ scores) {
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int e = wid % E;
  const int t0 = (wid / E) * tokens_per_wave;
  if (t0 >= T) return;
  const int t1 = min(T, t0 + tokens_per_wave);
  float4 w[MMAX];
  load_router_row<MMAX>(wg + (size_t)e * H, H, lane, w);
  for (int t = t0; t < t1; t++) {
    const float p = router_logit<MMAX>(x + (size_t)t * H, H, lane, w);
    if (lane == 0) scores[(size_t)t * E + e] = sigmoid_fixed(p);
  }
}

// Batched calls: one wavefront per block of TT tokens x TE experts, four per
// workgroup as 2 x 2 blocks (so that each token row and each router row a
// workgroup reads serves two wavefronts).  Lane j keeps the partial sum p_j of
// every (token, expert) pair of its block in registers, each walking the same
// elements 256m + 4j + c in the same (m, c) order as the single-row logit, so
// every partial is the one the per-row form computes; the operands of step
// m + 1 are requested before step m is computed.  The 64 lane partials of each
// pair then go through LDS and one lane per pair adds them in the butterfly's
// tree: level s pairs index j with j + s for s = 32, 16, ..., 1 (fp32 addition
// commutes, so this is exactly the value every lane of the shuffle butterfly
// ends with).
constexpr int kRtStride = 68;

// The 64 lane partials of each of the wavefront's TT x TE pairs through the
// wavefront's LDS area pw, then one lane per pair: the butterfly's tree, the
// sigmoid, the store.  Every wavefront of the workgroup calls it (barrier).
template <int TT, int TE>
__device__ __forceinline__ void pair_sums(const float (&acc)[TT][TE], float* pw, int lane, int t0, int e0, int T,
                                          int E, float* __restrict__ scores) {
#pragma clang fp contract(off)
  static_assert(TT * TE <= 64, "one lane per pair in the final sums");
#pragma unroll
  for (int a = 0; a < TT; a++)
#pragma unroll
    for (int b = 0; b < TE; b++) pw[(a * TE + b) * kRtStride + lane] = acc[a][b];
  __syncthreads();
  if (lane >= TT * TE) return;
  float p[64];
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const float4 q = *reinterpret_cast<const float4*>(pw + lane * kRtStride + 4 * i);
    p[4 * i] = q.x;
    p[4 * i + 1] = q.y;
    p[4 * i + 2] = q.z;
    p[4 * i + 3] = q.w;
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1)
#pragma unroll
    for (int j = 0; j < s; j++) p[j] = p[j] + p[j + s];
  const int t = t0 + lane / TE, e = e0 + lane % TE;
  if (t < T && e < E) scores[(size_t)t * E + e] = sigmoid_fixed(p[0]);
}

// The same blocks of 2 x 2 pairs with every operand of the row requested at
// once (H <= 256 MMAX), for calls whose blocks of 4 x 4 would leave the
// wavefronts waiting for one 256-element step after another.
template <int MMAX>
__global__ __launch_bounds__(256) void k_router_scores_resident(const uint16_t* __restrict__ x,
                                                               const float* __restrict__ wg, int T, int H, int E,
                                                               float* __restrict__ scores) {
#pragma clang fp contract(off)
  constexpr int TT = 2, TE = 2;
  __shared__ __attribute__((aligned(16))) float part[4][TT * TE * kRtStride];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = (2 * blockIdx.x + (wave >> 1)) * TT, e0 = (2 * blockIdx.y + (wave & 1)) * TE;
  const int M = H >> 8;
  uint2 xv[MMAX][TT];
  float4 wv[MMAX][TE];
#pragma unroll
  for (int m = 0; m < MMAX; m++) {
    const int mm = 256 * min(m, M - 1) + 4 * lane;  // steps past H repeat the last one (never used)
#pragma unroll
    for (int i = 0; i < TT; i++) xv[m][i] = *reinterpret_cast<const uint2*>(x + (size_t)min(t0 + i, T - 1) * H + mm);
#pragma unroll
    for (int i = 0; i < TE; i++) wv[m][i] = *reinterpret_cast<const float4*>(wg + (size_t)min(e0 + i, E - 1) * H + mm);
  }
  float acc[TT][TE];
#pragma unroll
  for (int a = 0; a < TT; a++)
#pragma unroll
    for (int b = 0; b < TE; b++) acc[a][b] = 0.0f;
#pragma unroll
  for (int m = 0; m < MMAX; m++) {
    if (m < M) {
#pragma unroll
      for (int c = 0; c < 4; c++) {
#pragma unroll
        for (int a = 0; a < TT; a++) {
          const uint32_t word = c < 2 ? xv[m][a].x : xv[m][a].y;
          const float xf = bf16_bits_to_f32((c & 1) ? word >> 16 : word & 0xffffu);
#pragma unroll
          for (int b = 0; b < TE; b++) {
            const float wf = c == 0 ? wv[m][b].x : c == 1 ? wv[m][b].y : c == 2 ? wv[m][b].z : wv[m][b].w;
            acc[a][b] = __builtin_fmaf(xf, wf, acc[a][b]);
          }
        }
      }
    }
  }
  pair_sums<TT, TE>(acc, part[wave], lane, t0, e0, T, E, scores);
}

template <int TT, int TE>
__global__ __launch_bounds__(256, 2) void k_router_scores_tiled(const uint16_t* __restrict__ x,
                                                              const float* __restrict__ wg, int T, int H, int E,
                                                              float* __restrict__ scores) {
#pragma clang fp contract(off)
  __shared__ __attribute__((aligned(16))) float part[4][TT * TE * kRtStride];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = (2 * blockIdx.x + (wave >> 1)) * TT, e0 = (2 * blockIdx.y + (wave & 1)) * TE;
  // rows past T or E repeat the last valid one (their sums are never stored);
  // such a wavefront runs too, so every wavefront reaches the barrier
  const uint16_t* xr[TT];
  const float* wr[TE];
#pragma unroll
  for (int i = 0; i < TT; i++) xr[i] = x + (size_t)min(t0 + i, T - 1) * H + 4 * lane;
#pragma unroll
  for (int i = 0; i < TE; i++) wr[i] = wg + (size_t)min(e0 + i, E - 1) * H + 4 * lane;
  float acc[TT][TE];
#pragma unroll
  for (int a = 0; a < TT; a++)
#pragma unroll
    for (int b = 0; b < TE; b++) acc[a][b] = 0.0f;
  uint2 xv[TT];
  float4 wv[TE];
#pragma unroll
  for (int i = 0; i < TT; i++) xv[i] = *reinterpret_cast<const uint2*>(xr[i]);
#pragma unroll
  for (int i = 0; i < TE; i++) wv[i] = *reinterpret_cast<const float4*>(wr[i]);
  const int M = H >> 8;
  for (int m = 0; m < M; m++) {
    const int mn = (m + 1 < M ? m + 1 : m) * 256;
    uint2 xn[TT];
    float4 wn[TE];
#pragma unroll
    for (int i = 0; i < TT; i++) xn[i] = *reinterpret_cast<const uint2*>(xr[i] + mn);
#pragma unroll
    for (int i = 0; i < TE; i++) wn[i] = *reinterpret_cast<const float4*>(wr[i] + mn);
#pragma unroll
    for (int c = 0; c < 4; c++) {
#pragma unroll
      for (int a = 0; a < TT; a++) {
        const uint32_t word = c < 2 ? xv[a].x : xv[a].y;
        const float xf = bf16_bits_to_f32((c & 1) ? word >> 16 : word & 0xffffu);
#pragma unroll
        for (int b = 0; b < TE; b++) {
          const float wf = c == 0 ? wv[b].x : c == 1 ? wv[b].y : c == 2 ? wv[b].z : wv[b].w;
          acc[a][b] = __builtin_fmaf(xf, wf, acc[a][b]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < TT; i++) xv[i] = xn[i];
#pragma unroll
    for (int i = 0; i < TE; i++) wv[i] = wn[i];
  }
  pair_sums<TT, TE>(acc, part[wave], lane, t0, e0, T, E, scores);
}

template <int TT, int TE>
void launch_router_tiled(const uint16_t* x, const float* wg, int T, int H, int E, float* scores_ws,
                         hipStream_t stream) {
  const dim3 grid((unsigned)((T + 2 * TT - 1) / (2 * TT)), (unsigned)((E + 2 * TE - 1) / (2 * TE)));
  hipLaunchKernelGGL((k_router_scores_tiled<TT, TE>), grid, dim3(256), 0, stream, x, wg, T, H, E, scores_ws);
}

// One wavefront per token.  scores rows hold E + gated values (the last one
// the shared expert's gate); weight rows K + gated.
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ scores, const float* __restrict__ bias, int T,
                                              int E, int K, int gated, float scale, int32_t* __restrict__ ids,
                                              float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_wave(scores + (size_t)t * (E + gated), bias, E, K, scale, lane, ids + (size_t)t * K,
            wout + (size_t)t * (K + gated), gated);
}

// Below this many tokens a wavefront per (expert, run of tokens) has more
// workgroups to spread over the chip than token x expert blocks.
constexpr int kRouterTiledMinTokens = 64;
// Blocks of 8 x 8 pairs once they give more than this many wavefronts (two
// per CU); below, blocks of 4 x 4 keep four times as many wavefronts busy,
// and blocks of 2 x 2 with every operand requested at once up to this many
// wavefronts (H <= 4096).
constexpr int64_t kRouterBigBlockWaves = 512;
constexpr int64_t kRouterResidentWaves = 2048;

hipError_t launch_router_scores(const uint16_t* x, const float* wg, int T, int H, int E, float* scores,
                                hipStream_t stream) {
  if (T == 0) return hipSuccess;
  int tpw = (int)(((int64_t)T * E) / 8192);
  tpw = tpw < 1 ? 1 : (tpw > 64 ? 64 : tpw);
  const int64_t waves = (int64_t)E * ((T + tpw - 1) / tpw);
  const int blocks = (int)((waves + 3) / 4);
  clear_last_error();
  if (T >= kRouterTiledMinTokens) {
    if ((int64_t)((T + 7) / 8) * ((E + 7) / 8) > kRouterBigBlockWaves) {
      launch_router_tiled<8, 8>(x, wg, T, H, E, scores, stream);
    } else if (H <= 16 * 256 && (int64_t)((T + 1) / 2) * ((E + 1) / 2) <= kRouterResidentWaves) {
      const dim3 grid((unsigned)((T + 3) / 4), (unsigned)((E + 3) / 4));
      if (H <= 8 * 256)
        hipLaunchKernelGGL(k_router_scores_resident<8>, grid, dim3(256), 0, stream, x, wg, T, H, E, scores);
      else
        hipLaunchKernelGGL(k_router_scores_resident<16>, grid, dim3(256), 0, stream, x, wg, T, H, E, scores);
    } else {
      launch_router_tiled<4, 4>(x, wg, T, H, E, scores, stream);
    }
  } else if (H <= 16 * 256)
    hipLaunchKernelGGL(k_router_scores<16>, dim3(blocks), dim3(256), 0, stream, x, wg, T, H, E, tpw, scores);
  else
    hipLaunchKernelGGL(k_router_scores<32>, dim3(blocks), dim3(256), 0, stream, x, wg, T, H, E, tpw, scores);
  return hipGetLastError();
}

hipError_t launch_router(const uint16_t* x, const float* wg, const float* bias, int T, int H, int E, int K,
                         int gated, float scale, float* scores_ws, int32_t* ids, float* w, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  hipError_t err = launch_router_scores(x, wg, T, H, E + gated, scores_ws, stream);
  if (err != hipSuccess) return err;
  clear_last_error();
  hipLaunchKernelGGL(k_topk, dim3((T + 3) / 4), dim3(256), 0, stream, scores_ws, bias, T, E, K, gated, scale, ids,
                     w);
  return hipGetLastError();
}

}  // namespace qmoe
