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
// sigmoid is evaluated in double by a fixed sequence of IEEE operations.
// Contraction is off in this file so that only the written fmas fuse.
#pragma clang fp contract(off)

#include "device.h"
#include "launch.h"

namespace qmoe {

// exp(y) in double: y = n ln2 + r (Cody-Waite with a two-part ln 2 and fused
// multiply-adds), Taylor polynomial of degree 13 for exp(r) in Horner form
// (|r| <= ln2/2, truncation error below 1e-17), times 2^n.
__device__ __forceinline__ double exp_fixed(double y) {
  constexpr double kLog2e = 0x1.71547652b82fep+0;  // nearest double to 1/ln 2
  constexpr double kLn2Hi = 0x1.62e42fefa39efp-1;  // nearest double to ln 2
  constexpr double kLn2Lo = 0x1.abc9e3b39803fp-56; // nearest double to (ln 2 - kLn2Hi)
  if (y > 200.0) return __builtin_inf();
  if (y < -200.0) return 0.0;
  const double n = __builtin_rint(y * kLog2e);
  double r = __builtin_fma(-n, kLn2Hi, y);
  r = __builtin_fma(-n, kLn2Lo, r);
  double inv_fact[14];
  double fact = 1.0;
#pragma unroll
  for (int k = 0; k < 14; k++) {
    if (k > 0) fact *= (double)k;
    inv_fact[k] = 1.0 / fact;
  }
  double p = inv_fact[13];
#pragma unroll
  for (int k = 12; k >= 0; k--) p = __builtin_fma(p, r, inv_fact[k]);
  return __builtin_ldexp(p, (int)n);
}

__device__ __forceinline__ float sigmoid_fixed(float l) { return (float)(1.0 / (1.0 + exp_fixed(-(double)l))); }

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
  const int M = H >> 8;
  float4 w[MMAX];
#pragma unroll
  for (int m = 0; m < MMAX; m++)
    if (m < M) w[m] = *reinterpret_cast<const float4*>(wg + (size_t)e * H + 256 * m + 4 * lane);
  for (int t = t0; t < t1; t++) {
    const uint16_t* xr = x + (size_t)t * H;
    float p = 0.0f;
#pragma unroll
    for (int m = 0; m < MMAX; m++) {
      if (m < M) {
        const uint2 xv = *reinterpret_cast<const uint2*>(xr + 256 * m + 4 * lane);
        p = __builtin_fmaf(bf16_bits_to_f32(xv.x & 0xffffu), w[m].x, p);
        p = __builtin_fmaf(bf16_bits_to_f32(xv.x >> 16), w[m].y, p);
        p = __builtin_fmaf(bf16_bits_to_f32(xv.y & 0xffffu), w[m].z, p);
        p = __builtin_fmaf(bf16_bits_to_f32(xv.y >> 16), w[m].w, p);
      }
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) p = p + __shfl_xor(p, s, 64);
    if (lane == 0) scores[(size_t)t * E + e] = sigmoid_fixed(p);
  }
}

// One wavefront per token: K rounds of a wave-wide arg-max under the order
// (selection score descending, expert index ascending), then the weights
// routed_scale * s_k / (((s_0 + s_1) + s_2) + ...).
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ scores, const float* __restrict__ bias, int T,
                                              int E, int K, float scale, int32_t* __restrict__ ids,
                                              float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float s[4], sel[4];
  bool avail[4];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const int e = lane + 64 * q;
    avail[q] = e < E;
    s[q] = avail[q] ? scores[(size_t)t * E + e] : 0.0f;
    sel[q] = avail[q] ? (bias ? s[q] + bias[e] : s[q]) : 0.0f;
  }
  int chosen[8];
  float chosen_s[8];
  for (int k = 0; k < K; k++) {
    bool have = false;
    float bs = 0.0f;
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      if (avail[q] && (!have || sel[q] > bs)) {
        have = true;
        bs = sel[q];
        be = lane + 64 * q;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float os = __shfl_xor(bs, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      const bool ohave = oe != 0x7fffffff;
      if (ohave && (!have || os > bs || (os == bs && oe < be))) {
        have = true;
        bs = os;
        be = oe;
      }
    }
    // every lane now holds the same winner
    float sw = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      if (lane + 64 * q == be) {
        avail[q] = false;
        sw = s[q];
      }
    }
    sw = __shfl(sw, be & 63, 64);
    chosen[k] = be;
    chosen_s[k] = sw;
  }
  if (lane == 0) {
    float S = 0.0f;
    for (int k = 0; k < K; k++) S = S + chosen_s[k];
    for (int k = 0; k < K; k++) {
      ids[(size_t)t * K + k] = chosen[k];
      wout[(size_t)t * K + k] = (chosen_s[k] / S) * scale;
    }
  }
}

hipError_t launch_router(const uint16_t* x, const float* wg, const float* bias, int T, int H, int E, int K,
                         float scale, float* scores_ws, int32_t* ids, float* w, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  int tpw = (int)(((int64_t)T * E) / 8192);
  tpw = tpw < 1 ? 1 : (tpw > 64 ? 64 : tpw);
  const int64_t waves = (int64_t)E * ((T + tpw - 1) / tpw);
  const int blocks = (int)((waves + 3) / 4);
  clear_last_error();
  if (H <= 16 * 256)
    hipLaunchKernelGGL(k_router_scores<16>, dim3(blocks), dim3(256), 0, stream, x, wg, T, H, E, tpw, scores_ws);
  else
    hipLaunchKernelGGL(k_router_scores<32>, dim3(blocks), dim3(256), 0, stream, x, wg, T, H, E, tpw, scores_ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  clear_last_error();
  hipLaunchKernelGGL(k_topk, dim3((T + 3) / 4), dim3(256), 0, stream, scores_ws, bias, T, E, K, scale, ids, w);
  return hipGetLastError();
}

}  // namespace qmoe
