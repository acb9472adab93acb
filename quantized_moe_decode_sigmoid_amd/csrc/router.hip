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

// One wavefront per token.
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ scores, const float* __restrict__ bias, int T,
                                              int E, int K, float scale, int32_t* __restrict__ ids,
                                              float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_wave(scores + (size_t)t * E, bias, E, K, scale, lane, ids + (size_t)t * K, wout + (size_t)t * K);
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
