// Router arithmetic shared by the standalone router kernels and the fused
// decode kernel: the fixed-order fp32 logit, the fixed-sequence sigmoid and
// the wavefront top-K.  Every function disables fp contraction in its body so
// that only the written fused multiply-adds fuse.
//
// Model card xing4_0-29b-IQ4_NL_EPQ, "Model and routing" table: sigmoid
// gating with the selection bias ffn_exp_probs_b (noaux_tc), top-K, weights
// normalised over the selected experts and scaled by expert_weights_scale.
#pragma once

#include "device.h"

namespace qmoe {

// exp(y) in double: y = n ln2 + r (Cody-Waite with a two-part ln 2 and fused
// multiply-adds), Taylor polynomial of degree 13 for exp(r) in Horner form
// (|r| <= ln2/2, truncation error below 1e-17), times 2^n.
__device__ __forceinline__ double exp_fixed(double y) {
#pragma clang fp contract(off)
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

// Sigmoid evaluated in double and rounded once to fp32.
__device__ __forceinline__ float sigmoid_fixed(float l) {
#pragma clang fp contract(off)
  return (float)(1.0 / (1.0 + exp_fixed(-(double)l)));
}

// The expert's router row in registers: lane j holds elements 256m + 4j + c.
// Every load is issued (slots m >= H/256 repeat the last valid one and are
// never used), so that no load sits behind a branch.
template <int MMAX>
__device__ __forceinline__ void load_router_row(const float* wrow, int H, int lane, float4 (&w)[MMAX]) {
  const int M = H >> 8;
#pragma unroll
  for (int m = 0; m < MMAX; m++) {
    const int mm = m < M ? m : M - 1;
    w[m] = *reinterpret_cast<const float4*>(wrow + 256 * mm + 4 * lane);
  }
}

// fp32 logit in the fixed order: lane j accumulates its elements with fused
// multiply-adds in (m, c) order, then p_j + p_{j xor s} for s = 32..1.  Every
// lane returns the same value.  xv[m] holds the lane's 4 bf16 activations
// 256m + 4j .. 256m + 4j + 3.
template <int MMAX>
__device__ __forceinline__ float router_logit_vals(const uint2 (&xv)[MMAX], int H, const float4 (&w)[MMAX]) {
#pragma clang fp contract(off)
  const int M = H >> 8;
  float p = 0.0f;
#pragma unroll
  for (int m = 0; m < MMAX; m++) {
    if (m < M) {
      p = __builtin_fmaf(bf16_bits_to_f32(xv[m].x & 0xffffu), w[m].x, p);
      p = __builtin_fmaf(bf16_bits_to_f32(xv[m].x >> 16), w[m].y, p);
      p = __builtin_fmaf(bf16_bits_to_f32(xv[m].y & 0xffffu), w[m].z, p);
      p = __builtin_fmaf(bf16_bits_to_f32(xv[m].y >> 16), w[m].w, p);
    }
  }
  return wave_xor_sum(p);
}

// The same with the lane's activations read from the row xrow.
template <int MMAX>
__device__ __forceinline__ float router_logit(const uint16_t* xrow, int H, int lane, const float4 (&w)[MMAX]) {
  const int M = H >> 8;
  uint2 xv[MMAX];
#pragma unroll
  for (int m = 0; m < MMAX; m++) {
    const int mm = m < M ? m : M - 1;
    xv[m] = *reinterpret_cast<const uint2*>(xrow + 256 * mm + 4 * lane);
  }
  return router_logit_vals<MMAX>(xv, H, w);
}

// A selection score's bits mapped so that unsigned order is float order (a
// selection score from finite inputs is never -0: a sigmoid is +0 or
// positive, and +0 plus a bias never rounds to -0, and never NaN).  Every such
// key is >= 1, so 0 is below every key (no candidate).  A NaN score (from a
// NaN input) gets a key too; the rankings compare keys and break ties by the
// expert index, so whatever the scores hold they pick K experts in range.
__device__ __forceinline__ uint32_t sel_order_bits(float s) {
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Largest key of the wavefront, as a scalar: within each quad (xor 1, xor 2),
// then half-rows of 8 and rows of 16 (mirrors), so that every lane holds its
// row's maximum; then the four row maxima read from lanes 0, 16, 32, 48.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t k) {
  constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kRowHalfMirror = 0x141, kRowMirror = 0x140;
  k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, kQuadXor1, 0xf, 0xf, false));
  k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, kQuadXor2, 0xf, 0xf, false));
  k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, kRowHalfMirror, 0xf, 0xf, false));
  k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, kRowMirror, 0xf, 0xf, false));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)k, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)k, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)k, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)k, 48);
  return max(max(r0, r1), max(r2, r3));
}

// One round of a wavefront's selection over NQ keys per lane (lane l holds
// experts l, l + 64, ...; key 0: no candidate): the largest key left, as a
// wave-wide maximum, and among equal keys the smallest expert index (first
// set bit of the first non-empty ballot, in expert order).  The owner lane
// retires it; every lane gets the expert index (returned) and its unbiased
// score s_win.
template <int NQ>
__device__ __forceinline__ int topk_take(uint32_t (&key)[NQ], const float (&s)[NQ], int lane, float& s_win) {
  uint32_t mk = key[0];
#pragma unroll
  for (int q = 1; q < NQ; q++) mk = max(mk, key[q]);
  const uint32_t m = wave_max_u32(mk);
  int e = 64 * NQ;
#pragma unroll
  for (int q = NQ - 1; q >= 0; q--) {
    const uint64_t b = __builtin_amdgcn_ballot_w64(key[q] == m);
    if (b) e = 64 * q + (int)__builtin_ctzll(b);
  }
  const int qe = e >> 6, le = e & 63;
  float sw = 0.0f;
#pragma unroll
  for (int q = 0; q < NQ; q++) {
    if (q == qe) {
      if (lane == le) key[q] = 0u;
      sw = s[q];
    }
  }
  s_win = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sw), le));
  return e;
}

// One wavefront selects the K experts of one token from its E sigmoid scores
// (E <= 256; lane l holds experts l, l + 64, l + 128, l + 192): K rounds of
// topk_take on the selection scores (s + bias), each taking the largest left
// (ties: the smallest expert index).  Lane 0 writes the slots to ids[0..K)
// and the weights scale * s_k / (((s_0 + s_1) + s_2) + ...) to w (either may
// point to global or LDS memory); with a sigmoid-gated shared expert
// (gated != 0) also w[K] = scores[E], the gate's own sigmoid score (not
// normalised or scaled).
__device__ __forceinline__ void topk_wave(const float* scores, const float* bias, int E, int K, float scale,
                                          int lane, int32_t* ids, float* wout, int gated = 0) {
#pragma clang fp contract(off)
  float s[4];
  uint32_t key[4];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const int e = lane + 64 * q;
    const bool avail = e < E;
    s[q] = avail ? scores[e] : 0.0f;
    const float sel = bias && avail ? s[q] + bias[e] : s[q];
    key[q] = avail ? sel_order_bits(sel) : 0u;
  }
  int chosen[8];
  float chosen_s[8];
  for (int k = 0; k < K; k++) chosen[k] = topk_take<4>(key, s, lane, chosen_s[k]);
  if (lane == 0) {
    float S = 0.0f;
    for (int k = 0; k < K; k++) S = S + chosen_s[k];
    for (int k = 0; k < K; k++) {
      ids[k] = chosen[k];
      wout[k] = (chosen_s[k] / S) * scale;
    }
    if (gated) wout[K] = scores[E];
  }
}

}  // namespace qmoe
