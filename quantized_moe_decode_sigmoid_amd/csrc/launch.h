// Host-side launchers of the libmoe kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"

namespace qmoe {

// The sigmoid scores [T][E] alone (the first half of launch_router).
hipError_t launch_router_scores(const uint16_t* x, const float* wg, int T, int H, int E, float* scores,
                                hipStream_t stream);

// Scores of E + gated router rows ([T][E + gated] in scores_ws), top-K of the
// first E into ids [T][K] and w [T][K + gated] (w[t][K] = the gate's score).
hipError_t launch_router(const uint16_t* x, const float* wg, const float* bias, int T, int H, int E, int K,
                         int gated, float scale, float* scores_ws, int32_t* ids, float* w, hipStream_t stream);

// chunk_rows: routes per work chunk (16 for the exact-weight kernels, kBfRows for the bf16 kernels)
hipError_t launch_bucket(const int32_t* ids, int T, int K, int E, int n_shared, int chunk_rows, int32_t* counts,
                         int32_t* offsets, int32_t* perm, int32_t* pos, Chunk* chunks, int32_t* n_chunks,
                         hipStream_t stream);

hipError_t launch_pack(const uint8_t* src, uint8_t* dst, int n_experts, int H, int F, hipStream_t stream);

hipError_t launch_dequant(const uint8_t* mat, int rows, int cols, int bf16, float* out, hipStream_t stream);

// out[t] = sum_k w[t][k] y[pos[t K + k]] + g_t y[T K + t]; w rows of K + gated
// values, g_t = w[t][K] when gated, else 1.
hipError_t launch_combine(const float* y, const int32_t* pos, const float* w, int T, int K, int H, int n_shared,
                          int gated, float* out, hipStream_t stream);

// ---- bf16 grouped MFMA path (ffn_bf16.hip)

constexpr int kBfRows = 128;  // routes per tile

hipError_t launch_ffn_bf16(const uint16_t* x, int T, int H, int F, int K, int n_shared, int gated, int max_tiles,
                           const uint8_t* arena, const uint8_t* shared, int64_t expert_bytes, const int32_t* perm,
                           const int32_t* pos, const float* w, const Chunk* tiles, const int32_t* n_tiles,
                           uint16_t* h, float* y, float* out, hipStream_t stream);

hipError_t launch_ffn_exact(const uint16_t* x, int T, int H, int F, int K, int n_shared, int gated, int max_chunks,
                            const uint8_t* arena, const uint8_t* shared, int64_t expert_bytes, const int32_t* perm,
                            const int32_t* pos, const float* w, const Chunk* chunks, const int32_t* n_chunks,
                            uint16_t* h_hi, uint16_t* h_lo, float* y, float* out, hipStream_t stream);

// ---- Q8_0 activations (ffn_w4a8.hip)

// n values (a multiple of 32; bf16 when src_bf16, else fp32) -> Q8_0 codes q [n] and fp16 scales d [n/32]
hipError_t launch_quantize_q8_0(const void* src, int src_bf16, int64_t n, int8_t* q, uint16_t* d,
                                hipStream_t stream);

hipError_t launch_ffn_w4a8(const uint16_t* x, int T, int H, int F, int K, int n_shared, int gated, int max_chunks,
                           const uint8_t* arena, const uint8_t* shared, int64_t expert_bytes, const int32_t* perm,
                           const int32_t* pos, const float* w, const Chunk* chunks, const int32_t* n_chunks,
                           int8_t* xq, uint16_t* xd, float* h, int8_t* hq, uint16_t* hd, float* y, float* out,
                           hipStream_t stream);

// ---- other expert codecs (ffn_codec.hip): 1 = IQ4_XS, 2 = packed 3-bit affine

int codec_tile_bytes(int codec);

hipError_t launch_pack_codec(int codec, const uint8_t* src, uint8_t* dst, int n_experts, int H, int F,
                             int64_t src_expert_bytes, int64_t dst_expert_bytes, hipStream_t stream);

hipError_t launch_dequant_codec(int codec, const uint8_t* mat, int rows, int cols, float* out, hipStream_t stream);

hipError_t launch_ffn_codec(int codec, const uint16_t* x, int T, int H, int F, int K, int n_shared, int gated,
                            int max_chunks, const uint8_t* arena, const uint8_t* shared, int64_t expert_bytes,
                            const int32_t* perm, const int32_t* pos, const float* w, const Chunk* chunks,
                            const int32_t* n_chunks, uint16_t* h_hi, uint16_t* h_lo, float* y, float* out,
                            hipStream_t stream);

// ---- one decode token in two launches (layer_decode.hip)

constexpr int kMaxDecodeK = 4;          // experts per token
constexpr int kMaxDecodeFfn = 1024;     // F
constexpr int kMaxDecodeHidden = 4096;  // H

struct DecodeArgs {
  const uint16_t* x;   // [H] bf16
  const float* wg;     // [E][H]
  const float* bias;   // [E] or null
  const uint8_t* arena;
  const uint8_t* shared;
  int64_t expert_bytes;
  int H, F, E, K, n_shared;
  int gated;           // the shared expert scaled by the sigmoid of router row E
  float scale;
  float* scores;       // [E + gated] sigmoid scores (first kernel -> second)
  int32_t* ids;        // [K] routing outputs
  float* w;            // [K + gated]
  uint32_t* hw;        // [hw_words(K, F, H)]: h words bf16(h) | bf16(h - bf16(h)) << 16 of the K + 1 slots
                       // ([K + 1][F]), then the shared expert's down rows y_s[H] (fp32 bits)
  float* out;          // [H]
  uint32_t* err;       // set to 1 if a wait gave up
  // chained input (x_prev non-null): the first kernel forms x = bf16(rmsnorm(x_prev + out_prev)) itself (the
  // arithmetic of k_residual_rmsnorm) and writes it to x (which must not overlap x_prev or out_prev)
  const uint16_t* x_prev;
  const float* out_prev;
  float eps;
  int n_router, n_shared_wg, n_routed_wg, n_down_wg;  // grid partition (set by the launcher)
  // stack steps: the first layer's scores kernel also copies x to x_copy
  // (when non-null) and clears the give-up word (when zero_err)
  uint16_t* x_copy = nullptr;
  int zero_err = 0;
};

// Words of the decode hand-off buffer: h of K + 1 slots, the shared expert's down rows.
__host__ __device__ inline int hw_words(int K, int F, int H) { return (K + 1) * F + H; }

hipError_t launch_layer_decode(DecodeArgs a, hipStream_t stream);

// Layers one moe_stack_decode call takes (two decode launches per layer).
constexpr int kMaxStackLayers = 64;

hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t stream);

// dst[i] = src[i] for i < n (device words; a kernel, so that it can sit in a captured graph)
hipError_t launch_copy_words(const uint32_t* src, uint32_t* dst, int64_t n, hipStream_t stream);

// Whether the k_decode_experts grid of this shape fits on the current device at
// once (occupancy x compute units >= workgroups).  Its down workgroups wait for
// data from its gate/up workgroups; co-residency makes every wait end whatever
// the dispatch order.  Queried once per device and shape class; false if the
// runtime cannot answer.
bool decode_grid_coresident(int F, int K, int H, int n_shared);

// ---- measurement (stream.hip) and the stack workload's chaining (chain.hip)

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);

hipError_t launch_residual_rmsnorm(const float* out, const uint16_t* x, int T, int H, float eps, uint16_t* y,
                                   hipStream_t stream);

}  // namespace qmoe
