// Expert FFN with Q8_0 activations and IQ4_NL weights (the W4A8 contract).
//
// The model card's CPU expert path dots IQ4_NL weights with activations
// quantized to Q8_0 (32 int8 codes and one fp16 scale per block) and reports
// the residual of its pure-NumPy checks as that quantization's error.  Here:
//   - x (bf16) and h = silu(g) * u (fp32) are quantized to Q8_0 per token row
//     in blocks of 32: d32 = max|v| / 127, stored scale fp16(d32), codes
//     round(v / d32) with halves away from zero (k_quantize_q8_0);
//   - every 32-weight block is one v_mfma_i32_16x16x32_i8: the integer levels
//     (IQ4_NL's 16-entry table holds integers of at most 8 bits) times the
//     codes, summed exactly in int32, then scaled by d_w * d_x in fp32 (the
//     product of two fp16 values is exact in fp32) and accumulated in fp32.
// So the block dots are exact; only the fp32 accumulation of the scaled
// blocks rounds.
//
// Work: the chunks of up to 16 routes of one expert (or 16 tokens of the
// shared expert) that the bucketing pass lists, as in the exact-weight FP32
// kernels: a gate/up workgroup owns (chunk, 32 rows of F) and splits the
// reduction dimension over 4 wavefronts; a down workgroup owns (chunk, 128
// rows of H) over 8.  A lane's operands of one block: the 8 levels of its
// nibble word (row lane % 16, weights 8 (lane / 16) .. + 7), decoded through
// an LDS table to int8; 8 codes of its route (lane % 16) at the same k.
#include "device.h"
#include "launch.h"

namespace qmoe {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- Q8_0 quantization

// One lane per element, the 32 lanes of a half wavefront per block.  n is a
// multiple of 32.  src is bf16 (src_bf16 != 0) or fp32.
__global__ __launch_bounds__(256) void k_quantize_q8_0(const void* __restrict__ src, int src_bf16, int64_t n,
                                                       int8_t* __restrict__ q, uint16_t* __restrict__ d) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool live = i < n;  // whole blocks: a half wavefront is all live or all not
  float v = 0.0f;
  if (live)
    v = src_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(src)[i]) : static_cast<const float*>(src)[i];
  float a = __builtin_fabsf(v);
#pragma unroll
  for (int s = 16; s >= 1; s >>= 1) a = __builtin_fmaxf(a, __shfl_xor(a, s, 32));
  const float d32 = a / 127.0f;
  const float id = d32 != 0.0f ? 1.0f / d32 : 0.0f;
  if (live) {
    q[i] = (int8_t)__builtin_roundf(v * id);
    if ((threadIdx.x & 31) == 0) d[i >> 5] = __builtin_bit_cast(uint16_t, (_Float16)d32);
  }
}

hipError_t launch_quantize_q8_0(const void* src, int src_bf16, int64_t n, int8_t* q, uint16_t* d,
                                hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  clear_last_error();
  hipLaunchKernelGGL(k_quantize_q8_0, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, src, src_bf16, n, q, d);
  return hipGetLastError();
}

// ---------------------------------------------------------------- int8 levels

// 256-entry table, one entry per byte of nibbles: the int8 level of its low
// nibble in bits 0..7, of its high nibble in bits 8..15; 32 replicas so that
// lane l reads bank l % 32.
__device__ __forceinline__ void build_i8_pair_table(uint32_t* tbl) {
  for (int i = threadIdx.x; i < kPairTableWords / 4; i += blockDim.x) {
    const int v = i >> 3;
    const uint32_t e = (uint32_t)(uint8_t)iq4nl_level(v & 15) | ((uint32_t)(uint8_t)iq4nl_level(v >> 4) << 8);
    uint32_t __attribute__((ext_vector_type(4))) w = {e, e, e, e};
    *reinterpret_cast<decltype(w)*>(tbl + 4 * i) = w;
  }
}

// One nibble word (weights 8w..8w+7 of a block, byte i = weights 8w+2i,
// 8w+2i+1) -> the lane's 8 int8 levels in weight order.
__device__ __forceinline__ long decode_word_i8(const uint32_t* tbl, uint32_t word, uint32_t lane32) {
  const uint32_t e0 = tbl[(word & 0xffu) * 32u + lane32];
  const uint32_t e1 = tbl[((word >> 8) & 0xffu) * 32u + lane32];
  const uint32_t e2 = tbl[((word >> 16) & 0xffu) * 32u + lane32];
  const uint32_t e3 = tbl[(word >> 24) * 32u + lane32];
  return (long)(((uint64_t)(e2 | (e3 << 16)) << 32) | (uint64_t)(e0 | (e1 << 16)));
}

__device__ __forceinline__ i32x4 mfma_i8(long a, long b) {
  const i32x4 z = {0, 0, 0, 0};
  return __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, z, 0, 0, 0);
}

// acc[i] (rows 4G+i) += d_w(row 4G+i) * dx * C[i]; d_w from the tile's scale
// word pair (rows 4G, 4G+1 | 4G+2, 4G+3).
__device__ __forceinline__ void scale_acc_i8(f32x4& acc, const i32x4& c, uint32_t s01, uint32_t s23, float dx) {
  acc[0] = __builtin_fmaf(half_bits_to_float(s01) * dx, (float)c[0], acc[0]);
  acc[1] = __builtin_fmaf(half_bits_to_float(s01 >> 16) * dx, (float)c[1], acc[1]);
  acc[2] = __builtin_fmaf(half_bits_to_float(s23) * dx, (float)c[2], acc[2]);
  acc[3] = __builtin_fmaf(half_bits_to_float(s23 >> 16) * dx, (float)c[3], acc[3]);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

// ---------------------------------------------------------------- gate / up

constexpr int kW8GuWaves = 4;
constexpr int kW8GuThreads = 64 * kW8GuWaves;
constexpr int kW8GuRowTiles = 2;  // 32 rows of F per workgroup
constexpr int kW8DnWaves = 8;
constexpr int kW8DnThreads = 64 * kW8DnWaves;
constexpr int kW8DnRowTiles = 8;  // 128 rows of H per workgroup

struct GateUpW8Lds {
  union {
    uint32_t scales[kW8GuWaves][256];           // per wavefront: 32 words of (row tile r, matrix m) at 32 (2r + m)
    f32x4 red[kW8GuRowTiles][kW8GuWaves][64];   // wavefront partials of one matrix
  } u;
  uint32_t tbl[kPairTableWords];
};

// Workgroup = (chunk, 2 row tiles of F).  Output h = silu(g) * u in fp32,
// row-major [route][F] (bucketed position, or T*K + token for the shared
// expert).  Wavefront w takes tile columns [w n/4, (w+1) n/4) of the n = H/128
// of a row, one column at a time: it requests the column's nibble words (2 row
// tiles x gate/up), codes and scales, then computes.
__global__ __launch_bounds__(kW8GuThreads) void k_gate_up_w4a8(
    const int8_t* __restrict__ xq, const uint16_t* __restrict__ xd, int H, int F, int K, int T,
    const uint8_t* __restrict__ arena, const uint8_t* __restrict__ shared, int64_t expert_bytes,
    const int32_t* __restrict__ perm, const Chunk* __restrict__ chunks, const int32_t* __restrict__ n_chunks,
    float* __restrict__ h) {
  __shared__ __attribute__((aligned(16))) GateUpW8Lds sh;
  const int n_rp = F / (16 * kW8GuRowTiles);
  const int chunk_id = blockIdx.x / n_rp;
  const int rt0 = kW8GuRowTiles * (blockIdx.x % n_rp);
  if (chunk_id >= *n_chunks) return;
  const Chunk ch = chunks[chunk_id];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = lane >> 4;
  const int64_t mat_bytes = expert_bytes / 3;
  const uint8_t* ex = ch.expert >= 0 ? arena + (int64_t)ch.expert * expert_bytes : shared;
  const int cc = (lane & 15) < ch.count ? (lane & 15) : 0;  // a column past the chunk reads column 0's token
  const int tok = ch.expert >= 0 ? perm[ch.first + cc] / K : ch.first + cc;
  const int nkg = H >> 7;
  const int kg0 = wave * nkg / kW8GuWaves, kg1 = (wave + 1) * nkg / kW8GuWaves;
  const int rt_bytes = nkg * kTileBytes;
  const uint8_t* gate_t = ex + rt0 * rt_bytes;  // row tile r: + r * rt_bytes; up: mat_bytes further
  const __amdgpu_buffer_rsrc_t w_rsrc = rsrc_of(gate_t);
  // this lane's 16-byte scale piece: piece lane % 8 of row tile (lane / 16) % 2,
  // matrix (lane / 8) % 2 (lanes 32-63 repeat lanes 0-31 into the unread half)
  const int sc_off =
      ((lane >> 4) & 1) * rt_bytes + ((lane >> 3) & 1) * (int)mat_bytes + kTileNibbleBytes + 16 * (lane & 7);
  const int8_t* xrow = xq + (int64_t)tok * H;
  const uint16_t* drow = xd + (int64_t)tok * (H / 32);
  uint32_t* sc = sh.u.scales[wave];

  build_i8_pair_table(sh.tbl);
  __syncthreads();
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[kW8GuRowTiles][2];
#pragma unroll
  for (int r = 0; r < kW8GuRowTiles; r++) acc[r][0] = acc[r][1] = zero;
  for (int kg = kg0; kg < kg1; kg++) {
    const u32x4 scw = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, sc_off, kg * kTileBytes, kNonTemporal));
    u32x4 nib[kW8GuRowTiles][2];
#pragma unroll
    for (int r = 0; r < kW8GuRowTiles; r++)
#pragma unroll
      for (int m = 0; m < 2; m++)
        nib[r][m] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, kg * kTileBytes + 16 * lane,
                                                         (int)(r * rt_bytes + m * mat_bytes), kNonTemporal));
    long xb[4];
#pragma unroll
    for (int b = 0; b < 4; b++) xb[b] = *reinterpret_cast<const long*>(xrow + 32 * (4 * kg + b) + 8 * G);
    const u32x2 dxw = *reinterpret_cast<const u32x2*>(drow + 4 * kg);  // the 4 blocks' fp16 scales
    *reinterpret_cast<u32x4*>(sc + 4 * lane) = scw;  // a wavefront's LDS operations run in order
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const float dx = half_bits_to_float(dxw[b >> 1] >> (16 * (b & 1)));
#pragma unroll
      for (int r = 0; r < kW8GuRowTiles; r++)
#pragma unroll
        for (int m = 0; m < 2; m++) {
          const i32x4 cr = mfma_i8(decode_word_i8(sh.tbl, nib[r][m][b], lane & 31), xb[b]);
          const uint32_t* sp = sc + 32 * (r * 2 + m) + 8 * G + 2 * b;
          scale_acc_i8(acc[r][m], cr, sp[0], sp[1], dx);
        }
    }
  }
  __syncthreads();  // the scale buffers become the reduction buffer
#pragma unroll
  for (int r = 0; r < kW8GuRowTiles; r++) sh.u.red[r][wave][lane] = acc[r][0];
  __syncthreads();
  f32x4 g = zero;
  if (wave < kW8GuRowTiles) {
    g = sh.u.red[wave][0][lane];
#pragma unroll
    for (int w = 1; w < kW8GuWaves; w++) g += sh.u.red[wave][w][lane];
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kW8GuRowTiles; r++) sh.u.red[r][wave][lane] = acc[r][1];
  __syncthreads();
  const int c = lane & 15;
  if (wave >= kW8GuRowTiles || c >= ch.count) return;
  f32x4 u = sh.u.red[wave][0][lane];
#pragma unroll
  for (int w = 1; w < kW8GuWaves; w++) u += sh.u.red[wave][w][lane];
  const int64_t hrow = (ch.expert >= 0 ? 0 : (int64_t)T * K) + ch.first + c;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int f = 16 * (rt0 + wave) + 4 * G + i;
    const float gv = g[i];
    h[hrow * F + f] = gv / (1.0f + expf(-gv)) * u[i];
  }
}

// ---------------------------------------------------------------- down

struct DownW8Lds {
  uint32_t scales[kW8DnWaves][256];                  // per wavefront: [row tile][32 words] of its tile column
  uint32_t tbl[kPairTableWords];
  f32x4 red[kW8DnWaves][kW8DnRowTiles / 2][64];    // the row tiles are reduced in two halves
};

// Workgroup = (chunk, 8 row tiles of H).  y[hrow][n] = sum_f W_down[n][f] h[f]
// with h as Q8_0 codes hq [row][F] and scales hd [row][F/32].
__global__ __launch_bounds__(kW8DnThreads) void k_down_w4a8(
    int H, int F, int K, int T, const uint8_t* __restrict__ arena, const uint8_t* __restrict__ shared,
    int64_t expert_bytes, const Chunk* __restrict__ chunks, const int32_t* __restrict__ n_chunks,
    const int8_t* __restrict__ hq, const uint16_t* __restrict__ hd, float* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) DownW8Lds sh;
  const int n_slab = H / (16 * kW8DnRowTiles);
  const int chunk_id = blockIdx.x / n_slab;
  const int slab = blockIdx.x % n_slab;
  if (chunk_id >= *n_chunks) return;
  const Chunk ch = chunks[chunk_id];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, G = lane >> 4;
  const int64_t mat_bytes = expert_bytes / 3;
  const uint8_t* ex = ch.expert >= 0 ? arena + (int64_t)ch.expert * expert_bytes : shared;
  const int TK = T * K;
  const int cc = c < ch.count ? c : 0;
  const int64_t hrow = ch.expert >= 0 ? (int64_t)(ch.first + cc) : (int64_t)TK + ch.first + cc;
  const int8_t* hqr = hq + hrow * F;
  const uint16_t* hdr = hd + hrow * (F / 32);
  const int nkg = F >> 7;
  const int kg0 = wave * nkg / kW8DnWaves, kg1 = (wave + 1) * nkg / kW8DnWaves;
  const int64_t rt_bytes = (int64_t)nkg * kTileBytes;
  const uint8_t* rows = ex + 2 * mat_bytes + (int64_t)slab * kW8DnRowTiles * rt_bytes;
  uint32_t* my_scales = sh.scales[wave];
  const __amdgpu_buffer_rsrc_t rows_rsrc = rsrc_of(rows);

  build_i8_pair_table(sh.tbl);
  __syncthreads();
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[kW8DnRowTiles];
#pragma unroll
  for (int t = 0; t < kW8DnRowTiles; t++) acc[t] = zero;
  for (int kg = kg0; kg < kg1; kg++) {
    dma16_stream(rows + min(lane >> 3, kW8DnRowTiles - 1) * rt_bytes + (int64_t)kg * kTileBytes + kTileNibbleBytes +
                     16 * (lane & 7),
                 my_scales);
    u32x4 nib[kW8DnRowTiles];
    const int voff = kg * kTileBytes + 16 * lane;
#pragma unroll
    for (int t = 0; t < kW8DnRowTiles; t++)
      nib[t] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rows_rsrc, voff, (int)(t * rt_bytes), kNonTemporal));
    long hb[4];
#pragma unroll
    for (int b = 0; b < 4; b++) hb[b] = *reinterpret_cast<const long*>(hqr + 32 * (4 * kg + b) + 8 * G);
    const u32x2 dhw = *reinterpret_cast<const u32x2*>(hdr + 4 * kg);
    wait_loads();  // the scale pieces (LDS DMA) with the rest
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const float dh = half_bits_to_float(dhw[b >> 1] >> (16 * (b & 1)));
#pragma unroll
      for (int t = 0; t < kW8DnRowTiles; t++) {
        const i32x4 cr = mfma_i8(decode_word_i8(sh.tbl, nib[t][b], lane & 31), hb[b]);
        const uint32_t* sd = my_scales + 32 * t + 8 * G + 2 * b;
        scale_acc_i8(acc[t], cr, sd[0], sd[1], dh);
      }
    }
  }
  const int64_t hrow_c = (ch.expert >= 0 ? 0 : (int64_t)TK) + ch.first + c;
#pragma unroll
  for (int half = 0; half < 2; half++) {
#pragma unroll
    for (int t = 0; t < kW8DnRowTiles / 2; t++) sh.red[wave][t][lane] = acc[(kW8DnRowTiles / 2) * half + t];
    __syncthreads();
    if (wave < kW8DnRowTiles / 2 && c < ch.count) {
      f32x4 s = sh.red[0][wave][lane];
#pragma unroll
      for (int w = 1; w < kW8DnWaves; w++) s += sh.red[w][wave][lane];
      const int rt = slab * kW8DnRowTiles + (kW8DnRowTiles / 2) * half + wave;
      *reinterpret_cast<f32x4*>(y + hrow_c * H + 16 * rt + 4 * G) = s;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- launcher

hipError_t launch_ffn_w4a8(const uint16_t* x, int T, int H, int F, int K, int n_shared, int gated, int max_chunks,
                           const uint8_t* arena, const uint8_t* shared, int64_t expert_bytes, const int32_t* perm,
                           const int32_t* pos, const float* w, const Chunk* chunks, const int32_t* n_chunks,
                           int8_t* xq, uint16_t* xd, float* h, int8_t* hq, uint16_t* hd, float* y, float* out,
                           hipStream_t stream) {
  if (T == 0) return hipSuccess;
  hipError_t err = launch_quantize_q8_0(x, 1, (int64_t)T * H, xq, xd, stream);
  if (err != hipSuccess) return err;
  clear_last_error();
  hipLaunchKernelGGL(k_gate_up_w4a8, dim3((unsigned)(max_chunks * (F / (16 * kW8GuRowTiles)))), dim3(kW8GuThreads), 0,
                     stream, xq, xd, H, F, K, T, arena, shared, expert_bytes, perm, chunks, n_chunks, h);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t rows = (int64_t)T * K + (n_shared ? T : 0);
  err = launch_quantize_q8_0(h, 0, rows * F, hq, hd, stream);
  if (err != hipSuccess) return err;
  clear_last_error();
  hipLaunchKernelGGL(k_down_w4a8, dim3((unsigned)(max_chunks * (H / (16 * kW8DnRowTiles)))), dim3(kW8DnThreads), 0,
                     stream, H, F, K, T, arena, shared, expert_bytes, chunks, n_chunks, hq, hd, y);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_combine(y, pos, w, T, K, H, n_shared, gated, out, stream);
}

}  // namespace qmoe
