// Expert FFN for the other expert codecs (FP32 contract: exact weights).
//
//   IQ4_XS  super-blocks of 256 weights: fp16 d, 6-bit sub-block scales ls,
//           IQ4_NL indices; weight = d * (ls - 32) * level (the zLLM feed and
//           the W7900D article name it beside IQ4_NL).
//   Q3      packed 3-bit affine groups of 64 weights: fp16 scale and bias,
//           3-bit codes q; weight = scale * q + bias (the SSD streaming page,
//           packed 3-bit section: 8 codes in 3 bytes, 4-bit element order).
//
// Packed layout (moe_pack_experts), per matrix tiles of 16 rows x 128 weights
// in the IQ4_NL tile order (tile (rt, kg) at rt * (cols / 128) + kg):
//   IQ4_XS  1120 bytes: [0, 1024) the indices as in an IQ4_NL tile (lane slot
//           s = row s % 16, word s / 16: 4 bytes per block b of weights
//           8w..8w+7, byte i = weight 8w+2i low nibble, 8w+2i+1 high);
//           [1024, 1056) the fp16 d of each row (row r at 1024 + 2r; both
//           tiles of a super-block repeat it); [1056, 1120) the 6-bit ls of
//           (row 4G + i, block b) as a byte at 1056 + 16G + 4b + i.
//   Q3      896 bytes: [0, 768) 12 bytes per lane slot, 3 per block b: the
//           codes of weights 8w..8w+7 of block b, code j at bits 3j of the
//           24-bit little-endian value (the source bytes of those weights,
//           unchanged); [768, 896) scale and bias (fp16) of (row 4G + i,
//           group g of the tile's two 64-weight groups) at 768 + 32G + 16g + 4i
//           and + 2.
//
// Arithmetic: every 32-weight block is one v_mfma_f32_16x16x32_bf16 of the
// exact small integers (levels; codes 0..7) against the activations, then in
// fp32 acc += s * C (IQ4_XS, s = d * (ls - 32), exact) or
// acc += scale * C + bias * S (Q3, S the block's sum of activations, from one
// more MFMA against a ones operand).  h is handed to down as bf16 hi + lo, as
// in the IQ4_NL FP32 kernels.  Work: the chunks of up to 16 routes of one
// expert from the bucketing pass; gate/up workgroups of (chunk, 32 rows of F)
// over 4 wavefronts, down workgroups of (chunk, 128 rows of H) over 8.
#include "device.h"
#include "launch.h"

namespace qmoe {

constexpr int kCodecXs = 1;
constexpr int kCodecQ3 = 2;

typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

template <int C>
struct Codec;

template <>
struct Codec<kCodecXs> {
  static constexpr int kTile = 1120, kCodeBytes = 1024, kScaleBytes = 96;
};

template <>
struct Codec<kCodecQ3> {
  static constexpr int kTile = 896, kCodeBytes = 768, kScaleBytes = 128;
};

int codec_tile_bytes(int codec) { return codec == kCodecXs ? Codec<kCodecXs>::kTile : Codec<kCodecQ3>::kTile; }

// ---------------------------------------------------------------- packing

// One thread per lane slot of a tile (64 per tile); src rows of `cols`
// weights in the codec's own byte order.
template <int C>
__global__ void k_pack_codec(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t n_tiles, int rows,
                             int cols) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t tile = gid >> 6;
  const int slot = (int)(gid & 63);
  if (tile >= n_tiles) return;
  const int nkg = cols >> 7;
  const int rt = (int)(tile / nkg), kg = (int)(tile % nkg);
  uint8_t* t_dst = dst + tile * Codec<C>::kTile;
  const int row = 16 * rt + (slot & 15), w = slot >> 4;
  if constexpr (C == kCodecXs) {
    const int64_t row_bytes = (int64_t)(cols / 256) * 136;
    const uint8_t* sb = src + row * row_bytes + (int64_t)(kg >> 1) * 136;
    uint8_t out[16];
    for (int b = 0; b < 4; b++) {
      const uint8_t* qs = sb + 8 + 16 * (4 * (kg & 1) + b);
      for (int i = 0; i < 4; i++) {
        const int k0 = 8 * w + 2 * i, k1 = k0 + 1;
        const int q0 = k0 < 16 ? (qs[k0] & 15) : (qs[k0 - 16] >> 4);
        const int q1 = k1 < 16 ? (qs[k1] & 15) : (qs[k1 - 16] >> 4);
        out[4 * b + i] = (uint8_t)(q0 | (q1 << 4));
      }
    }
    uint4 v;
    __builtin_memcpy(&v, out, 16);
    *reinterpret_cast<uint4*>(t_dst + 16 * slot) = v;
    if (slot < 16) {  // this row's d and its 4 sub-block scales
      const int r = slot;
      const uint8_t* sr = src + (int64_t)(16 * rt + r) * row_bytes + (int64_t)(kg >> 1) * 136;
      t_dst[1024 + 2 * r] = sr[0];
      t_dst[1024 + 2 * r + 1] = sr[1];
      const unsigned sh = (unsigned)sr[2] | ((unsigned)sr[3] << 8);
      for (int b = 0; b < 4; b++) {
        const int ib = 4 * (kg & 1) + b;
        const int ls = ((sr[4 + ib / 2] >> (4 * (ib % 2))) & 15) | (((sh >> (2 * ib)) & 3) << 4);
        t_dst[1056 + 16 * (r >> 2) + 4 * b + (r & 3)] = (uint8_t)ls;
      }
    }
  } else {
    const int64_t row_bytes = (int64_t)(cols / 64) * 28;
    const uint8_t* sr = src + row * row_bytes;
    for (int b = 0; b < 4; b++) {
      const uint8_t* g = sr + (int64_t)(2 * kg + (b >> 1)) * 28;
      const int j0 = 32 * (b & 1) + 8 * w;  // multiple of 8: its codes start on a byte
      for (int i = 0; i < 3; i++) t_dst[12 * slot + 3 * b + i] = g[4 + 3 * j0 / 8 + i];
    }
    if (slot < 16) {
      const int r = slot;
      const uint8_t* s2 = src + (int64_t)(16 * rt + r) * row_bytes;
      for (int gi = 0; gi < 2; gi++) {
        const uint8_t* g = s2 + (int64_t)(2 * kg + gi) * 28;
        for (int i = 0; i < 4; i++) t_dst[768 + 32 * (r >> 2) + 16 * gi + 4 * (r & 3) + i] = g[i];
      }
    }
  }
}

hipError_t launch_pack_codec(int codec, const uint8_t* src, uint8_t* dst, int n_experts, int H, int F,
                             int64_t src_expert_bytes, int64_t dst_expert_bytes, hipStream_t stream) {
  for (int e = 0; e < n_experts; e++) {
    int64_t s_off = (int64_t)e * src_expert_bytes, d_off = (int64_t)e * dst_expert_bytes;
    for (int m = 0; m < 3; m++) {
      const int rows = m < 2 ? F : H, cols = m < 2 ? H : F;
      const int64_t tiles = (int64_t)(rows / 16) * (cols / 128);
      const int64_t src_mat = codec == kCodecXs ? (int64_t)rows * (cols / 256) * 136 : (int64_t)rows * (cols / 64) * 28;
      clear_last_error();
      if (codec == kCodecXs)
        hipLaunchKernelGGL(k_pack_codec<kCodecXs>, dim3((unsigned)((tiles * 64 + 255) / 256)), dim3(256), 0, stream,
                           src + s_off, dst + d_off, tiles, rows, cols);
      else
        hipLaunchKernelGGL(k_pack_codec<kCodecQ3>, dim3((unsigned)((tiles * 64 + 255) / 256)), dim3(256), 0, stream,
                           src + s_off, dst + d_off, tiles, rows, cols);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
      s_off += src_mat;
      d_off += tiles * codec_tile_bytes(codec);
    }
  }
  return hipSuccess;
}

// ---------------------------------------------------------------- decoding

// Q3: 64-entry table of code pairs (bf16 of the low code in bits 0..15, of the
// high code in 16..31), 32 replicas (lane l reads bank l % 32).
constexpr int kQ3TableWords = 64 * 32;

__device__ __forceinline__ void build_q3_table(uint32_t* tbl) {
  for (int i = threadIdx.x; i < kQ3TableWords; i += blockDim.x) {
    const int v = i >> 5;
    tbl[i] = small_int_bf16(v & 7) | (small_int_bf16(v >> 3) << 16);
  }
}

// The 24-bit code value of block b from a lane's 12 code bytes.
__device__ __forceinline__ uint32_t q3_codes(const u32x3& raw, int b) {
  const uint64_t lo = ((uint64_t)raw[1] << 32) | raw[0];
  const uint64_t hi = ((uint64_t)raw[2] << 32) | raw[1];
  switch (b) {
    case 0: return (uint32_t)(lo & 0xffffffu);
    case 1: return (uint32_t)((lo >> 24) & 0xffffffu);
    case 2: return (uint32_t)((hi >> 16) & 0xffffffu);
    default: return (uint32_t)((hi >> 40) & 0xffffffu);
  }
}

// 8 codes -> the bf16 operand (code j -> slot j).
__device__ __forceinline__ bf16x8 decode_q3(const uint32_t* tbl, uint32_t v, uint32_t lane32) {
  union {
    uint32_t u[4];
    bf16x8 b;
  } r;
#pragma unroll
  for (int p = 0; p < 4; p++) r.u[p] = tbl[((v >> (6 * p)) & 63u) * 32u + lane32];
  return r.b;
}

// The scale words of one tile's scale area (as staged in LDS, 32 words) for
// the lane's rows 4G + i and block b: IQ4_XS -> s (acc += s * C), Q3 -> scale
// and bias (acc += scale * C + bias * S).
__device__ __forceinline__ float xs_scale(const uint32_t* sw, int G, int i, int b) {
  const float d = half_bits_to_float(sw[2 * G + (i >> 1)] >> (16 * (i & 1)));
  const int ls = (int)((sw[8 + 4 * G + b] >> (8 * i)) & 0xffu);
  return d * (float)(ls - 32);
}

__device__ __forceinline__ uint32_t q3_scale_word(const uint32_t* sw, int G, int i, int b) {
  return sw[8 * G + 4 * (b >> 1) + i];
}

template <int C>
__device__ __forceinline__ void codec_acc(f32x4& acc, const f32x4& c, const f32x4& s, const uint32_t* sw, int G,
                                          int b) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    if constexpr (C == kCodecXs) {
      acc[i] = __builtin_fmaf(xs_scale(sw, G, i, b), c[i], acc[i]);
    } else {
      const uint32_t wd = q3_scale_word(sw, G, i, b);
      acc[i] = __builtin_fmaf(half_bits_to_float(wd), c[i], acc[i]);
      acc[i] = __builtin_fmaf(half_bits_to_float(wd >> 16), s[i], acc[i]);
    }
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t codec_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

// The lane's code data of a tile: IQ4_XS 16 bytes (a nibble word per block),
// Q3 12 bytes.
template <int C>
struct LaneCodes {
  u32x4 v;
};

template <int C>
__device__ __forceinline__ LaneCodes<C> load_codes(__amdgpu_buffer_rsrc_t r, int tile_off, int soff, int lane) {
  LaneCodes<C> t;
  if constexpr (C == kCodecXs) {
    t.v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, tile_off + 16 * lane, soff, kNonTemporal));
  } else {
    const u32x3 q = __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(r, tile_off + 12 * lane, soff,
                                                                                   kNonTemporal));
    t.v = u32x4{q[0], q[1], q[2], 0u};
  }
  return t;
}

template <int C>
__device__ __forceinline__ bf16x8 decode_block(const uint32_t* tbl, const LaneCodes<C>& t, int b, uint32_t lane32) {
  if constexpr (C == kCodecXs) return decode_word(tbl, t.v[b], lane32);
  else return decode_q3(tbl, q3_codes(u32x3{t.v[0], t.v[1], t.v[2]}, b), lane32);
}

template <int C>
__device__ __forceinline__ void build_codec_table(uint32_t* tbl) {
  if constexpr (C == kCodecXs) build_pair_table(tbl);
  else build_q3_table(tbl);
}

__device__ __forceinline__ bf16x8 ones_operand() {
  const short one = (short)0x3f80;
  bf16x8 o = {one, one, one, one, one, one, one, one};
  return o;
}

// ---------------------------------------------------------------- dequant (one wavefront per tile)

template <int C>
__global__ __launch_bounds__(256) void k_dequant_codec(const uint8_t* __restrict__ mat, int rows, int cols,
                                                       float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint32_t tbl[kPairTableWords];
  build_codec_table<C>(tbl);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int nkg = cols >> 7;
  const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= (int64_t)(rows >> 4) * nkg) return;
  const int rt = (int)(tile / nkg), kg = (int)(tile % nkg);
  const uint8_t* t = mat + tile * Codec<C>::kTile;
  const LaneCodes<C> codes = load_codes<C>(codec_rsrc(t), 0, 0, lane);
  const int r = lane & 15, w = lane >> 4, G = r >> 2, i = r & 3;
  const uint32_t* sw = reinterpret_cast<const uint32_t*>(t + Codec<C>::kCodeBytes);
  for (int b = 0; b < 4; b++) {
    union {
      bf16x8 v;
      uint32_t u[4];
    } a;
    a.v = decode_block<C>(tbl, codes, b, lane & 31);
    float* o = out + (size_t)(16 * rt + r) * cols + 32 * (4 * kg + b) + 8 * w;
    for (int k = 0; k < 8; k++) {
      const float q = bf16_bits_to_f32((a.u[k >> 1] >> (16 * (k & 1))) & 0xffffu);
      if constexpr (C == kCodecXs) {
        o[k] = xs_scale(sw, G, i, b) * q;
      } else {
        const uint32_t wd = q3_scale_word(sw, G, i, b);
        o[k] = __builtin_fmaf(half_bits_to_float(wd), q, half_bits_to_float(wd >> 16));
      }
    }
  }
}

hipError_t launch_dequant_codec(int codec, const uint8_t* mat, int rows, int cols, float* out, hipStream_t stream) {
  const int64_t tiles = (int64_t)(rows / 16) * (cols / 128);
  clear_last_error();
  if (codec == kCodecXs)
    hipLaunchKernelGGL(k_dequant_codec<kCodecXs>, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0, stream, mat, rows,
                       cols, out);
  else
    hipLaunchKernelGGL(k_dequant_codec<kCodecQ3>, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0, stream, mat, rows,
                       cols, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------- gate / up

constexpr int kCdGuWaves = 4;
constexpr int kCdGuRowTiles = 2;
constexpr int kCdDnWaves = 8;
constexpr int kCdDnRowTiles = 8;

struct GateUpCodecLds {
  union {
    uint32_t scales[kCdGuWaves][256];         // per wavefront: 32 words of (row tile r, matrix m) at 32 (2r + m)
    f32x4 red[kCdGuRowTiles][kCdGuWaves][64];  // wavefront partials of one matrix
  } u;
  uint32_t tbl[kPairTableWords];
};

template <int C>
__global__ __launch_bounds__(64 * kCdGuWaves) void k_gate_up_codec(
    const uint16_t* __restrict__ x, int H, int F, int K, int T, const uint8_t* __restrict__ arena,
    const uint8_t* __restrict__ shared, int64_t expert_bytes, const int32_t* __restrict__ perm,
    const Chunk* __restrict__ chunks, const int32_t* __restrict__ n_chunks, uint16_t* __restrict__ h_hi,
    uint16_t* __restrict__ h_lo) {
  __shared__ __attribute__((aligned(16))) GateUpCodecLds sh;
  const int n_rp = F / (16 * kCdGuRowTiles);
  const int chunk_id = blockIdx.x / n_rp;
  const int rt0 = kCdGuRowTiles * (blockIdx.x % n_rp);
  if (chunk_id >= *n_chunks) return;
  const Chunk ch = chunks[chunk_id];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = lane >> 4;
  const int64_t mat_bytes = expert_bytes / 3;
  const uint8_t* ex = ch.expert >= 0 ? arena + (int64_t)ch.expert * expert_bytes : shared;
  const int cc = (lane & 15) < ch.count ? (lane & 15) : 0;
  const int tok = ch.expert >= 0 ? perm[ch.first + cc] / K : ch.first + cc;
  const int nkg = H >> 7;
  const int kg0 = wave * nkg / kCdGuWaves, kg1 = (wave + 1) * nkg / kCdGuWaves;
  const int rt_bytes = nkg * Codec<C>::kTile;
  const __amdgpu_buffer_rsrc_t w_rsrc = codec_rsrc(ex + rt0 * rt_bytes);
  // this lane's 16-byte scale piece: piece (lane % 8, clamped to the scale
  // area) of row tile (lane / 16) % 2, matrix (lane / 8) % 2
  const int piece = min(lane & 7, Codec<C>::kScaleBytes / 16 - 1);
  const int sc_off = ((lane >> 4) & 1) * rt_bytes + ((lane >> 3) & 1) * (int)mat_bytes + Codec<C>::kCodeBytes +
                     16 * piece;
  const uint16_t* xrow = x + (int64_t)tok * H;
  uint32_t* sc = sh.u.scales[wave];

  build_codec_table<C>(sh.tbl);
  __syncthreads();
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[kCdGuRowTiles][2];
#pragma unroll
  for (int r = 0; r < kCdGuRowTiles; r++) acc[r][0] = acc[r][1] = zero;
  for (int kg = kg0; kg < kg1; kg++) {
    const int toff = kg * Codec<C>::kTile;
    const u32x4 scw =
        __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, sc_off, toff, kNonTemporal));
    LaneCodes<C> codes[kCdGuRowTiles][2];
#pragma unroll
    for (int r = 0; r < kCdGuRowTiles; r++)
#pragma unroll
      for (int m = 0; m < 2; m++) codes[r][m] = load_codes<C>(w_rsrc, toff, (int)(r * rt_bytes + m * mat_bytes), lane);
    bf16x8 xb[4];
#pragma unroll
    for (int b = 0; b < 4; b++) xb[b] = load_x_operand(xrow, 4 * kg + b, G);
    *reinterpret_cast<u32x4*>(sc + 4 * lane) = scw;  // a wavefront's LDS operations run in order
#pragma unroll
    for (int b = 0; b < 4; b++) {
      f32x4 s = zero;
      if constexpr (C == kCodecQ3) s = mfma16x16x32(ones_operand(), xb[b], zero);
#pragma unroll
      for (int r = 0; r < kCdGuRowTiles; r++)
#pragma unroll
        for (int m = 0; m < 2; m++) {
          const f32x4 cr = mfma16x16x32(decode_block<C>(sh.tbl, codes[r][m], b, lane & 31), xb[b], zero);
          codec_acc<C>(acc[r][m], cr, s, sc + 32 * (r * 2 + m), G, b);
        }
    }
  }
  __syncthreads();  // the scale buffers become the reduction buffer
#pragma unroll
  for (int r = 0; r < kCdGuRowTiles; r++) sh.u.red[r][wave][lane] = acc[r][0];
  __syncthreads();
  f32x4 g = zero;
  if (wave < kCdGuRowTiles) {
    g = sh.u.red[wave][0][lane];
#pragma unroll
    for (int w = 1; w < kCdGuWaves; w++) g += sh.u.red[wave][w][lane];
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kCdGuRowTiles; r++) sh.u.red[r][wave][lane] = acc[r][1];
  __syncthreads();
  const int c = lane & 15;
  if (wave >= kCdGuRowTiles || c >= ch.count) return;
  f32x4 u = sh.u.red[wave][0][lane];
#pragma unroll
  for (int w = 1; w < kCdGuWaves; w++) u += sh.u.red[wave][w][lane];
  const int64_t hrow = (ch.expert >= 0 ? 0 : (int64_t)T * K) + ch.first + c;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int f = 16 * (rt0 + wave) + 4 * G + i;
    const float gv = g[i];
    const float hv = gv / (1.0f + expf(-gv)) * u[i];
    const uint32_t hb = f32_to_bf16_rne(hv);
    h_hi[hrow * F + f] = (uint16_t)hb;
    h_lo[hrow * F + f] = (uint16_t)f32_to_bf16_rne(hv - bf16_bits_to_f32(hb));
  }
}

// ---------------------------------------------------------------- down

struct DownCodecLds {
  uint32_t scales[kCdDnWaves][256];                 // per wavefront: [row tile][32 words] of its tile column
  uint32_t tbl[kPairTableWords];
  f32x4 red[kCdDnWaves][kCdDnRowTiles / 2][64];   // the row tiles are reduced in two halves
};

template <int C>
__global__ __launch_bounds__(64 * kCdDnWaves) void k_down_codec(
    int H, int F, int K, int T, const uint8_t* __restrict__ arena, const uint8_t* __restrict__ shared,
    int64_t expert_bytes, const Chunk* __restrict__ chunks, const int32_t* __restrict__ n_chunks,
    const uint16_t* __restrict__ h_hi, const uint16_t* __restrict__ h_lo, float* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) DownCodecLds sh;
  const int n_slab = H / (16 * kCdDnRowTiles);
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
  const uint16_t* hh = h_hi + hrow * F;
  const uint16_t* hl = h_lo + hrow * F;
  const int nkg = F >> 7;
  const int kg0 = wave * nkg / kCdDnWaves, kg1 = (wave + 1) * nkg / kCdDnWaves;
  const int64_t rt_bytes = (int64_t)nkg * Codec<C>::kTile;
  const uint8_t* rows = ex + 2 * mat_bytes + (int64_t)slab * kCdDnRowTiles * rt_bytes;
  uint32_t* my_scales = sh.scales[wave];
  const __amdgpu_buffer_rsrc_t rows_rsrc = codec_rsrc(rows);

  build_codec_table<C>(sh.tbl);
  __syncthreads();
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[kCdDnRowTiles];
#pragma unroll
  for (int t = 0; t < kCdDnRowTiles; t++) acc[t] = zero;
  for (int kg = kg0; kg < kg1; kg++) {
    const int toff = kg * Codec<C>::kTile;
    // lane l: piece (l % 8, clamped) of the scale area of row tile l / 8
    const int piece = min(lane & 7, Codec<C>::kScaleBytes / 16 - 1);
    dma16_stream(rows + min(lane >> 3, kCdDnRowTiles - 1) * rt_bytes + toff + Codec<C>::kCodeBytes + 16 * piece,
                 my_scales);
    LaneCodes<C> codes[kCdDnRowTiles];
#pragma unroll
    for (int t = 0; t < kCdDnRowTiles; t++) codes[t] = load_codes<C>(rows_rsrc, toff, (int)(t * rt_bytes), lane);
    bf16x8 bh[4], bl[4];
#pragma unroll
    for (int b = 0; b < 4; b++) {
      bh[b] = load_x_operand(hh, 4 * kg + b, G);
      bl[b] = load_x_operand(hl, 4 * kg + b, G);
    }
    wait_loads();  // the scale pieces (LDS DMA) with the rest
#pragma unroll
    for (int b = 0; b < 4; b++) {
      f32x4 s = zero;
      if constexpr (C == kCodecQ3) s = mfma16x16x32(ones_operand(), bl[b], mfma16x16x32(ones_operand(), bh[b], zero));
#pragma unroll
      for (int t = 0; t < kCdDnRowTiles; t++) {
        const bf16x8 a = decode_block<C>(sh.tbl, codes[t], b, lane & 31);
        const f32x4 cr = mfma16x16x32(a, bl[b], mfma16x16x32(a, bh[b], zero));
        codec_acc<C>(acc[t], cr, s, my_scales + 32 * t, G, b);
      }
    }
  }
  const int64_t hrow_c = (ch.expert >= 0 ? 0 : (int64_t)TK) + ch.first + c;
#pragma unroll
  for (int half = 0; half < 2; half++) {
#pragma unroll
    for (int t = 0; t < kCdDnRowTiles / 2; t++) sh.red[wave][t][lane] = acc[(kCdDnRowTiles / 2) * half + t];
    __syncthreads();
    if (wave < kCdDnRowTiles / 2 && c < ch.count) {
      f32x4 s = sh.red[0][wave][lane];
#pragma unroll
      for (int w = 1; w < kCdDnWaves; w++) s += sh.red[w][wave][lane];
      const int rt = slab * kCdDnRowTiles + (kCdDnRowTiles / 2) * half + wave;
      *reinterpret_cast<f32x4*>(y + hrow_c * H + 16 * rt + 4 * G) = s;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- launcher

hipError_t launch_ffn_codec(int codec, const uint16_t* x, int T, int H, int F, int K, int n_shared, int gated,
                            int max_chunks, const uint8_t* arena, const uint8_t* shared, int64_t expert_bytes,
                            const int32_t* perm, const int32_t* pos, const float* w, const Chunk* chunks,
                            const int32_t* n_chunks, uint16_t* h_hi, uint16_t* h_lo, float* y, float* out,
                            hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 gu((unsigned)(max_chunks * (F / (16 * kCdGuRowTiles)))), dn((unsigned)(max_chunks * (H / (16 * kCdDnRowTiles))));
  clear_last_error();
  if (codec == kCodecXs)
    hipLaunchKernelGGL(k_gate_up_codec<kCodecXs>, gu, dim3(64 * kCdGuWaves), 0, stream, x, H, F, K, T, arena, shared,
                       expert_bytes, perm, chunks, n_chunks, h_hi, h_lo);
  else
    hipLaunchKernelGGL(k_gate_up_codec<kCodecQ3>, gu, dim3(64 * kCdGuWaves), 0, stream, x, H, F, K, T, arena, shared,
                       expert_bytes, perm, chunks, n_chunks, h_hi, h_lo);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  clear_last_error();
  if (codec == kCodecXs)
    hipLaunchKernelGGL(k_down_codec<kCodecXs>, dn, dim3(64 * kCdDnWaves), 0, stream, H, F, K, T, arena, shared,
                       expert_bytes, chunks, n_chunks, h_hi, h_lo, y);
  else
    hipLaunchKernelGGL(k_down_codec<kCodecQ3>, dn, dim3(64 * kCdDnWaves), 0, stream, H, F, K, T, arena, shared,
                       expert_bytes, chunks, n_chunks, h_hi, h_lo, y);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_combine(y, pos, w, T, K, H, n_shared, gated, out, stream);
}

}  // namespace qmoe
