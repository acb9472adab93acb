// Expert FFN with exact IQ4_NL weights (the decode / small-batch path).
//
// The FFN is the gated MLP y = W_down(silu(W_gate x) * (W_up x)) (zLLM
// "Algorithm Layer", FFN section), silu(g) * u handed to the down projection
// in fp32 and the routed + shared sum formed in fp32 (PocketLLM design record,
// section 2).
//
// Work is a list of chunks, each up to 16 routes of one expert (or up to 16
// tokens of the shared expert), produced by the bucketing pass: an expert's
// weights are streamed once per chunk, not once per route.  Every 16x32
// weight fragment (16 rows, one 32-weight block) is one v_mfma_f32_16x16x32_bf16
// against the chunk's 16 activation columns:
//   A = the block's levels (exact in bf16, decoded two at a time from LDS),
//   B = the activations (bf16) -- or, for the down projection, the fp32
//       product h split exactly enough as h_hi + h_lo (two bf16, two MFMAs),
//   then acc += d * C with the block's fp16 scale d, in fp32.
// So the weights are the exact values d*level; products of levels and bf16
// activations are exact; only fp32 accumulation rounds.
//
// Memory: a packed tile (16 rows x 4 blocks, 1152 bytes) is read by one
// wavefront with one 16-byte load per lane for the nibbles (into registers);
// the scales of a wavefront's tiles of one column come as one 16-byte piece
// per lane (gate/up: into a register, then the wavefront's LDS; down: by LDS
// DMA), fully coalesced.  A gate/up workgroup owns one (chunk, 32 rows of F)
// and splits the reduction dimension over 4 wavefronts, a down workgroup one
// (chunk, 128 rows of H) over 8.
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace qmoe {

// ---------------------------------------------------------------- packing

// One thread per 16-byte lane slot of a tile.  src: GGUF order, rows of
// NB = cols/32 blocks of 18 bytes, byte j of a block holding the index of
// weight j (low nibble) and of weight j+16 (high nibble).  Lane slot s (row
// s%16, word w = s/16) receives, per block, the indices of weights
// 8w..8w+7 as 4 bytes (weight 8w+2i low, 8w+2i+1 high in byte i).  Threads
// with slot < 16 also place the four scales of (rows 4G..4G+3, block b),
// G = slot/4, b = slot%4.
__global__ void k_pack(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t n_tiles_total,
                       int rows, int nb, int64_t matrix_bytes) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t tile = gid >> 6;
  const int slot = (int)(gid & 63);
  if (tile >= n_tiles_total) return;
  const int nkg = nb >> 2;
  const int64_t tiles_per_matrix = (int64_t)(rows >> 4) * nkg;
  const int64_t mat = tile / tiles_per_matrix;
  const int64_t tin = tile % tiles_per_matrix;
  const int rt = (int)(tin / nkg), kg = (int)(tin % nkg);
  const uint8_t* m_src = src + mat * matrix_bytes;
  uint8_t* t_dst = dst + mat * matrix_bytes + tin * kTileBytes;
  {
    const int row = 16 * rt + (slot & 15), w = slot >> 4;
    uint8_t out[16];
    for (int b = 0; b < 4; b++) {
      const uint8_t* blk = m_src + ((int64_t)row * nb + 4 * kg + b) * 18;
      for (int i = 0; i < 4; i++) {
        const int k0 = 8 * w + 2 * i, k1 = k0 + 1;  // weight indices, 0..31
        const int q0 = k0 < 16 ? (blk[2 + k0] & 15) : (blk[2 + k0 - 16] >> 4);
        const int q1 = k1 < 16 ? (blk[2 + k1] & 15) : (blk[2 + k1 - 16] >> 4);
        out[4 * b + i] = (uint8_t)(q0 | (q1 << 4));
      }
    }
    uint4 v;
    __builtin_memcpy(&v, out, 16);
    *reinterpret_cast<uint4*>(t_dst + 16 * slot) = v;
  }
  if (slot < 16) {
    const int G = slot >> 2, b = slot & 3;
    uint8_t out[8];
    for (int i = 0; i < 4; i++) {
      const uint8_t* blk = m_src + ((int64_t)(16 * rt + 4 * G + i) * nb + 4 * kg + b) * 18;
      out[2 * i] = blk[0];
      out[2 * i + 1] = blk[1];
    }
    uint2 v;
    __builtin_memcpy(&v, out, 8);
    *reinterpret_cast<uint2*>(t_dst + kTileNibbleBytes + 32 * G + 8 * b) = v;
  }
}

// ---------------------------------------------------------------- dequant

// One wavefront per tile; writes the 16 x 128 weights of the tile.
// bf16 = 0: exact d*level in fp32; bf16 = 1: that value rounded to bf16.
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ mat, int rows, int cols, int bf16,
                                                 float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint32_t tbl[kPairTableWords];
  build_pair_table(tbl);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int nkg = cols >> 7;
  const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= (int64_t)(rows >> 4) * nkg) return;
  const int rt = (int)(tile / nkg), kg = (int)(tile % nkg);
  const uint8_t* t = mat + tile * kTileBytes;
  const uint4 nib = *reinterpret_cast<const uint4*>(t + 16 * lane);
  const int r = lane & 15, w = lane >> 4;
  const int row = 16 * rt + r;
  const uint32_t words[4] = {nib.x, nib.y, nib.z, nib.w};
  for (int b = 0; b < 4; b++) {
    // the scale of (row, block 4kg+b): G = r/4, i = r%4
    const uint16_t dh = *reinterpret_cast<const uint16_t*>(t + kTileNibbleBytes + 32 * (r >> 2) + 8 * b + 2 * (r & 3));
    const float d = half_bits_to_float(dh);
    union {
      bf16x8 v;
      uint32_t u[4];
    } a;
    a.v = decode_word(tbl, words[b], lane & 31);
    float* o = out + (size_t)row * cols + 32 * (4 * kg + b) + 8 * w;
    for (int i = 0; i < 4; i++) {
      float lo = d * bf16_bits_to_f32(a.u[i] & 0xffffu);
      float hi = d * bf16_bits_to_f32(a.u[i] >> 16);
      if (bf16) {  // the conversion the bf16-contract FFN kernels use
        const uint32_t pk = pack_bf16x2(lo, hi);
        lo = bf16_bits_to_f32(pk & 0xffffu);
        hi = bf16_bits_to_f32(pk >> 16);
      }
      o[2 * i] = lo;
      o[2 * i + 1] = hi;
    }
  }
}

// ---------------------------------------------------------------- gate / up

// Both FFN kernels split the reduction dimension over the W wavefronts of a
// workgroup (W = 4 for gate/up, 8 for down): wavefront w takes packed tiles
// [w n/W, (w+1) n/W) of the n tiles of a row (n = H/128 for gate/up, F/128
// for down), so each activation (or h) element is read once per workgroup.
// A wavefront requests everything a tile column needs -- the nibble words and
// the B operands into registers, the tiles' scales for its own LDS -- before
// it computes on it; partial sums are added in wavefront order through LDS,
// so results are deterministic.
constexpr int kExWaves = 8;  // down
constexpr int kExThreads = 64 * kExWaves;
// gate/up: 4 wavefronts (Xing4: 7 tile columns each); with the reduction
// buffer holding one matrix at a time a workgroup needs 40 KB of LDS, so 4
// workgroups (16 wavefronts, 118 VGPRs each) fit on a CU.
constexpr int kGuWaves = 4;
constexpr int kGuThreads = 64 * kGuWaves;
// gate/up: a workgroup covers 2 row tiles of F (32 rows), so that each
// activation operand a wavefront loads serves 4 tiles (2 row tiles x gate/up).
// A wavefront walks its tile columns with two sets of registers: the loads of
// column j + 1 are in flight while column j is computed.  The scales travel
// through registers too and are written to the wavefront's LDS when their
// column starts (an LDS DMA would make the compiler wait for every load in
// flight before any LDS read).
constexpr int kGuRowTiles = 2;
constexpr int kDnRowTiles = 8;  // down: 16-row tiles of H per workgroup

struct GateUpExactLds {
  union {
    uint32_t scales[kGuWaves][256];        // per wavefront: 32 words of (row tile r, matrix m) at 32 (2r + m)
    f32x4 red[kGuRowTiles][kGuWaves][64];  // wavefront partials of one matrix, after the last column
  } u;
  uint32_t tbl[kPairTableWords];
};
static_assert(kGuRowTiles * 2 * 8 == 32, "32 lanes of 16 bytes cover the scales of a column");

struct DownExactLds {
  uint32_t scales[kExWaves][256];  // per wavefront: [row tile][32 words] of its current tile column
  uint32_t tbl[kPairTableWords];
  f32x4 red[kExWaves][kDnRowTiles / 2][64];  // the row tiles are reduced in two halves
};

// acc[0..3] (rows 4G..4G+3) += d * c, d from the word pair (rows 4G, 4G+1 | 4G+2, 4G+3).
__device__ __forceinline__ void scale_acc_words(f32x4& acc, const f32x4& c, uint32_t s01, uint32_t s23) {
  acc[0] = __builtin_fmaf(half_bits_to_float(s01), c[0], acc[0]);
  acc[1] = __builtin_fmaf(half_bits_to_float(s01 >> 16), c[1], acc[1]);
  acc[2] = __builtin_fmaf(half_bits_to_float(s23), c[2], acc[2]);
  acc[3] = __builtin_fmaf(half_bits_to_float(s23 >> 16), c[3], acc[3]);
}

template <int B>
using BufferIndex = std::integral_constant<int, B>;

// Workgroup = (chunk, 2 row tiles of F).  Output: the product h = silu(g)*u
// of route column c, row f, as two bf16 halves h_hi = bf16(h), h_lo = bf16(h -
// h_hi), row-major [route][F].
__global__ __launch_bounds__(kGuThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_gate_up_exact(
    const uint16_t* __restrict__ x, int H, int F, int K, int T, const uint8_t* __restrict__ arena,
    const uint8_t* __restrict__ shared, int64_t expert_bytes, const int32_t* __restrict__ perm,
    const Chunk* __restrict__ chunks, const int32_t* __restrict__ n_chunks, uint16_t* __restrict__ h_hi,
    uint16_t* __restrict__ h_lo) {
  __shared__ __attribute__((aligned(16))) GateUpExactLds sh;
  const int n_rp = F / (16 * kGuRowTiles);
  const int chunk_id = blockIdx.x / n_rp;
  const int rt0 = kGuRowTiles * (blockIdx.x % n_rp);
  if (chunk_id >= *n_chunks) return;
  const Chunk ch = chunks[chunk_id];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar buffer offsets
  const int G = lane >> 4;
  const int64_t mat_bytes = expert_bytes / 3;
  const uint8_t* ex = ch.expert >= 0 ? arena + (int64_t)ch.expert * expert_bytes : shared;
  const int cc = (lane & 15) < ch.count ? (lane & 15) : 0;  // a column past the chunk reads column 0's token
  const int tok = ch.expert >= 0 ? perm[ch.first + cc] / K : ch.first + cc;
  const int nkg = H >> 7;
  const int kg0 = wave * nkg / kGuWaves, n_cols = (wave + 1) * nkg / kGuWaves - kg0;
  const int rt_bytes = nkg * kTileBytes;
  const uint8_t* gate_t = ex + rt0 * rt_bytes;  // row tile r: + r * rt_bytes; up: mat_bytes further

  // The weight rows and the activations through buffer resources (byte
  // offsets fit in 32 bits: an expert matrix is < 2 GB, T * H * 2 <= 1 GB).
  const __amdgpu_buffer_rsrc_t w_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(gate_t), (short)0, 0x7fffffff, 0x00020000);
  const __amdgpu_buffer_rsrc_t x_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), (short)0, 0x7fffffff, 0x00020000);
  const int x_off = 2 * (tok * H + 8 * G);  // + 256 kg + 64 b: elements 32 (4 kg + b) + 8 G .. + 7

  u32x4 nib[2][kGuRowTiles][2];
  bf16x8 xb[2][4];
  u32x4 scw[2];
  // this lane's 16-byte scale piece: piece lane % 8 of row tile (lane / 16) %
  // 2, matrix (lane / 8) % 2 (lanes 32-63 repeat lanes 0-31; their copy lands
  // in the second half of the LDS buffer and is never read)
  const int sc_off = ((lane >> 4) & 1) * rt_bytes + ((lane >> 3) & 1) * (int)mat_bytes + kTileNibbleBytes + 16 * (lane & 7);
  // The loads of tile column kg into register set B.  A column past this
  // wavefront's range (valid false) gets a byte offset past the buffer's
  // range: such a load returns zeros and makes no memory request, so the
  // loop below can issue unconditionally and keep no old values alive.
  auto issue = [&](auto bc, int kg, bool valid) {
    constexpr int B = decltype(bc)::value;
    const int oob = valid ? 0 : INT32_MIN;  // 0x80000000 >= the range 0x7fffffff
    const int voff = (kg * kTileBytes + 16 * lane) | oob;
    scw[B] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, sc_off | oob, kg * kTileBytes, kNonTemporal));
#pragma unroll
    for (int r = 0; r < kGuRowTiles; r++)
#pragma unroll
      for (int m = 0; m < 2; m++)
        nib[B][r][m] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, voff, (int)(r * rt_bytes + m * mat_bytes), kNonTemporal));
    const int xo = (x_off + 256 * kg) | oob;
#pragma unroll
    for (int b = 0; b < 4; b++)
      xb[B][b] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, xo + 64 * b, 0, 0));
  };
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[kGuRowTiles][2];
#pragma unroll
  for (int r = 0; r < kGuRowTiles; r++) acc[r][0] = acc[r][1] = zero;
  uint32_t* sc = sh.u.scales[wave];
  // one column from register set B; a wavefront's LDS operations run in
  // order, so the scale words are written after the previous column's reads
  // and read after this write
  auto compute = [&](auto bc) {
    constexpr int B = decltype(bc)::value;
    *reinterpret_cast<u32x4*>(sc + 4 * lane) = scw[B];
#pragma unroll
    for (int b = 0; b < 4; b++)
#pragma unroll
      for (int r = 0; r < kGuRowTiles; r++)
#pragma unroll
        for (int m = 0; m < 2; m++) {
          const f32x4 cr = mfma16x16x32(decode_word(sh.tbl, nib[B][r][m][b], lane & 31), xb[B][b], zero);
          const uint32_t* sp = sc + 32 * (r * 2 + m) + 8 * G + 2 * b;
          scale_acc_words(acc[r][m], cr, sp[0], sp[1]);
        }
  };
  const BufferIndex<0> b0;
  const BufferIndex<1> b1;
  issue(b0, kg0, n_cols > 0);
  issue(b1, kg0 + 1, n_cols > 1);
  build_pair_table(sh.tbl);
  __syncthreads();
  // columns j (set 0) and j + 1 (set 1) are in flight at the top of a pass;
  // each set is refilled with the column two ahead once computed
  for (int j = 0; j < n_cols; j += 2) {
    compute(b0);
    issue(b0, kg0 + j + 2, j + 2 < n_cols);
    if (j + 1 < n_cols) compute(b1);
    issue(b1, kg0 + j + 3, j + 3 < n_cols);
  }
  __syncthreads();  // the scale buffers become the reduction buffer
#pragma unroll
  for (int r = 0; r < kGuRowTiles; r++) sh.u.red[r][wave][lane] = acc[r][0];
  __syncthreads();
  // wavefront r finishes row tile r (gate sums, then up sums through the same
  // buffer); the lane's column and row group are recomputed (mbcnt) instead of
  // kept live through the loop
  const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int c_e = lane_e & 15, G_e = lane_e >> 4;
  f32x4 g = zero;
  if (wave < kGuRowTiles) {
    g = sh.u.red[wave][0][lane_e];
#pragma unroll
    for (int w = 1; w < kGuWaves; w++) g += sh.u.red[wave][w][lane_e];
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kGuRowTiles; r++) sh.u.red[r][wave][lane] = acc[r][1];
  __syncthreads();
  if (wave >= kGuRowTiles || c_e >= ch.count) return;
  f32x4 u = sh.u.red[wave][0][lane_e];
#pragma unroll
  for (int w = 1; w < kGuWaves; w++) u += sh.u.red[wave][w][lane_e];
  // bucketed position of the route, or T*K + token for the shared expert
  const int64_t hrow = (ch.expert >= 0 ? 0 : (int64_t)T * K) + ch.first + c_e;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int f = 16 * (rt0 + wave) + 4 * G_e + i;
    const float gv = g[i];
    const float h = gv / (1.0f + expf(-gv)) * u[i];
    const uint32_t hb = f32_to_bf16_rne(h);
    const uint32_t lb = f32_to_bf16_rne(h - bf16_bits_to_f32(hb));
    h_hi[hrow * F + f] = (uint16_t)hb;
    h_lo[hrow * F + f] = (uint16_t)lb;
  }
}

// ---------------------------------------------------------------- down

// Workgroup = (chunk, kDnRowTiles row tiles of H).  y[hrow][n] = sum_f
// W_down[n][f] h[f] in fp32, one row per route (bucketed position) or per
// shared-expert token.  Wavefront w takes tile columns [w n/8, (w+1) n/8) of
// F for all the workgroup's row tiles, one tile column at a time, so its h
// operands serve each of them.
__global__ __launch_bounds__(kExThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_down_exact(
    int H, int F, int K, int T, const uint8_t* __restrict__ arena, const uint8_t* __restrict__ shared,
    int64_t expert_bytes, const Chunk* __restrict__ chunks, const int32_t* __restrict__ n_chunks,
    const uint16_t* __restrict__ h_hi, const uint16_t* __restrict__ h_lo, float* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) DownExactLds sh;
  const int n_slab = H / (16 * kDnRowTiles);
  const int chunk_id = blockIdx.x / n_slab;
  const int slab = blockIdx.x % n_slab;
  if (chunk_id >= *n_chunks) return;
  const Chunk ch = chunks[chunk_id];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, G = lane >> 4;
  const int64_t mat_bytes = expert_bytes / 3;
  const uint8_t* ex = ch.expert >= 0 ? arena + (int64_t)ch.expert * expert_bytes : shared;
  const int TK = T * K;
  const bool live = c < ch.count;
  const int cc = live ? c : 0;  // a column past the chunk reads column 0's h (never stored)
  const int64_t hrow = ch.expert >= 0 ? (int64_t)(ch.first + cc) : (int64_t)TK + ch.first + cc;
  const uint16_t* hh = h_hi + hrow * F;
  const uint16_t* hl = h_lo + hrow * F;
  const int nkg = F >> 7;
  const int kg0 = wave * nkg / kExWaves, kg1 = (wave + 1) * nkg / kExWaves;
  const int64_t rt_bytes = (int64_t)nkg * kTileBytes;
  const uint8_t* rows = ex + 2 * mat_bytes + (int64_t)slab * kDnRowTiles * rt_bytes;
  uint32_t* my_scales = sh.scales[wave];

  u32x4 nib[kDnRowTiles];
  bf16x8 bh[4], bl[4];
  // the row tiles' nibble words through one buffer resource: row tile t at
  // scalar offset t * rt_bytes, so one lane offset serves all of them
  const __amdgpu_buffer_rsrc_t rows_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(rows), (short)0, 0x7fffffff, 0x00020000);
  auto issue = [&](int kg) {
    dma16_stream(rows + min(lane >> 3, kDnRowTiles - 1) * rt_bytes + (int64_t)kg * kTileBytes + kTileNibbleBytes +
                     16 * (lane & 7),
                 my_scales);
    const int voff = kg * kTileBytes + 16 * lane;
#pragma unroll
    for (int t = 0; t < kDnRowTiles; t++)
      nib[t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rows_rsrc, voff, (int)(t * rt_bytes), kNonTemporal));
#pragma unroll
    for (int b = 0; b < 4; b++) {
      bh[b] = *reinterpret_cast<const bf16x8*>(hh + 32 * (4 * kg + b) + 8 * G);
      bl[b] = *reinterpret_cast<const bf16x8*>(hl + 32 * (4 * kg + b) + 8 * G);
    }
  };
  issue(min(kg0, nkg - 1));
  build_pair_table(sh.tbl);
  wait_loads();  // as in k_gate_up_exact: a full wait before the scales are read
  __syncthreads();
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[kDnRowTiles];
#pragma unroll
  for (int t = 0; t < kDnRowTiles; t++) acc[t] = zero;
  for (int kg = kg0; kg < kg1; kg++) {
    if (kg != kg0) {  // only when F > 1024: this wavefront's own scales, no barrier needed
      issue(kg);
      wait_loads();
    }
#pragma unroll
    for (int b = 0; b < 4; b++)
#pragma unroll
      for (int t = 0; t < kDnRowTiles; t++) {
        const bf16x8 a = decode_word(sh.tbl, nib[t][b], lane & 31);
        f32x4 cr = mfma16x16x32(a, bh[b], zero);
        cr = mfma16x16x32(a, bl[b], cr);
        const uint32_t* sd = my_scales + 32 * t + 8 * G + 2 * b;
        scale_acc_words(acc[t], cr, sd[0], sd[1]);
      }
  }
  // wavefront-order sums, half of the row tiles at a time; wavefront t stores
  // row tile t.  The lane's column, row group and output row are recomputed
  // (mbcnt) instead of kept live through the loop, which needs every register.
  const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int c_e = lane_e & 15, G_e = lane_e >> 4;
  const int64_t hrow_e = (ch.expert >= 0 ? 0 : (int64_t)TK) + ch.first + c_e;
#pragma unroll
  for (int half = 0; half < 2; half++) {
#pragma unroll
    for (int t = 0; t < kDnRowTiles / 2; t++) sh.red[wave][t][lane_e] = acc[(kDnRowTiles / 2) * half + t];
    __syncthreads();
    if (wave < kDnRowTiles / 2 && c_e < ch.count) {
      f32x4 s = sh.red[0][wave][lane_e];
#pragma unroll
      for (int w = 1; w < kExWaves; w++) s += sh.red[w][wave][lane_e];
      const int rt = slab * kDnRowTiles + (kDnRowTiles / 2) * half + wave;
      *reinterpret_cast<f32x4*>(y + hrow_e * H + 16 * rt + 4 * G_e) = s;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- combine

// out[t][n] = sum_k w[t][k] * y[pos[t*K+k]][n]  (slot order)  + g_t * y[TK + t][n],
// w rows of K + gated values, g_t = w[t][K] for a gated shared expert, else 1.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y, const int32_t* __restrict__ pos,
                                                 const float* __restrict__ w, int T, int K, int H, int n_shared,
                                                 int gated, float* __restrict__ out) {
  const int t = blockIdx.y;
  const int n = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
  if (n >= H) return;
  const int TK = T * K;
  const int WK = K + gated;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < K; k++) {
    const float wk = w[(size_t)t * WK + k];
    const float4 v = *reinterpret_cast<const float4*>(y + (size_t)pos[(size_t)t * K + k] * H + n);
    acc.x = __builtin_fmaf(wk, v.x, acc.x);
    acc.y = __builtin_fmaf(wk, v.y, acc.y);
    acc.z = __builtin_fmaf(wk, v.z, acc.z);
    acc.w = __builtin_fmaf(wk, v.w, acc.w);
  }
  if (n_shared) {
    const float4 v = *reinterpret_cast<const float4*>(y + ((size_t)TK + t) * H + n);
    if (gated) {
      const float g = w[(size_t)t * WK + K];
      acc.x = __builtin_fmaf(g, v.x, acc.x);
      acc.y = __builtin_fmaf(g, v.y, acc.y);
      acc.z = __builtin_fmaf(g, v.z, acc.z);
      acc.w = __builtin_fmaf(g, v.w, acc.w);
    } else {
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
  }
  *reinterpret_cast<float4*>(out + (size_t)t * H + n) = acc;
}

// ---------------------------------------------------------------- launchers

hipError_t launch_pack(const uint8_t* src, uint8_t* dst, int n_experts, int H, int F, hipStream_t stream) {
  const int64_t mat_bytes = (int64_t)F * (H / 32) * 18;
  // gate and up: F rows x H/32 blocks; down: H rows x F/32 blocks.  The two
  // shapes differ, so launch per matrix kind with a matrix stride of 3.
  for (int m = 0; m < 3; m++) {
    const int rows = m < 2 ? F : H;
    const int nb = m < 2 ? H / 32 : F / 32;
    const int64_t tiles = (int64_t)(rows / 16) * (nb / 4);
    for (int e = 0; e < n_experts; e++) {
      const int64_t off = (int64_t)e * 3 * mat_bytes + m * mat_bytes;
      const int64_t threads = tiles * 64;
      clear_last_error();
      hipLaunchKernelGGL(k_pack, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, src + off, dst + off,
                         tiles, rows, nb, mat_bytes);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
  }
  return hipSuccess;
}

hipError_t launch_dequant(const uint8_t* mat, int rows, int cols, int bf16, float* out, hipStream_t stream) {
  const int64_t tiles = (int64_t)(rows / 16) * (cols / 128);
  clear_last_error();
  hipLaunchKernelGGL(k_dequant, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0, stream, mat, rows, cols, bf16, out);
  return hipGetLastError();
}

hipError_t launch_ffn_exact(const uint16_t* x, int T, int H, int F, int K, int n_shared, int gated, int max_chunks,
                            const uint8_t* arena, const uint8_t* shared, int64_t expert_bytes, const int32_t* perm,
                            const int32_t* pos, const float* w, const Chunk* chunks, const int32_t* n_chunks,
                            uint16_t* h_hi, uint16_t* h_lo, float* y, float* out, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  clear_last_error();
  hipLaunchKernelGGL(k_gate_up_exact, dim3((unsigned)(max_chunks * (F / (16 * kGuRowTiles)))), dim3(kGuThreads), 0,
                     stream, x, H, F, K, T, arena, shared, expert_bytes, perm, chunks, n_chunks, h_hi, h_lo);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  clear_last_error();
  hipLaunchKernelGGL(k_down_exact, dim3((unsigned)(max_chunks * (H / (16 * kDnRowTiles)))), dim3(kExThreads), 0, stream,
                     H, F, K, T, arena, shared, expert_bytes, chunks, n_chunks, h_hi, h_lo, y);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_combine(y, pos, w, T, K, H, n_shared, gated, out, stream);
}

hipError_t launch_combine(const float* y, const int32_t* pos, const float* w, int T, int K, int H, int n_shared,
                          int gated, float* out, hipStream_t stream) {
  clear_last_error();
  hipLaunchKernelGGL(k_combine, dim3((unsigned)((H / 4 + 255) / 256), (unsigned)T), dim3(256), 0, stream, y, pos, w, T,
                     K, H, n_shared, gated, out);
  return hipGetLastError();
}

}  // namespace qmoe
