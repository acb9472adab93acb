// Expert FFN with bf16 weights on MFMA: the batched / prefill path.
//
// Arithmetic (bf16 contract): every weight is the IQ4_NL value d*level
// (model card xing4_0-29b-IQ4_NL_EPQ, pure-NumPy parity section) rounded to
// bf16, nearest even; products run on v_mfma_f32_16x16x32_bf16 with fp32
// accumulation; h = silu(g)*u (zLLM "Algorithm Layer", FFN section) is
// rounded to bf16 before the down projection; y and the routed + shared sum
// stay fp32 (PocketLLM design record, section 2).
//
// Work: tiles of up to 128 routes of one expert (bucketed order, design
// record section 4) or 128 tokens of the shared expert, largest first.  A
// workgroup of 16 wavefronts owns one tile and one slab of output columns;
// wavefront w owns 16 gate columns and the same 16 up columns (gate/up, 256 +
// 256 per workgroup) or 32 output columns (down, 512 per workgroup), over all
// rows of the tile.  Per 128-wide step of the reduction:
//   - the tile's activation rows (the A operand, the same for every
//     wavefront) go from global memory straight into LDS (LDS DMA loads,
//     double buffered, one step ahead): gathered rows of x for gate/up,
//     consecutive rows of h for down;
//   - each wavefront loads its packed weight tiles (one 16-byte word per lane
//     per 16 columns) and dequantizes every word straight into its lane's
//     bf16 B operand (levels from the LDS pair table, times the fp16 scale,
//     rounded to bf16).  Each weight feeds exactly one wavefront, so the
//     dequantized tile needs no trip through LDS; it is dequantized once per
//     workgroup and reused by every 16-row sub-tile of the tile;
//   - 16-row sub-tiles past the tile's last row are skipped: the k-loop is
//     instantiated for each count of active sub-tiles (1 .. 8) and the tile
//     picks its instance once, so that the loop body has no per-sub-tile
//     branch and its LDS reads and MFMAs can be scheduled together.
#include "device.h"
#include "launch.h"

namespace qmoe {

constexpr int kBfThreads = 1024;
constexpr int kBfWaves = kBfThreads / 64;
constexpr int kBfSub = kBfRows / 16;        // 16-row MFMA sub-tiles per tile
constexpr int kBfStep = 128;                // reduction elements per step (one packed tile)
constexpr int kGuCols = 16;                 // gate (and up) columns per wavefront
constexpr int kDnCols = 32;                 // down output columns per wavefront
constexpr int kGuTiles = kGuCols / 16;      // gate tiles per wavefront (as many up tiles)
constexpr int kDnTiles = kDnCols / 16;      // down tiles per wavefront
constexpr int kStageLoads = kBfRows / 4 / kBfWaves;  // 1 KB LDS DMA loads per wavefront and step

// LDS: two buffers of activation rows, then the level pair table.  A buffer
// row is 256 bytes (one step); its 16-byte slots are permuted by the row
// index (slot = piece ^ (row % 16)), so that the 16 rows read by one A
// operand fetch fall into distinct banks.  The buffers come first: the LDS
// address of an LDS DMA load is taken from the low 16 bits of M0, so its
// destinations must lie in the first 64 KB of the workgroup's LDS.
//
// The table starts at 64 KB: 256 entries (one per byte of nibbles: the fp16
// levels of its low and high nibble) x 64 replicas, entry e of lane l at byte
// 65536 + 256 e + 4 l.  That address is one v_perm_b32 of the nibble word
// and a per-lane constant, and the 64 lanes of a lookup hit 64 banks.
constexpr int kTblReplicas = 64;
constexpr int kTblWords = 256 * kTblReplicas;
struct BfLds {
  uint16_t a[2][kBfRows * kBfStep];
  __attribute__((aligned(16))) uint32_t tbl[kTblWords];
  int32_t src[kBfRows];  // source row of each tile row (x row or h row)
};
static_assert(sizeof(uint16_t) * 2 * kBfRows * kBfStep == 65536, "the table starts at 64 KB");
static_assert(offsetof(BfLds, tbl) == 65536, "the table starts at 64 KB");

// The fp16 level pairs (exact), kTblReplicas copies of each entry.
__device__ __forceinline__ void build_pair_table_f16_64(uint32_t* tbl) {
  for (int i = threadIdx.x; i < kTblWords / 4; i += blockDim.x) {
    const int v = i / (kTblReplicas / 4);
    const uint32_t e = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)iq4nl_level(v & 15)) |
                       ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)iq4nl_level(v >> 4)) << 16);
    uint32_t __attribute__((ext_vector_type(4))) q = {e, e, e, e};
    *reinterpret_cast<decltype(q)*>(tbl + 4 * i) = q;
  }
}
static_assert(kBfSub == 8, "the k-loop is instantiated for 1 .. 8 sub-tiles");

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// One nibble word -> the lane's 8-element bf16 operand, each weight
// bf16(d * level): the fp16 level pair from the LDS table times the fp16
// scale in fp32 (v_fma_mix_f32 with addend +0: the product is exact; a zero
// product comes out +0 whatever its sign, which no sum can tell apart), both
// rounded to nearest even by one v_cvt_pk_bf16_f32.
// lane_sel = 4 * lane | 1 << 16: the address of byte i of word is
// perm(word, lane_sel) with bytes (lane_sel.b0, word.b_i, lane_sel.b2, 0).
__device__ __forceinline__ bf16x8 dequant_bf16(const BfLds& sh, uint32_t word, _Float16 d, uint32_t lane_sel) {
  const char* lds0 = reinterpret_cast<const char*>(sh.tbl) - 65536;
  union {
    uint32_t u[4];
    bf16x8 v;
  } r;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint32_t addr = __builtin_amdgcn_perm(word, lane_sel, 0x0c020400u + 0x100u * i);
    const uint32_t e = *reinterpret_cast<const uint32_t*>(lds0 + addr);
    const _Float16 l0 = __builtin_bit_cast(_Float16, (uint16_t)(e & 0xffffu));
    const _Float16 l1 = __builtin_bit_cast(_Float16, (uint16_t)(e >> 16));
    const f32x2 w = {__builtin_fmaf((float)l0, (float)d, 0.0f), __builtin_fmaf((float)l1, (float)d, 0.0f)};
    r.u[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(w, bf16x2v));
  }
  return r.v;
}

// The packed tile of 16 columns that a lane reads: its nibble word and the
// fp16 scales of its column (lane % 16) for the tile's 4 blocks, two per
// register (each loaded into its half).  Ordinary (temporal) loads: every
// tile of 128 routes of an expert reads the expert's weights, and a popular
// expert (or the shared one) has many tiles, which then hit in L2.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
struct LaneTile {
  u32x4 nib;
  f16x2 sc[2];  // blocks 0, 1 | 2, 3
};

__device__ __forceinline__ LaneTile load_lane_tile(const uint8_t* tile, int lane) {
  LaneTile t;
  t.nib = *reinterpret_cast<const u32x4*>(tile + 16 * lane);
  const int n = lane & 15;
  const _Float16* sp = reinterpret_cast<const _Float16*>(tile + kTileNibbleBytes + 32 * (n >> 2) + 2 * (n & 3));
#pragma unroll
  for (int h = 0; h < 2; h++) {
    t.sc[h].x = *(sp + 8 * h);
    t.sc[h].y = *(sp + 8 * h + 4);
  }
  return t;
}

__device__ __forceinline__ _Float16 lane_scale(const LaneTile& t, int b) {
  return (b & 1) ? t.sc[b >> 1].y : t.sc[b >> 1].x;
}

// Activation rows of one step, global memory straight into LDS
// (global_load_lds_dwordx4): load j of wavefront w fills rows 4q..4q+3,
// q = j*8 + w, lane i writing slot i%16 of row 4q + i/16.  Loads of rows at
// or past n_rows (16 x active sub-tiles) are not issued.
__device__ __forceinline__ void stage_rows(uint16_t* a, const uint16_t* base, int64_t ld, const int32_t* src, int k0,
                                           int n_rows, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < kStageLoads; j++) {
    const int q = j * kBfWaves + wave;
    if (4 * q < n_rows) {
      const int row = 4 * q + (lane >> 4);
      const int piece = (lane & 15) ^ (row & 15);
      const uint16_t* g = base + (int64_t)src[row] * ld + k0 + 8 * piece;
      __builtin_amdgcn_global_load_lds(g, a + 4 * kBfStep * q, 16, 0, 0);
    }
  }
}

// A operand of sub-tile s, block b: row 16s + lane%16, elements 32b + 8*(lane/16) .. +7.
__device__ __forceinline__ bf16x8 a_operand(const uint16_t* a, int s, int b, int lane) {
  const int r = lane & 15;
  return *reinterpret_cast<const bf16x8*>(a + (16 * s + r) * kBfStep + 8 * ((4 * b + (lane >> 4)) ^ r));
}

// acc[s][c] += A(s) x B(c) over one step for the NS active sub-tiles and the
// NC column tiles in wt.
template <int NS, int NC>
__device__ __forceinline__ void step_mfma(const BfLds& sh, const uint16_t* a, const LaneTile (&wt)[NC], int lane,
                                          f32x4 (&acc)[NS][NC]) {
#pragma unroll
  for (int b = 0; b < 4; b++) {
    bf16x8 bop[NC];
#pragma unroll
    for (int c = 0; c < NC; c++) bop[c] = dequant_bf16(sh, wt[c].nib[b], lane_scale(wt[c], b), (lane << 2) | 0x10000u);
#pragma unroll
    for (int s = 0; s < NS; s++) {
      const bf16x8 aop = a_operand(a, s, b, lane);
#pragma unroll
      for (int c = 0; c < NC; c++) acc[s][c] = mfma16x16x32(aop, bop[c], acc[s][c]);
    }
  }
}

// ---------------------------------------------------------------- gate / up

// Workgroup = (tile, slab of 256 gate columns).  h[hrow][f] = bf16(silu(g) * u)
// for hrow = bucketed position (routed) or T*K + token (shared).
template <int NS>
__device__ void gate_up_tile(BfLds& sh, const Chunk& ch, const uint16_t* __restrict__ x, int H, int F, int K, int T,
                             const uint8_t* ex, int64_t mat_bytes, int col0, bool routed, int lane, int wave,
                             uint16_t* __restrict__ h) {
  const int n_rows = 16 * NS;
  const bool cols_on = col0 < F;
  const int nkg = H / kBfStep;
  const int rt0 = (cols_on ? col0 : 0) >> 4;
  // column tiles: c < kGuTiles = gate rows rt0 + c; kGuTiles + c = up rows rt0 + c
  constexpr int NC = 2 * kGuTiles;
  const uint8_t* wbase[NC];
#pragma unroll
  for (int c = 0; c < kGuTiles; c++) {
    wbase[c] = ex + (int64_t)(rt0 + c) * nkg * kTileBytes;
    wbase[kGuTiles + c] = ex + mat_bytes + (int64_t)(rt0 + c) * nkg * kTileBytes;
  }

  f32x4 acc[NS][NC];
#pragma unroll
  for (int s = 0; s < NS; s++)
#pragma unroll
    for (int c = 0; c < NC; c++) acc[s][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  stage_rows(sh.a[0], x, H, sh.src, 0, n_rows, wave, lane);
  LaneTile wt[NC];
#pragma unroll
  for (int c = 0; c < NC; c++) wt[c] = load_lane_tile(wbase[c], lane);
  wait_loads();
  __syncthreads();

  for (int kt = 0; kt < nkg; kt++) {
    const bool more = kt + 1 < nkg;
    LaneTile wn[NC];
    if (more) {
      stage_rows(sh.a[(kt + 1) & 1], x, H, sh.src, (kt + 1) * kBfStep, n_rows, wave, lane);
#pragma unroll
      for (int c = 0; c < NC; c++) wn[c] = load_lane_tile(wbase[c] + (int64_t)(kt + 1) * kTileBytes, lane);
    }
    if (cols_on) step_mfma<NS, NC>(sh, sh.a[kt & 1], wt, lane, acc);
    if (more) {
#pragma unroll
      for (int c = 0; c < NC; c++) wt[c] = wn[c];
    }
    wait_loads();
    __syncthreads();
  }

  if (!cols_on) return;
  const int TK = T * K;
#pragma unroll
  for (int s = 0; s < NS; s++) {
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const int m = 16 * s + 4 * (lane >> 4) + v;
      if (m < ch.count) {
        const int64_t hrow = routed ? (int64_t)ch.first + m : (int64_t)TK + ch.first + m;
#pragma unroll
        for (int c = 0; c < kGuTiles; c++) {
          const float g = acc[s][c][v], u = acc[s][c + kGuTiles][v];
          const float hv = g / (1.0f + expf(-g)) * u;
          h[hrow * F + col0 + 16 * c + (lane & 15)] = __builtin_bit_cast(uint16_t, (__bf16)hv);
        }
      }
    }
  }
}

__global__ __launch_bounds__(kBfThreads) void k_gate_up_bf16(
    const uint16_t* __restrict__ x, int H, int F, int K, int T, const uint8_t* __restrict__ arena,
    const uint8_t* __restrict__ shared, int64_t expert_bytes, const int32_t* __restrict__ perm,
    const Chunk* __restrict__ tiles, const int32_t* __restrict__ n_tiles, int max_tiles, uint16_t* __restrict__ h) {
  __shared__ BfLds sh;
  const int tile_id = blockIdx.x % max_tiles;
  const int slab = blockIdx.x / max_tiles;
  if (tile_id >= *n_tiles) return;
  const Chunk ch = tiles[tile_id];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool routed = ch.expert >= 0;
  if (threadIdx.x < kBfRows) {
    const int i = min((int)threadIdx.x, ch.count - 1);
    sh.src[threadIdx.x] = routed ? perm[ch.first + i] / K : ch.first + i;
  }
  build_pair_table_f16_64(sh.tbl);
  __syncthreads();
  const int col0 = slab * (kBfWaves * kGuCols) + wave * kGuCols;
  const int64_t mat_bytes = expert_bytes / 3;
  const uint8_t* ex = routed ? arena + (int64_t)ch.expert * expert_bytes : shared;
  switch ((ch.count + 15) >> 4) {
#define QMOE_GU_CASE(n) \
  case n: gate_up_tile<n>(sh, ch, x, H, F, K, T, ex, mat_bytes, col0, routed, lane, wave, h); break;
    QMOE_GU_CASE(1) QMOE_GU_CASE(2) QMOE_GU_CASE(3) QMOE_GU_CASE(4)
    QMOE_GU_CASE(5) QMOE_GU_CASE(6) QMOE_GU_CASE(7) QMOE_GU_CASE(8)
#undef QMOE_GU_CASE
    default: break;
  }
}

// ---------------------------------------------------------------- down

// Workgroup = (tile, slab of 512 output columns).  y[hrow][n] = sum_f Wd[n][f] h[hrow][f].
template <int NS>
__device__ void down_tile(BfLds& sh, const Chunk& ch, int H, int F, const uint8_t* ex, int64_t row0, int col0,
                          int lane, int wave, const uint16_t* __restrict__ h, float* __restrict__ y) {
  const int n_rows = 16 * NS;
  const bool cols_on = col0 < H;
  const int nkg = F / kBfStep;
  const int rt0 = (cols_on ? col0 : 0) >> 4;
  constexpr int NC = kDnTiles;
  const uint8_t* wbase[NC];
#pragma unroll
  for (int c = 0; c < NC; c++) wbase[c] = ex + (int64_t)(rt0 + c) * nkg * kTileBytes;

  f32x4 acc[NS][NC];
#pragma unroll
  for (int s = 0; s < NS; s++)
#pragma unroll
    for (int c = 0; c < NC; c++) acc[s][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  stage_rows(sh.a[0], h, F, sh.src, 0, n_rows, wave, lane);
  LaneTile wt[NC];
#pragma unroll
  for (int c = 0; c < NC; c++) wt[c] = load_lane_tile(wbase[c], lane);
  wait_loads();
  __syncthreads();

  for (int kt = 0; kt < nkg; kt++) {
    const bool more = kt + 1 < nkg;
    LaneTile wn[NC];
    if (more) {
      stage_rows(sh.a[(kt + 1) & 1], h, F, sh.src, (kt + 1) * kBfStep, n_rows, wave, lane);
#pragma unroll
      for (int c = 0; c < NC; c++) wn[c] = load_lane_tile(wbase[c] + (int64_t)(kt + 1) * kTileBytes, lane);
    }
    if (cols_on) step_mfma<NS, NC>(sh, sh.a[kt & 1], wt, lane, acc);
    if (more) {
#pragma unroll
      for (int c = 0; c < NC; c++) wt[c] = wn[c];
    }
    wait_loads();
    __syncthreads();
  }

  if (!cols_on) return;
#pragma unroll
  for (int s = 0; s < NS; s++) {
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const int m = 16 * s + 4 * (lane >> 4) + v;
      if (m < ch.count) {
        float* yr = y + (row0 + m) * H + col0 + (lane & 15);
#pragma unroll
        for (int c = 0; c < NC; c++) yr[16 * c] = acc[s][c][v];
      }
    }
  }
}

__global__ __launch_bounds__(kBfThreads) void k_down_bf16(
    int H, int F, int K, int T, const uint8_t* __restrict__ arena, const uint8_t* __restrict__ shared,
    int64_t expert_bytes, const Chunk* __restrict__ tiles, const int32_t* __restrict__ n_tiles, int max_tiles,
    const uint16_t* __restrict__ h, float* __restrict__ y) {
  __shared__ BfLds sh;
  const int tile_id = blockIdx.x % max_tiles;
  const int slab = blockIdx.x / max_tiles;
  if (tile_id >= *n_tiles) return;
  const Chunk ch = tiles[tile_id];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool routed = ch.expert >= 0;
  const int TK = T * K;
  const int64_t row0 = routed ? (int64_t)ch.first : (int64_t)TK + ch.first;
  if (threadIdx.x < kBfRows) sh.src[threadIdx.x] = (int32_t)(row0 + min((int)threadIdx.x, ch.count - 1));
  build_pair_table_f16_64(sh.tbl);
  __syncthreads();
  const int col0 = slab * (kBfWaves * kDnCols) + wave * kDnCols;
  const int64_t mat_bytes = expert_bytes / 3;
  const uint8_t* ex = (routed ? arena + (int64_t)ch.expert * expert_bytes : shared) + 2 * mat_bytes;
  switch ((ch.count + 15) >> 4) {
#define QMOE_DN_CASE(n) \
  case n: down_tile<n>(sh, ch, H, F, ex, row0, col0, lane, wave, h, y); break;
    QMOE_DN_CASE(1) QMOE_DN_CASE(2) QMOE_DN_CASE(3) QMOE_DN_CASE(4)
    QMOE_DN_CASE(5) QMOE_DN_CASE(6) QMOE_DN_CASE(7) QMOE_DN_CASE(8)
#undef QMOE_DN_CASE
    default: break;
  }
}

// ---------------------------------------------------------------- launcher

hipError_t launch_ffn_bf16(const uint16_t* x, int T, int H, int F, int K, int n_shared, int gated, int max_tiles,
                           const uint8_t* arena, const uint8_t* shared, int64_t expert_bytes, const int32_t* perm,
                           const int32_t* pos, const float* w, const Chunk* tiles, const int32_t* n_tiles,
                           uint16_t* h, float* y, float* out, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int gu_slabs = (F + kBfWaves * kGuCols - 1) / (kBfWaves * kGuCols);
  const int dn_slabs = (H + kBfWaves * kDnCols - 1) / (kBfWaves * kDnCols);
  clear_last_error();
  hipLaunchKernelGGL(k_gate_up_bf16, dim3((unsigned)(max_tiles * gu_slabs)), dim3(kBfThreads), 0, stream, x, H, F, K,
                     T, arena, shared, expert_bytes, perm, tiles, n_tiles, max_tiles, h);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  clear_last_error();
  hipLaunchKernelGGL(k_down_bf16, dim3((unsigned)(max_tiles * dn_slabs)), dim3(kBfThreads), 0, stream, H, F, K, T,
                     arena, shared, expert_bytes, tiles, n_tiles, max_tiles, h, y);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_combine(y, pos, w, T, K, H, n_shared, gated, out, stream);
}

}  // namespace qmoe
