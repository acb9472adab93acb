// Device-side building blocks shared by the libmoe kernels (gfx950 / CDNA4).
//
// IQ4_NL decode (model card xing4_0-29b-IQ4_NL_EPQ, pure-NumPy parity section:
// a 16-entry non-linear lookup times one fp16 scale per 32-weight block).
// Every level is an integer of at most 7 significant bits, so it is exact in
// bf16; the kernels feed the levels to bf16 MFMA and apply the fp16 scale to
// the fp32 block result (exact-weight contract), or round d*level to bf16
// (bf16 contract).
//
// In the packed arena (moe_pack_experts) the 4-bit indices of a block are
// regrouped so that nibble word w (4 bytes) holds weights 8w..8w+7, byte i
// holding weight 8w+2i in its low nibble and 8w+2i+1 in its high nibble.
// Bytes are decoded two weights at a time through a 256-entry table in LDS:
// entry v = bf16(level[v & 15]) | bf16(level[v >> 4]) << 16, i.e. one dword
// of an MFMA operand with its two k slots in natural order.  The table is
// replicated 32 times so that lane l always reads bank l % 32: lookups never
// conflict.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // a native 16-byte vector (not a struct)

// Cache policy bit of a non-temporal access (gfx950): weights are streamed
// once per call, so their loads should not displace reused data in the caches
// (a plain read stream of this GPU runs at about 5.6 TB/s, a non-temporal one
// at about 6.5 TB/s).
constexpr int kNonTemporal = 2;

// 16-byte load of streamed weight data into a native vector (non-temporal)
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

constexpr int kTileBytes = 1152;       // 16 rows x 4 blocks of 18 bytes
constexpr int kTileNibbleBytes = 1024; // 64 lane slots x 16 bytes
constexpr int kPairTableWords = 256 * 32;

// The IQ4_NL levels (ggml definition of the format).
constexpr int kIq4nlLevels[16] = {-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113};

// Levels 4w..4w+3 as signed bytes of one word.
constexpr uint32_t iq4nl_level_word(int w) {
  return (uint32_t)(uint8_t)kIq4nlLevels[4 * w] | ((uint32_t)(uint8_t)kIq4nlLevels[4 * w + 1] << 8) |
         ((uint32_t)(uint8_t)kIq4nlLevels[4 * w + 2] << 16) | ((uint32_t)(uint8_t)kIq4nlLevels[4 * w + 3] << 24);
}

// Level of index q, selected from immediate words: no memory access (a table
// in memory would make every table build wait behind the weight loads that
// are already in flight).
__device__ __forceinline__ int iq4nl_level(int q) {
  const uint32_t lo = (q & 4) ? iq4nl_level_word(1) : iq4nl_level_word(0);
  const uint32_t hi = (q & 4) ? iq4nl_level_word(3) : iq4nl_level_word(2);
  const uint32_t w = (q & 8) ? hi : lo;
  return (int)(int8_t)(uint8_t)(w >> (8 * (q & 3)));
}

// bf16 bits of a small integer (exact: at most 8 significant bits).
__device__ __forceinline__ uint32_t small_int_bf16(int v) { return __float_as_uint((float)v) >> 16; }

// Fill the replicated pair table; every thread of the block takes part.  Each
// step computes one entry and writes 4 of its 32 copies with one 16-byte
// store.
__device__ __forceinline__ void build_pair_table(uint32_t* tbl) {
  for (int i = threadIdx.x; i < kPairTableWords / 4; i += blockDim.x) {
    const int v = i >> 3;
    const uint32_t e = small_int_bf16(iq4nl_level(v & 15)) | (small_int_bf16(iq4nl_level(v >> 4)) << 16);
    uint32_t __attribute__((ext_vector_type(4))) q = {e, e, e, e};
    *reinterpret_cast<decltype(q)*>(tbl + 4 * i) = q;
  }
}

// The same table with fp16 levels (also exact), for the kernels that scale
// each weight: a half of an entry feeds v_fma_mix_f32 directly.
__device__ __forceinline__ void build_pair_table_f16(uint32_t* tbl) {
  for (int i = threadIdx.x; i < kPairTableWords / 4; i += blockDim.x) {
    const int v = i >> 3;
    const uint32_t e = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)iq4nl_level(v & 15)) |
                       ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)iq4nl_level(v >> 4)) << 16);
    uint32_t __attribute__((ext_vector_type(4))) q = {e, e, e, e};
    *reinterpret_cast<decltype(q)*>(tbl + 4 * i) = q;
  }
}

// One nibble word (weights 8w..8w+7 of a block) -> the 4 dwords of an 8-slot
// bf16 operand: dword i = (level of weight 8w+2i, level of weight 8w+2i+1).
__device__ __forceinline__ bf16x8 decode_word(const uint32_t* tbl, uint32_t word, uint32_t lane32) {
  union {
    uint32_t u[4];
    bf16x8 v;
  } r;
  r.u[0] = tbl[((word)&0xffu) * 32u + lane32];
  r.u[1] = tbl[((word >> 8) & 0xffu) * 32u + lane32];
  r.u[2] = tbl[((word >> 16) & 0xffu) * 32u + lane32];
  r.u[3] = tbl[(word >> 24) * 32u + lane32];
  return r.v;
}

// 16 bytes per lane from global memory straight into LDS (LDS DMA): lane i
// writes bytes [16i, 16i + 16) of the wavefront's 1 KB at lds (uniform over
// the wavefront; the address comes from the low 16 bits of M0, so every
// destination lies in the first 64 KB of LDS).
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}

// The same for streamed weight data (the scale bytes of weight tiles): non-temporal.
__device__ __forceinline__ void dma16_stream(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, kNonTemporal);
}

// Cross-lane partners without a trip through LDS memory: lane i gets the
// value of lane i ^ M -- M = 1, 2 (DPP quad permutes), 8 (DPP rotation by 8
// inside a row of 16), 4 and 16 (ds_swizzle with an xor mask, which stays in
// the LDS unit's crossbar), 32 (v_permlane32_swap: lanes below 32 take the
// swapped-in upper half, the others the lower half).
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  const int u = __builtin_bit_cast(int, v);
  int r;
  if constexpr (M == 1) {
    r = __builtin_amdgcn_update_dpp(0, u, 0xB1, 0xf, 0xf, false);
  } else if constexpr (M == 2) {
    r = __builtin_amdgcn_update_dpp(0, u, 0x4E, 0xf, 0xf, false);
  } else if constexpr (M == 4) {
    r = __builtin_amdgcn_ds_swizzle(u, 0x101f);
  } else if constexpr (M == 8) {
    r = __builtin_amdgcn_update_dpp(0, u, 0x128, 0xf, 0xf, false);
  } else if constexpr (M == 16) {
    r = __builtin_amdgcn_ds_swizzle(u, 0x401f);
  } else {
    static_assert(M == 32, "xor partners 1 .. 32");
    const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    r = (threadIdx.x & 32) ? (int)p[0] : (int)p[1];
  }
  return __builtin_bit_cast(float, r);
}

// The wavefront's xor butterfly: v + v(lane ^ 32), then partners 16, 8, 4, 2
// and 1 -- the same additions in the same order as a loop of xor shuffles;
// every lane ends with the same value.
__device__ __forceinline__ float wave_xor_sum(float v) {
  v = v + lane_xor<32>(v);
  v = v + lane_xor<16>(v);
  v = v + lane_xor<8>(v);
  v = v + lane_xor<4>(v);
  v = v + lane_xor<2>(v);
  v = v + lane_xor<1>(v);
  return v;
}

// Lane i gets the value of lane i + 1 of its row of 16 (DPP row shift; lane
// 15 of a row gets 0).
__device__ __forceinline__ float lane_next_in_row(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x101, 0xf, 0xf, false));
}

// Every load of this wavefront (LDS DMA included) has landed.
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Every load of this wavefront but the last N has landed (vector memory loads
// complete in order): e.g. the LDS DMA issued before N register loads.
template <int N>
__device__ __forceinline__ void wait_dma_before() {
  static_assert(N >= 0 && N <= 63, "vmcnt immediate (6 bits)");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// fp16 bits -> fp32.
__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xffffu));
}

// fp32 -> bf16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two fp32 values -> one dword of bf16 (lo in bits 0..15), each rounded to
// nearest even by the hardware conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

// bf16 activations of one row for block b, in the operand slot order of
// decode_word: elements 32b + 8w .. 32b + 8w + 7, one 16-byte load.
__device__ __forceinline__ bf16x8 load_x_operand(const uint16_t* xrow, int b, int w) {
  return *reinterpret_cast<const bf16x8*>(xrow + 32 * b + 8 * w);
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 zero_operand() {
  bf16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
  return z;
}

// Scales of one packed tile as seen by MFMA C-register group G (rows 4G..4G+3).

struct TileScales {
  uint32_t s[8];  // fp16 pairs: block b -> s[2b] (rows 4G, 4G+1), s[2b+1] (rows 4G+2, 4G+3)
};

__device__ __forceinline__ TileScales load_scales(const uint8_t* tile, int G) {
  const uint4 a = *reinterpret_cast<const uint4*>(tile + kTileNibbleBytes + 32 * G);
  const uint4 b = *reinterpret_cast<const uint4*>(tile + kTileNibbleBytes + 32 * G + 16);
  TileScales t;
  t.s[0] = a.x;
  t.s[1] = a.y;
  t.s[2] = a.z;
  t.s[3] = a.w;
  t.s[4] = b.x;
  t.s[5] = b.y;
  t.s[6] = b.z;
  t.s[7] = b.w;
  return t;
}

// acc[i] += d(row 4G+i, block b) * c[i]
__device__ __forceinline__ void scale_acc(f32x4& acc, const f32x4& c, const TileScales& sc, int b) {
  const uint32_t p = sc.s[2 * b], q = sc.s[2 * b + 1];
  acc[0] = __builtin_fmaf(half_bits_to_float(p), c[0], acc[0]);
  acc[1] = __builtin_fmaf(half_bits_to_float(p >> 16), c[1], acc[1]);
  acc[2] = __builtin_fmaf(half_bits_to_float(q), c[2], acc[2]);
  acc[3] = __builtin_fmaf(half_bits_to_float(q >> 16), c[3], acc[3]);
}

__device__ __forceinline__ uint32_t uword(const uint4& v, int b) {
  return b == 0 ? v.x : (b == 1 ? v.y : (b == 2 ? v.z : v.w));
}
__device__ __forceinline__ uint32_t uword(const u32x4& v, int b) { return v[b]; }

// HIP keeps the last error of any runtime call per thread; clear it before a
// launch so that the check after the launch reports that launch only.
inline void clear_last_error() { (void)hipGetLastError(); }

// Work item of the expert FFN: up to 16 routes of one expert (expert >= 0,
// first = start position in the bucketed route order) or up to 16 tokens of
// the shared expert (expert == -1, first = first token).
struct Chunk {
  int32_t expert;
  int32_t first;
  int32_t count;
  int32_t pad;
};

}  // namespace qmoe
