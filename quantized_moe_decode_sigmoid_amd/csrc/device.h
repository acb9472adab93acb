// Device-side building blocks shared by the libmoe kernels (gfx950 / CDNA4).
//
// IQ4_NL decode (model card xing4_0-29b-IQ4_NL_EPQ, pure-NumPy parity section:
// a 16-entry non-linear lookup times one fp16 scale per 32-weight block).
// Every level is an integer of at most 7 significant bits, so it is exact in
// bf16; the kernels feed the levels to bf16 MFMA and apply the fp16 scale to
// the fp32 block result (exact-weight contract), or round d*level to bf16
// (bf16 contract).
//
// Nibble bytes are decoded two weights at a time through a 256-entry table in
// LDS: entry v = bf16(level[v & 15]) | bf16(level[v >> 4]) << 16, i.e. the
// pair (weight j, weight j+16) of a block, ready to be one dword of an MFMA
// operand.  The table is replicated 32 times so that lane l always reads bank
// l % 32: lookups never conflict.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kTileBytes = 1152;       // 16 rows x 4 blocks of 18 bytes
constexpr int kTileNibbleBytes = 1024; // 64 lane slots x 16 bytes
constexpr int kPairTableWords = 256 * 32;

// The IQ4_NL levels (ggml definition of the format).
__device__ __forceinline__ int iq4nl_level(int q) {
  constexpr int kLevels[16] = {-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113};
  return kLevels[q & 15];
}

// bf16 bits of a small integer (exact: at most 8 significant bits).
__device__ __forceinline__ uint32_t small_int_bf16(int v) { return __float_as_uint((float)v) >> 16; }

// Fill the replicated pair table; every thread of the block takes part.
__device__ __forceinline__ void build_pair_table(uint32_t* tbl) {
  for (int i = threadIdx.x; i < kPairTableWords; i += blockDim.x) {
    const int v = i >> 5;
    tbl[i] = small_int_bf16(iq4nl_level(v & 15)) | (small_int_bf16(iq4nl_level(v >> 4)) << 16);
  }
}

// One nibble word (bytes 4w..4w+3 of a block) -> the 4 dwords of an 8-slot
// bf16 operand: dword i = (level of weight 4w+i, level of weight 16+4w+i).
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

// bf16 activations of one row for block b, in the operand slot order of
// decode_word: dword i = (x[32b + 4w + i], x[32b + 16 + 4w + i]).
__device__ __forceinline__ bf16x8 load_x_operand(const uint16_t* xrow, int b, int w) {
  const uint2 a = *reinterpret_cast<const uint2*>(xrow + 32 * b + 4 * w);
  const uint2 c = *reinterpret_cast<const uint2*>(xrow + 32 * b + 16 + 4 * w);
  union {
    uint32_t u[4];
    bf16x8 v;
  } r;
  r.u[0] = (a.x & 0xffffu) | (c.x << 16);
  r.u[1] = (a.x >> 16) | (c.x & 0xffff0000u);
  r.u[2] = (a.y & 0xffffu) | (c.y << 16);
  r.u[3] = (a.y >> 16) | (c.y & 0xffff0000u);
  return r.v;
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 zero_operand() {
  bf16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
  return z;
}

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
