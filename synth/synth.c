/*
 * Seeded synthetic inputs for the quantized MoE layer.
 *
 * This module only *makes inputs*: counter-based normal variates, their
 * rounding to the storage types the layer consumes (fp32, bf16), and the
 * encoding of N(0, sigma) weight matrices into IQ4_NL blocks.  It holds none
 * of the layer's arithmetic (no dequantization, routing, FFN or combine) and
 * is shared, as plain bytes, by the CPU oracle and the GPU library alike.
 *
 * Random numbers: SplitMix64 (Steele, Lea & Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator: draw i of a stream is mix(key + (i + 1) * gamma).  Normals come
 * from the Box-Muller transform in single precision, one draw per pair.  Every element is a pure
 * function of (seed, stream, index), so results do not depend on the number
 * of threads.
 *
 * IQ4_NL block (the GGUF type used by the model card's checkpoint): 2 bytes
 * little-endian fp16 scale d, then 16 bytes of 4-bit indices into a fixed
 * 16-entry non-linear table; byte j holds weight j in its low nibble and
 * weight j + 16 in its high nibble.  The encoder below is the plain one the
 * pages leave open: d maps the largest-magnitude weight onto the table's
 * largest-magnitude entry (-127), each weight takes the nearest table value.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static const int kCodebook[16] = {-127, -104, -83, -65, -49, -35, -22, -10,
                                  1,    13,   25,  38,  53,  69,  89,  113};

#define GAMMA 0x9e3779b97f4a7c15ULL

static inline uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return sm_mix(sm_mix(seed + GAMMA) + (stream + 1) * GAMMA);
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return sm_mix(key + (i + 1) * GAMMA); }

/* Normal pair p of a stream: one 64-bit draw gives two 24-bit uniforms
 * u1 in (0, 1] and u2 in [0, 1); Box-Muller in single precision. */
static inline void normal_pair(uint64_t key, uint64_t p, float* z0, float* z1) {
  uint64_t a = draw(key, p);
  float u1 = (float)((a >> 40) + 1) * 0x1.0p-24f;
  float u2 = (float)((a >> 8) & 0xffffffu) * 0x1.0p-24f;
  float r = sqrtf(-2.0f * logf(u1)), sn, cs;
  sincosf(6.28318530717958648f * u2, &sn, &cs);
  *z0 = r * cs;
  *z1 = r * sn;
}

/* Element n of the normal stream: component n%2 of pair n/2. */
static inline float normal_at(uint64_t key, uint64_t n) {
  float z0, z1;
  normal_pair(key, n >> 1, &z0, &z1);
  return (n & 1) ? z1 : z0;
}

static inline uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

/* fp32 -> bf16, round to nearest even (inputs here are finite). */
static inline uint16_t to_bf16(float f) {
  uint32_t u = f32_bits(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* fp32 -> IEEE binary16, round to nearest even, with subnormals. */
static uint16_t to_f16(float f) {
  uint32_t u = f32_bits(f);
  uint32_t sign = (u >> 16) & 0x8000u;
  uint32_t a = u & 0x7fffffffu;
  if (a >= 0x7f800000u) return (uint16_t)(sign | 0x7c00u | (a > 0x7f800000u ? 0x200u : 0));
  int e = (int)(a >> 23) - 127;
  uint32_t m = (a & 0x7fffffu) | 0x800000u;
  if (e > 15) return (uint16_t)(sign | 0x7c00u);
  if (e >= -14) { /* normal range: keep 10 fraction bits of 23 */
    uint32_t rest = m & 0x1fffu, keep = m >> 13;
    if (rest > 0x1000u || (rest == 0x1000u && (keep & 1u))) keep++;
    uint32_t h = ((uint32_t)(e + 15) << 10) + (keep - 0x400u);
    if (keep == 0x800u) h = ((uint32_t)(e + 16) << 10); /* carry into exponent */
    return (uint16_t)(sign | h);
  }
  if (e < -25) return (uint16_t)sign;
  /* subnormal: value = m * 2^(e-23); unit = 2^-24 -> shift by (-e - 1) */
  int sh = -e - 1; /* 14..24 */
  uint32_t keep = m >> sh;
  uint32_t rest = m & ((1u << sh) - 1u), half = 1u << (sh - 1);
  if (rest > half || (rest == half && (keep & 1u))) keep++;
  return (uint16_t)(sign | keep);
}

static double f16_value(uint16_t h) {
  int e = (h >> 10) & 0x1f, m = h & 0x3ff;
  double v = e == 0 ? ldexp((double)m, -24) : ldexp((double)(m | 0x400), e - 25);
  return (h & 0x8000) ? -v : v;
}

int synth_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void synth_normal_f32(uint64_t seed, uint64_t stream, int64_t n, double mean, double std, float* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < (n + 1) / 2; p++) {
    float z0, z1;
    normal_pair(key, (uint64_t)p, &z0, &z1);
    out[2 * p] = (float)(mean + std * (double)z0);
    if (2 * p + 1 < n) out[2 * p + 1] = (float)(mean + std * (double)z1);
  }
}

void synth_normal_bf16(uint64_t seed, uint64_t stream, int64_t n, double mean, double std, uint16_t* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = to_bf16((float)(mean + std * (double)normal_at(key, (uint64_t)i)));
}

/* Codebook midpoints, as doubles (exact: halves of small integers). */
static const double kMid[15] = {-115.5, -93.5, -74.0, -57.0, -42.0, -28.5, -16.0, -4.5,
                                7.0,    19.0,  31.5,  45.5,  61.0,  79.0,  101.0};

/* Nearest codebook entry to w for scale d, by |w - d*T[i]| in double, ties to
 * the lower index.  The candidate is the number of midpoints below w/d; its
 * two neighbours are then compared by the exact distance. */
static inline int nearest_index(double w, double d) {
  double y = w / d;
  int i = 0;
  for (int k = 0; k < 15; k++) i += y > kMid[k];
  int best = i > 0 ? i - 1 : 0;
  double bd = fabs(w - d * kCodebook[best]);
  int last = i + 1 < 15 ? i + 1 : 15;
  for (int j = best + 1; j <= last; j++) {
    double dj = fabs(w - d * kCodebook[j]);
    if (dj < bd) { bd = dj; best = j; }
  }
  return best;
}

static void encode_block(const float* w, uint8_t* out) {
  int imax = 0;
  float amax = fabsf(w[0]);
  for (int j = 1; j < 32; j++)
    if (fabsf(w[j]) > amax) { amax = fabsf(w[j]); imax = j; }
  uint16_t dh = to_f16(w[imax] / -127.0f);
  double d = f16_value(dh);
  uint8_t idx[32];
  if (d == 0.0)
    for (int j = 0; j < 32; j++) idx[j] = 8;
  else
    for (int j = 0; j < 32; j++) idx[j] = (uint8_t)nearest_index((double)w[j], d);
  out[0] = (uint8_t)(dh & 0xff);
  out[1] = (uint8_t)(dh >> 8);
  for (int j = 0; j < 16; j++) out[2 + j] = (uint8_t)(idx[j] | (idx[j + 16] << 4));
}

/* n_blocks consecutive IQ4_NL blocks encoding N(0, std) weights, weight k of
 * block b being normal element 32*b + k of the stream.  A row-major matrix of
 * R rows by C columns (C % 32 == 0) is R*C/32 blocks in row order. */
void synth_iq4nl(uint64_t seed, uint64_t stream, int64_t n_blocks, double std, uint8_t* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < n_blocks; b++) {
    float w[32];
    for (int k = 0; k < 32; k += 2) {
      float z0, z1;
      normal_pair(key, (uint64_t)(16 * b + k / 2), &z0, &z1);
      w[k] = (float)(std * (double)z0);
      w[k + 1] = (float)(std * (double)z1);
    }
    encode_block(w, out + 18 * b);
  }
}

/* Encode caller-given fp32 weights (n_blocks * 32 values) into IQ4_NL. */
void synth_encode_iq4nl(const float* w, int64_t n_blocks, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < n_blocks; b++) encode_block(w + 32 * b, out + 18 * b);
}

/* ---- other expert codecs (input generation only) ----------------------- */

/* IQ4_XS super-block of 256 weights: fp16 d, the high 2 bits of eight 6-bit
 * sub-block scales (uint16, sub-block i at bits 2i), their low 4 bits (nibble
 * i % 2 of byte 4 + i / 2), then 8 x 16 index bytes in IQ4_NL order; weight =
 * d * (ls - 32) * table[index].  The plain encoder: each sub-block's ideal
 * scale s_i maps its largest-magnitude weight onto -127 (as for IQ4_NL),
 * d = fp16(max_i |s_i| / 31), ls_i = clamp(round(s_i / d) + 32, 0, 63), and
 * each weight takes the nearest table value for the sub-block's scale. */
static void encode_iq4xs(const float* w, uint8_t* out) {
  double s[8];
  double smax = 0.0;
  for (int ib = 0; ib < 8; ib++) {
    int imax = 0;
    float amax = fabsf(w[32 * ib]);
    for (int j = 1; j < 32; j++)
      if (fabsf(w[32 * ib + j]) > amax) { amax = fabsf(w[32 * ib + j]); imax = j; }
    s[ib] = (double)w[32 * ib + imax] / -127.0;
    if (fabs(s[ib]) > smax) smax = fabs(s[ib]);
  }
  uint16_t dh = to_f16((float)(smax / 31.0));
  double d = f16_value(dh);
  memset(out, 0, 136);
  out[0] = (uint8_t)(dh & 0xff);
  out[1] = (uint8_t)(dh >> 8);
  unsigned sh = 0;
  for (int ib = 0; ib < 8; ib++) {
    int ls = d == 0.0 ? 32 : (int)lround(s[ib] / d) + 32;
    ls = ls < 0 ? 0 : (ls > 63 ? 63 : ls);
    sh |= (unsigned)((ls >> 4) & 3) << (2 * ib);
    out[4 + ib / 2] |= (uint8_t)((ls & 15) << (4 * (ib % 2)));
    double dl = d * (double)(ls - 32);
    uint8_t idx[32];
    for (int j = 0; j < 32; j++) idx[j] = dl == 0.0 ? 8 : (uint8_t)nearest_index((double)w[32 * ib + j], dl);
    for (int j = 0; j < 16; j++) out[8 + 16 * ib + j] = (uint8_t)(idx[j] | (idx[j + 16] << 4));
  }
  out[2] = (uint8_t)(sh & 0xff);
  out[3] = (uint8_t)(sh >> 8);
}

/* Packed 3-bit affine group of 64 weights: fp16 scale, fp16 bias, then 24
 * bytes with code j (0..7) at bits 3j..3j+2 of the little-endian bit string;
 * weight = scale * code + bias.  The plain min/max encoder: bias = fp16(min),
 * scale = fp16((max - min) / 7), code = clamp(round((w - bias) / scale), 0, 7). */
static void encode_q3(const float* w, uint8_t* out) {
  float lo = w[0], hi = w[0];
  for (int j = 1; j < 64; j++) {
    if (w[j] < lo) lo = w[j];
    if (w[j] > hi) hi = w[j];
  }
  uint16_t sh = to_f16((hi - lo) / 7.0f), bh = to_f16(lo);
  double scale = f16_value(sh), bias = f16_value(bh);
  memset(out, 0, 28);
  out[0] = (uint8_t)(sh & 0xff);
  out[1] = (uint8_t)(sh >> 8);
  out[2] = (uint8_t)(bh & 0xff);
  out[3] = (uint8_t)(bh >> 8);
  for (int j = 0; j < 64; j++) {
    int q = scale == 0.0 ? 0 : (int)lround(((double)w[j] - bias) / scale);
    q = q < 0 ? 0 : (q > 7 ? 7 : q);
    for (int k = 0; k < 3; k++)
      if ((q >> k) & 1) out[4 + (3 * j + k) / 8] |= (uint8_t)(1u << ((3 * j + k) % 8));
  }
}

/* n_units consecutive super-blocks (IQ4_XS, 256 weights) or groups (3-bit, 64
 * weights) encoding N(0, std) weights, weight k of unit u being normal element
 * (unit size) * u + k of the stream. */
void synth_codec(int codec, uint64_t seed, uint64_t stream, int64_t n_units, double std, uint8_t* out) {
  uint64_t key = stream_key(seed, stream);
  const int unit = codec == 1 ? 256 : 64;
  const int bytes = codec == 1 ? 136 : 28;
#pragma omp parallel for schedule(static)
  for (int64_t u = 0; u < n_units; u++) {
    float w[256];
    for (int k = 0; k < unit; k += 2) {
      float z0, z1;
      normal_pair(key, (uint64_t)(unit / 2 * u + k / 2), &z0, &z1);
      w[k] = (float)(std * (double)z0);
      w[k + 1] = (float)(std * (double)z1);
    }
    if (codec == 1)
      encode_iq4xs(w, out + bytes * u);
    else
      encode_q3(w, out + bytes * u);
  }
}
