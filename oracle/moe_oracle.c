/*
 * CPU oracle for the quantized MoE layer.  TEST INFRASTRUCTURE ONLY: it is
 * called by the test suite, the smoke check and the benchmark's CPU-baseline
 * leg, never by the product path.  It shares no code with the GPU library.
 *
 * Plain C, built with -O2 -ffp-contract=off -fno-fast-math: every fp32
 * operation below is one IEEE operation in the written order; fma() is used
 * only where written.  Floating point is double except where the method fixes
 * a narrower type (the fp32 router, the bf16 activations, the IQ4_NL weights).
 *
 * Sources (the pages are the web pages on Xing4.0-29B-A4B and on IQ4_NL MoE
 * decoding; see the per-function comments):
 *  - PocketLLM "Xing4.0-29B-A4B: the design record", section 1 (shape table:
 *    64 routed top-4 + 1 shared, expert_ffn 1,024, sigmoid router,
 *    routed_scaling_factor 2.0), section 2 (routed + shared summed in fp32,
 *    silu(gate)*up handed to the down projection in fp32) and section 4
 *    (routes sorted by expert, top-k summed in slot order).
 *  - HelloSun "xing4_0-29b-IQ4_NL_EPQ" model card, "Model and routing" table
 *    (sigmoid + ffn_exp_probs_b (noaux_tc), weights normalised and scaled by
 *    2.0, one expert group) and the "pure NumPy" parity sections (IQ4_NL
 *    dequantized by the ggml definition: 16-entry non-linear lookup times one
 *    fp16 scale; whole-layer check = sigmoid + bias + top-4 + sum
 *    normalisation + scale 2.0, weighted sum of the experts).
 *  - zLLM "Algorithm Layer" article, FFN section (gated MLP
 *    y = W_down(act(x W_gate) * (x W_up)), SiLU for this model).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - router logits: fp32, in one fixed summation order (oracle_router_logits);
 *  - sigmoid: evaluated in double by exp_spec below, then rounded to fp32;
 *  - selection order: score descending, expert index ascending;
 *  - the selection bias changes selection only; weights use the plain sigmoid;
 *  - normalisation over the K selected scores, no epsilon; scale applied
 *    after the division, to routed experts only; the shared expert has weight 1;
 *  - precision mode 2 (the grouped bf16 path) rounds dequantized weights and
 *    the SiLU*up product to bf16, nearest-even, as that path specifies.
 *
 * Parity pins: every function here is checked by the CPU tests against
 * brute force, closed forms or invariants (tests/test_oracle_pins.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_FP32 1
#define ORACLE_BF16 2
#define ORACLE_W4A8 3

/* IQ4_NL's 16-entry non-linear codebook (model card: IQ4_NL, 4.5 bpw). */
static const int kIQ4NL[16] = {-127, -104, -83, -65, -49, -35, -22, -10,
                               1,    13,   25,  38,  53,  69,  89,  113};

int oracle_codebook(int i) { return kIQ4NL[i & 15]; }

/* ---- storage types ---------------------------------------------------- */

/* IEEE binary16 -> double, by the format's definition. */
double oracle_f16_value(uint16_t h) {
  int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp(1024.0 + m, e - 25);
  return sign ? -v : v;
}

/* bf16 bit pattern -> fp32 (the upper half of an fp32). */
float oracle_bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* fp32 -> bf16, round to nearest, ties to even (finite inputs).  Written as
 * the choice between the two bf16 neighbours of f. */
uint16_t oracle_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lower = u & 0xffff0000u;         /* truncation toward zero */
  uint32_t rem = u & 0x0000ffffu;           /* distance to it, in fp32 units */
  uint32_t pick = lower;
  if (rem > 0x8000u || (rem == 0x8000u && ((lower >> 16) & 1u))) pick = lower + 0x10000u;
  return (uint16_t)(pick >> 16);
}

/* fp32 -> IEEE binary16, round to nearest, ties to even, by the format's
 * definition: the representable neighbours are multiples of the spacing of
 * f's binade (2^(e-10) for normal results, 2^-24 for subnormal ones);
 * results above the largest finite value round to infinity. */
uint16_t oracle_to_f16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  double a = fabs((double)f);
  if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);               /* a = m * 2^e, 0.5 <= m < 1: leading bit 2^(e-1) */
  int lead = e - 1;           /* exponent of the leading bit */
  if (lead < -14) lead = -14; /* subnormal range: spacing 2^-24 */
  double spacing = ldexp(1.0, lead - 10);
  double k = a / spacing;     /* exact: a is an fp32 value, spacing a power of two */
  double kf = floor(k);
  double rem = k - kf;
  if (rem > 0.5 || (rem == 0.5 && fmod(kf, 2.0) != 0.0)) kf += 1.0;
  double r = kf * spacing;    /* the rounded magnitude */
  if (r >= 65536.0 - 16.0) return (uint16_t)(sign | 0x7c00u); /* above 65504 + half a spacing: infinity */
  /* encode r */
  if (r < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, -24)));
  frexp(r, &e);
  lead = e - 1;
  uint16_t mant = (uint16_t)(r / ldexp(1.0, lead - 10) - 1024.0);
  return (uint16_t)(sign | ((uint16_t)(lead + 15) << 10) | mant);
}

/* ---- Q8_0 activations (the model card's CPU expert path quantizes each
 * matrix product's activation to Q8_0 -- the ggml block format: 32 values,
 * one fp16 scale, 32 int8 codes -- and attributes the residual of its
 * pure-NumPy checks to it; "對純 NumPy：單一 expert" and 整層).  The pages give
 * the format by name only; the reading here: per block, amax = max |x_j| in
 * fp32, d32 = amax / 127 (fp32), stored scale d = fp16(d32) (nearest even),
 * id = 1 / d32 (0 when d32 == 0), q_j = x_j * id rounded to the nearest
 * integer, halves away from zero (|q_j| <= 127 by construction); the value a
 * code stands for is d * q_j. */
void oracle_quantize_q8_0(int64_t n_blocks, const float* x, int8_t* q, uint16_t* d) {
  for (int64_t b = 0; b < n_blocks; b++) {
    float amax = 0.0f;
    for (int j = 0; j < 32; j++) {
      float v = fabsf(x[32 * b + j]);
      if (v > amax) amax = v;
    }
    float d32 = amax / 127.0f;
    float id = d32 != 0.0f ? 1.0f / d32 : 0.0f;
    d[b] = oracle_to_f16(d32);
    for (int j = 0; j < 32; j++) {
      float t = x[32 * b + j] * id;
      q[32 * b + j] = (int8_t)roundf(t);
    }
  }
}

/* ---- IQ4_NL dequantization (model card, parity section: 16-entry lookup
 * times one fp16 scale) ------------------------------------------------- */

/* Weight k (0..31) of an 18-byte block: fp16 d, then byte j holds weight j in
 * the low nibble and weight j+16 in the high nibble.  d (11-bit significand)
 * times a table entry (at most 7 significant bits) is exact in fp32. */
static float block_weight(const uint8_t* blk, int k, int mode) {
  uint16_t dh = (uint16_t)(blk[0] | (blk[1] << 8));
  uint8_t byte = blk[2 + (k & 15)];
  int q = k < 16 ? (byte & 15) : (byte >> 4);
  float w = (float)(oracle_f16_value(dh) * (double)kIQ4NL[q]);
  if (mode == ORACLE_BF16) w = oracle_bf16_value(oracle_to_bf16(w));
  return w;
}

void oracle_dequant(const uint8_t* blocks, int64_t n_blocks, int mode, float* out) {
  for (int64_t b = 0; b < n_blocks; b++)
    for (int k = 0; k < 32; k++) out[32 * b + k] = block_weight(blocks + 18 * b, k, mode);
}

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---- router ----------------------------------------------------------- */

/* Router logits l[t][e] = sum_i x[t][i] * Wg[e][i] in fp32 (the router is an
 * fp32 GEMV: model card weight table lists ffn_gate_inp; the research log
 * names the F32 router GEMVs).  The pages fix no summation order; this one is
 * the method's: 64 partial sums, partial j taking the elements
 * i = 256*m + 4*j + c in the order (m ascending, c ascending) with fused
 * multiply-add, then the 64 partials combined by pairwise sums
 * p[j] <- p[j] + p[j xor s] for s = 32, 16, 8, 4, 2, 1, the result being p[0].
 * Requires H % 256 == 0. */
void oracle_router_logits(int T, int H, int E, const uint16_t* x, const float* Wg, float* logits) {
  for (int t = 0; t < T; t++) {
    for (int e = 0; e < E; e++) {
      float p[64];
      for (int j = 0; j < 64; j++) p[j] = 0.0f;
      for (int m = 0; m < H / 256; m++)
        for (int j = 0; j < 64; j++)
          for (int c = 0; c < 4; c++) {
            int i = 256 * m + 4 * j + c;
            p[j] = fmaf(oracle_bf16_value(x[(int64_t)t * H + i]), Wg[(int64_t)e * H + i], p[j]);
          }
      for (int s = 32; s >= 1; s >>= 1) {
        float q[64];
        for (int j = 0; j < 64; j++) q[j] = p[j] + p[j ^ s];
        memcpy(p, q, sizeof p);
      }
      logits[(int64_t)t * E + e] = p[0];
    }
  }
}

/* exp(y) for double y, evaluated by one fixed sequence of IEEE double
 * operations: range reduction y = n*ln2 + r (Cody & Waite, with a two-part
 * ln 2 and fused multiply-add), the Taylor polynomial of degree 13 for exp(r)
 * in Horner form (|r| <= ln2/2, truncation below 1e-17), and scaling by 2^n. */
static double exp_spec(double y) {
  static const double kLog2e = 0x1.71547652b82fep+0;  /* nearest double to 1/ln 2 */
  static const double kLn2Hi = 0x1.62e42fefa39efp-1;  /* nearest double to ln 2 */
  static const double kLn2Lo = 0x1.abc9e3b39803fp-56; /* nearest double to ln 2 - kLn2Hi */
  if (y > 200.0) return INFINITY;
  if (y < -200.0) return 0.0;
  double n = rint(y * kLog2e);
  double r = fma(-n, kLn2Hi, y);
  r = fma(-n, kLn2Lo, r);
  /* coefficients 1/k!, each the nearest double (exact k! divided once) */
  double fact = 1.0;
  double c[14];
  for (int k = 0; k < 14; k++) {
    if (k > 0) fact *= (double)k;
    c[k] = 1.0 / fact;
  }
  double p = c[13];
  for (int k = 12; k >= 0; k--) p = fma(p, r, c[k]);
  return ldexp(p, (int)n);
}

double oracle_exp_spec(double y) { return exp_spec(y); }

/* Router score: sigmoid (model card: expert_gating_func = sigmoid) evaluated
 * in double and rounded once to fp32. */
float oracle_sigmoid(float l) { return (float)(1.0 / (1.0 + exp_spec(-(double)l))); }

/* Sigmoid scores, biased selection, top-K, normalisation and scaling
 * (model card: sigmoid + ffn_exp_probs_b, top-4, sum normalisation,
 * routed_scaling_factor 2.0).  Slot k holds the k-th selected expert in the
 * order (selection score descending, expert index ascending).  Weights:
 * S = ((s_0 + s_1) + s_2) + ... in fp32 over the slots, w_k = (s_k / S) * scale.
 * bias may be NULL (zero).  logits_out / scores_out may be NULL. */
void oracle_route(int T, int H, int E, int K, float scale, const uint16_t* x, const float* Wg,
                  const float* bias, int32_t* ids, float* w, float* logits_out, float* scores_out) {
  float* logits = (float*)malloc(sizeof(float) * (size_t)T * E);
  oracle_router_logits(T, H, E, x, Wg, logits);
  float* s = (float*)malloc(sizeof(float) * E);
  float* sel = (float*)malloc(sizeof(float) * E);
  char* taken = (char*)malloc((size_t)E);
  for (int t = 0; t < T; t++) {
    for (int e = 0; e < E; e++) {
      s[e] = oracle_sigmoid(logits[(int64_t)t * E + e]);
      sel[e] = bias ? s[e] + bias[e] : s[e];
      taken[e] = 0;
      if (logits_out) logits_out[(int64_t)t * E + e] = logits[(int64_t)t * E + e];
      if (scores_out) scores_out[(int64_t)t * E + e] = s[e];
    }
    for (int k = 0; k < K; k++) {
      int best = -1;
      for (int e = 0; e < E; e++) {
        if (taken[e]) continue;
        if (best < 0 || sel[e] > sel[best]) best = e; /* strict: lower index wins ties */
      }
      taken[best] = 1;
      ids[(int64_t)t * K + k] = best;
    }
    float S = 0.0f;
    for (int k = 0; k < K; k++) S = S + s[ids[(int64_t)t * K + k]];
    for (int k = 0; k < K; k++) w[(int64_t)t * K + k] = (s[ids[(int64_t)t * K + k]] / S) * scale;
  }
  free(logits);
  free(s);
  free(sel);
  free(taken);
}

/* ---- bucketing (design record section 4: routes sorted by expert) ------ */

/* Route r = t*K + k goes to expert ids[r].  counts[e] = number of routes of
 * expert e; offsets = exclusive prefix sum (offsets[E] = T*K); perm lists the
 * routes grouped by expert in ascending expert order, ascending r within an
 * expert; pos is the inverse permutation (pos[perm[i]] = i), may be NULL. */
void oracle_bucket(int T, int K, int E, const int32_t* ids, int32_t* counts, int32_t* offsets,
                   int32_t* perm, int32_t* pos) {
  int64_t R = (int64_t)T * K;
  for (int e = 0; e < E; e++) counts[e] = 0;
  for (int64_t r = 0; r < R; r++) counts[ids[r]]++;
  offsets[0] = 0;
  for (int e = 0; e < E; e++) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * (E > 0 ? E : 1));
  for (int e = 0; e < E; e++) fill[e] = offsets[e];
  for (int64_t r = 0; r < R; r++) {
    int32_t at = fill[ids[r]]++;
    perm[at] = (int32_t)r;
    if (pos) pos[r] = at;
  }
  free(fill);
}

/* ---- expert FFN (zLLM FFN section; design record section 2) ----------- */

/* One expert on one token: g = W_gate x, u = W_up x, h = silu(g) * u,
 * y = W_down h, with silu(g) = g / (1 + exp(-g)).  expert points at
 * [gate F x H | up F x H | down H x F] in IQ4_NL blocks, rows in order.
 * Sums in double.  Mode 1: h kept in double.  Mode 2: weights rounded to bf16
 * and h rounded to fp32 then bf16.  y is [H] doubles. */
/* IQ4_NL block in parts: its scale d (exact, double) and its 32 levels. */
static double block_levels(const uint8_t* blk, int levels[32]) {
  uint16_t dh = (uint16_t)(blk[0] | (blk[1] << 8));
  for (int k = 0; k < 32; k++) {
    uint8_t byte = blk[2 + (k & 15)];
    levels[k] = kIQ4NL[k < 16 ? (byte & 15) : (byte >> 4)];
  }
  return oracle_f16_value(dh);
}

/* Row of IQ4_NL blocks dotted with a Q8_0 vector, block by block: the integer
 * sum s = sum_j level_j * q_j (exact), times d_w * d_x, summed in double. */
static double dot_w4a8(const uint8_t* row, const int8_t* q, const uint16_t* dq, int n_blocks) {
  double acc = 0.0;
  int levels[32];
  for (int b = 0; b < n_blocks; b++) {
    double dw = block_levels(row + 18 * b, levels);
    int64_t s = 0;
    for (int j = 0; j < 32; j++) s += (int64_t)levels[j] * q[32 * b + j];
    acc += dw * oracle_f16_value(dq[b]) * (double)s;
  }
  return acc;
}

/* The W4A8 variant of one expert (mode 3): x (bf16, as fp32) quantized to
 * Q8_0 for gate and up; h = silu(g) * u formed in double, rounded to fp32
 * and quantized to Q8_0 for down; every product an integer block dot as in
 * dot_w4a8. */
static void expert_w4a8(int H, int F, const uint8_t* expert, const uint16_t* x, double* y) {
  if (H < 32 || F < 32) return;
  const int64_t mat_bytes = (int64_t)F * (H / 32) * 18;
  const uint8_t* gate = expert;
  const uint8_t* up = expert + mat_bytes;
  const uint8_t* down = expert + 2 * mat_bytes;
  float* xf = (float*)malloc(sizeof(float) * H);
  int8_t* xq = (int8_t*)malloc((size_t)H);
  uint16_t* xd = (uint16_t*)malloc(sizeof(uint16_t) * (H / 32));
  float* h = (float*)malloc(sizeof(float) * F);
  int8_t* hq = (int8_t*)malloc((size_t)F);
  uint16_t* hd = (uint16_t*)malloc(sizeof(uint16_t) * (F / 32));
  for (int i = 0; i < H; i++) xf[i] = oracle_bf16_value(x[i]);
  oracle_quantize_q8_0(H / 32, xf, xq, xd);
  for (int f = 0; f < F; f++) {
    double g = dot_w4a8(gate + (int64_t)f * (H / 32) * 18, xq, xd, H / 32);
    double u = dot_w4a8(up + (int64_t)f * (H / 32) * 18, xq, xd, H / 32);
    h[f] = (float)(g / (1.0 + exp(-g)) * u);
  }
  oracle_quantize_q8_0(F / 32, h, hq, hd);
  for (int n = 0; n < H; n++) y[n] = dot_w4a8(down + (int64_t)n * (F / 32) * 18, hq, hd, F / 32);
  free(xf);
  free(xq);
  free(xd);
  free(h);
  free(hq);
  free(hd);
}

void oracle_expert(int H, int F, const uint8_t* expert, const uint16_t* x, int mode, double* y) {
  if (mode == ORACLE_W4A8) {
    expert_w4a8(H, F, expert, x, y);
    return;
  }
  const int64_t mat_bytes = (int64_t)F * (H / 32) * 18;
  const uint8_t* gate = expert;
  const uint8_t* up = expert + mat_bytes;
  const uint8_t* down = expert + 2 * mat_bytes;
  double* xv = (double*)malloc(sizeof(double) * H);
  double* h = (double*)malloc(sizeof(double) * F);
  float* wg = (float*)malloc(sizeof(float) * H);
  float* wu = (float*)malloc(sizeof(float) * H);
  float* wd = (float*)malloc(sizeof(float) * F);
  for (int i = 0; i < H; i++) xv[i] = oracle_bf16_value(x[i]);
  for (int f = 0; f < F; f++) {
    oracle_dequant(gate + (int64_t)f * (H / 32) * 18, H / 32, mode, wg);
    oracle_dequant(up + (int64_t)f * (H / 32) * 18, H / 32, mode, wu);
    double g = 0.0, u = 0.0;
    for (int i = 0; i < H; i++) {
      g += (double)wg[i] * xv[i];
      u += (double)wu[i] * xv[i];
    }
    double hv = g / (1.0 + exp(-g)) * u;
    if (mode == ORACLE_BF16) hv = oracle_bf16_value(oracle_to_bf16((float)hv));
    h[f] = hv;
  }
  for (int n = 0; n < H; n++) {
    oracle_dequant(down + (int64_t)n * (F / 32) * 18, F / 32, mode, wd);
    double acc = 0.0;
    for (int f = 0; f < F; f++) acc += (double)wd[f] * h[f];
    y[n] = acc;
  }
  free(xv);
  free(h);
  free(wg);
  free(wu);
  free(wd);
}

/* ---- other expert codecs ------------------------------------------------ */

#define CODEC_IQ4_NL 0
#define CODEC_IQ4_XS 1
#define CODEC_Q3_AFFINE 2

/* IQ4_XS (the zLLM feed's "Quantization Is Not a Zip File" and the W7900D
 * article name it beside IQ4_NL: the same 16-entry non-linear table with a
 * finer scale hierarchy).  The pages name the format only; the reading is
 * ggml's definition: a super-block of 256 weights = fp16 d (2 bytes), the
 * high 2 bits of eight 6-bit sub-block scales (uint16, sub-block i at bits
 * 2i..2i+1), their low 4 bits (4 bytes, sub-block i in nibble i % 2 of byte
 * i / 2, low nibble first), then 8 x 16 bytes of indices, each 16 bytes laid
 * out as an IQ4_NL block (byte j: weight j low nibble, weight j + 16 high).
 * Weight = d * (ls - 32) * level, with ls the 6-bit sub-block scale: an
 * 11-bit times a 6-bit times a 7-bit integer, exact in fp32. */
static void dequant_iq4xs_row(const uint8_t* row, int cols, double* out) {
  for (int sb = 0; sb < cols / 256; sb++) {
    const uint8_t* s = row + 136 * sb;
    double d = oracle_f16_value((uint16_t)(s[0] | (s[1] << 8)));
    unsigned sh = (unsigned)(s[2] | (s[3] << 8));
    for (int ib = 0; ib < 8; ib++) {
      int lo = (s[4 + ib / 2] >> (4 * (ib % 2))) & 15;
      int hi = (sh >> (2 * ib)) & 3;
      double dl = d * (double)((lo | (hi << 4)) - 32);
      const uint8_t* qs = s + 8 + 16 * ib;
      for (int j = 0; j < 32; j++) {
        int q = j < 16 ? (qs[j] & 15) : (qs[j - 16] >> 4);
        out[256 * sb + 32 * ib + j] = dl * (double)kIQ4NL[q];
      }
    }
  }
}

/* Packed 3-bit affine (the SSD streaming page, section on packed 3-bit
 * experts: w = scale * q + bias, eight codes in three bytes instead of four,
 * the same element order as the 4-bit layout; its expert-bytes formula
 * E = P (b + g) / 8 with g = 0.5 bit of scale data per weight).  Reading: a
 * group of 64 weights = fp16 scale, fp16 bias, then 24 bytes holding the 64
 * 3-bit codes q in [0, 7], weight j in bits 3j .. 3j + 2 of the bytes read as
 * one little-endian bit string (so each 3 bytes hold 8 consecutive weights).
 * 28 bytes per 64 weights: 3.5 bits per weight. */
static void dequant_q3_row(const uint8_t* row, int cols, double* out) {
  for (int g = 0; g < cols / 64; g++) {
    const uint8_t* s = row + 28 * g;
    double scale = oracle_f16_value((uint16_t)(s[0] | (s[1] << 8)));
    double bias = oracle_f16_value((uint16_t)(s[2] | (s[3] << 8)));
    for (int j = 0; j < 64; j++) {
      int bit = 3 * j;
      unsigned two = (unsigned)s[4 + bit / 8] | ((bit / 8 + 1 < 24) ? (unsigned)s[4 + bit / 8 + 1] << 8 : 0u);
      int q = (two >> (bit % 8)) & 7;
      out[64 * g + j] = scale * (double)q + bias;
    }
  }
}

/* Bytes of one row of `cols` weights in a codec. */
int64_t oracle_codec_row_bytes(int codec, int cols) {
  if (codec == CODEC_IQ4_XS) return (int64_t)cols / 256 * 136;
  if (codec == CODEC_Q3_AFFINE) return (int64_t)cols / 64 * 28;
  return (int64_t)cols / 32 * 18;
}

/* Bytes of one expert ([gate F x H | up F x H | down H x F], rows in order). */
int64_t oracle_codec_expert_bytes(int codec, int H, int F) {
  return 2 * (int64_t)F * oracle_codec_row_bytes(codec, H) + (int64_t)H * oracle_codec_row_bytes(codec, F);
}

/* Weights of one row, exact, in double. */
void oracle_dequant_codec(int codec, const uint8_t* row, int cols, double* out) {
  if (codec == CODEC_IQ4_XS) {
    dequant_iq4xs_row(row, cols, out);
  } else if (codec == CODEC_Q3_AFFINE) {
    dequant_q3_row(row, cols, out);
  } else {
    for (int b = 0; b < cols / 32; b++)
      for (int k = 0; k < 32; k++) out[32 * b + k] = block_weight(row + 18 * b, k, ORACLE_FP32);
  }
}

/* One expert in another codec (FP32 contract: exact weights, h in double). */
static void expert_codec(int H, int F, int codec, const uint8_t* expert, const uint16_t* x, double* y) {
  const int64_t rbh = oracle_codec_row_bytes(codec, H), rbf = oracle_codec_row_bytes(codec, F);
  const uint8_t* gate = expert;
  const uint8_t* up = expert + F * rbh;
  const uint8_t* down = expert + 2 * F * rbh;
  double* xv = (double*)malloc(sizeof(double) * H);
  double* h = (double*)malloc(sizeof(double) * F);
  double* wg = (double*)malloc(sizeof(double) * H);
  double* wu = (double*)malloc(sizeof(double) * H);
  double* wd = (double*)malloc(sizeof(double) * F);
  for (int i = 0; i < H; i++) xv[i] = oracle_bf16_value(x[i]);
  for (int f = 0; f < F; f++) {
    oracle_dequant_codec(codec, gate + f * rbh, H, wg);
    oracle_dequant_codec(codec, up + f * rbh, H, wu);
    double g = 0.0, u = 0.0;
    for (int i = 0; i < H; i++) {
      g += wg[i] * xv[i];
      u += wu[i] * xv[i];
    }
    h[f] = g / (1.0 + exp(-g)) * u;
  }
  for (int n = 0; n < H; n++) {
    oracle_dequant_codec(codec, down + n * rbf, F, wd);
    double acc = 0.0;
    for (int f = 0; f < F; f++) acc += wd[f] * h[f];
    y[n] = acc;
  }
  free(xv);
  free(h);
  free(wg);
  free(wu);
  free(wd);
}

void oracle_expert_codec(int H, int F, int codec, const uint8_t* expert, const uint16_t* x, double* y) {
  expert_codec(H, F, codec, expert, x, y);
}

/* ---- whole layer -------------------------------------------------------- */

/* out[t] = sum over slots k (ascending) of w[t][k] * y_{ids[t][k]}(x_t)
 *          + g_t * y_shared(x_t)   (when n_shared == 1),
 * accumulated in double and rounded once to fp32 (design record section 2:
 * the routed + shared sum is carried in fp32 or wider).  Routing as in
 * oracle_route.  arena: E experts back to back, expert_bytes = 3*F*H/32*18.
 *
 * The shared expert's weight g_t is 1, or, when shared_gate (an fp32 [H]
 * row) is given, the sigmoid of its logit: g_t = oracle_sigmoid(x_t . shared_gate)
 * with the logit in the router's fixed fp32 order -- the sigmoid-gated shared
 * expert (the research log's shared_expert_gate GEMV, "Where decode time
 * actually goes"; an fp32 GEMV of width H like the router's, its fourth
 * section's ffn_gate_inp_shexp).  Read as: the same sigmoid as the routed
 * scores, no normalisation, no routed_scale.
 *
 * E == 0 with K == 0 and n_shared == 1 is a dense FFN block (model card,
 * "Model and routing": hidden / dense FFN / expert FFN 3584 / 9216 / 1024, the
 * two leading dense blocks): no routing, out[t] = y_shared(x_t).
 * ids_out / w_out may be NULL. */
static void layer_any(int T, int H, int F, int E, int K, int n_shared, float scale, int mode, int codec,
                      const uint16_t* x, const float* Wg, const float* bias, const float* shared_gate,
                      const uint8_t* arena, const uint8_t* shared, float* out, int32_t* ids_out, float* w_out);

void oracle_layer_gated(int T, int H, int F, int E, int K, int n_shared, float scale, int mode,
                        const uint16_t* x, const float* Wg, const float* bias, const float* shared_gate,
                        const uint8_t* arena, const uint8_t* shared, float* out, int32_t* ids_out,
                        float* w_out) {
  layer_any(T, H, F, E, K, n_shared, scale, mode, CODEC_IQ4_NL, x, Wg, bias, shared_gate, arena, shared, out, ids_out,
            w_out);
}

/* The layer with experts in another codec (codec 1 IQ4_XS, 2 packed 3-bit
 * affine; FP32 contract only: mode is ignored). */
void oracle_layer_codec(int T, int H, int F, int E, int K, int n_shared, float scale, int codec,
                        const uint16_t* x, const float* Wg, const float* bias, const float* shared_gate,
                        const uint8_t* arena, const uint8_t* shared, float* out, int32_t* ids_out,
                        float* w_out) {
  layer_any(T, H, F, E, K, n_shared, scale, ORACLE_FP32, codec, x, Wg, bias, shared_gate, arena, shared, out, ids_out,
            w_out);
}

static void layer_any(int T, int H, int F, int E, int K, int n_shared, float scale, int mode, int codec,
                      const uint16_t* x, const float* Wg, const float* bias, const float* shared_gate,
                      const uint8_t* arena, const uint8_t* shared, float* out, int32_t* ids_out, float* w_out) {
  const int64_t eb = oracle_codec_expert_bytes(codec, H, F);
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * ((size_t)T * K + 1));
  float* w = (float*)malloc(sizeof(float) * ((size_t)T * K + 1));
  float* g = (float*)malloc(sizeof(float) * ((size_t)T + 1));
  if (K > 0) oracle_route(T, H, E, K, scale, x, Wg, bias, ids, w, NULL, NULL);
  if (shared_gate) {
    oracle_router_logits(T, H, 1, x, shared_gate, g);
    for (int t = 0; t < T; t++) g[t] = oracle_sigmoid(g[t]);
  }
  /* tokens are independent: the threads split them, each token's sum is
   * formed in the same order whatever the thread count */
#pragma omp parallel for schedule(dynamic, 1)
  for (int t = 0; t < T; t++) {
    double* acc = (double*)malloc(sizeof(double) * H);
    double* y = (double*)malloc(sizeof(double) * H);
    const uint16_t* xt = x + (int64_t)t * H;
    for (int n = 0; n < H; n++) acc[n] = 0.0;
    for (int k = 0; k < K; k++) {
      int e = ids[(int64_t)t * K + k];
      double wk = w[(int64_t)t * K + k];
      if (codec == CODEC_IQ4_NL)
        oracle_expert(H, F, arena + e * eb, xt, mode, y);
      else
        expert_codec(H, F, codec, arena + e * eb, xt, y);
      for (int n = 0; n < H; n++) acc[n] += wk * y[n];
    }
    if (n_shared) {
      const double gs = shared_gate ? (double)g[t] : 1.0;
      if (codec == CODEC_IQ4_NL)
        oracle_expert(H, F, shared, xt, mode, y);
      else
        expert_codec(H, F, codec, shared, xt, y);
      for (int n = 0; n < H; n++) acc[n] += gs * y[n];
    }
    for (int n = 0; n < H; n++) out[(int64_t)t * H + n] = (float)acc[n];
    free(acc);
    free(y);
  }
  if (ids_out && K > 0) memcpy(ids_out, ids, sizeof(int32_t) * (size_t)T * K);
  if (w_out && K > 0) memcpy(w_out, w, sizeof(float) * (size_t)T * K);
  free(ids);
  free(w);
  free(g);
}

/* The layer with an ungated shared expert (weight 1). */
void oracle_layer(int T, int H, int F, int E, int K, int n_shared, float scale, int mode,
                  const uint16_t* x, const float* Wg, const float* bias, const uint8_t* arena,
                  const uint8_t* shared, float* out, int32_t* ids_out, float* w_out) {
  oracle_layer_gated(T, H, F, E, K, n_shared, scale, mode, x, Wg, bias, NULL, arena, shared, out, ids_out, w_out);
}

/* ---- helpers for the test suite and the benchmark's CPU leg ------------ */

/* oracle_sigmoid over n values (the same function, one call per element). */
void oracle_sigmoid_many(int64_t n, const float* l, float* s) {
  for (int64_t i = 0; i < n; i++) s[i] = oracle_sigmoid(l[i]);
}

/* Threads the token loop of oracle_layer may use (OpenMP); n <= 0 leaves
 * the setting unchanged.  Results do not depend on it. */
void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Chaining between the layers of a stack (not part of the MoE layer; harness
 * glue for the 38-layer workload): per row,
 *   h = x + out, y = bf16(h / sqrt(mean(h^2) + eps))
 * with x the layer's bf16 input and out its fp32 output, an unweighted RMS
 * norm (the model card's attention-free stand-in for the rest of a decoder
 * block), evaluated in double and rounded once to bf16 (nearest even). */
void oracle_residual_rmsnorm(int T, int H, const uint16_t* x, const float* out, double eps, uint16_t* y) {
  double* h = (double*)malloc(sizeof(double) * H);
  for (int t = 0; t < T; t++) {
    double ss = 0.0;
    for (int i = 0; i < H; i++) {
      h[i] = (double)oracle_bf16_value(x[(int64_t)t * H + i]) + (double)out[(int64_t)t * H + i];
      ss += h[i] * h[i];
    }
    double r = 1.0 / sqrt(ss / H + eps);
    for (int i = 0; i < H; i++) y[(int64_t)t * H + i] = oracle_to_bf16((float)(h[i] * r));
  }
  free(h);
}
