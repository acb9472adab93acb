/*
 * moe.h -- C ABI of libmoe: one quantized Mixture-of-Experts FFN layer on an
 * MI355X (gfx950) GPU.
 *
 * The layer (shape of Xing4.0-29B-A4B: PocketLLM design record, section 1
 * shape table; HelloSun xing4_0-29b-IQ4_NL_EPQ model card, "Model and
 * routing" table):
 *   - a sigmoid router over E experts with an optional selection-only bias
 *     (ffn_exp_probs_b, "noaux_tc"), top-K, weights normalised over the K
 *     selected scores and multiplied by routed_scale (2.0);
 *   - per selected expert a SwiGLU FFN y = W_down(silu(W_gate x) * (W_up x))
 *     (zLLM "Algorithm Layer", FFN section) with IQ4_NL weights (32-weight
 *     blocks, one fp16 scale, 4-bit indices into a 16-entry non-linear table);
 *   - an always-on shared expert of weight 1;
 *   - the routed + shared sum in fp32 (design record, section 2), the top-K
 *     summed in slot order with no atomics (design record, section 4).
 *
 * Conventions for every entry point:
 *   - Pointers named *_dev are device pointers; the caller owns all memory
 *     (inputs, outputs, arenas, workspace).  The library keeps no device
 *     state, allocates nothing and never synchronizes: each call validates its
 *     arguments on the host, then enqueues kernels on `stream` (0 = the null
 *     stream) and returns.  Device memory is never read back to the host.
 *   - Validation failures return a negative status before anything is
 *     enqueued.  Every device pointer must be 16-byte aligned (MOE_EALIGN).
 *     A call with T == 0 tokens is a no-op that checks only cfg and T
 *     (except moe_bucket, which then writes all-zero counts and offsets).
 *   - Workspaces are caller-owned scratch; no state is kept in them between
 *     calls (beyond the status word, see moe_workspace_init).
 *   - Values that are only known on the device (expert ids outside [0, E),
 *     non-finite activations) are not checked: behaviour is undefined.
 *   - Row-major layouts.  bf16 is the upper half of an IEEE fp32, fp16 is
 *     IEEE binary16, both little-endian.
 *   - Calls on one stream are ordered; calls sharing a workspace must not
 *     overlap in time.
 */
#ifndef QMOE_MOE_H
#define QMOE_MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 4

/* Status codes. */
typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,       /* a null required pointer, a bad size or shape */
  MOE_EALIGN = -2,       /* a device pointer not 16-byte aligned */
  MOE_EWORKSPACE = -3,   /* workspace smaller than moe_workspace_bytes() */
  MOE_EUNSUPPORTED = -4, /* a shape outside the supported set (see moe_config) */
  MOE_ELAUNCH = -5       /* the HIP runtime refused a launch */
} moe_status;

/* Arithmetic contract of the expert FFN.
 * FP32: weights are the exact IQ4_NL values d*level; g, u, y and the combine
 *       are fp32 sums; h = silu(g)*u is formed in fp32 and handed to the down
 *       projection as two bf16 terms, h_hi = bf16(h) and h_lo = bf16(h - h_hi)
 *       (nearest even), whose sum is within 2^-16 * |h| of h (decode-sized
 *       calls).  Against a double-precision evaluation with exact weights the
 *       output then differs by fp32 summation order, the fp32 SiLU and this
 *       split.
 * BF16: weights are the exact values rounded to bf16 (nearest even), the
 *       product silu(g)*u is rounded to bf16 before the down projection;
 *       products run on bf16 MFMA with fp32 accumulation (batched / prefill
 *       calls: tiles of up to 128 routes of one expert).
 * W4A8: the exact IQ4_NL weights against activations quantized to Q8_0 --
 *       the model card's CPU expert path, whose pure-NumPy checks attribute
 *       their ~1 % residual to this quantization: x and h are quantized per
 *       token row in blocks of 32 (fp16 scale d = fp16(max|v| / 127), int8
 *       codes round(v * 127 / max|v|) with halves away from zero), every
 *       32-weight block is an exact integer dot of levels and codes on int8
 *       MFMA, scaled by d_w * d_x and accumulated in fp32.  Only when asked
 *       for (AUTO never picks it); takes the multi-kernel plan at every T.
 * AUTO: FP32 when T*K <= 16*E (at most 16 routes per expert on average;
 *       for a dense block, T <= 16), else BF16.  The router and the combine are fp32 in every mode. */
typedef enum { MOE_PREC_AUTO = 0, MOE_PREC_FP32 = 1, MOE_PREC_BF16 = 2, MOE_PREC_W4A8 = 3 } moe_precision;

/* Expert weight codecs (input layout of moe_pack_experts, per expert
 * [gate F x H | up F x H | down H x F], rows in order):
 * IQ4_NL    18-byte blocks of 32 weights (see "expert arena" below).
 * IQ4_XS    136-byte super-blocks of 256 weights: fp16 d, uint16 with the high
 *           2 bits of eight 6-bit sub-block scales ls (sub-block i at bits 2i),
 *           4 bytes with their low 4 bits (nibble i % 2 of byte i / 2, low
 *           first), then 8 x 16 index bytes in IQ4_NL order; weight =
 *           d * (ls - 32) * level (named beside IQ4_NL by the zLLM feed,
 *           "Quantization Is Not a Zip File"; ggml's layout).  Needs ffn % 256.
 * Q3_AFFINE 28-byte groups of 64 weights: fp16 scale, fp16 bias, then 24 bytes
 *           of 3-bit codes q, weight j in bits 3j..3j+2 of the little-endian
 *           bit string; weight = scale * q + bias (the SSD streaming page,
 *           packed 3-bit section: 8 codes in 3 bytes, 3.5 bits per weight).
 * IQ4_XS and Q3_AFFINE run the exact-weight (FP32) contract on the
 * multi-kernel plan at every T (precision AUTO or FP32 only). */
typedef enum { MOE_CODEC_IQ4_NL = 0, MOE_CODEC_IQ4_XS = 1, MOE_CODEC_Q3_AFFINE = 2 } moe_codec;

/* Layer shape.  Supported: hidden % 256 == 0, ffn % 128 == 0,
 * 1 <= n_experts <= 256, 1 <= top_k <= min(n_experts, 8), n_shared in {0, 1},
 * routed_scale finite.  Tokens per call: 0 <= T <= 65536.
 *
 * shared_gate = 1 (needs n_shared = 1): the shared expert's output is scaled
 * by g_t = sigmoid(x_t . gate_w[E]) -- a sigmoid-gated shared expert (the
 * FlashNext research log's shared_expert_gate, "Where decode time actually
 * goes") -- instead of 1.  gate_w then has E + 1 rows, row E being the gate;
 * its logit and sigmoid are computed exactly like the routed scores (fixed
 * fp32 order, see moe_route) and the routing weights carry it as one more
 * value per token: topk_w is [T][K + 1] with topk_w[t][K] = g_t.
 *
 * n_experts = 0 (with top_k = 0, n_shared = 1, shared_gate = 0) is a dense
 * FFN block (model card "Model and routing": the two leading dense blocks,
 * hidden / dense FFN 3584 / 9216): out[t] = FFN(x_t) with the one always-on
 * expert's weights in shared_dev; no router weight, routing or arena is read
 * (those pointers may be NULL) and moe_route / moe_bucket / moe_router_scores
 * refuse it (MOE_EINVAL). */
typedef struct {
  int32_t hidden;      /* H: model width */
  int32_t ffn;         /* F: expert intermediate width */
  int32_t n_experts;   /* E: routed experts (0: a dense FFN block) */
  int32_t top_k;       /* K: experts per token */
  int32_t n_shared;    /* shared experts (0 or 1) */
  float routed_scale;  /* multiplies the normalised routed weights (2.0) */
  int32_t precision;   /* moe_precision */
  int32_t shared_gate; /* 1: the shared expert is scaled by sigmoid(x . gate_w[E]); 0: weight 1 */
  int32_t codec;       /* moe_codec of the expert weights */
} moe_config;

/* ---- queries (host only, no GPU work) ----------------------------------- */

int moe_abi_version(void);

/* Static description of a status code; never NULL. */
const char* moe_status_string(int status);

/* MOE_OK if the shape is supported, else MOE_EINVAL / MOE_EUNSUPPORTED. */
moe_status moe_check_config(const moe_config* cfg);

/* Bytes of one expert in its codec's input layout: for IQ4_NL 3 matrices of
 * F*H/32 blocks of 18 bytes (the model card's 6,193,152 B for H=3584,
 * F=1024).  0 if the configuration is invalid. */
size_t moe_expert_bytes(const moe_config* cfg);

/* Bytes of one expert in the packed layout (what moe_pack_experts writes and
 * the compute entry points read, expert e at e * this): moe_expert_bytes for
 * IQ4_NL and Q3_AFFINE; for IQ4_XS 1120 bytes per 16 x 128 tile, 32 more than
 * the format (each of a super-block's two tiles repeats its d).  0 if the
 * configuration is invalid. */
size_t moe_packed_expert_bytes(const moe_config* cfg);

/* Precision the expert FFN will use for T tokens (resolves AUTO). */
int32_t moe_resolved_precision(const moe_config* cfg, int32_t T);

/* Workspace bytes moe_route / moe_expert_forward / moe_layer_forward need for
 * T tokens (the maximum of the three).  0 if the configuration is invalid. */
size_t moe_workspace_bytes(const moe_config* cfg, int32_t T);

/* Zero the status word of a workspace (its first 4 bytes).  The decode path
 * of moe_layer_forward (T = 1, K <= 4, H <= 4096, F <= 1024, H <= 4 F with a shared
 * expert, FP32 contract)
 * hands data between workgroups of one kernel and bounds every wait; a wait
 * that gives up (which a correct launch never does) sets this word to 1.
 * Workspaces need no other preparation. */
moe_status moe_workspace_init(const moe_config* cfg, int32_t T, void* ws_dev, size_t ws_bytes, hipStream_t stream);

/* Copy the status word of a workspace (see moe_workspace_init: 0 = every wait
 * of the decode path ended normally, 1 = one gave up and that call's outputs are
 * not valid) to status_dev, a device int32, on `stream` (a kernel: no host
 * synchronization, no readback).  The word is sticky until the next
 * moe_workspace_init. */
moe_status moe_workspace_status(const moe_config* cfg, int32_t T, const void* ws_dev, size_t ws_bytes,
                                int32_t* status_dev, hipStream_t stream);

/* ---- expert arena --------------------------------------------------------
 * GGUF order (input of moe_pack_experts): expert e starts at e*expert_bytes;
 * inside it W_gate [F rows][H/32 blocks], W_up [F][H/32], W_down [H][F/32],
 * each block 18 bytes: fp16 scale d, then 16 bytes where byte j holds the
 * index of weight j in its low nibble and of weight j+16 in its high nibble
 * (the ggml IQ4_NL definition the model card's checker follows).
 *
 * Packed order (what the compute entry points read): the same information
 * regrouped per matrix into 1152-byte tiles of 16 rows x 4 blocks, so that a
 * wavefront streams each tile with one 16-byte load per lane: tile (rt, kg)
 * covers rows 16*rt..16*rt+15 and blocks 4*kg..4*kg+3 and sits at tile index
 * rt*(NB/4) + kg (NB = blocks per row).  Bytes [0, 1024): lane slot s
 * (row 16*rt + s%16, word w = s/16) holds, for blocks 4kg+0..4kg+3 in turn,
 * 4 bytes with the indices of weights 8w..8w+7 of that block: byte i holds
 * weight 8w+2i in its low nibble and 8w+2i+1 in its high nibble.  Bytes
 * [1024, 1152): the 64 fp16 scales, scale of (row 16*rt + 4*G + i,
 * block 4*kg + b) at 1024 + 32*G + 8*b + 2*i.  An expert keeps
 * moe_expert_bytes() bytes and the same start offset. */

/* Repack n_experts consecutive experts from GGUF order (src_dev) into packed
 * order (dst_dev).  src and dst must not overlap.  Run once at load. */
moe_status moe_pack_experts(const moe_config* cfg, int32_t n_experts, const void* src_dev, void* dst_dev,
                            hipStream_t stream);

/* Dequantize one matrix of one packed expert to fp32, row-major:
 * matrix 0 = W_gate [F][H], 1 = W_up [F][H], 2 = W_down [H][F].
 * precision FP32: the exact weights d*level.  BF16: those weights rounded to
 * bf16 (nearest even), returned widened to fp32.  Uses the same decode as the
 * FFN kernels (model card, pure-NumPy parity section: 16-entry non-linear
 * lookup times one fp16 scale). */
moe_status moe_dequant(const moe_config* cfg, const void* packed_expert_dev, int32_t matrix, int32_t precision,
                       float* out_dev, hipStream_t stream);

/* The W4A8 contract's activation quantizer alone: n values (a multiple of 32,
 * src_bf16 = 1: bf16, 0: fp32) -> Q8_0 blocks of 32: q_dev int8 [n] codes and
 * d_dev fp16 [n/32] scales, as stated for MOE_PREC_W4A8. */
moe_status moe_quantize_q8_0(const void* src_dev, int32_t src_bf16, int64_t n, int8_t* q_dev, uint16_t* d_dev,
                             hipStream_t stream);

/* ---- the layer's steps ---------------------------------------------------- */

/* Router (model card "Model and routing": sigmoid + ffn_exp_probs_b, top-K,
 * sum normalisation, expert_weights_scale 2.0).
 *   x_dev       bf16 [T][H] activations
 *   gate_w_dev  fp32 [E][H] router weight
 *   sel_bias_dev fp32 [E] selection bias, or NULL for none
 *   topk_ids_dev int32 [T][K] out: slot k = k-th expert by
 *               (sigmoid(logit) + bias) descending, expert index ascending
 *   topk_w_dev  fp32 [T][K] out: routed_scale * s_k / (s_0 + ... + s_{K-1})
 *               with s the unbiased sigmoid scores, sums left to right.
 * Logits are fp32 dot products in one fixed order (64 partial sums of
 * elements 256m+4j+c, fused multiply-adds over (m, c), then pairwise sums
 * p[j] + p[j^s], s = 32..1); the sigmoid is evaluated in double by a fixed
 * sequence of IEEE operations and rounded to fp32; so the outputs are
 * bit-reproducible and equal to the CPU reference.  ws: >= moe_workspace_bytes. */
moe_status moe_route(const moe_config* cfg, int32_t T, const void* x_dev, const float* gate_w_dev,
                     const float* sel_bias_dev, int32_t* topk_ids_dev, float* topk_w_dev, void* ws_dev,
                     size_t ws_bytes, hipStream_t stream);

/* The router's first half alone: scores_dev fp32 [T][E] receives
 * s[t][e] = sigmoid(x[t] . gate_w[e]), the fp32 logit in the fixed order stated
 * for moe_route and the sigmoid evaluated as stated there (model card
 * xing4_0-29b-IQ4_NL_EPQ, "Model and routing": expert_gating_func = sigmoid).
 * These are the scores moe_route selects from and normalises (before the
 * selection bias).  Needs no workspace. */
moe_status moe_router_scores(const moe_config* cfg, int32_t T, const void* x_dev, const float* gate_w_dev,
                             float* scores_dev, hipStream_t stream);

/* Token-to-expert bucketing (design record, section 4: routes sorted by
 * expert so each output has one writer).  Route r = t*K + k.
 *   counts_dev  int32 [E]     routes per expert
 *   offsets_dev int32 [E+1]   exclusive prefix sum, offsets[E] = T*K
 *   perm_dev    int32 [T*K]   routes grouped by expert (ascending), ascending r
 *                             inside an expert
 *   pos_dev     int32 [T*K]   inverse permutation, or NULL
 * Bit-exact (integer).  Needs no workspace. */
moe_status moe_bucket(const moe_config* cfg, int32_t T, const int32_t* topk_ids_dev, int32_t* counts_dev,
                      int32_t* offsets_dev, int32_t* perm_dev, int32_t* pos_dev, hipStream_t stream);

/* Expert FFN and combine for given routing (FFN(x) = W_down (silu(W_gate x) *
 * (W_up x)): zLLM "Algorithm Layer", FFN section; IQ4_NL weights: model card,
 * pure-NumPy parity section; weighting after the down projection, fp32 sum:
 * design record, section 2; slot-order sum over the bucketed routes, no
 * atomics: design record, section 4):
 *   out[t] = sum_{k=0..K-1} topk_w[t][k] * FFN_{topk_ids[t][k]}(x[t])
 *            + FFN_shared(x[t])                     (if n_shared == 1)
 *   x_dev        bf16 [T][H]
 *   arena_dev    E experts, packed order (moe_pack_experts)
 *   shared_dev   one packed expert, or NULL when n_shared == 0
 *   out_dev      fp32 [T][H], fully overwritten
 * Deterministic: the same inputs give the same bits on every run; the slot
 * sum runs in slot order.  ws: >= moe_workspace_bytes(cfg, T). */
moe_status moe_expert_forward(const moe_config* cfg, int32_t T, const void* x_dev, const int32_t* topk_ids_dev,
                              const float* topk_w_dev, const void* arena_dev, const void* shared_dev,
                              float* out_dev, void* ws_dev, size_t ws_bytes, hipStream_t stream);

/* The whole layer (model card "Model and routing": sigmoid router with
 * selection bias, top-K of E routed experts plus the shared expert, weights
 * times routed_scale; design record, section 1, for the Xing4 layer):
 * moe_route then moe_expert_forward.  topk_ids_out_dev and
 * topk_w_out_dev receive the routing when non-NULL (else the workspace holds
 * it).  ws: >= moe_workspace_bytes(cfg, T).  A token whose activations hold
 * a NaN has NaN scores, which all tie: it takes the K lowest expert indices
 * (on every plan) and its output row is NaN; no other token is affected and
 * no access leaves the given buffers. */
moe_status moe_layer_forward(const moe_config* cfg, int32_t T, const void* x_dev, const float* gate_w_dev,
                             const float* sel_bias_dev, const void* arena_dev, const void* shared_dev,
                             float* out_dev, int32_t* topk_ids_out_dev, float* topk_w_out_dev, void* ws_dev,
                             size_t ws_bytes, hipStream_t stream);

/* A layer of a stack of MoE layers, its input formed in the same call from
 * the previous layer's input and output:
 *   x = bf16(h / sqrt(mean(h^2) + eps)) with h = fp32(x_prev) + out_prev
 * per token row (an unweighted RMS norm after the residual add: the chaining
 * that stands in for the rest of a decoder block between two MoE layers of
 * Xing4.0-29B-A4B, design record section 1), then moe_layer_forward on x.
 *   x_prev_dev   bf16 [T][H]   the previous layer's input
 *   out_prev_dev fp32 [T][H]   the previous layer's output
 *   x_dev        bf16 [T][H]   out: this layer's input (the next call's
 *                x_prev); must not overlap x_prev_dev or out_prev_dev
 * x is bit-identical to moe_residual_rmsnorm(out_prev, x_prev, T, H, eps, x)
 * and the outputs to moe_layer_forward on that x.  On the decode plan
 * (T = 1) the norm runs inside the router kernel (no extra launch).  Other
 * arguments as moe_layer_forward; eps >= 0 and finite. */
moe_status moe_layer_forward_chained(const moe_config* cfg, int32_t T, const void* x_prev_dev,
                                     const float* out_prev_dev, float eps, void* x_dev, const float* gate_w_dev,
                                     const float* sel_bias_dev, const void* arena_dev, const void* shared_dev,
                                     float* out_dev, int32_t* topk_ids_out_dev, float* topk_w_out_dev, void* ws_dev,
                                     size_t ws_bytes, hipStream_t stream);

/* ---- a stack of layers ----------------------------------------------------
 * One decode token (T = 1) through L layers chained as in
 * moe_layer_forward_chained (design record, section 6: the decode step
 * captured as a whole rather than call by call):
 *   x_0 = x0;  out_l = moe_layer_forward on x_l with layer l's weights;
 *   x_{l+1} = bf16(rmsnorm(x_l + out_l)) with eps (moe_residual_rmsnorm).
 * 2 L launches on `stream`: per layer the decode plan's two kernels, the
 * layer's input formed in the first (as in moe_layer_forward_chained: 256
 * threads per router row form bf16(rmsnorm(x + out)) and the logit); layer 0
 * reads x0, copies it to row 0 of x_all and clears the status word.  Results
 * are bit-identical to L calls of moe_layer_forward_chained (layer 0:
 * moe_layer_forward on x0) with the same weights: the same routing, x and
 * outputs.  One token's decode workspace is reused by every layer.
 *   layers_host  host array of L layer descriptions (device pointers inside;
 *                gate_w fp32 [E + shared_gate][H], sel_bias fp32 [E] or
 *                NULL, arena and shared packed by moe_pack_experts; shared
 *                may be NULL without a shared expert), read during the
 *                call only
 *   x0_dev       bf16 [H]        layer 0's input
 *   x_all_dev    bf16 [L][H]     out: every layer's input (row 0 = x0); must
 *                                not overlap x0_dev
 *   out_all_dev  fp32 [L][H]     out: every layer's output
 *   ids_all_dev  int32 [L][K]    out, or NULL
 *   w_all_dev    fp32 [L][K + shared_gate]  out, or NULL
 *   ws           >= moe_stack_workspace_bytes(cfg, L)
 * Supported (else MOE_EUNSUPPORTED): the decode plan's shapes (precision AUTO
 * or FP32, IQ4_NL, n_experts >= 1, top_k <= 4, ffn <= 1024, hidden <= 4096,
 * hidden <= 4 ffn with a shared expert; gated or not), 1 <= L <= 64, and the
 * decode kernel's grid resident on the device at once.  Every wait is
 * bounded; if one gives up, the outputs are wrong and the status word is 1
 * (moe_stack_status).  eps >= 0 and finite. */
typedef struct {
  const float* gate_w;
  const float* sel_bias;
  const void* arena;
  const void* shared;
} moe_stack_layer;

moe_status moe_stack_workspace_bytes(const moe_config* cfg, int32_t L, size_t* bytes);

moe_status moe_stack_decode(const moe_config* cfg, int32_t L, const moe_stack_layer* layers_host, const void* x0_dev,
                            float eps, void* x_all_dev, float* out_all_dev, int32_t* ids_all_dev, float* w_all_dev,
                            void* ws_dev, size_t ws_bytes, hipStream_t stream);

/* Copy the last moe_stack_decode's status word (0: every wait ended in time,
 * 1: one gave up) to status_dev (int32, device), on `stream` (one small
 * kernel, no synchronization). */
moe_status moe_stack_status(const moe_config* cfg, int32_t L, const void* ws_dev, size_t ws_bytes,
                            int32_t* status_dev, hipStream_t stream);

/* moe_layer_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, validation, kernels and
 * results as moe_layer_forward; the workspace is instead a device array of
 * 64 MiB inside the library, one per GPU it runs on, held until the process
 * ends.  Calls whose workspace (moe_workspace_bytes(cfg, T)) exceeds it return
 * MOE_EWORKSPACE (the Xing4 layer fits up to a few hundred tokens per call).
 * Allocates nothing: the array's address is looked up once per device, and the
 * first call on a device also clears its status word (one small kernel on
 * `stream`).  Every call on one GPU uses that GPU's array: calls that overlap
 * in time on one GPU (other streams, other threads) race and give undefined
 * results.  The array keeps the last call's contents. */
moe_status moe_layer_forward_noalloc(const moe_config* cfg, int32_t T, const void* x_dev, const float* gate_w_dev,
                                     const float* sel_bias_dev, const void* arena_dev, const void* shared_dev,
                                     float* out_dev, int32_t* topk_ids_out_dev, float* topk_w_out_dev,
                                     hipStream_t stream);

/* ---- measurement ----------------------------------------------------------
 * Not part of the layer: a kernel of known traffic for reporting achieved
 * bandwidth against this GPU's own streaming rate as well as the vendor peak.
 *
 * Read bytes of src_dev exactly once (16-byte vector loads, a grid-stride walk
 * over the whole GPU) and write nothing except, with negligible probability,
 * one word to sink_dev (so the reads cannot be optimised away).  bytes must be
 * a multiple of 16; src_dev and sink_dev 16-byte aligned. */
moe_status moe_stream_read(const void* src_dev, size_t bytes, uint32_t* sink_dev, hipStream_t stream);

/* Not part of the layer either: the chaining between consecutive layers of a
 * stack, y = bf16(rmsnorm(x + out)) with no weight, one fused kernel.
 *   out_dev fp32 [T][H] (a layer's output), x_dev bf16 [T][H] (its input),
 *   y_dev   bf16 [T][H] (the next layer's input; may alias x_dev)
 * Per row: h = fp32(x) + out, r = 1 / sqrt(mean(h^2) + eps) in fp32, y =
 * bf16(h * r) rounded to nearest even.  H % 256 == 0 as for the layer. */
moe_status moe_residual_rmsnorm(const float* out_dev, const void* x_dev, int32_t T, int32_t H, float eps,
                                void* y_dev, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QMOE_MOE_H */
