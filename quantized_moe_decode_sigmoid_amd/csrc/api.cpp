// C ABI of libmoe (declared in include/moe.h): host-side validation, the
// workspace plan, and the dispatch of the kernels onto the caller's stream.
// Nothing here allocates device memory, synchronizes, or reads device memory.
#include "moe.h"

#include <math.h>
#include <stdio.h>
#include <stdint.h>
#include <string.h>

#include "launch.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kMaxTokens = 65536;
constexpr int kMaxHidden = 8192;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

moe_status check_cfg(const moe_config* c) {
  if (!c) return MOE_EINVAL;
  if (c->hidden <= 0 || c->ffn <= 0 || c->n_experts < 0 || c->top_k < 0) return MOE_EINVAL;
  if (c->n_shared != 0 && c->n_shared != 1) return MOE_EUNSUPPORTED;
  if (c->shared_gate != 0 && c->shared_gate != 1) return MOE_EINVAL;
  if (c->hidden % 256 != 0 || c->hidden > kMaxHidden) return MOE_EUNSUPPORTED;
  if (c->ffn % 128 != 0 || c->ffn > 65536) return MOE_EUNSUPPORTED;
  if (c->codec < MOE_CODEC_IQ4_NL || c->codec > MOE_CODEC_Q3_AFFINE) return MOE_EINVAL;
  if (c->codec != MOE_CODEC_IQ4_NL) {
    // the other codecs run the exact-weight (FP32) kernels only
    if (c->precision != MOE_PREC_AUTO && c->precision != MOE_PREC_FP32) return MOE_EUNSUPPORTED;
    if (c->codec == MOE_CODEC_IQ4_XS && c->ffn % 256 != 0) return MOE_EUNSUPPORTED;  // down rows: 256-weight blocks
  }
  if (c->n_experts > 256) return MOE_EUNSUPPORTED;
  if (c->n_experts == 0) {
    // a dense FFN block: the always-on expert alone, nothing to route or gate
    if (c->top_k != 0 || c->n_shared != 1 || c->shared_gate != 0) return MOE_EUNSUPPORTED;
  } else {
    if (c->top_k == 0) return MOE_EINVAL;
    if (c->top_k > 8 || c->top_k > c->n_experts) return MOE_EUNSUPPORTED;
    if (c->shared_gate && !c->n_shared) return MOE_EUNSUPPORTED;
  }
  if (!isfinite(c->routed_scale)) return MOE_EINVAL;
  if (c->precision < MOE_PREC_AUTO || c->precision > MOE_PREC_W4A8) return MOE_EINVAL;
  return MOE_OK;
}

// AUTO: the exact-weight contract while an expert serves at most 16 routes on
// average (a dense block: its one expert at most 16 tokens), else bf16 tiles.
int resolve_precision(const moe_config* c, int T) {
  if (c->codec != MOE_CODEC_IQ4_NL) return MOE_PREC_FP32;
  if (c->precision != MOE_PREC_AUTO) return c->precision;
  if (c->n_experts == 0) return T <= 16 ? MOE_PREC_FP32 : MOE_PREC_BF16;
  return (int64_t)T * c->top_k <= 16 * (int64_t)c->n_experts ? MOE_PREC_FP32 : MOE_PREC_BF16;
}

// Values per row of the routing weights: K, plus the shared expert's gate.
int weight_cols(const moe_config* c) { return c->top_k + c->shared_gate; }

// Bytes of one expert in the codec's own (input) layout.
int64_t expert_bytes(const moe_config* c) {
  const int64_t w = 3 * (int64_t)c->ffn * c->hidden;
  if (c->codec == MOE_CODEC_IQ4_XS) return w / 256 * 136;
  if (c->codec == MOE_CODEC_Q3_AFFINE) return w / 64 * 28;
  return w / 32 * 18;
}

// Bytes of one expert in the packed layout the kernels read (IQ4_XS repeats a
// super-block's d in both of its tiles).
int64_t packed_expert_bytes(const moe_config* c) {
  if (c->codec == MOE_CODEC_IQ4_NL) return expert_bytes(c);
  return 3 * (int64_t)(c->ffn / 16) * (c->hidden / 128) * qmoe::codec_tile_bytes(c->codec);
}

// Routes per work chunk of the FFN kernels of each contract (W4A8 uses the
// exact-weight kernels' chunks).
int chunk_rows(int precision) { return precision == MOE_PREC_BF16 ? qmoe::kBfRows : 16; }

// Upper bound on the chunks of T tokens: at most one partial chunk per
// non-empty expert beyond the full ones, plus the shared expert's.
int max_chunks(const moe_config* c, int T, int rows) {
  const int64_t R = (int64_t)T * c->top_k;
  const int64_t nonempty = R < c->n_experts ? R : c->n_experts;
  return (int)(R / rows + nonempty + (c->n_shared ? (T + rows - 1) / rows : 0));
}

int max_chunks(const moe_config* c, int T) { return max_chunks(c, T, chunk_rows(resolve_precision(c, T))); }

// The two-launch decode path covers one token with the exact-weight contract.
// Its second kernel hands data between workgroups, so it is taken only when
// the device holds that kernel's whole grid at once.  The shared expert's
// down rows are split over its F/16 gate/up workgroups, at most 4 row tiles
// of 16 each: hidden <= 4 ffn.
bool decode_shape(const moe_config* c) {
  return c->n_experts > 0 && c->codec == MOE_CODEC_IQ4_NL && c->top_k <= qmoe::kMaxDecodeK &&
         c->ffn <= qmoe::kMaxDecodeFfn && (c->n_shared == 0 || c->hidden <= 4 * c->ffn) &&
         c->hidden <= qmoe::kMaxDecodeHidden && resolve_precision(c, 1) == MOE_PREC_FP32;
}

bool decode_path(const moe_config* c, int T) {
  return T == 1 && decode_shape(c) && qmoe::decode_grid_coresident(c->ffn, c->top_k, c->hidden, c->n_shared);
}

// Workspace plan: 256-byte aligned sub-buffers.
struct Plan {
  size_t status;                               // error word of the decode path
  size_t hw;                                   // decode path: h words of one token
  size_t scores, ids, w;                       // router
  size_t counts, offsets, perm, pos, chunks, n_chunks;  // bucketing
  size_t h_hi, h_lo, y;                        // exact-weight FFN
  size_t xq, xd, h32, hq, hd;                  // W4A8: Q8_0 x, fp32 h, Q8_0 h
  size_t total;
};

Plan make_plan(const moe_config* c, int T) {
  const size_t R = (size_t)T * c->top_k, E = c->n_experts, S = c->n_shared ? (size_t)T : 0;
  const size_t H = c->hidden, F = c->ffn;
  Plan p;
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t here = at;
    at += align_up(bytes > 0 ? bytes : 1);
    return here;
  };
  p.status = take(4);
  p.hw = take((size_t)qmoe::hw_words(c->top_k, (int)F, (int)H) * 4);
  p.scores = take((size_t)T * (E + c->shared_gate) * 4);
  p.ids = take(R * 4);
  p.w = take((size_t)T * weight_cols(c) * 4);
  p.counts = take(E * 4);
  p.offsets = take((E + 1) * 4);
  p.perm = take(R * 4);
  p.pos = take(R * 4);
  const size_t nch = (size_t)max_chunks(c, T);
  p.chunks = take(nch * sizeof(qmoe::Chunk));
  p.n_chunks = take(4);
  const int prec = resolve_precision(c, T);
  const bool w4a8 = prec == MOE_PREC_W4A8;
  p.h_hi = take(w4a8 ? 0 : (R + S) * F * 2);  // h (bf16 contract) or its high half (exact contract)
  p.h_lo = take(prec == MOE_PREC_FP32 ? (R + S) * F * 2 : 0);
  p.y = take((R + S) * H * 4);
  p.xq = take(w4a8 ? (size_t)T * H : 0);
  p.xd = take(w4a8 ? (size_t)T * H / 16 : 0);
  p.h32 = take(w4a8 ? (R + S) * F * 4 : 0);
  p.hq = take(w4a8 ? (R + S) * F : 0);
  p.hd = take(w4a8 ? (R + S) * F / 16 : 0);
  p.total = at;
  return p;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

moe_status check_common(const moe_config* cfg, int32_t T) {
  const moe_status s = check_cfg(cfg);
  if (s != MOE_OK) return s;
  if (T < 0 || T > kMaxTokens) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

moe_status need(const void* p) {
  if (!p) return MOE_EINVAL;
  if (!aligned16(p)) return MOE_EALIGN;
  return MOE_OK;
}

moe_status optional_ptr(const void* p) { return (p && !aligned16(p)) ? MOE_EALIGN : MOE_OK; }

#define TRY(expr)                          \
  do {                                     \
    const moe_status _s = (expr);          \
    if (_s != MOE_OK) return _s;           \
  } while (0)

moe_status launched(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  fprintf(stderr, "libmoe: launch failed: %s\n", hipGetErrorString(e));
  return MOE_ELAUNCH;
}

// Arguments of the two-launch decode plan (plain input x).
qmoe::DecodeArgs decode_args(const moe_config* cfg, const void* x_dev, const float* gate_w_dev,
                             const float* sel_bias_dev, const void* arena_dev, const void* shared_dev, float* out_dev,
                             int32_t* ids, float* w, void* ws_dev, const Plan& p) {
  qmoe::DecodeArgs a;
  a.x = static_cast<const uint16_t*>(x_dev);
  a.wg = gate_w_dev;
  a.bias = sel_bias_dev;
  a.arena = static_cast<const uint8_t*>(arena_dev);
  a.shared = static_cast<const uint8_t*>(shared_dev);
  a.expert_bytes = expert_bytes(cfg);
  a.H = cfg->hidden;
  a.F = cfg->ffn;
  a.E = cfg->n_experts;
  a.K = cfg->top_k;
  a.n_shared = cfg->n_shared;
  a.gated = cfg->shared_gate;
  a.scale = cfg->routed_scale;
  a.scores = at<float>(ws_dev, p.scores);
  a.ids = ids;
  a.w = w;
  a.hw = at<uint32_t>(ws_dev, p.hw);
  a.out = out_dev;
  a.err = at<uint32_t>(ws_dev, p.status);
  a.x_prev = nullptr;
  a.out_prev = nullptr;
  a.eps = 0.0f;
  return a;
}

// Expert FFN + combine after validation; ids and w are device pointers.
moe_status run_expert_forward(const moe_config* cfg, int32_t T, const void* x, const int32_t* ids, const float* w,
                              const void* arena, const void* shared, float* out, void* ws, hipStream_t stream) {
  if (T == 0) return MOE_OK;
  const Plan p = make_plan(cfg, T);
  const int H = cfg->hidden, F = cfg->ffn, E = cfg->n_experts, K = cfg->top_k;
  const int prec = resolve_precision(cfg, T);
  TRY(launched(qmoe::launch_bucket(ids, T, K, E, cfg->n_shared, chunk_rows(prec), at<int32_t>(ws, p.counts),
                                   at<int32_t>(ws, p.offsets), at<int32_t>(ws, p.perm), at<int32_t>(ws, p.pos),
                                   at<qmoe::Chunk>(ws, p.chunks), at<int32_t>(ws, p.n_chunks), stream)));
  if (cfg->codec != MOE_CODEC_IQ4_NL)
    return launched(qmoe::launch_ffn_codec(
        cfg->codec, static_cast<const uint16_t*>(x), T, H, F, K, cfg->n_shared, cfg->shared_gate, max_chunks(cfg, T),
        static_cast<const uint8_t*>(arena), static_cast<const uint8_t*>(shared), packed_expert_bytes(cfg),
        at<int32_t>(ws, p.perm), at<int32_t>(ws, p.pos), w, at<qmoe::Chunk>(ws, p.chunks),
        at<int32_t>(ws, p.n_chunks), at<uint16_t>(ws, p.h_hi), at<uint16_t>(ws, p.h_lo), at<float>(ws, p.y), out,
        stream));
  if (prec == MOE_PREC_W4A8)
    return launched(qmoe::launch_ffn_w4a8(
        static_cast<const uint16_t*>(x), T, H, F, K, cfg->n_shared, cfg->shared_gate, max_chunks(cfg, T),
        static_cast<const uint8_t*>(arena), static_cast<const uint8_t*>(shared), packed_expert_bytes(cfg),
        at<int32_t>(ws, p.perm), at<int32_t>(ws, p.pos), w, at<qmoe::Chunk>(ws, p.chunks),
        at<int32_t>(ws, p.n_chunks), at<int8_t>(ws, p.xq), at<uint16_t>(ws, p.xd), at<float>(ws, p.h32),
        at<int8_t>(ws, p.hq), at<uint16_t>(ws, p.hd), at<float>(ws, p.y), out, stream));
  if (prec == MOE_PREC_BF16)
    return launched(qmoe::launch_ffn_bf16(
        static_cast<const uint16_t*>(x), T, H, F, K, cfg->n_shared, cfg->shared_gate, max_chunks(cfg, T),
        static_cast<const uint8_t*>(arena), static_cast<const uint8_t*>(shared), packed_expert_bytes(cfg),
        at<int32_t>(ws, p.perm), at<int32_t>(ws, p.pos), w, at<qmoe::Chunk>(ws, p.chunks),
        at<int32_t>(ws, p.n_chunks), at<uint16_t>(ws, p.h_hi), at<float>(ws, p.y), out, stream));
  return launched(qmoe::launch_ffn_exact(
      static_cast<const uint16_t*>(x), T, H, F, K, cfg->n_shared, cfg->shared_gate, max_chunks(cfg, T),
      static_cast<const uint8_t*>(arena), static_cast<const uint8_t*>(shared), packed_expert_bytes(cfg),
      at<int32_t>(ws, p.perm), at<int32_t>(ws, p.pos), w, at<qmoe::Chunk>(ws, p.chunks), at<int32_t>(ws, p.n_chunks),
      at<uint16_t>(ws, p.h_hi), at<uint16_t>(ws, p.h_lo), at<float>(ws, p.y), out, stream));
}

}  // namespace

MOE_API int moe_abi_version(void) { return MOE_ABI_VERSION; }

MOE_API const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null pointer, bad size or shape)";
    case MOE_EALIGN: return "device pointer not 16-byte aligned";
    case MOE_EWORKSPACE: return "workspace smaller than moe_workspace_bytes()";
    case MOE_EUNSUPPORTED: return "unsupported configuration";
    case MOE_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

MOE_API moe_status moe_check_config(const moe_config* cfg) { return check_cfg(cfg); }

MOE_API size_t moe_expert_bytes(const moe_config* cfg) {
  return check_cfg(cfg) == MOE_OK ? (size_t)expert_bytes(cfg) : 0;
}

MOE_API size_t moe_packed_expert_bytes(const moe_config* cfg) {
  return check_cfg(cfg) == MOE_OK ? (size_t)packed_expert_bytes(cfg) : 0;
}

MOE_API int32_t moe_resolved_precision(const moe_config* cfg, int32_t T) {
  return check_cfg(cfg) == MOE_OK ? resolve_precision(cfg, T) : 0;
}

MOE_API size_t moe_workspace_bytes(const moe_config* cfg, int32_t T) {
  if (check_common(cfg, T) != MOE_OK) return 0;
  return make_plan(cfg, T).total;
}

MOE_API moe_status moe_workspace_init(const moe_config* cfg, int32_t T, void* ws_dev, size_t ws_bytes,
                                      hipStream_t stream) {
  TRY(check_common(cfg, T));
  TRY(need(ws_dev));
  const Plan p = make_plan(cfg, T);
  if (ws_bytes < p.total) return MOE_EWORKSPACE;
  return launched(qmoe::launch_zero_words(at<uint32_t>(ws_dev, p.status), 1, stream));
}

MOE_API moe_status moe_workspace_status(const moe_config* cfg, int32_t T, const void* ws_dev, size_t ws_bytes,
                                        int32_t* status_dev, hipStream_t stream) {
  TRY(check_common(cfg, T));
  TRY(need(ws_dev));
  TRY(need(status_dev));
  const Plan p = make_plan(cfg, T);
  if (ws_bytes < p.total) return MOE_EWORKSPACE;
  return launched(qmoe::launch_copy_words(at<const uint32_t>(const_cast<void*>(ws_dev), p.status),
                                          reinterpret_cast<uint32_t*>(status_dev), 1, stream));
}

MOE_API moe_status moe_pack_experts(const moe_config* cfg, int32_t n_experts, const void* src_dev, void* dst_dev,
                                    hipStream_t stream) {
  TRY(check_cfg(cfg));
  if (n_experts < 0) return MOE_EINVAL;
  if (n_experts == 0) return MOE_OK;
  TRY(need(src_dev));
  TRY(need(dst_dev));
  const char* s = static_cast<const char*>(src_dev);
  const char* d = static_cast<const char*>(dst_dev);
  const int64_t sbytes = (int64_t)n_experts * expert_bytes(cfg), dbytes = (int64_t)n_experts * packed_expert_bytes(cfg);
  if (s < d + dbytes && d < s + sbytes) return MOE_EINVAL;  // overlap
  if (cfg->codec != MOE_CODEC_IQ4_NL)
    return launched(qmoe::launch_pack_codec(cfg->codec, static_cast<const uint8_t*>(src_dev),
                                            static_cast<uint8_t*>(dst_dev), n_experts, cfg->hidden, cfg->ffn,
                                            expert_bytes(cfg), packed_expert_bytes(cfg), stream));
  return launched(qmoe::launch_pack(static_cast<const uint8_t*>(src_dev), static_cast<uint8_t*>(dst_dev), n_experts,
                                    cfg->hidden, cfg->ffn, stream));
}

MOE_API moe_status moe_dequant(const moe_config* cfg, const void* packed_expert_dev, int32_t matrix, int32_t precision,
                               float* out_dev, hipStream_t stream) {
  TRY(check_cfg(cfg));
  if (matrix < 0 || matrix > 2) return MOE_EINVAL;
  if (precision != MOE_PREC_FP32 && precision != MOE_PREC_BF16) return MOE_EINVAL;
  TRY(need(packed_expert_dev));
  TRY(need(out_dev));
  const int64_t mat_bytes = packed_expert_bytes(cfg) / 3;
  const int rows = matrix < 2 ? cfg->ffn : cfg->hidden;
  const int cols = matrix < 2 ? cfg->hidden : cfg->ffn;
  if (cfg->codec != MOE_CODEC_IQ4_NL) {
    if (precision != MOE_PREC_FP32) return MOE_EUNSUPPORTED;
    return launched(qmoe::launch_dequant_codec(cfg->codec, static_cast<const uint8_t*>(packed_expert_dev) +
                                                               matrix * mat_bytes,
                                               rows, cols, out_dev, stream));
  }
  return launched(qmoe::launch_dequant(static_cast<const uint8_t*>(packed_expert_dev) + matrix * mat_bytes, rows,
                                       cols, precision == MOE_PREC_BF16 ? 1 : 0, out_dev, stream));
}

MOE_API moe_status moe_quantize_q8_0(const void* src_dev, int32_t src_bf16, int64_t n, int8_t* q_dev,
                                     uint16_t* d_dev, hipStream_t stream) {
  if (n < 0 || n % 32 != 0 || (src_bf16 != 0 && src_bf16 != 1)) return MOE_EINVAL;
  if (n == 0) return MOE_OK;
  TRY(need(src_dev));
  TRY(need(q_dev));
  TRY(need(d_dev));
  return launched(qmoe::launch_quantize_q8_0(src_dev, src_bf16, n, q_dev, d_dev, stream));
}

MOE_API moe_status moe_stream_read(const void* src_dev, size_t bytes, uint32_t* sink_dev, hipStream_t stream) {
  if (bytes % 16 != 0) return MOE_EINVAL;
  TRY(need(src_dev));
  TRY(need(sink_dev));
  return launched(qmoe::launch_stream_read(src_dev, (int64_t)bytes, sink_dev, stream));
}

MOE_API moe_status moe_residual_rmsnorm(const float* out_dev, const void* x_dev, int32_t T, int32_t H, float eps,
                                        void* y_dev, hipStream_t stream) {
  if (T < 0 || T > kMaxTokens || H <= 0 || H % 256 != 0 || H > kMaxHidden) return MOE_EUNSUPPORTED;
  if (!(eps >= 0.0f) || !isfinite(eps)) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  TRY(need(out_dev));
  TRY(need(x_dev));
  TRY(need(y_dev));
  return launched(qmoe::launch_residual_rmsnorm(out_dev, static_cast<const uint16_t*>(x_dev), T, H, eps,
                                                static_cast<uint16_t*>(y_dev), stream));
}

MOE_API moe_status moe_route(const moe_config* cfg, int32_t T, const void* x_dev, const float* gate_w_dev,
                             const float* sel_bias_dev, int32_t* topk_ids_dev, float* topk_w_dev, void* ws_dev,
                             size_t ws_bytes, hipStream_t stream) {
  TRY(check_common(cfg, T));
  if (cfg->n_experts == 0) return MOE_EINVAL;  // a dense block has nothing to route
  if (T == 0) return MOE_OK;  // nothing to read or write
  TRY(need(x_dev));
  TRY(need(gate_w_dev));
  TRY(optional_ptr(sel_bias_dev));
  TRY(need(topk_ids_dev));
  TRY(need(topk_w_dev));
  TRY(need(ws_dev));
  const Plan p = make_plan(cfg, T);
  if (ws_bytes < p.total) return MOE_EWORKSPACE;
  return launched(qmoe::launch_router(static_cast<const uint16_t*>(x_dev), gate_w_dev, sel_bias_dev, T, cfg->hidden,
                                      cfg->n_experts, cfg->top_k, cfg->shared_gate, cfg->routed_scale,
                                      at<float>(ws_dev, p.scores), topk_ids_dev, topk_w_dev, stream));
}

MOE_API moe_status moe_router_scores(const moe_config* cfg, int32_t T, const void* x_dev, const float* gate_w_dev,
                                     float* scores_dev, hipStream_t stream) {
  TRY(check_common(cfg, T));
  if (cfg->n_experts == 0) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  TRY(need(x_dev));
  TRY(need(gate_w_dev));
  TRY(need(scores_dev));
  return launched(qmoe::launch_router_scores(static_cast<const uint16_t*>(x_dev), gate_w_dev, T, cfg->hidden,
                                             cfg->n_experts + cfg->shared_gate, scores_dev, stream));
}

MOE_API moe_status moe_bucket(const moe_config* cfg, int32_t T, const int32_t* topk_ids_dev, int32_t* counts_dev,
                              int32_t* offsets_dev, int32_t* perm_dev, int32_t* pos_dev, hipStream_t stream) {
  TRY(check_common(cfg, T));
  if (cfg->n_experts == 0) return MOE_EINVAL;
  TRY(need(counts_dev));
  TRY(need(offsets_dev));
  if (T > 0) {  // with no routes only the (all-zero) counts and offsets are written
    TRY(need(topk_ids_dev));
    TRY(need(perm_dev));
    TRY(optional_ptr(pos_dev));
  }
  return launched(qmoe::launch_bucket(topk_ids_dev, T, cfg->top_k, cfg->n_experts, cfg->n_shared, 16, counts_dev,
                                      offsets_dev, perm_dev, pos_dev, nullptr, nullptr, stream));
}

MOE_API moe_status moe_expert_forward(const moe_config* cfg, int32_t T, const void* x_dev, const int32_t* topk_ids_dev,
                                      const float* topk_w_dev, const void* arena_dev, const void* shared_dev,
                                      float* out_dev, void* ws_dev, size_t ws_bytes, hipStream_t stream) {
  TRY(check_common(cfg, T));
  if (T == 0) return MOE_OK;  // nothing to read or write
  TRY(need(x_dev));
  if (cfg->n_experts > 0) {  // a dense block reads no routing and no routed arena
    TRY(need(topk_ids_dev));
    TRY(need(topk_w_dev));
    TRY(need(arena_dev));
  }
  if (cfg->n_shared) TRY(need(shared_dev));
  TRY(need(out_dev));
  TRY(need(ws_dev));
  if (ws_bytes < make_plan(cfg, T).total) return MOE_EWORKSPACE;
  return run_expert_forward(cfg, T, x_dev, topk_ids_dev, topk_w_dev, arena_dev, shared_dev, out_dev, ws_dev, stream);
}

namespace {

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const char* p = static_cast<const char*>(a);
  const char* q = static_cast<const char*>(b);
  return p < q + nb && q < p + na;
}

}  // namespace

// ---- the stack kernel

namespace {

// Workspace of moe_stack_decode: the decode plan's workspace of one token
// (scores, hand-off words, status word), which every layer reuses, then the
// routing outputs of every layer for a caller that passes none.
struct StackPlan {
  Plan dec;
  size_t ids, w, total;
};

StackPlan make_stack_plan(const moe_config* c, int L) {
  StackPlan p;
  p.dec = make_plan(c, 1);
  size_t off = align_up(p.dec.total);
  p.ids = off;
  off += align_up((size_t)L * c->top_k * 4);
  p.w = off;
  off += align_up((size_t)L * weight_cols(c) * 4);
  p.total = off;
  return p;
}

// The shapes of the decode plan (the device check comes in moe_stack_decode).
moe_status check_stack(const moe_config* cfg, int32_t L) {
  TRY(check_common(cfg, 1));
  if (L < 1 || L > qmoe::kMaxStackLayers) return MOE_EUNSUPPORTED;
  if (!decode_shape(cfg)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

}  // namespace

MOE_API moe_status moe_stack_workspace_bytes(const moe_config* cfg, int32_t L, size_t* bytes) {
  if (!bytes) return MOE_EINVAL;
  TRY(check_stack(cfg, L));
  *bytes = make_stack_plan(cfg, L).total;
  return MOE_OK;
}

MOE_API moe_status moe_stack_decode(const moe_config* cfg, int32_t L, const moe_stack_layer* layers_host,
                                    const void* x0_dev, float eps, void* x_all_dev, float* out_all_dev,
                                    int32_t* ids_all_dev, float* w_all_dev, void* ws_dev, size_t ws_bytes,
                                    hipStream_t stream) {
  TRY(check_stack(cfg, L));
  if (!(eps >= 0.0f) || !isfinite(eps)) return MOE_EINVAL;
  if (!layers_host) return MOE_EINVAL;
  for (int l = 0; l < L; l++) {
    TRY(need(layers_host[l].gate_w));
    TRY(optional_ptr(layers_host[l].sel_bias));
    TRY(need(layers_host[l].arena));
    if (cfg->n_shared) TRY(need(layers_host[l].shared));
    else TRY(optional_ptr(layers_host[l].shared));
  }
  TRY(need(x0_dev));
  TRY(need(x_all_dev));
  TRY(need(out_all_dev));
  TRY(optional_ptr(ids_all_dev));
  TRY(optional_ptr(w_all_dev));
  TRY(need(ws_dev));
  const size_t H = cfg->hidden;
  if (overlaps(x_all_dev, (size_t)L * H * 2, x0_dev, H * 2) ||
      overlaps(out_all_dev, (size_t)L * H * 4, x0_dev, H * 2) ||
      overlaps(out_all_dev, (size_t)L * H * 4, x_all_dev, (size_t)L * H * 2))
    return MOE_EINVAL;
  const StackPlan sp = make_stack_plan(cfg, L);
  if (ws_bytes < sp.total) return MOE_EWORKSPACE;
  if (overlaps(ws_dev, sp.total, out_all_dev, (size_t)L * H * 4) || overlaps(ws_dev, sp.total, x_all_dev, (size_t)L * H * 2))
    return MOE_EINVAL;
  if (!qmoe::decode_grid_coresident(cfg->ffn, cfg->top_k, cfg->hidden, cfg->n_shared)) return MOE_EUNSUPPORTED;

  // Per layer the decode plan's two launches, the layer's input formed in the
  // first (as moe_layer_forward_chained); layer 0 reads x0, copies it to row 0
  // of x_all and clears the give-up word.
  int32_t* ids_all = ids_all_dev ? ids_all_dev : at<int32_t>(ws_dev, sp.ids);
  float* w_all = w_all_dev ? w_all_dev : at<float>(ws_dev, sp.w);
  uint16_t* x_all = static_cast<uint16_t*>(x_all_dev);
  const int WK = weight_cols(cfg);
  for (int l = 0; l < L; l++) {
    const moe_stack_layer& ly = layers_host[l];
    qmoe::DecodeArgs a = decode_args(cfg, l == 0 ? x0_dev : x_all + (size_t)l * H, ly.gate_w, ly.sel_bias, ly.arena,
                                     ly.shared, out_all_dev + (size_t)l * H, ids_all + (size_t)l * cfg->top_k,
                                     w_all + (size_t)l * WK, ws_dev, sp.dec);
    if (l == 0) {
      a.x_copy = x_all;
      a.zero_err = 1;
    } else {
      a.x_prev = x_all + (size_t)(l - 1) * H;
      a.out_prev = out_all_dev + (size_t)(l - 1) * H;
      a.eps = eps;
    }
    TRY(launched(qmoe::launch_layer_decode(a, stream)));
  }
  return MOE_OK;
}

MOE_API moe_status moe_stack_status(const moe_config* cfg, int32_t L, const void* ws_dev, size_t ws_bytes,
                                    int32_t* status_dev, hipStream_t stream) {
  TRY(check_stack(cfg, L));
  TRY(need(ws_dev));
  TRY(need(status_dev));
  const StackPlan sp = make_stack_plan(cfg, L);
  if (ws_bytes < sp.total) return MOE_EWORKSPACE;
  return launched(qmoe::launch_copy_words(at<const uint32_t>(const_cast<void*>(ws_dev), sp.dec.status),
                                          reinterpret_cast<uint32_t*>(status_dev), 1, stream));
}

MOE_API moe_status moe_layer_forward_chained(const moe_config* cfg, int32_t T, const void* x_prev_dev,
                                             const float* out_prev_dev, float eps, void* x_dev,
                                             const float* gate_w_dev, const float* sel_bias_dev,
                                             const void* arena_dev, const void* shared_dev, float* out_dev,
                                             int32_t* topk_ids_out_dev, float* topk_w_out_dev, void* ws_dev,
                                             size_t ws_bytes, hipStream_t stream) {
  TRY(check_common(cfg, T));
  if (!(eps >= 0.0f) || !isfinite(eps)) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  TRY(need(x_prev_dev));
  TRY(need(out_prev_dev));
  TRY(need(x_dev));
  const size_t xb = (size_t)T * cfg->hidden * 2;
  if (overlaps(x_dev, xb, x_prev_dev, xb) || overlaps(x_dev, xb, out_prev_dev, 2 * xb)) return MOE_EINVAL;
  if (cfg->n_experts > 0) {
    TRY(need(gate_w_dev));
    TRY(optional_ptr(sel_bias_dev));
    TRY(need(arena_dev));
  }
  if (cfg->n_shared) TRY(need(shared_dev));
  TRY(need(out_dev));
  TRY(optional_ptr(topk_ids_out_dev));
  TRY(optional_ptr(topk_w_out_dev));
  TRY(need(ws_dev));
  const Plan p = make_plan(cfg, T);
  if (ws_bytes < p.total) return MOE_EWORKSPACE;
  if (decode_path(cfg, T)) {
    qmoe::DecodeArgs a = decode_args(cfg, x_dev, gate_w_dev, sel_bias_dev, arena_dev, shared_dev, out_dev,
                                     topk_ids_out_dev ? topk_ids_out_dev : at<int32_t>(ws_dev, p.ids),
                                     topk_w_out_dev ? topk_w_out_dev : at<float>(ws_dev, p.w), ws_dev, p);
    a.x_prev = static_cast<const uint16_t*>(x_prev_dev);
    a.out_prev = out_prev_dev;
    a.eps = eps;
    return launched(qmoe::launch_layer_decode(a, stream));
  }
  TRY(launched(qmoe::launch_residual_rmsnorm(out_prev_dev, static_cast<const uint16_t*>(x_prev_dev), T, cfg->hidden,
                                             eps, static_cast<uint16_t*>(x_dev), stream)));
  return moe_layer_forward(cfg, T, x_dev, gate_w_dev, sel_bias_dev, arena_dev, shared_dev, out_dev, topk_ids_out_dev,
                           topk_w_out_dev, ws_dev, ws_bytes, stream);
}

MOE_API moe_status moe_layer_forward(const moe_config* cfg, int32_t T, const void* x_dev, const float* gate_w_dev,
                                     const float* sel_bias_dev, const void* arena_dev, const void* shared_dev,
                                     float* out_dev, int32_t* topk_ids_out_dev, float* topk_w_out_dev, void* ws_dev,
                                     size_t ws_bytes, hipStream_t stream) {
  TRY(check_common(cfg, T));
  if (T == 0) return MOE_OK;  // nothing to read or write
  const bool dense = cfg->n_experts == 0;
  TRY(need(x_dev));
  if (!dense) {
    TRY(need(gate_w_dev));
    TRY(optional_ptr(sel_bias_dev));
    TRY(need(arena_dev));
  }
  if (cfg->n_shared) TRY(need(shared_dev));
  TRY(need(out_dev));
  TRY(optional_ptr(topk_ids_out_dev));
  TRY(optional_ptr(topk_w_out_dev));
  TRY(need(ws_dev));
  const Plan p = make_plan(cfg, T);
  if (ws_bytes < p.total) return MOE_EWORKSPACE;
  if (dense)
    return run_expert_forward(cfg, T, x_dev, nullptr, nullptr, nullptr, shared_dev, out_dev, ws_dev, stream);
  int32_t* ids = topk_ids_out_dev ? topk_ids_out_dev : at<int32_t>(ws_dev, p.ids);
  float* w = topk_w_out_dev ? topk_w_out_dev : at<float>(ws_dev, p.w);
  if (decode_path(cfg, T))
    return launched(qmoe::launch_layer_decode(
        decode_args(cfg, x_dev, gate_w_dev, sel_bias_dev, arena_dev, shared_dev, out_dev, ids, w, ws_dev, p), stream));
  TRY(launched(qmoe::launch_router(static_cast<const uint16_t*>(x_dev), gate_w_dev, sel_bias_dev, T, cfg->hidden,
                                   cfg->n_experts, cfg->top_k, cfg->shared_gate, cfg->routed_scale,
                                   at<float>(ws_dev, p.scores), ids, w, stream)));
  return run_expert_forward(cfg, T, x_dev, ids, w, arena_dev, shared_dev, out_dev, ws_dev, stream);
}
