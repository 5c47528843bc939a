// Host side of the C ABI declared in include/flint_moe.h: argument checks,
// workspace carve-up and kernel dispatch.  No allocation, no host sync.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "common.hpp"
#include "prefill_ws.hpp"

namespace flint {

namespace {

constexpr int64_t kAlign = 256;

inline int64_t align_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Checks common to decode and prefill; returns FLINT_OK or an error code.
int check_shape(const flint_moe_shape* s) {
  if (!s) return FLINT_ERR_INVALID_ARG;
  if (s->hidden <= 0 || s->n_experts <= 0 || s->inter <= 0 || s->shared_inter < 0 || s->top_k <= 0)
    return FLINT_ERR_INVALID_ARG;
  if (s->hidden % 64 || s->inter % 64 || s->shared_inter % 64) return FLINT_ERR_UNSUPPORTED;
  if (s->hidden > 4096) return FLINT_ERR_UNSUPPORTED;
  if (s->n_experts > FLINT_MAX_EXPERTS) return FLINT_ERR_UNSUPPORTED;
  if (s->top_k > FLINT_MAX_TOP_K || s->top_k > s->n_experts) return FLINT_ERR_UNSUPPORTED;
  if (s->flags & ~(FLINT_RENORM | FLINT_W_BF16 | FLINT_PRE_RMSNORM | FLINT_RESIDUAL | FLINT_SPLIT))
    return FLINT_ERR_UNSUPPORTED;
  if ((s->flags & FLINT_PRE_RMSNORM) && !(s->rms_eps >= 0.0f)) return FLINT_ERR_INVALID_ARG;
  return FLINT_OK;
}

#define FLINT_NEED(p)                      \
  do {                                     \
    if (!(p)) return FLINT_ERR_INVALID_ARG; \
    if (!aligned16(p)) return FLINT_ERR_ALIGNMENT; \
  } while (0)

int check_weights(const flint_moe_shape* s, const flint_moe_weights* w) {
  if (!w) return FLINT_ERR_INVALID_ARG;
  FLINT_NEED(w->router);
  const bool sh = s->shared_inter > 0;
  if (s->flags & FLINT_W_BF16) {
    FLINT_NEED(w->gu_bf16);
    FLINT_NEED(w->d_bf16);
    if (sh) {
      FLINT_NEED(w->sh_gu_bf16);
      FLINT_NEED(w->sh_d_bf16);
    }
  } else {
    FLINT_NEED(w->gu_codes);
    FLINT_NEED(w->gu_scales);
    FLINT_NEED(w->d_codes);
    FLINT_NEED(w->d_scales);
    FLINT_NEED(w->gscale);
    if (sh) {
      FLINT_NEED(w->sh_gu_codes);
      FLINT_NEED(w->sh_gu_scales);
      FLINT_NEED(w->sh_d_codes);
      FLINT_NEED(w->sh_d_scales);
      FLINT_NEED(w->sh_gscale);
    }
  }
  return FLINT_OK;
}

LayerArgs make_args(const flint_moe_shape* s, const flint_moe_weights* w, const void* x, int batch,
                    void* out, const void* gamma) {
  LayerArgs a;
  std::memset(&a, 0, sizeof(a));
  a.H = s->hidden; a.E = s->n_experts; a.I = s->inter; a.SI = s->shared_inter;
  a.K = s->top_k; a.B = batch; a.flags = s->flags; a.eps = s->rms_eps;
  a.router = static_cast<const uint16_t*>(w->router);
  a.gu_codes = static_cast<const uint8_t*>(w->gu_codes);
  a.gu_scales = static_cast<const uint8_t*>(w->gu_scales);
  a.d_codes = static_cast<const uint8_t*>(w->d_codes);
  a.d_scales = static_cast<const uint8_t*>(w->d_scales);
  a.gscale = w->gscale;
  a.sh_gu_codes = static_cast<const uint8_t*>(w->sh_gu_codes);
  a.sh_gu_scales = static_cast<const uint8_t*>(w->sh_gu_scales);
  a.sh_d_codes = static_cast<const uint8_t*>(w->sh_d_codes);
  a.sh_d_scales = static_cast<const uint8_t*>(w->sh_d_scales);
  a.sh_gscale = w->sh_gscale;
  a.gu_bf16 = static_cast<const uint16_t*>(w->gu_bf16);
  a.d_bf16 = static_cast<const uint16_t*>(w->d_bf16);
  a.sh_gu_bf16 = static_cast<const uint16_t*>(w->sh_gu_bf16);
  a.sh_d_bf16 = static_cast<const uint16_t*>(w->sh_d_bf16);
  a.x = static_cast<const uint16_t*>(x);
  a.gamma = static_cast<const uint16_t*>(gamma);
  a.out = static_cast<uint16_t*>(out);
  return a;
}

int to_status(hipError_t e) { return e == hipSuccess ? FLINT_OK : FLINT_ERR_DEVICE; }

}  // namespace

int decode_max_slots(const flint_moe_shape& s, int batch);

int64_t prefill_ws_bytes(const flint_moe_shape& s, int T) {
  return carve_prefill_ws(nullptr, s, T).bytes;
}

int64_t decode_ws_bytes(const flint_moe_shape& s, int max_batch) {
  DecodeWs ws = carve_decode_ws(nullptr, s, max_batch);
  return ws.bytes;
}

DecodeWs carve_decode_ws(void* base, const flint_moe_shape& s, int max_batch) {
  const int B = FLINT_MAX_DECODE_BATCH;
  (void)max_batch;   // the layout always holds 8 tokens, so one workspace serves any batch
  const int S = decode_max_slots(s, B);
  const int imax = s.inter > s.shared_inter ? s.inter : s.shared_inter;
  char* b = static_cast<char*>(base);
  int64_t off = 0;
  DecodeWs w;
  auto take = [&](int64_t bytes) {
    char* p = b ? b + off : nullptr;
    off = align_up(off + bytes);
    return p;
  };
  // the header: four words, 256 bytes apart (offsets fixed in the ABI)
  w.ticket = reinterpret_cast<uint32_t*>(take(4));
  w.epoch = reinterpret_cast<uint32_t*>(take(4));
  w.error = reinterpret_cast<uint32_t*>(take(4));
  w.wait_limit = reinterpret_cast<uint32_t*>(take(4));
  static_assert(FLINT_WS_ERROR_OFFSET == 2 * kAlign && FLINT_WS_WAIT_LIMIT_OFFSET == 3 * kAlign &&
                    FLINT_WS_HEADER_BYTES == 4 * kAlign,
                "workspace header offsets");
  // the single-launch path's logit words, [replicas][E] (its readers each
  // take their own copy; the three-kernel path uses the first [B][E]),
  // then one arrival word per workgroup beyond E, at most 256
  w.logit_words = reinterpret_cast<uint64_t*>(take(((int64_t)8 * B * s.n_experts + 256) * 8));
  w.xn = reinterpret_cast<uint16_t*>(take((int64_t)B * s.hidden * 2));
  w.idx = reinterpret_cast<int32_t*>(take((int64_t)B * FLINT_MAX_TOP_K * 4));
  w.wgt = reinterpret_cast<float*>(take((int64_t)B * FLINT_MAX_TOP_K * 4));
  w.nslot = reinterpret_cast<int32_t*>(take(4));
  w.slot_expert = reinterpret_cast<int32_t*>(take((int64_t)S * 4));
  w.slot_mask = reinterpret_cast<uint32_t*>(take((int64_t)S * 4));
  w.slot_w = reinterpret_cast<float*>(take((int64_t)S * B * 4));
  w.h_words = reinterpret_cast<uint64_t*>(take((int64_t)8 * (FLINT_MAX_TOP_K + 1) * (imax / 2) * 8));
  w.x_words = reinterpret_cast<uint64_t*>(take((int64_t)8 * (s.hidden / 2) * 8));
  w.h = reinterpret_cast<uint16_t*>(take((int64_t)S * B * imax * 2));
  // the batch single launch's routed h words and partial sums (Flint shape only)
  w.hb_words = w.p_words = nullptr;
  if (flint_b8_shape(s)) {
    const int routed = S - (s.shared_inter > 0 ? 1 : 0);
    w.hb_words = reinterpret_cast<uint64_t*>(take((int64_t)routed * B * (imax / 2) * 8));
    w.p_words = reinterpret_cast<uint64_t*>(take((int64_t)B * (FLINT_MAX_TOP_K + 1) * s.hidden * 8));
  }
  w.bytes = off;
  return w;
}

}  // namespace flint

namespace flint {
int32_t decode_common(int32_t stage, const flint_moe_shape* shape, const flint_moe_weights* weights,
                      const void* x, int32_t batch, void* out, int32_t* topk_idx, float* topk_w,
                      const void* gamma, void* ws, int64_t ws_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != FLINT_OK) return st;
  st = check_weights(shape, weights);
  if (st != FLINT_OK) return st;
  if (batch <= 0) return FLINT_ERR_INVALID_ARG;
  if (batch > FLINT_MAX_DECODE_BATCH) return FLINT_ERR_UNSUPPORTED;
  if (stage < -1 || stage > 2) return FLINT_ERR_INVALID_ARG;
  FLINT_NEED(x);
  FLINT_NEED(out);
  if (out == x && !(shape->flags & FLINT_RESIDUAL)) return FLINT_ERR_INVALID_ARG;
  if (shape->flags & FLINT_PRE_RMSNORM) FLINT_NEED(gamma);
  if (topk_idx && !aligned4(topk_idx)) return FLINT_ERR_ALIGNMENT;
  if (topk_w && !aligned4(topk_w)) return FLINT_ERR_ALIGNMENT;
  if (!ws) return FLINT_ERR_WORKSPACE;
  if (!aligned16(ws)) return FLINT_ERR_ALIGNMENT;
  const int64_t need = decode_ws_bytes(*shape, FLINT_MAX_DECODE_BATCH);
  if (ws_bytes < need) return FLINT_ERR_WORKSPACE;

  DecodeWs w = carve_decode_ws(ws, *shape, FLINT_MAX_DECODE_BATCH);
  LayerArgs a = make_args(shape, weights, x, batch, out, gamma);
  a.topk_idx = topk_idx ? topk_idx : w.idx;
  a.topk_w = topk_w ? topk_w : w.wgt;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (stage < 0 && !(shape->flags & FLINT_SPLIT)) {
    if (flint_b1_supported(a)) return to_status(launch_flint_b1(a, w, s));
    if (flint_b8_supported(a)) return to_status(launch_flint_b8(a, w, s));
    if (fused_decode_supported(a)) return to_status(launch_fused_decode(a, w, s));
  }
  if (stage < 0 || stage == 0) e = launch_route(a, w, s);
  if (e == hipSuccess && (stage < 0 || stage == 1)) e = launch_gate_up(a, w, false, false, s);
  if (e == hipSuccess && (stage < 0 || stage == 2)) e = launch_down(a, w, false, 0, nullptr, nullptr, s);
  return to_status(e);
}
}  // namespace flint

using namespace flint;

extern "C" {

const char* flint_version(void) { return "flint-moe 0.1.0 (gfx950)"; }

const char* flint_status_string(int32_t st) {
  switch (st) {
    case FLINT_OK: return "ok";
    case FLINT_ERR_INVALID_ARG: return "invalid argument";
    case FLINT_ERR_ALIGNMENT: return "device pointer not 16-byte aligned";
    case FLINT_ERR_UNSUPPORTED: return "unsupported shape, batch or flags";
    case FLINT_ERR_WORKSPACE: return "workspace missing or too small";
    case FLINT_ERR_DEVICE: return "HIP launch error";
    default: return "unknown";
  }
}

int32_t flint_nvfp4_packed_bytes(int64_t n_mats, int64_t rows, int64_t cols, int64_t* code_bytes,
                                 int64_t* scale_bytes) {
  if (!code_bytes || !scale_bytes || n_mats <= 0 || rows <= 0 || cols <= 0)
    return FLINT_ERR_INVALID_ARG;
  if (cols % 64) return FLINT_ERR_UNSUPPORTED;
  *code_bytes = n_mats * rows * cols / 2;
  *scale_bytes = n_mats * rows * cols / 16;
  return FLINT_OK;
}

int64_t flint_moe_workspace_bytes(const flint_moe_shape* shape, int32_t max_tokens) {
  const int st = check_shape(shape);
  if (st != FLINT_OK) return -(int64_t)st;
  if (max_tokens <= 0) return -(int64_t)FLINT_ERR_INVALID_ARG;
  // the decode layout first (its launch counters and hand-off words), the
  // prefill layout after it, so the two never overlap
  return decode_ws_bytes(*shape, FLINT_MAX_DECODE_BATCH) + prefill_ws_bytes(*shape, max_tokens);
}

int32_t flint_moe_workspace_error(const void* ws, int64_t ws_bytes, uint32_t* dst, void* stream) {
  if (!ws || !dst) return FLINT_ERR_INVALID_ARG;
  if (!aligned16(ws)) return FLINT_ERR_ALIGNMENT;
  if (!aligned4(dst)) return FLINT_ERR_ALIGNMENT;
  if (ws_bytes < FLINT_WS_HEADER_BYTES) return FLINT_ERR_WORKSPACE;
  return to_status(hipMemcpyAsync(dst, static_cast<const char*>(ws) + FLINT_WS_ERROR_OFFSET, 4,
                                  hipMemcpyDefault, static_cast<hipStream_t>(stream)));
}

int32_t flint_moe_repack(const void* src, int64_t n_mats, int32_t rows, int32_t cols,
                         int32_t src_layout, void* dst_codes, void* dst_scales,
                         int64_t dst_mat_stride, void* stream) {
  if (n_mats <= 0 || rows <= 0 || cols <= 0 || dst_mat_stride <= 0) return FLINT_ERR_INVALID_ARG;
  if (cols % 64) return FLINT_ERR_UNSUPPORTED;
  if (src_layout != FLINT_SRC_INTERLEAVED && src_layout != FLINT_SRC_SCALES_FIRST)
    return FLINT_ERR_UNSUPPORTED;
  FLINT_NEED(src);
  FLINT_NEED(dst_codes);
  FLINT_NEED(dst_scales);
  return to_status(launch_repack(static_cast<const uint8_t*>(src), n_mats, rows, cols, src_layout,
                                 static_cast<uint8_t*>(dst_codes),
                                 static_cast<uint8_t*>(dst_scales), dst_mat_stride,
                                 static_cast<hipStream_t>(stream)));
}

int32_t flint_moe_unpack(const void* codes, const void* scales, int64_t n_mats, int32_t rows,
                         int32_t cols, int32_t src_layout, int64_t src_mat_stride, void* dst,
                         void* stream) {
  if (n_mats <= 0 || rows <= 0 || cols <= 0 || src_mat_stride <= 0) return FLINT_ERR_INVALID_ARG;
  if (cols % 64) return FLINT_ERR_UNSUPPORTED;
  if (src_layout != FLINT_SRC_INTERLEAVED && src_layout != FLINT_SRC_SCALES_FIRST)
    return FLINT_ERR_UNSUPPORTED;
  FLINT_NEED(codes);
  FLINT_NEED(scales);
  FLINT_NEED(dst);
  return to_status(launch_unpack(static_cast<const uint8_t*>(codes),
                                 static_cast<const uint8_t*>(scales), n_mats, rows, cols,
                                 src_layout, src_mat_stride, static_cast<uint8_t*>(dst),
                                 static_cast<hipStream_t>(stream)));
}

int32_t flint_nvfp4_dequant(const void* codes, const void* scales, int64_t n_mats, int32_t rows,
                            int32_t cols, const float* tensor_scale, float* out, void* stream) {
  if (n_mats <= 0 || rows <= 0 || cols <= 0) return FLINT_ERR_INVALID_ARG;
  if (cols % 64) return FLINT_ERR_UNSUPPORTED;
  FLINT_NEED(codes);
  FLINT_NEED(scales);
  FLINT_NEED(out);
  if (tensor_scale && !aligned16(tensor_scale)) return FLINT_ERR_ALIGNMENT;
  return to_status(launch_dequant(static_cast<const uint8_t*>(codes),
                                  static_cast<const uint8_t*>(scales), n_mats, rows, cols,
                                  tensor_scale, out, static_cast<hipStream_t>(stream)));
}


int32_t flint_moe_decode(const flint_moe_shape* shape, const flint_moe_weights* weights,
                         const void* x, int32_t batch, void* out, int32_t* topk_idx,
                         float* topk_w, const void* gamma, void* ws, int64_t ws_bytes,
                         void* stream) {
  return decode_common(-1, shape, weights, x, batch, out, topk_idx, topk_w, gamma, ws, ws_bytes,
                       stream);
}

int32_t flint_moe_decode_stack(const flint_moe_shape* shape, const flint_moe_weights* layers,
                               int32_t n_layers, const void* gammas, const void* x, void* out,
                               int32_t* topk_idx, float* topk_w, void* layer_out, void* ws,
                               int64_t ws_bytes, void* stream) {
  const int st = check_shape(shape);
  if (st != FLINT_OK) return st;
  if (shape->flags & ~FLINT_RENORM) return FLINT_ERR_UNSUPPORTED;
  if (n_layers <= 0) return FLINT_ERR_INVALID_ARG;
  if (n_layers > FLINT_MAX_STACK_LAYERS) return FLINT_ERR_UNSUPPORTED;
  FLINT_NEED(layers);
  FLINT_NEED(gammas);
  FLINT_NEED(x);
  FLINT_NEED(out);
  if (!topk_idx || !topk_w) return FLINT_ERR_INVALID_ARG;
  if (!aligned4(topk_idx) || !aligned4(topk_w)) return FLINT_ERR_ALIGNMENT;
  if (layer_out && !aligned16(layer_out)) return FLINT_ERR_ALIGNMENT;
  if (!ws) return FLINT_ERR_WORKSPACE;
  if (!aligned16(ws)) return FLINT_ERR_ALIGNMENT;
  if (ws_bytes < decode_ws_bytes(*shape, FLINT_MAX_DECODE_BATCH)) return FLINT_ERR_WORKSPACE;
  DecodeWs w = carve_decode_ws(ws, *shape, FLINT_MAX_DECODE_BATCH);
  StackArgs sa;
  std::memset(&sa, 0, sizeof(sa));
  LayerArgs& a = sa.base;
  a.H = shape->hidden; a.E = shape->n_experts; a.I = shape->inter; a.SI = shape->shared_inter;
  a.K = shape->top_k; a.B = 1; a.eps = shape->rms_eps;
  a.flags = shape->flags | FLINT_PRE_RMSNORM | FLINT_RESIDUAL;
  const bool flint = !(a.flags & FLINT_W_BF16) && flint_b1_supported(a);   // the stack reads NVFP4 planes
  if (!flint && !fused_stack_supported(a)) return FLINT_ERR_UNSUPPORTED;
  sa.layers = layers;
  sa.gammas = static_cast<const uint16_t*>(gammas);
  sa.x_in = static_cast<const uint16_t*>(x);
  sa.x_out = static_cast<uint16_t*>(out);
  sa.topk_idx = topk_idx;
  sa.topk_w = topk_w;
  sa.layer_out = static_cast<uint16_t*>(layer_out);
  sa.L = n_layers;
  return to_status(flint ? launch_flint_stack(sa, w, static_cast<hipStream_t>(stream))
                         : launch_fused_stack(sa, w, static_cast<hipStream_t>(stream)));
}

int32_t flint_moe_decode_stage(int32_t stage, const flint_moe_shape* shape,
                               const flint_moe_weights* weights, const void* x, int32_t batch,
                               void* out, int32_t* topk_idx, float* topk_w, const void* gamma,
                               void* ws, int64_t ws_bytes, void* stream) {
  if (stage < 0 || stage > 2) return FLINT_ERR_INVALID_ARG;
  return decode_common(stage, shape, weights, x, batch, out, topk_idx, topk_w, gamma, ws, ws_bytes,
                       stream);
}

int32_t flint_moe_decode_path(const flint_moe_shape* shape, int32_t batch) {
  const int st = check_shape(shape);
  if (st != FLINT_OK) return -st;
  if (batch < 1 || batch > FLINT_MAX_DECODE_BATCH) return -FLINT_ERR_UNSUPPORTED;
  if (shape->flags & FLINT_SPLIT) return FLINT_PATH_SPLIT;
  LayerArgs a;
  std::memset(&a, 0, sizeof(a));
  a.H = shape->hidden; a.E = shape->n_experts; a.I = shape->inter; a.SI = shape->shared_inter;
  a.K = shape->top_k; a.B = batch; a.flags = shape->flags; a.eps = shape->rms_eps;
  if (flint_b1_supported(a) || fused_decode_supported(a)) return FLINT_PATH_SINGLE_ONE;
  if (flint_b8_supported(a)) return FLINT_PATH_SINGLE_BATCH;
  return FLINT_PATH_SPLIT;
}

int32_t flint_moe_prefill(const flint_moe_shape* shape, const flint_moe_weights* weights,
                          const void* x, int32_t n_tokens, void* out, int32_t* topk_idx,
                          float* topk_w, const void* gamma, void* ws, int64_t ws_bytes,
                          void* stream) {
  return flint_moe_prefill_tiled(shape, weights, nullptr, x, n_tokens, out, topk_idx, topk_w, gamma, ws,
                                 ws_bytes, stream);
}

int32_t flint_moe_prefill_tiled(const flint_moe_shape* shape, const flint_moe_weights* weights,
                                const flint_moe_prefill_planes* planes, const void* x, int32_t n_tokens,
                                void* out, int32_t* topk_idx, float* topk_w, const void* gamma, void* ws,
                                int64_t ws_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != FLINT_OK) return st;
  st = check_weights(shape, weights);
  if (st != FLINT_OK) return st;
  if (planes) {
    const bool sh = shape->shared_inter > 0;
    const void* c[4] = {planes->gu_codes, planes->d_codes, sh ? planes->sh_gu_codes : nullptr,
                        sh ? planes->sh_d_codes : nullptr};
    const void* sc[4] = {planes->gu_scales, planes->d_scales, sh ? planes->sh_gu_scales : nullptr,
                         sh ? planes->sh_d_scales : nullptr};
    for (int i = 0; i < (sh ? 4 : 2); ++i) {
      FLINT_NEED(c[i]);
      FLINT_NEED(sc[i]);
    }
  }
  if (n_tokens <= 0) return FLINT_ERR_INVALID_ARG;
  if (n_tokens > (1 << 22)) return FLINT_ERR_UNSUPPORTED;
  FLINT_NEED(x);
  FLINT_NEED(out);
  if (out == x && !(shape->flags & FLINT_RESIDUAL)) return FLINT_ERR_INVALID_ARG;
  if (shape->flags & FLINT_PRE_RMSNORM) FLINT_NEED(gamma);
  if (topk_idx && !aligned4(topk_idx)) return FLINT_ERR_ALIGNMENT;
  if (topk_w && !aligned4(topk_w)) return FLINT_ERR_ALIGNMENT;
  if (!ws) return FLINT_ERR_WORKSPACE;
  if (!aligned16(ws)) return FLINT_ERR_ALIGNMENT;
  const int64_t dec = decode_ws_bytes(*shape, FLINT_MAX_DECODE_BATCH);
  if (ws_bytes < dec + prefill_ws_bytes(*shape, n_tokens)) return FLINT_ERR_WORKSPACE;
  PrefillWs w = carve_prefill_ws(static_cast<char*>(ws) + dec, *shape, n_tokens);
  LayerArgs a = make_args(shape, weights, x, n_tokens < 8 ? n_tokens : 8, out, gamma);
  a.topk_idx = topk_idx ? topk_idx : w.idx;
  a.topk_w = topk_w ? topk_w : w.wgt;
  if (planes) {
    auto u8 = [](const void* p) { return static_cast<const uint8_t*>(p); };
    a.pf_gu_codes = u8(planes->gu_codes); a.pf_gu_scales = u8(planes->gu_scales);
    a.pf_d_codes = u8(planes->d_codes);   a.pf_d_scales = u8(planes->d_scales);
    if (shape->shared_inter > 0) {
      a.pf_sh_gu_codes = u8(planes->sh_gu_codes); a.pf_sh_gu_scales = u8(planes->sh_gu_scales);
      a.pf_sh_d_codes = u8(planes->sh_d_codes);   a.pf_sh_d_scales = u8(planes->sh_d_scales);
    }
  }
  return to_status(launch_prefill(a, w, n_tokens, static_cast<hipStream_t>(stream)));
}

int32_t flint_moe_prefill_layout(const void* codes, const void* scales, int64_t n_mats, int32_t rows,
                                 int32_t cols, int32_t interleave, void* out_codes, void* out_scales,
                                 void* stream) {
  if (n_mats <= 0 || rows <= 0 || cols <= 0 || (interleave != 0 && interleave != 1)) return FLINT_ERR_INVALID_ARG;
  if (cols % 128 || ((int64_t)rows * (1 + interleave)) % 32 || (interleave && n_mats % 2)) return FLINT_ERR_INVALID_ARG;
  FLINT_NEED(codes);
  FLINT_NEED(scales);
  FLINT_NEED(out_codes);
  FLINT_NEED(out_scales);
  const int64_t cb = n_mats * rows * (int64_t)cols / 2, sb = cb / 8;
  auto apart = [](const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x + (uint64_t)na <= y || y + (uint64_t)nb <= x;
  };
  if (!apart(codes, cb, out_codes, cb) || !apart(codes, cb, out_scales, sb) || !apart(scales, sb, out_codes, cb) ||
      !apart(scales, sb, out_scales, sb))
    return FLINT_ERR_INVALID_ARG;
  return to_status(launch_prefill_layout(static_cast<const uint8_t*>(codes), static_cast<const uint8_t*>(scales),
                                         n_mats, rows, cols, interleave, static_cast<uint8_t*>(out_codes),
                                         static_cast<uint8_t*>(out_scales), static_cast<hipStream_t>(stream)));
}

int32_t flint_dense_gemv(const void* codes, const void* scales, const float* gscale,
                         const void* w_bf16, int32_t rows, int32_t cols, uint32_t flags,
                         const void* x, int32_t batch, void* y, int32_t epilogue,
                         const void* aux, const void* gamma, float rms_eps, void* stream) {
  if (rows <= 0 || cols <= 0 || batch <= 0) return FLINT_ERR_INVALID_ARG;
  if (cols % 64) return FLINT_ERR_UNSUPPORTED;
  if (batch > FLINT_MAX_DECODE_BATCH) return FLINT_ERR_UNSUPPORTED;
  if (flags & ~(FLINT_W_BF16 | FLINT_PRE_RMSNORM)) return FLINT_ERR_UNSUPPORTED;
  if (epilogue != FLINT_EPI_NONE && epilogue != FLINT_EPI_SWIGLU && epilogue != FLINT_EPI_RESIDUAL)
    return FLINT_ERR_UNSUPPORTED;
  const bool norm = (flags & FLINT_PRE_RMSNORM) != 0;
  if (norm && epilogue != FLINT_EPI_SWIGLU) return FLINT_ERR_UNSUPPORTED;
  if (flags & FLINT_W_BF16) {
    FLINT_NEED(w_bf16);
  } else {
    FLINT_NEED(codes);
    FLINT_NEED(scales);
    FLINT_NEED(gscale);
  }
  FLINT_NEED(x);
  FLINT_NEED(y);
  if (y == x) return FLINT_ERR_INVALID_ARG;
  if (epilogue == FLINT_EPI_RESIDUAL) FLINT_NEED(aux);
  if (norm) {
    FLINT_NEED(gamma);
    if (!(rms_eps >= 0.0f)) return FLINT_ERR_INVALID_ARG;
  }

  // The dense matrix runs as the single "shared" expert of a layer with no
  // routed experts.
  LayerArgs a;
  std::memset(&a, 0, sizeof(a));
  a.B = batch;
  a.flags = flags & FLINT_W_BF16;
  a.eps = rms_eps;
  a.sh_gu_codes = static_cast<const uint8_t*>(codes);
  a.sh_gu_scales = static_cast<const uint8_t*>(scales);
  a.sh_d_codes = static_cast<const uint8_t*>(codes);
  a.sh_d_scales = static_cast<const uint8_t*>(scales);
  a.sh_gscale = gscale;
  a.sh_gu_bf16 = static_cast<const uint16_t*>(w_bf16);
  a.sh_d_bf16 = static_cast<const uint16_t*>(w_bf16);
  a.x = static_cast<const uint16_t*>(x);
  a.gamma = static_cast<const uint16_t*>(gamma);
  a.out = static_cast<uint16_t*>(y);
  DecodeWs w;
  std::memset(&w, 0, sizeof(w));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (epilogue == FLINT_EPI_SWIGLU) {
    a.H = cols; a.I = 0; a.SI = rows;   // gate/up pair [2][rows][cols] -> y [B][rows]
    return to_status(launch_gate_up(a, w, true, norm, s));
  }
  a.H = rows; a.I = 0; a.SI = cols;     // W [rows][cols] . x[B][cols] -> y [B][rows]
  return to_status(launch_down(a, w, true, epilogue, static_cast<const uint16_t*>(x),
                               static_cast<const uint16_t*>(aux), s));
}

}  // extern "C"
