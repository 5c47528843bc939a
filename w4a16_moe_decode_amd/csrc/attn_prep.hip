// flint_qk_norm_rope_kv: the per-head Q/K RMSNorm, rotary position
// embedding and KV-cache write of an attention layer's projected heads, in
// one kernel ("Day-0 Support for Flint on vLLM", "Optimizations": the three
// steps fused into one kernel; "Model architecture": GQA with 32 query and
// 4 KV heads of dimension 128, per-head Q/K RMSNorm, RoPE on the
// sliding-window layers, BF16 KV cache).
//
// One wave per (token, head) of the projection row [q heads | k heads |
// v heads]; lane l holds the pair (x_l, x_{l+64}) of its head, which is
// exactly the pair the rotate-half RoPE mixes, so the rotation needs no
// exchange between lanes.  Per q or k head: the mean of squares over the
// head (float64 wave sum), BF16(BF16(x / rms) * gamma) with the library's
// RMSNorm rounding, then (with FLINT_ATTN_ROPE) the rotation by the table
// row of the token's position, taken in float64 (the products of a BF16
// value and a float32 table entry are exact there) and rounded to BF16
// once.  V heads are copied to the cache unchanged.
#include <hip/hip_runtime.h>

#include "common.hpp"

namespace flint {
namespace {

constexpr int kHeadDim = 128;

struct AttnArgs {
  const uint16_t* qkv;
  const int32_t* positions;
  const float* cos_sin;
  const int32_t* slots;
  uint16_t* k_cache;
  uint16_t* v_cache;
  const uint16_t* gamma_q;
  const uint16_t* gamma_k;
  uint16_t* q_out;
  int32_t* error;
  int n_tokens, n_q, n_kv, n_positions, n_slots;
  uint32_t flags;
  float eps;
};

__global__ __launch_bounds__(256) void qk_norm_rope_kv_kernel(AttnArgs a) {
  constexpr int D = kHeadDim, HALF = D / 2;
  const int t = blockIdx.x;
  const int head = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n_heads = a.n_q + 2 * a.n_kv;
  if (head >= n_heads) return;                     // the whole wave
  const bool rope = (a.flags & FLINT_ATTN_ROPE) != 0;
  const int slot = a.slots[t];
  const int pos = rope ? a.positions[t] : 0;
  // an index outside its table or cache: nothing of this token is written
  if ((rope && (pos < 0 || pos >= a.n_positions)) || slot >= a.n_slots) {
    if (a.error && head == 0 && lane == 0) *a.error = 1;
    return;
  }
  const uint16_t* row = a.qkv + (size_t)t * n_heads * D + (size_t)head * D;
  const uint32_t xa = row[lane], xb = row[lane + HALF];
  const bool is_q = head < a.n_q, is_k = !is_q && head < a.n_q + a.n_kv;
  if (!is_q && !is_k) {                            // V head: to the cache, unchanged
    if (slot >= 0) {
      uint16_t* dst = a.v_cache + ((size_t)slot * a.n_kv + (head - a.n_q - a.n_kv)) * D;
      dst[lane] = (uint16_t)xa;
      dst[lane + HALF] = (uint16_t)xb;
    }
    return;
  }
  const uint16_t* gamma = is_q ? a.gamma_q : a.gamma_k;
  // RMSNorm of the head: the pair as one packed word (low: x_l, high: x_{l+64})
  uint32_t v[1] = {xa | (xb << 16)};
  const uint32_t g[1] = {(uint32_t)gamma[lane] | ((uint32_t)gamma[lane + HALF] << 16)};
  const double lo = bf16_lo(v[0]), hi = bf16_hi(v[0]);
  const double ss = wave_sum_f64(lo * lo + hi * hi);
  rms_norm_words<1>(v, g, make_rms(sqrt(ss / (double)D + (double)a.eps)));
  uint16_t ya = (uint16_t)(v[0] & 0xffffu), yb = (uint16_t)(v[0] >> 16);
  if (rope) {
    const float* cs = a.cos_sin + (size_t)pos * D;
    const double c = cs[lane], s = cs[HALF + lane];
    const double p = bf16_lo(v[0]), q = bf16_hi(v[0]);
    ya = f64_to_bf16_bits(p * c - q * s);
    yb = f64_to_bf16_bits(q * c + p * s);
  }
  uint16_t* dst;
  if (is_q) {
    dst = a.q_out + ((size_t)t * a.n_q + head) * D;
  } else {
    if (slot < 0) return;                          // a padding token keeps no KV
    dst = a.k_cache + ((size_t)slot * a.n_kv + (head - a.n_q)) * D;
  }
  dst[lane] = ya;
  dst[lane + HALF] = yb;
}

}  // namespace
}  // namespace flint

extern "C" int32_t flint_qk_norm_rope_kv(const flint_attn_shape* shape, const void* qkv, int32_t n_tokens,
                                         const int32_t* positions, const float* cos_sin, int32_t n_positions,
                                         const int32_t* slots, void* k_cache, void* v_cache, int32_t n_slots,
                                         const void* gamma_q, const void* gamma_k, void* q_out, int32_t* error,
                                         void* stream) {
  using namespace flint;
  if (!shape || !qkv || !slots || !k_cache || !v_cache || !gamma_q || !gamma_k || !q_out)
    return FLINT_ERR_INVALID_ARG;
  if (n_tokens <= 0 || n_slots <= 0 || shape->n_q_heads <= 0 || shape->n_kv_heads <= 0)
    return FLINT_ERR_INVALID_ARG;
  if (shape->head_dim != kHeadDim || (shape->flags & ~FLINT_ATTN_ROPE) || shape->n_q_heads % shape->n_kv_heads ||
      shape->n_q_heads + 2 * shape->n_kv_heads > 4096 || !(shape->rms_eps >= 0.f))
    return FLINT_ERR_UNSUPPORTED;
  const bool rope = (shape->flags & FLINT_ATTN_ROPE) != 0;
  if (rope && (!positions || !cos_sin || n_positions <= 0)) return FLINT_ERR_INVALID_ARG;
  auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  auto a4 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; };
  if (!a16(qkv) || !a16(k_cache) || !a16(v_cache) || !a16(q_out) || !a16(gamma_q) || !a16(gamma_k) ||
      !a4(slots) || (rope && (!a16(cos_sin) || !a4(positions))) || (error && !a4(error)))
    return FLINT_ERR_ALIGNMENT;
  AttnArgs a;
  a.qkv = static_cast<const uint16_t*>(qkv);
  a.positions = positions;
  a.cos_sin = cos_sin;
  a.slots = slots;
  a.k_cache = static_cast<uint16_t*>(k_cache);
  a.v_cache = static_cast<uint16_t*>(v_cache);
  a.gamma_q = static_cast<const uint16_t*>(gamma_q);
  a.gamma_k = static_cast<const uint16_t*>(gamma_k);
  a.q_out = static_cast<uint16_t*>(q_out);
  a.error = error;
  a.n_tokens = n_tokens;
  a.n_q = shape->n_q_heads;
  a.n_kv = shape->n_kv_heads;
  a.n_positions = rope ? n_positions : 0;
  a.n_slots = n_slots;
  a.flags = shape->flags;
  a.eps = shape->rms_eps;
  const int heads = a.n_q + 2 * a.n_kv;
  hipLaunchKernelGGL(qk_norm_rope_kv_kernel, dim3(n_tokens, (heads + 3) / 4), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? FLINT_OK : FLINT_ERR_DEVICE;
}
