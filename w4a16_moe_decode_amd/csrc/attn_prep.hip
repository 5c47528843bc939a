// flint_qk_norm_rope_kv: the per-head Q/K RMSNorm, rotary position
// embedding and KV-cache write of an attention layer's projected heads, in
// one kernel ("Day-0 Support for Flint on vLLM", "Optimizations": the three
// steps fused into one kernel; "Model architecture": GQA with 32 query and
// 4 KV heads of dimension 128, per-head Q/K RMSNorm, RoPE on the
// sliding-window layers, BF16 KV cache).
//
// 64 / NP lanes per (token, head) of the projection row [q heads | k heads |
// v heads]: lane j of a head holds elements NP j .. NP j + NP - 1 and
// 64 + NP j .. 64 + NP j + NP - 1, i.e. the pairs (x_i, x_{i+64}) that the
// rotate-half RoPE mixes, so the rotation needs no exchange between lanes.
// NP = 8 (16-byte accesses, eight heads per wave) for many tokens; NP = 1
// (one head per wave, the shortest dependent chain per lane) for a few
// decode tokens, where the launch is latency-bound.  Per q or k head: the mean of squares
// over the head (float64), BF16(BF16(x / rms) * gamma) with the library's
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

// a float64 value of the lane paired by a DPP pattern (two 32-bit moves)
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)b, CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, 0xf, 0xf, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
// v plus the value of the paired row (W = 16) or half wave (W = 32),
// through permlane swaps of the two 32-bit halves (the swap returns both
// values, the lane's own and its partner's)
template <int W>
__device__ __forceinline__ double swap_sum_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)b, hi = (uint32_t)(b >> 32);
  uint32_t l0, l1, h0, h1;
  if constexpr (W == 16) {
    const auto rl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto rh = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    l0 = rl[0]; l1 = rl[1]; h0 = rh[0]; h1 = rh[1];
  } else {
    const auto rl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto rh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    l0 = rl[0]; l1 = rl[1]; h0 = rh[0]; h1 = rh[1];
  }
  return __longlong_as_double((long long)(((uint64_t)h0 << 32) | l0)) +
         __longlong_as_double((long long)(((uint64_t)h1 << 32) | l1));
}
// Sum over the head's LPH lanes, the same in each: blocks of 2, 4, ..
// lanes, each the sum of its two halves (DPP within a row of 16, permlane
// swaps across rows), the pairing of an xor butterfly without the LDS
// crossbar.
template <int LPH>
__device__ __forceinline__ double group_sum_f64(double v) {
  static_assert(LPH == 8 || LPH == 64, "heads of 8 or 64 lanes");
  v += dpp_f64<0xB1>(v);                           // quad_perm [1, 0, 3, 2]
  v += dpp_f64<0x4E>(v);                           // quad_perm [2, 3, 0, 1]
  v += dpp_f64<0x141>(v);                          // row_half_mirror
  if constexpr (LPH == 64) {
    v += dpp_f64<0x140>(v);                        // row_mirror
    v = swap_sum_f64<16>(v);                       // rows 0 <-> 1, 2 <-> 3
    v = swap_sum_f64<32>(v);                       // halves of the wave
  }
  return v;
}

// the lane's NP elements at p (NP = 8: 16 bytes; NP = 1: 2 bytes) as NP / 2
// words, and back
template <int NP>
__device__ __forceinline__ void load_half(uint32_t (&w)[NP > 1 ? NP / 2 : 1], const uint16_t* p) {
  if constexpr (NP == 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else {
    w[0] = *p;
  }
}
// NP = 8 stores are non-temporal: the rows are read by a later kernel, and
// without write-back lines left in L2 the 8,192-token call ran 49.5 -> 43.1 us
template <int NP>
__device__ __forceinline__ void store_half(uint16_t* p, const uint32_t (&w)[NP > 1 ? NP / 2 : 1]) {
  if constexpr (NP == 8)
    __builtin_nontemporal_store(__builtin_bit_cast(f32x4_t, make_uint4(w[0], w[1], w[2], w[3])),
                                reinterpret_cast<f32x4_t*>(p));
  else *p = (uint16_t)w[0];
}
// (low: x_i, high: x_{i+64}) words of the lane's NP pairs
template <int NP>
__device__ __forceinline__ void pair_words(uint32_t (&w)[NP], const uint32_t (&lo)[NP > 1 ? NP / 2 : 1],
                                           const uint32_t (&hi)[NP > 1 ? NP / 2 : 1]) {
  if constexpr (NP == 1) {
    w[0] = (lo[0] & 0xffffu) | (hi[0] << 16);
  } else {
#pragma unroll
    for (int k = 0; k < NP / 2; ++k) {
      w[2 * k] = (lo[k] & 0xffffu) | (hi[k] << 16);
      w[2 * k + 1] = (lo[k] >> 16) | (hi[k] & 0xffff0000u);
    }
  }
}

// grid (tokens, head groups of blockDim / LPH): lane group hg (LPH lanes)
// takes head (blockDim / LPH) blockIdx.y + hg
template <int NP>
__global__ __launch_bounds__(256) void qk_norm_rope_kv_kernel(AttnArgs a) {
  constexpr int D = kHeadDim, HALF = D / 2, LPH = HALF / NP, NW = NP > 1 ? NP / 2 : 1;
  const int t = blockIdx.x;
  const int head = blockIdx.y * (blockDim.x / LPH) + threadIdx.x / LPH;
  const int j = threadIdx.x % LPH;
  const int n_heads = a.n_q + 2 * a.n_kv;
  if (head >= n_heads) return;                     // whole lane groups
  const bool rope = (a.flags & FLINT_ATTN_ROPE) != 0;
  const int slot = a.slots[t];
  const int pos = rope ? a.positions[t] : 0;
  // an index outside its table or cache: nothing of this token is written
  if ((rope && (pos < 0 || pos >= a.n_positions)) || slot >= a.n_slots) {
    if (a.error && head == 0 && j == 0) *a.error = 1;
    return;
  }
  const uint16_t* row = a.qkv + (size_t)t * n_heads * D + (size_t)head * D;
  uint32_t xa[NW], xb[NW];
  load_half<NP>(xa, row + NP * j);                 // x_{NP j} ..
  load_half<NP>(xb, row + HALF + NP * j);          // x_{64 + NP j} ..
  const bool is_q = head < a.n_q, is_k = !is_q && head < a.n_q + a.n_kv;
  if (!is_q && !is_k) {                            // V head: to the cache, unchanged
    if (slot >= 0) {
      uint16_t* dst = a.v_cache + ((size_t)slot * a.n_kv + (head - a.n_q - a.n_kv)) * D;
      store_half<NP>(dst + NP * j, xa);
      store_half<NP>(dst + HALF + NP * j, xb);
    }
    return;
  }
  const uint16_t* gamma = is_q ? a.gamma_q : a.gamma_k;
  uint32_t ga[NW], gb[NW], v[NP], g[NP];
  load_half<NP>(ga, gamma + NP * j);
  load_half<NP>(gb, gamma + HALF + NP * j);
  pair_words<NP>(v, xa, xb);
  pair_words<NP>(g, ga, gb);
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const double lo = bf16_lo(v[i]), hi = bf16_hi(v[i]);
    ss = fma(lo, lo, ss);
    ss = fma(hi, hi, ss);
  }
  ss = group_sum_f64<LPH>(ss);
  rms_norm_words<NP>(v, g, make_rms(sqrt(ss / (double)D + (double)a.eps)));
  uint32_t ya[NP], yb[NP];                          // BF16 bits of y_i, y_{i+64}
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    ya[i] = v[i] & 0xffffu;
    yb[i] = v[i] >> 16;
  }
  if (rope) {
    const float* cs = a.cos_sin + (size_t)pos * D;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const double p = bf16_lo(v[i]), q = bf16_hi(v[i]), c = cs[NP * j + i], sv = cs[HALF + NP * j + i];
      ya[i] = f64_to_bf16_bits(p * c - q * sv);
      yb[i] = f64_to_bf16_bits(q * c + p * sv);
    }
  }
  uint16_t* dst;
  if (is_q) {
    dst = a.q_out + ((size_t)t * a.n_q + head) * D;
  } else {
    if (slot < 0) return;                          // a padding token keeps no KV
    dst = a.k_cache + ((size_t)slot * a.n_kv + (head - a.n_q)) * D;
  }
  uint32_t oa[NW], ob[NW];
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    oa[k] = NP > 1 ? ya[2 * k] | (ya[2 * k + 1] << 16) : ya[0];
    ob[k] = NP > 1 ? yb[2 * k] | (yb[2 * k + 1] << 16) : yb[0];
  }
  store_half<NP>(dst + NP * j, oa);
  store_half<NP>(dst + HALF + NP * j, ob);
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
  // a few decode tokens: one head per wave, four per workgroup (the shortest
  // chain per lane, the most workgroups); many tokens: 16-byte accesses, 32
  // heads per workgroup
  if (n_tokens < 256)
    hipLaunchKernelGGL(qk_norm_rope_kv_kernel<1>, dim3(n_tokens, (heads + 3) / 4), dim3(256), 0,
                       static_cast<hipStream_t>(stream), a);
  else
    hipLaunchKernelGGL(qk_norm_rope_kv_kernel<8>, dim3(n_tokens, (heads + 31) / 32), dim3(256), 0,
                       static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? FLINT_OK : FLINT_ERR_DEVICE;
}
