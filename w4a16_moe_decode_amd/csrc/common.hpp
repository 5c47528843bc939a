// Device helpers and internal launch interfaces of the MI355X (gfx950) MoE
// library: BF16 rounding, NVFP4 chunk decode, wave reductions, workspace
// layout.  Internal header (the public ABI is include/flint_moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flint_moe.h"

namespace flint {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// two floats -> packed BF16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// ------------------------------------------------------------- BF16 ------

// float -> BF16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float round_bf16(float f) { return bf16_bits_to_f32(f32_to_bf16_bits(f)); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// float64 -> BF16 bits, round to nearest even, directly from the double
// (no intermediate float rounding).  For finite values in float's range.
__device__ __forceinline__ uint16_t f64_to_bf16_bits(double d) {
  uint64_t b = (uint64_t)__double_as_longlong(d);
  b += 0x0fffffffffffull + ((b >> 45) & 1ull);           // half of bit 45, ties to even
  b &= ~0x1fffffffffffull;
  return (uint16_t)(__float_as_uint((float)__longlong_as_double((long long)b)) >> 16);
}

// RMSNorm of packed BF16 pairs: BF16(BF16(x / rms) * gamma), with
// rms = sqrt(mean(x^2) + eps) in float64 and x / rms rounded once, from
// float64, like the definition; the second step (times gamma) is exact in
// float32 before its rounding.  The quotient is first taken as
// x * float(1/rms) in float32, which is within 1.5 float32 ulps of x / rms;
// both therefore round to the same BF16 value unless that product lies
// within a few ulps of a BF16 rounding midpoint (its 16 bits below the BF16
// mantissa near 0x8000).  Only such values -- a few in ten thousand -- are
// recomputed as a float64 division.  When 1/rms is outside float32's
// comfortable range every value takes the division.
struct Rms { double rms; float rinv; bool fast; };
__device__ __forceinline__ Rms make_rms(double rms) {
  const float ri = (float)(1.0 / rms);
  return Rms{rms, ri, ri >= 0x1p-100f && ri <= 0x1p100f};
}
__device__ __forceinline__ bool near_bf16_midpoint(float f) {
  return ((__float_as_uint(f) - 0x7ffcu) & 0xffffu) <= 8u;
}
__device__ __forceinline__ uint32_t bf16_quotient_bits(float x, double rms) {
  double q = (double)x / rms;
  asm volatile("" : "+v"(q));                     // keeps the division on the rare path
  return f64_to_bf16_bits(q);
}
template <int N>
__device__ __forceinline__ void rms_norm_words(uint32_t (&v)[N], const uint32_t (&g)[N], const Rms& r) {
  uint32_t y[N];
  bool nlo[N], nhi[N];
  bool any = false;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float lo = bf16_lo(v[i]) * r.rinv, hi = bf16_hi(v[i]) * r.rinv;
    nlo[i] = near_bf16_midpoint(lo) || !r.fast;
    nhi[i] = near_bf16_midpoint(hi) || !r.fast;
    any = any || nlo[i] || nhi[i];
    y[i] = pack_bf16x2_rne(lo, hi);
  }
  if (__ballot(any) != 0ull) {                    // wave-wide branch, rarely taken
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (nlo[i]) y[i] = (y[i] & 0xffff0000u) | bf16_quotient_bits(bf16_lo(v[i]), r.rms);
      if (nhi[i]) y[i] = (y[i] & 0x0000ffffu) | (bf16_quotient_bits(bf16_hi(v[i]), r.rms) << 16);
    }
  }
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = pack_bf16x2_rne(bf16_lo(y[i]) * bf16_lo(g[i]), bf16_hi(y[i]) * bf16_hi(g[i]));
}
// the same for one uint4 (8 values)
__device__ __forceinline__ uint4 rms_norm_8(uint4 x, uint4 g, const Rms& r) {
  uint32_t v[4] = {x.x, x.y, x.z, x.w};
  const uint32_t gv[4] = {g.x, g.y, g.z, g.w};
  rms_norm_words<4>(v, gv, r);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// SiLU(z) = z / (1 + e^-z) in fp32 (expf: the HIP device function).
__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }
// SiLU from the hardware base-2 exponential and reciprocal (each within about
// 1 ulp): within a few fp32 ulps of silu_f32, for epilogues that round the
// result to BF16 right after.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

// ------------------------------------------------------------ NVFP4 ------

// Two E2M1 codes (byte `sel` of w; low nibble = even column) -> two exact
// BF16 values.  The f32 operand of the gfx950 conversion only contributes
// its exponent, so it stays 1.0 and the UE4M3 block scale is applied to the
// fp32 partial sum of its 16 columns instead.
template <int SEL>
__device__ __forceinline__ bf16x2_t fp4x2_to_bf16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
}

// UE4M3 scale byte `SEL` of w -> float (hardware OCP E4M3FN decode: bias 7,
// subnormals, 0x7F/0xFF NaN, bit 7 sign).
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8((int)w, SEL);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ __forceinline__ float dot2_bf16v(bf16x2_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Weight formats of the GEMV engine.  A "chunk" is the 16 bytes of one row a
// lane loads at once: 32 NVFP4 codes (+2 scale bytes) or 8 BF16 weights.
enum { FMT_NVFP4 = 0, FMT_BF16 = 1 };
template <int WF> struct Fmt;
template <> struct Fmt<FMT_NVFP4> { static constexpr int VALS = 32; };
template <> struct Fmt<FMT_BF16> { static constexpr int VALS = 8; };

// Decoded chunk, reusable for every token routed to the row.
template <int WF> struct DChunk;
template <> struct DChunk<FMT_NVFP4> {
  bf16x2_t w[16];   // columns (2m, 2m+1), m = 0..15
  float s0, s1;     // scales of columns 0..15 and 16..31
};
template <> struct DChunk<FMT_BF16> {
  uint32_t w[4];
};

// Activation chunk matching one weight chunk: 32 (NVFP4) or 8 (BF16) BF16
// values as packed pairs.
template <int WF> struct XChunk { uint32_t v[Fmt<WF>::VALS / 2]; };

__device__ __forceinline__ DChunk<FMT_NVFP4> decode_nvfp4(uint4 c, uint32_t sc2) {
  DChunk<FMT_NVFP4> d;
  const uint32_t q[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    d.w[4 * i + 0] = fp4x2_to_bf16x2<0>(q[i]);
    d.w[4 * i + 1] = fp4x2_to_bf16x2<1>(q[i]);
    d.w[4 * i + 2] = fp4x2_to_bf16x2<2>(q[i]);
    d.w[4 * i + 3] = fp4x2_to_bf16x2<3>(q[i]);
  }
  d.s0 = e4m3_to_f32<0>(sc2);
  d.s1 = e4m3_to_f32<1>(sc2);
  return d;
}

// sum over the chunk of weight * x, block scales applied per 16 columns.
__device__ __forceinline__ float chunk_dot(const DChunk<FMT_NVFP4>& d, const XChunk<FMT_NVFP4>& x) {
  float p0 = 0.f, p1 = 0.f;
#pragma unroll
  for (int m = 0; m < 8; ++m) p0 = dot2_bf16v(d.w[m], x.v[m], p0);
#pragma unroll
  for (int m = 8; m < 16; ++m) p1 = dot2_bf16v(d.w[m], x.v[m], p1);
  return fmaf(d.s1, p1, d.s0 * p0);
}
__device__ __forceinline__ float chunk_dot(const DChunk<FMT_BF16>& d, const XChunk<FMT_BF16>& x) {
  float p = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) p = dot2_bf16(d.w[m], x.v[m], p);
  return p;
}

template <int WF>
__device__ __forceinline__ XChunk<WF> load_x(const uint16_t* row, int j) {
  XChunk<WF> x;
  const uint4* p = reinterpret_cast<const uint4*>(row + (size_t)j * Fmt<WF>::VALS);
#pragma unroll
  for (int i = 0; i < Fmt<WF>::VALS / 8; ++i) {
    uint4 v = p[i];
    x.v[4 * i + 0] = v.x; x.v[4 * i + 1] = v.y; x.v[4 * i + 2] = v.z; x.v[4 * i + 3] = v.w;
  }
  return x;
}

// Load of a T from device memory through a global-qualified pointer.  For
// pointers the compiler cannot trace to a kernel argument (read from an
// array of per-layer pointers, say) a plain dereference becomes a flat load,
// which counts against the LDS counter too, so every later LDS read would
// wait for it.
template <class T>
__device__ __forceinline__ T ldg(const void* p) {
  typedef __attribute__((address_space(1))) const T GT;
  return *(GT*)p;
}
// uint4's copy constructor takes a generic reference, so 16 bytes are loaded
// as a native vector
template <>
__device__ __forceinline__ uint4 ldg<uint4>(const void* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(1))) const v4u GV;
  const v4u v = *(GV*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}

// The same 16 bytes as a non-temporal load, for data that streams through
// once (weight rows of a decode layer, KV rows): the batch-8 layer ran
// 31.07 -> 30.13 us with them, the batch-1 layer 11.08 -> 10.92 us and a
// 513-token window of attention 9.16 -> 8.53 us.  Data that many
// workgroups read (a token, hand-off words) keeps plain loads: the batch-1
// layer with every load non-temporal ran 11.1 -> 14.5 us; so does the LM
// head's stream (33 -> 49 us as non-temporal loads).
__device__ __forceinline__ uint4 ldg_nt(const void* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(1))) const v4u GV;
  const v4u v = __builtin_nontemporal_load((GV*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt 0 and leaves
// expcnt and lgkmcnt unconstrained.
constexpr int kWaitVmcnt0 = 0x0F70;

// ------------------------------------------------------- wave reductions --

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G lanes (G a power of two <= 64); every lane
// of a group ends with the group's sum.  Fixed order: bit-reproducible.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp_f<0xB1>(v);     // quad_perm [1,0,3,2]
  if constexpr (G >= 4) v += dpp_f<0x4E>(v);     // quad_perm [2,3,0,1]
  if constexpr (G >= 8) v += dpp_f<0x141>(v);    // row_half_mirror
  if constexpr (G >= 16) v += dpp_f<0x140>(v);   // row_mirror
  if constexpr (G >= 32) {    // rows 0<->1, 2<->3: v_permlane16_swap
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if constexpr (G >= 64) {    // halves 0..31 <-> 32..63: v_permlane32_swap
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return v;
}

// Sum of a double over the 64 lanes of a wave (fixed order), all lanes.
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Maximum over the wave of 64-bit keys, every lane ends with the result.
// In-row steps use DPP; the four row maxima are combined with readlane.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint64_t o;
  o = dpp_u64<0xB1>(v);  v = o > v ? o : v;     // quad_perm [1,0,3,2]
  o = dpp_u64<0x4E>(v);  v = o > v ? o : v;     // quad_perm [2,3,0,1]
  o = dpp_u64<0x141>(v); v = o > v ? o : v;     // row_half_mirror
  o = dpp_u64<0x140>(v); v = o > v ? o : v;     // row_mirror
  uint64_t m = readlane_u64(v, 0);
  o = readlane_u64(v, 16); m = o > m ? o : m;
  o = readlane_u64(v, 32); m = o > m ? o : m;
  o = readlane_u64(v, 48); m = o > m ? o : m;
  return m;
}

// Maximum over the wave of a 32-bit value (DPP max steps within rows, then
// the four row maxima), the same in every lane.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));
  v = max(v, dpp_u32<0x4E>(v));
  v = max(v, dpp_u32<0x141>(v));
  v = max(v, dpp_u32<0x140>(v));
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

// Wave maximum of 64-bit keys (order key << 32 | inverted index) whose high
// halves are usually distinct: the high half is reduced with 32-bit steps,
// and the low half only among the lanes that hold the maximal high half.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t key) {
  const uint32_t hi = (uint32_t)(key >> 32);
  const uint32_t mhi = wave_max_u32(hi);
  const bool at = hi == mhi;
  const unsigned long long bal = __ballot(at);
  uint32_t mlo;
  if (__popcll(bal) == 1) {
    mlo = __builtin_amdgcn_readlane((uint32_t)key, __ffsll((long long)bal) - 1);
  } else {
    mlo = wave_max_u32(at ? (uint32_t)key : 0u);
  }
  return ((uint64_t)mhi << 32) | mlo;
}

// Order-preserving map of a float to uint32 (larger float -> larger key);
// NaN is treated as -inf.
__device__ __forceinline__ uint32_t float_order_key(float f) {
  if (f != f) f = -INFINITY;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float float_from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// ------------------------------------------------------ decode workspace --

// Device-side view of the decode workspace (offsets computed on the host).
struct DecodeWs {
  uint32_t* ticket;      // [1] arrival counter of the route kernel, left at zero
  uint32_t* epoch;       // [1] number of route launches so far
  uint32_t* error;       // [1] set to 1 if a routing hand-off ever timed out
  uint32_t* wait_limit;  // [1] bound of each wait in reloads (0: the default), set by the host
  uint64_t* logit_words; // [B][E] (epoch << 32) | fp32 logit bits
  uint16_t* xn;          // [B][H] BF16 normalised input (PRE_RMSNORM)
  int32_t* idx;          // [B][K] selected experts (when the caller passes none)
  float* wgt;            // [B][K] combine weights
  int32_t* nslot;        // [1] number of distinct routed experts U
  int32_t* slot_expert;  // [S] routed expert of routed slot r (ascending)
  uint32_t* slot_mask;   // [S] bit t set = token t routed to routed slot r
  float* slot_w;         // [S][8] combine weight of token t at routed slot r
  uint64_t* h_words;     // [K+1][Imax/2] (epoch << 32) | two BF16 of h, single-launch path
  uint64_t* x_words;     // [8][H/2] (epoch << 32) | two BF16 of the residual, layer stack
  uint64_t* hb_words;    // [S_routed][8][Imax/2] (epoch << 32) | two BF16 of h, batch single launch
  uint64_t* p_words;     // [8][K_max+1][H] (epoch << 32) | fp32 partial sum, batch single launch
                         // (both null unless the shape takes that path)
  uint16_t* h;           // [S][8][Imax] BF16 SiLU(g)*u per slot and token; slot 0
                         // is the shared expert when there is one, routed
                         // slot r is slot r + (shared ? 1 : 0)
  int64_t bytes;
};

DecodeWs carve_decode_ws(void* base, const flint_moe_shape& s, int max_batch);
int64_t decode_ws_bytes(const flint_moe_shape& s, int max_batch);
int decode_max_slots(const flint_moe_shape& s, int batch);

// -------------------------------------------------------- launch surface --

// Arguments shared by the decode kernels (device pointers).
struct LayerArgs {
  int H, E, I, SI, K, B;
  uint32_t flags;
  float eps;
  const uint16_t* router;
  const uint8_t* gu_codes; const uint8_t* gu_scales;
  const uint8_t* d_codes;  const uint8_t* d_scales;
  const float* gscale;
  const uint8_t* sh_gu_codes; const uint8_t* sh_gu_scales;
  const uint8_t* sh_d_codes;  const uint8_t* sh_d_scales;
  const float* sh_gscale;
  const uint16_t* gu_bf16; const uint16_t* d_bf16;
  const uint16_t* sh_gu_bf16; const uint16_t* sh_d_bf16;
  // the NVFP4 planes in the prefill layout (flint_moe_prefill_tiled), or null
  const uint8_t* pf_gu_codes; const uint8_t* pf_gu_scales;
  const uint8_t* pf_d_codes;  const uint8_t* pf_d_scales;
  const uint8_t* pf_sh_gu_codes; const uint8_t* pf_sh_gu_scales;
  const uint8_t* pf_sh_d_codes;  const uint8_t* pf_sh_d_scales;
  const uint16_t* x;       // [B][H] layer input (residual with PRE_RMSNORM)
  const uint16_t* gamma;   // [H]
  uint16_t* out;           // [B][H]
  int32_t* topk_idx;       // [B][K] (user or workspace)
  float* topk_w;           // [B][K]
};

// flint_moe_decode (stage -1) or one of its stages, on a given workspace.
int32_t decode_common(int32_t stage, const flint_moe_shape* shape, const flint_moe_weights* weights,
                      const void* x, int32_t batch, void* out, int32_t* topk_idx, float* topk_w,
                      const void* gamma, void* ws, int64_t ws_bytes, void* stream);

hipError_t launch_route(const LayerArgs& a, const DecodeWs& ws, hipStream_t st);
bool fused_decode_supported(const LayerArgs& a);
// The single-launch batch-1 layer specialised to the Flint shape (hidden
// 2048, 256 experts, intermediate 512 routed and shared, top-k <= 8).
bool flint_b1_supported(const LayerArgs& a);
bool flint_b8_shape(const flint_moe_shape& s);
bool flint_b8_supported(const LayerArgs& a);   // the workspace of such a shape holds its buffers
hipError_t launch_flint_b8(const LayerArgs& a, const DecodeWs& ws, hipStream_t st);
hipError_t launch_flint_b1(const LayerArgs& a, const DecodeWs& ws, hipStream_t st);
hipError_t launch_fused_decode(const LayerArgs& a, const DecodeWs& ws, hipStream_t st);
// A stack of MoE layers for one token in one launch (flint_moe_decode_stack).
struct StackArgs {
  LayerArgs base;                      // shape, flags, eps; pointers set per layer
  const flint_moe_weights* layers;     // device array [L]
  const uint16_t* gammas;              // [L][H]
  const uint16_t* x_in;                // [H]
  uint16_t* x_out;                     // [H]
  int32_t* topk_idx;                   // [L][K]
  float* topk_w;                       // [L][K]
  uint16_t* layer_out;                 // [L][H] or null
  int L;
};
bool fused_stack_supported(const LayerArgs& a);
hipError_t launch_flint_stack(const StackArgs& sa, const DecodeWs& ws, hipStream_t st);
hipError_t launch_fused_stack(const StackArgs& sa, const DecodeWs& ws, hipStream_t st);
hipError_t launch_gate_up(const LayerArgs& a, const DecodeWs& ws, bool dense, bool norm_on_the_fly,
                          hipStream_t st);
hipError_t launch_down(const LayerArgs& a, const DecodeWs& ws, bool dense, int dense_epilogue,
                       const uint16_t* dense_in, const uint16_t* aux, hipStream_t st);

struct PrefillWs;
PrefillWs carve_prefill_ws(void* base, const flint_moe_shape& s, int T);
hipError_t launch_prefill(const LayerArgs& a, const PrefillWs& ws, int T, hipStream_t st);

hipError_t launch_repack(const uint8_t* src, int64_t n_mats, int rows, int cols, int layout,
                         uint8_t* codes, uint8_t* scales, int64_t mat_stride, hipStream_t st);
hipError_t launch_unpack(const uint8_t* codes, const uint8_t* scales, int64_t n_mats, int rows,
                         int cols, int layout, int64_t mat_stride, uint8_t* dst, hipStream_t st);
// The prefill layout of packed planes (flint_moe_prefill_layout).
hipError_t launch_prefill_layout(const uint8_t* codes, const uint8_t* scales, int64_t n_mats, int rows, int cols,
                                 int interleave, uint8_t* out_codes, uint8_t* out_scales, hipStream_t st);
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, int64_t n_mats, int rows,
                          int cols, const float* tscale, float* out, hipStream_t st);

}  // namespace flint
