// Single-launch decode MoE layer for one token at the Flint shape: hidden
// 2048, 256 routed experts of intermediate 512, a shared expert of
// intermediate 512, top-k (k <= 8) -- the layer of "Day-0 Support for Flint
// on vLLM" ("Model architecture": 256 experts, sigmoid top-6 plus an
// always-on shared expert, hidden 2048; the expert intermediate is not
// printed and 512 is this library's reading), on a GPU with at least 256
// compute units.
//
// Same arithmetic as the general single-launch kernel (fused.hip), with
// every size a compile-time constant so that each wave runs straight-line
// code whose memory waits are exact, and with 8 waves per workgroup, each
// with its own role:
//
//   all waves  load their lane's 32 columns of x (and gamma) and normalise
//              them independently (every wave holds the whole token), so no
//              exchange is needed inside the workgroup before the router
//   wave 0     router row b (workgroup b owns expert b): dot product, wave
//              reduction, publish; then it polls all 256 logits, selects
//              the top-k and writes the slot table
//   wave 1     the shared expert's gate/up rows 2b, 2b+1
//   after the top-k: wave w < K takes routed gate/up item K*b + w (rows of
//   one routed expert); routed slot s (1..K, ascending expert) has its
//   down rows on wave 7 - s, and wave 7 the shared expert's (slot 0) and,
//   when k = 8, routed slot 8's
//   all waves  poll every h word, then the waves holding down rows compute
//              their partial sums of the workgroup's 8 output rows
//
// Hand-offs between workgroups are the epoch-tagged 64-bit words of the
// general kernel (one copy per XCD), with the same bounded waits.
//
// The same kernel runs the W16A16 form (BF16 expert weights, no tensor
// scales): a lane then holds its 32 columns of each row as four 16-byte
// words instead of one word of codes and its block scales.
#include "flint_common.hpp"

namespace flint {
namespace {

constexpr int FL_SLOTS = FLINT_MAX_TOP_K + 1;      // shared slot 0, routed slots 1..K

// acc[rw] += f * (down row chunk . h chunk) for the lane's two rows.
__device__ __forceinline__ void down_dot(float (&acc)[2], const DownRows& d, const uint32_t* hrow, float f, int lane) {
  const int li = lane & 15;
  XChunk<FMT_NVFP4> hx;
  const uint4* hp = reinterpret_cast<const uint4*>(hrow + 16 * li);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = hp[i];
    hx.v[4 * i] = v.x; hx.v[4 * i + 1] = v.y; hx.v[4 * i + 2] = v.z; hx.v[4 * i + 3] = v.w;
  }
#pragma unroll
  for (int rw = 0; rw < 2; ++rw) acc[rw] = fmaf(f, chunk_dot(decode_nvfp4(d.c[rw], d.s[rw]), hx), acc[rw]);
}

// h pair of one gate/up item (rows 2p, 2p+1) from the lane's chunk of the
// normalised token: BF16(BF16(SiLU(BF16(g))) * BF16(u)) per row.
__device__ __forceinline__ uint32_t item_h(const GUItem<1>& it, float gsc, float usc, const XChunk<FMT_NVFP4>& xn) {
  float h[2];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const float g = group_sum<64>(chunk_dot(decode_nvfp4(it.c[rr][0][0], it.s[rr][0][0]), xn));
    const float u = group_sum<64>(chunk_dot(decode_nvfp4(it.c[rr][1][0], it.s[rr][1][0]), xn));
    const float gv = round_bf16(g * gsc), uv = round_bf16(u * usc);
    h[rr] = round_bf16(silu_f32(gv)) * uv;
  }
  return pack_bf16x2(h[0], h[1]);
}

__device__ __forceinline__ void item_load(GUItem<1>& it, const uint8_t* gc, const uint8_t* gs, int p, int lane) {
  // gate rows of the pair, then the up rows (matrix stride I x H)
  constexpr size_t MC = (size_t)FL_I * FL_H / 2, MS = (size_t)FL_I * FL_H / 16;
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int row = 2 * p + rr;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      it.c[rr][m][0] = ldg_nt(gc + m * MC + (size_t)row * (FL_H / 2) + 16 * lane);
      it.s[rr][m][0] = ldg<uint16_t>(gs + m * MS + (size_t)row * (FL_H / 16) + 2 * lane);
    }
  }
}

// W16A16 (BF16 weights, no tensor scales): a lane holds the same 32
// columns of each row as in the NVFP4 form, as four 16-byte words.
struct GUItemBF { uint4 c[2][2][4]; };   // [row][gate|up][16-byte word]
struct DownRowsBF { uint4 c[2][4]; };    // [row][16-byte word]: columns 32 li .. + 31
template <int WF> struct FlRows;
template <> struct FlRows<FMT_NVFP4> { using Item = GUItem<1>; using Down = DownRows; };
template <> struct FlRows<FMT_BF16> { using Item = GUItemBF; using Down = DownRowsBF; };

// 32 BF16 weights (four words) . 32 BF16 values (16 packed pairs), fp32.
__device__ __forceinline__ float dot32_bf16(const uint4 (&w)[4], const uint32_t* v) {
  float p0 = 0.f, p1 = 0.f;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    p0 = dot2_bf16(w[q].x, v[4 * q], p0);
    p0 = dot2_bf16(w[q].y, v[4 * q + 1], p0);
    p0 = dot2_bf16(w[q].z, v[4 * q + 2], p0);
    p0 = dot2_bf16(w[q].w, v[4 * q + 3], p0);
  }
#pragma unroll
  for (int q = 2; q < 4; ++q) {
    p1 = dot2_bf16(w[q].x, v[4 * q], p1);
    p1 = dot2_bf16(w[q].y, v[4 * q + 1], p1);
    p1 = dot2_bf16(w[q].z, v[4 * q + 2], p1);
    p1 = dot2_bf16(w[q].w, v[4 * q + 3], p1);
  }
  return p0 + p1;
}

// rows 2p, 2p + 1 of the gate matrix at g and of the up matrix `up` elements
// after it
__device__ __forceinline__ void item_load(GUItemBF& it, const uint16_t* g, size_t up, int p, int lane) {
#pragma unroll
  for (int rr = 0; rr < 2; ++rr)
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        it.c[rr][m][q] = ldg_nt(g + m * up + (size_t)(2 * p + rr) * FL_H + 32 * lane + 8 * q);
}

__device__ __forceinline__ uint32_t item_h(const GUItemBF& it, float gsc, float usc, const XChunk<FMT_NVFP4>& xn) {
  float h[2];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const float g = group_sum<64>(dot32_bf16(it.c[rr][0], xn.v));
    const float u = group_sum<64>(dot32_bf16(it.c[rr][1], xn.v));
    const float gv = round_bf16(g * gsc), uv = round_bf16(u * usc);
    h[rr] = round_bf16(silu_f32(gv)) * uv;
  }
  return pack_bf16x2(h[0], h[1]);
}

// rows row0 + 4 rw + grp of the [H][I] matrix w, columns 32 li .. + 31
__device__ __forceinline__ void down_load(DownRowsBF& d, const uint16_t* w, int row0, int lane) {
  const int grp = lane >> 4, li = lane & 15;
#pragma unroll
  for (int rw = 0; rw < 2; ++rw)
#pragma unroll
    for (int q = 0; q < 4; ++q) d.c[rw][q] = ldg_nt(w + (size_t)(row0 + 4 * rw + grp) * FL_I + 32 * li + 8 * q);
}

__device__ __forceinline__ void down_dot(float (&acc)[2], const DownRowsBF& d, const uint32_t* hrow, float f, int lane) {
  const int li = lane & 15;
  uint32_t hx[16];
  const uint4* hp = reinterpret_cast<const uint4*>(hrow + 16 * li);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = hp[i];
    hx[4 * i] = v.x; hx[4 * i + 1] = v.y; hx[4 * i + 2] = v.z; hx[4 * i + 3] = v.w;
  }
#pragma unroll
  for (int rw = 0; rw < 2; ++rw) acc[rw] = fmaf(f, dot32_bf16(d.c[rw], hx), acc[rw]);
}

// Loads of a layer that do not depend on its input, issued early: this
// lane's 32 columns of gamma and of router row b (wave 0), the shared
// expert's gate/up item b and its two tensor scales (wave 1), the
// tensor-scale table entries.
template <int WF>
struct FlintPreT {
  uint4 g[4], r[4];
  typename FlRows<WF>::Item sh;
  GsPre gs;
  float shs[2];
};
using FlintPre = FlintPreT<FMT_NVFP4>;

template <int WF>
__device__ __forceinline__ void flint_prefetch(FlintPreT<WF>& p, const LayerArgs& a, bool norm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.x;
  const uint16_t* gsrc = norm ? a.gamma : a.x;     // without the norm the gamma loads are dummies
#pragma unroll
  for (int i = 0; i < 4; ++i) p.g[i] = ldg<uint4>(gsrc + 32 * lane + 8 * i);
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) p.r[i] = ldg<uint4>(a.router + (size_t)b * FL_H + 32 * lane + 8 * i);
  }
  if constexpr (WF == FMT_NVFP4) {
    if (wave == 1) {
      item_load(p.sh, a.sh_gu_codes, a.sh_gu_scales, b, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j) p.shs[j] = __hip_atomic_load(a.sh_gscale + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    gs_prefetch(p.gs, a.gscale, a.sh_gscale, FL_E);
  } else {                                         // BF16 weights carry no tensor scales
    if (wave == 1) item_load(p.sh, a.sh_gu_bf16, (size_t)FL_I * FL_H, b, lane);
    p.shs[0] = p.shs[1] = 1.f;
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int j = 0; j < 3; ++j) p.gs.v[q][j] = 1.f;
  }
}

// One layer; returns the epoch its hand-off words carry.  In a layer stack
// (STACK) the token comes from LDS (lds_x) and the workgroup's output rows
// go to LDS (lds_out); otherwise both are a.x and a.out in global memory.
template <bool STACK, int KC, int WF = FMT_NVFP4>
__device__ __forceinline__ uint32_t flint_layer(const LayerArgs& a, const DecodeWs& ws, const FlintPreT<WF>& pre,
                                                uint32_t epoch, uint32_t lim, const uint16_t* lds_x,
                                                uint16_t* lds_out) {
  __shared__ float s_gs[FL_E + 1][3];
  __shared__ int s_exp[FL_SLOTS];
  __shared__ float s_w[FL_SLOTS];
  __shared__ int s_sel_e[FLINT_MAX_TOP_K];
  __shared__ float s_sel_w[FLINT_MAX_TOP_K];
  __shared__ __align__(16) uint32_t s_h[FL_SLOTS][FL_IW];
  __shared__ float s_red[FL_NW][FL_ROWS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.x;
  const int K = KC ? KC : a.K;                     // the top-k, a constant when KC > 0
  const bool norm = (a.flags & FLINT_PRE_RMSNORM) != 0;
  const bool resid = (a.flags & FLINT_RESIDUAL) != 0;
  uint64_t* lw_all = ws.logit_words;               // [replica][E]
  uint64_t* hw_all = ws.h_words;                   // [replica][slot][IW]
  constexpr size_t HREP = (size_t)FL_SLOTS * FL_IW;
  const int rep = b % kReplicas;

  // ---- the token: every wave holds columns 32 lane .. 32 lane + 31 -------
  XChunk<FMT_NVFP4> xn;
  {
    uint4 xv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      xv[i] = STACK ? reinterpret_cast<const uint4*>(lds_x)[4 * lane + i] : ldg<uint4>(a.x + 32 * lane + 8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xn.v[4 * i] = xv[i].x; xn.v[4 * i + 1] = xv[i].y; xn.v[4 * i + 2] = xv[i].z; xn.v[4 * i + 3] = xv[i].w;
    }
  }
  // residual of output row 8b + (threadIdx.x & 7): an unconditional load (a
  // conditional one would be waited for at once)
  const int xr = FL_ROWS * b + (threadIdx.x & (FL_ROWS - 1));
  const float xres = bf16_bits_to_f32(STACK ? lds_x[xr] : ldg<uint16_t>(a.x + xr));
  gs_store(pre.gs, s_gs, FL_E);
  if (norm) {
    double ss = 0.0;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const double lo = bf16_lo(xn.v[m]), hi = bf16_hi(xn.v[m]);
      ss = fma(lo, lo, ss);
      ss = fma(hi, hi, ss);
    }
    ss = wave_sum_f64(ss);
    const Rms rms = make_rms(sqrt(ss / (double)FL_H + (double)a.eps));
    uint32_t gv[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gv[4 * i] = pre.g[i].x; gv[4 * i + 1] = pre.g[i].y; gv[4 * i + 2] = pre.g[i].z; gv[4 * i + 3] = pre.g[i].w;
    }
    rms_norm_words<16>(xn.v, gv, rms);
  }

  // ---- phase 1 --------------------------------------------------------------
  if (wave == 0) {                                 // router logit of expert b
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      part = dot2_bf16(pre.r[i].x, xn.v[4 * i], part);
      part = dot2_bf16(pre.r[i].y, xn.v[4 * i + 1], part);
      part = dot2_bf16(pre.r[i].z, xn.v[4 * i + 2], part);
      part = dot2_bf16(pre.r[i].w, xn.v[4 * i + 3], part);
    }
    put_word_all(lw_all, FL_E, b, epoch, __float_as_uint(group_sum<64>(part)));
  } else if (wave == 1) {                          // shared expert item b
    put_word_all(hw_all, HREP, b, epoch, item_h(pre.sh, pre.shs[0], pre.shs[1], xn));
  }

  // ---- phase 2: top-k on wave 0 ---------------------------------------------
  // Lane l holds the logits of experts 4l..4l+3.  Each round takes the wave
  // maximum of the lanes' best 32-bit logit keys; among the lanes holding
  // it, the lowest lane has the lowest expert index (experts rise with the
  // lane), so it wins and pops its key: equal logits go to the lower index
  // with no second reduction and no branch.  Wave 0 then writes the slot
  // table (expert ids in ascending order) and the other waves start their
  // loads; the combine weights (sigmoid, renorm) are computed afterwards,
  // while those loads are in flight.
  float my_logit = 0.f;
  int my_e = 0, my_rank = 0;
  if (wave == 0) {
    uint64_t wd[4];
    poll_lane_words4(wd, lw_all + (size_t)rep * FL_E, epoch, ws.error, lim);
    uint64_t key[4];
    logit_keys(key, wd);
    const uint64_t my_key = topk_lane_key<KC>(key, K);   // lane k: the k-th selected key
    my_e = (int)~(uint32_t)my_key;
    my_logit = float_from_order_key((uint32_t)(my_key >> 32));
#pragma unroll
    for (int k = 0; k < FLINT_MAX_TOP_K; ++k)      // rank among the selected: ascending slot
      if (k < K) my_rank += __builtin_amdgcn_readlane(my_e, k) < my_e ? 1 : 0;
    if (lane < K) {
      s_exp[1 + my_rank] = my_e;
      s_sel_e[lane] = my_e;
    }
    if (lane == 0) s_exp[0] = -1;
  }
  __syncthreads();

  // ---- phase 3: routed gate/up items and down rows ---------------------------
  // wave w < K: item K b + w (every workgroup takes K of the K * 256 items);
  // down slot ds = 7 - w (slot 0 the shared expert, loaded in phase 1 by
  // wave 7; routed slots 1..K), and on wave 7 slot 8 when k = 8.
  const bool has_item = wave < K;
  const int item = K * b + (has_item ? wave : 0);
  const int islot = item / FL_IW, ip = item - islot * FL_IW;
  const int ie = __builtin_amdgcn_readfirstlane(s_exp[1 + islot]);
  typename FlRows<WF>::Item it;
  if (has_item) {
    constexpr size_t MC = (size_t)FL_I * FL_H / 2, MS = (size_t)FL_I * FL_H / 16, MB = (size_t)FL_I * FL_H;
    if constexpr (WF == FMT_NVFP4)
      item_load(it, a.gu_codes + (size_t)(2 * ie) * MC, a.gu_scales + (size_t)(2 * ie) * MS, ip, lane);
    else
      item_load(it, a.gu_bf16 + (size_t)(2 * ie) * MB, MB, ip, lane);
  }
  if (wave == 0) {                                 // combine weights, off the load path
    const float my_s = lane < K ? 1.0f / (1.0f + expf(-my_logit)) : 0.f;
    float ssum = 0.f;
#pragma unroll
    for (int k = 0; k < FLINT_MAX_TOP_K; ++k)     // selection order, like the split path
      if (k < K) ssum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), k));
    const float w = (a.flags & FLINT_RENORM) ? my_s / ssum : my_s;
    if (lane < K) {
      s_w[1 + my_rank] = w;
      s_sel_w[lane] = w;
    }
    if (lane == 0) s_w[0] = 1.f;
  }
  if (has_item)
    put_word_all(hw_all, HREP, (size_t)(1 + islot) * FL_IW + ip, epoch, item_h(it, s_gs[ie][0], s_gs[ie][1], xn));

  // ---- phase 4: every h word, then down + combine ----------------------------
  // Polling starts once this workgroup's own items are out: waves without
  // an item would otherwise re-request unready words every round trip while
  // the weights are still streaming.  The down rows are requested only now
  // too (they are needed after the h exchange, and requested earlier they
  // would take bandwidth from the gate/up rows that the exchange waits for).
  __syncthreads();
  const int ds1 = 7 - wave;
  const bool has_d1 = ds1 >= 1 && ds1 <= K, has_d2 = wave == 7 && K == 8;
  const int de1 = __builtin_amdgcn_readfirstlane(s_exp[has_d1 ? ds1 : 1]);
  const int de2 = __builtin_amdgcn_readfirstlane(s_exp[has_d2 ? 8 : 1]);
  typename FlRows<WF>::Down d1, d2, dsh;           // dsh: the shared expert's (slot 0) on wave 7
  constexpr size_t DC = (size_t)FL_H * FL_I / 2, DS = (size_t)FL_H * FL_I / 16, DB = (size_t)FL_H * FL_I;
  if constexpr (WF == FMT_NVFP4) {
    if (has_d1) down_load(d1, a.d_codes + (size_t)de1 * DC, a.d_scales + (size_t)de1 * DS, FL_ROWS * b, lane);
    if (wave == 7) down_load(dsh, a.sh_d_codes, a.sh_d_scales, FL_ROWS * b, lane);
    if (has_d2) down_load(d2, a.d_codes + (size_t)de2 * DC, a.d_scales + (size_t)de2 * DS, FL_ROWS * b, lane);
  } else {
    if (has_d1) down_load(d1, a.d_bf16 + (size_t)de1 * DB, FL_ROWS * b, lane);
    if (wave == 7) down_load(dsh, a.sh_d_bf16, FL_ROWS * b, lane);
    if (has_d2) down_load(d2, a.d_bf16 + (size_t)de2 * DB, FL_ROWS * b, lane);
  }
  {
    const uint64_t* hw = hw_all + (size_t)rep * HREP;
    // words per thread: (1 + k) slots of 256 words over 512 threads
    constexpr int NPOLL = ((1 + (KC ? KC : FLINT_MAX_TOP_K)) * FL_IW + 511) / 512;
    const int nw = (1 + K) * FL_IW;
    uint64_t wd[NPOLL];
    const uint64_t* ptr[NPOLL];
    bool ok[NPOLL];
#pragma unroll
    for (int u = 0; u < NPOLL; ++u) {
      const int q = threadIdx.x + 512 * u;
      ok[u] = q < nw;
      ptr[u] = hw + (ok[u] ? q : 0);
    }
    poll_words<NPOLL>(wd, ptr, ok, epoch, ws.error, lim);
#pragma unroll
    for (int u = 0; u < NPOLL; ++u)
      if (ok[u]) (&s_h[0][0])[threadIdx.x + 512 * u] = (uint32_t)wd[u];
  }
  __syncthreads();
  float acc[2] = {0.f, 0.f};
  if (wave == 7) down_dot(acc, dsh, s_h[0], s_gs[FL_E][2], lane);
  if (has_d1) down_dot(acc, d1, s_h[ds1], s_w[ds1] * s_gs[de1][2], lane);
  if (has_d2) down_dot(acc, d2, s_h[8], s_w[8] * s_gs[de2][2], lane);
  {
    const int grp = lane >> 4;
#pragma unroll
    for (int rw = 0; rw < 2; ++rw) {
      const float v = group_sum<16>(acc[rw]);
      if ((lane & 15) == 0) s_red[wave][4 * rw + grp] = v;
    }
  }
  __syncthreads();
  if (threadIdx.x < FL_ROWS) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < FL_NW; ++w) v += s_red[w][threadIdx.x];
    float o = round_bf16(v);
    if (resid) o = xres + o;
    if constexpr (STACK) lds_out[FL_ROWS * b + threadIdx.x] = f32_to_bf16_bits(o);
    else a.out[FL_ROWS * b + threadIdx.x] = f32_to_bf16_bits(o);
  }
  if (b == 0 && (int)threadIdx.x < K) {
    a.topk_idx[threadIdx.x] = s_sel_e[threadIdx.x];
    a.topk_w[threadIdx.x] = s_sel_w[threadIdx.x];
  }
  return epoch;
}

template <int KC, int WF>
__global__ __launch_bounds__(512) void flint_b1_kernel(LayerArgs a_arg, DecodeWs ws_arg) {
  const LayerArgs a = pin_layer_args(a_arg);
  const DecodeWs ws = pin_decode_ws(ws_arg);
  FlintPreT<WF> pre;
  flint_prefetch(pre, a, (a.flags & FLINT_PRE_RMSNORM) != 0);
  const uint32_t epoch = __hip_atomic_load(ws.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  const uint32_t lim = wait_limit(ws);
  flint_layer<false, KC, WF>(a, ws, pre, epoch, lim, nullptr, nullptr);
  // Every workgroup published its logit with the epoch it read at its start,
  // and workgroup 0 saw all of them before its top-k: none of this launch can
  // still be about to read the old value.
  if (blockIdx.x == 0 && threadIdx.x == 0) *ws.epoch = epoch;
}

// A wave-uniform 64-bit value read from LDS, into scalar registers.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32) |
         (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
}

// A stack of pre-norm residual layers for one token (flint_moe_decode_stack)
// at the Flint shape: the layer body above, run layer after layer by the
// same grid.  The residual lives in LDS; after layer l each workgroup
// publishes its 8 output rows (two BF16 per tagged word, one copy per XCD)
// and polls every row before layer l + 1 starts.  While it waits, the next
// layer's input-independent loads (router row, gamma, shared-expert item,
// tensor-scale table) are already in flight, and the weight pointers of the
// layer after it are read (vector loads into LDS, never scalar loads).
// Layer l's words carry epoch + 1 + l; a workgroup reaches layer l + 1's
// hand-offs only after every workgroup has finished reading layer l's
// (it needs all of their output rows first), so no word is overwritten
// while another workgroup still needs it.
template <int KC>
__global__ __launch_bounds__(512) void flint_stack_kernel(StackArgs sa_arg, DecodeWs ws_arg) {
  constexpr int NPTR = sizeof(flint_moe_weights) / sizeof(uint64_t);
  static_assert(NPTR <= 16, "pointer table");
  __shared__ __align__(16) uint16_t s_x[FL_H];      // the residual entering the layer
  __shared__ __align__(16) uint16_t s_xo[FL_H];     // this workgroup's rows of its output
  __shared__ uint64_t s_lp[2][16];                  // weight pointers of layer l in slot l & 1
  StackArgs sa = sa_arg;
  sa.base.K = pin_sgpr(sa_arg.base.K); sa.base.flags = pin_sgpr(sa_arg.base.flags);
  sa.base.eps = pin_sgpr(sa_arg.base.eps);
  sa.layers = pin_sgpr(sa_arg.layers); sa.gammas = pin_sgpr(sa_arg.gammas);
  sa.x_in = pin_sgpr(sa_arg.x_in); sa.x_out = pin_sgpr(sa_arg.x_out);
  sa.topk_idx = pin_sgpr(sa_arg.topk_idx); sa.topk_w = pin_sgpr(sa_arg.topk_w);
  sa.layer_out = pin_sgpr(sa_arg.layer_out); sa.L = pin_sgpr(sa_arg.L);
  const DecodeWs ws = pin_decode_ws(ws_arg);
  const int K = sa.base.K, L = sa.L;
  const int b = blockIdx.x, rep = b % kReplicas;
  const uint64_t* tab = reinterpret_cast<const uint64_t*>(sa.layers);
  reinterpret_cast<uint64_t*>(s_x)[threadIdx.x] = ldg<uint64_t>(sa.x_in + 4 * threadIdx.x);
  if (threadIdx.x < NPTR) {
    s_lp[0][threadIdx.x] = ldg<uint64_t>(tab + threadIdx.x);
    s_lp[1][threadIdx.x] = ldg<uint64_t>(tab + (size_t)(L > 1 ? 1 : 0) * NPTR + threadIdx.x);
  }
  const uint32_t epoch0 = __hip_atomic_load(ws.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t lim = wait_limit(ws);
  __syncthreads();
  // the layer arguments of slot s (pointers from LDS, shape from the base)
  auto layer_args = [&](int s, int l) {
    const uint64_t* lp = s_lp[s];
    LayerArgs a = sa.base;
    a.router = reinterpret_cast<const uint16_t*>(uniform_u64(lp[0]));
    a.gu_codes = reinterpret_cast<const uint8_t*>(uniform_u64(lp[1]));
    a.gu_scales = reinterpret_cast<const uint8_t*>(uniform_u64(lp[2]));
    a.d_codes = reinterpret_cast<const uint8_t*>(uniform_u64(lp[3]));
    a.d_scales = reinterpret_cast<const uint8_t*>(uniform_u64(lp[4]));
    a.gscale = reinterpret_cast<const float*>(uniform_u64(lp[5]));
    a.sh_gu_codes = reinterpret_cast<const uint8_t*>(uniform_u64(lp[6]));
    a.sh_gu_scales = reinterpret_cast<const uint8_t*>(uniform_u64(lp[7]));
    a.sh_d_codes = reinterpret_cast<const uint8_t*>(uniform_u64(lp[8]));
    a.sh_d_scales = reinterpret_cast<const uint8_t*>(uniform_u64(lp[9]));
    a.sh_gscale = reinterpret_cast<const float*>(uniform_u64(lp[10]));
    a.gamma = sa.gammas + (size_t)l * FL_H;
    a.topk_idx = sa.topk_idx + (size_t)l * K;
    a.topk_w = sa.topk_w + (size_t)l * K;
    return a;
  };
  FlintPre pre;
  flint_prefetch(pre, layer_args(0, 0), true);
  uint64_t nxt = 0;                                // layer l + 2's pointer (lanes < NPTR)
  uint32_t epoch = epoch0;
  for (int l = 0; l < L; ++l) {
    // layer l + 1's pointers, read during the previous exchange, go to the
    // slot layer l - 1 used
    if (l >= 1 && l + 1 < L && threadIdx.x < NPTR) s_lp[(l + 1) & 1][threadIdx.x] = nxt;
    const LayerArgs a = layer_args(l & 1, l);
    epoch = flint_layer<true, KC>(a, ws, pre, epoch0 + 1u + (uint32_t)l, lim, s_x, s_xo);
    if (l + 1 < L) {
      flint_prefetch(pre, layer_args((l + 1) & 1, l + 1), true);
      // unconditional (clamped): a conditional load merged with the old
      // value would be waited for at once
      const int l2 = l + 2 < L ? l + 2 : L - 1;
      const int f = (int)threadIdx.x < NPTR ? (int)threadIdx.x : NPTR - 1;
      nxt = ldg<uint64_t>(tab + (size_t)l2 * NPTR + f);
    }
    __syncthreads();                               // this workgroup's rows of x_{l+1} are in s_xo
    if (threadIdx.x < FL_ROWS) {
      const int n = FL_ROWS * b + threadIdx.x;
      if (sa.layer_out) sa.layer_out[(size_t)l * FL_H + n] = s_xo[n];
      if (l + 1 == L) sa.x_out[n] = s_xo[n];
    }
    if (l + 1 == L) break;
    // publish this workgroup's rows (pairs n, n+1), one replica per thread
    if (threadIdx.x < (FL_ROWS / 2) * kReplicas) {
      const int wq = threadIdx.x / kReplicas, r = threadIdx.x % kReplicas, n = FL_ROWS * b + 2 * wq;
      put_word(ws.x_words + (size_t)r * (FL_H / 2) + n / 2, epoch,
               (uint32_t)s_xo[n] | ((uint32_t)s_xo[n + 1] << 16));
    }
    // and take every row of x_{l+1}
    {
      const uint64_t* xw = ws.x_words + (size_t)rep * (FL_H / 2);
      uint64_t wd[2];
      const uint64_t* ptr[2] = {xw + threadIdx.x, xw + threadIdx.x + 512};
      const bool ok[2] = {true, true};
      poll_words<2>(wd, ptr, ok, epoch, ws.error, lim);
      reinterpret_cast<uint32_t*>(s_x)[threadIdx.x] = (uint32_t)wd[0];
      reinterpret_cast<uint32_t*>(s_x)[threadIdx.x + 512] = (uint32_t)wd[1];
    }
    __syncthreads();
  }
  if (b == 0 && threadIdx.x == 0) *ws.epoch = epoch;
}

}  // namespace

bool flint_b1_supported(const LayerArgs& a) {
  if (a.B != 1) return false;
  if (a.H != FL_H || a.E != FL_E || a.I != FL_I || a.SI != FL_I || a.K > FLINT_MAX_TOP_K) return false;
  if (device_num_cu() < FL_G) return false;
  static int per_cu = -1;                          // co-residency of the grid (see fused.hip), every form
  if (per_cu == -1) {
    int ndev = 0, n[4] = {0, 0, 0, 0};
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0) per_cu = -2;
    else {
      const bool ok =
          hipOccupancyMaxActiveBlocksPerMultiprocessor(&n[0], flint_b1_kernel<0, FMT_NVFP4>, 512, 0) == hipSuccess &&
          hipOccupancyMaxActiveBlocksPerMultiprocessor(&n[1], flint_b1_kernel<6, FMT_NVFP4>, 512, 0) == hipSuccess &&
          hipOccupancyMaxActiveBlocksPerMultiprocessor(&n[2], flint_b1_kernel<0, FMT_BF16>, 512, 0) == hipSuccess &&
          hipOccupancyMaxActiveBlocksPerMultiprocessor(&n[3], flint_b1_kernel<6, FMT_BF16>, 512, 0) == hipSuccess;
      int m = n[0];
      for (int i = 1; i < 4; ++i) m = n[i] < m ? n[i] : m;
      per_cu = ok ? m : -2;
    }
  }
  return per_cu == -2 || (int64_t)per_cu * device_num_cu() >= FL_G;
}

hipError_t launch_flint_b1(const LayerArgs& a, const DecodeWs& ws, hipStream_t st) {
  // the usual top-6 as a compile-time constant (straight-line selection)
  const bool bf = (a.flags & FLINT_W_BF16) != 0;
  if (a.K == 6 && bf) hipLaunchKernelGGL((flint_b1_kernel<6, FMT_BF16>), dim3(FL_G), dim3(512), 0, st, a, ws);
  else if (bf) hipLaunchKernelGGL((flint_b1_kernel<0, FMT_BF16>), dim3(FL_G), dim3(512), 0, st, a, ws);
  else if (a.K == 6) hipLaunchKernelGGL((flint_b1_kernel<6, FMT_NVFP4>), dim3(FL_G), dim3(512), 0, st, a, ws);
  else hipLaunchKernelGGL((flint_b1_kernel<0, FMT_NVFP4>), dim3(FL_G), dim3(512), 0, st, a, ws);
  return hipGetLastError();
}

hipError_t launch_flint_stack(const StackArgs& sa, const DecodeWs& ws, hipStream_t st) {
  if (sa.base.K == 6) hipLaunchKernelGGL(flint_stack_kernel<6>, dim3(FL_G), dim3(512), 0, st, sa, ws);
  else hipLaunchKernelGGL(flint_stack_kernel<0>, dim3(FL_G), dim3(512), 0, st, sa, ws);
  return hipGetLastError();
}

}  // namespace flint
