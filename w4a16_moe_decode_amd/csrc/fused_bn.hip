// Single-launch decode MoE layer for 2..8 tokens, NVFP4 weights.
//
// The same layer as the three-kernel path (decode.hip) and the one-token
// single launch (fused.hip), for the rest of the low-latency path of "Day-0
// Support for Flint on vLLM" ("Optimizations": up to 8 concurrent requests,
// routing and the expert combine fused into the neighbouring GEMVs, each
// selected expert's weights read once for every token routed to it):
//
//   phase 0  the tokens (RMS-normalised when asked) are staged in LDS
//   phase 1  router logits of every token (one expert per workgroup, a
//            quarter row per wave) and the shared expert's gate/up rows
//   phase 2  every workgroup waits for all logits; wave w selects the top-k
//            of tokens w and w + 4.  The union of the selected experts, in
//            ascending index order, is the slot table: each slot holds its
//            token mask and, per token, the (token, k) pair its h goes to
//   phase 3  routed gate/up row pairs, dealt round-robin over all waves with
//            three items in flight per wave; an item's weights are read once
//            and applied to every token routed to its expert
//   phase 4  every workgroup waits for the h of all (token, expert) pairs,
//            then computes its output rows for every token: weighted combine
//            of the selected experts and the shared expert, one BF16
//            rounding (+ residual)
//
// Hand-offs use the epoch-tagged words of the one-token kernel; every wait is
// bounded.  Loads whose item does not exist are pointed at the first item
// (an L2 hit) instead of being skipped, so that no load is conditional and
// the in-order completion count lets each item wait only for its own rows.
#include "fused_common.hpp"

namespace flint {
namespace {

constexpr int kBT = FLINT_MAX_DECODE_BATCH;
constexpr int kKM = FLINT_MAX_TOP_K;
constexpr int kPairStride = kBT * (kKM + 1);       // pairs per h-word replica
constexpr int kSlotsBn = kBT * kKM + 1;
constexpr int kPoolWords = 64 * 1024 / 4;          // tokens, then h (packed BF16 pairs)
constexpr int kDownSlots = 6;                      // down items in flight per wave

// Pointers of the gate and up planes of a selected expert (-1 = shared).
__device__ __forceinline__ GURows bn_rows(const LayerArgs& a, int expert) {
  GURows r;
  const int H = a.H;
  r.inter = expert < 0 ? a.SI : a.I;
  const size_t mc = (size_t)r.inter * H / 2, ms = (size_t)r.inter * H / 16;
  if (expert < 0) {
    r.gc = a.sh_gu_codes;
    r.gs = a.sh_gu_scales;
  } else {
    r.gc = a.gu_codes + (size_t)(2 * expert) * mc;
    r.gs = a.gu_scales + (size_t)(2 * expert) * ms;
  }
  r.uc = r.gc + mc;
  r.us = r.gs + ms;
  r.g_scale = r.u_scale = 0.f;
  return r;
}

// Gate/up of one row pair for the tokens of `mask`, one token at a time (a
// loop, not unrolled, so that the code stays small).  Token j of the mask
// (j-th set bit) has its packed BF16 pair h[2p], h[2p+1] stored by lanes
// 8j..8j+7, one replica each, at pair `pair[t]` (pair t when pair is null).
// The loop holds no global memory access and reads no register that a
// pending load writes, and there is exactly one store per item: the
// compiler can then wait for each item's own loads only.
template <int NCH>
__device__ __forceinline__ void gu_tokens(const GUItem<NCH>& it, float gsg_in, float gsu_in, const uint32_t* s_x,
                                          int Hw, uint32_t mask, const uint8_t* pair, uint64_t* hw_all,
                                          size_t hrep, int hstride, int p, uint32_t epoch) {
  const int lane = threadIdx.x & 63;
  const float gsg = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gsg_in)));
  const float gsu = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gsu_in)));
  DChunk<FMT_NVFP4> d[2][2][NCH];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr)
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int c = 0; c < NCH; ++c) d[rr][m][c] = decode_nvfp4(it.c[rr][m][c], it.s[rr][m][c]);
  uint32_t myword = 0u;
  int mypair = 0, j = 0;
#pragma unroll 1
  for (uint32_t rest = mask; rest != 0u; rest &= rest - 1u, ++j) {
    const int t = __builtin_ctz(rest);             // the same in every lane
    float acc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      XChunk<FMT_NVFP4> xc;
      const uint4* xp = reinterpret_cast<const uint4*>(s_x + t * Hw + 16 * (lane + 64 * c));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = xp[i];
        xc.v[4 * i + 0] = v.x; xc.v[4 * i + 1] = v.y; xc.v[4 * i + 2] = v.z; xc.v[4 * i + 3] = v.w;
      }
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
#pragma unroll
        for (int m = 0; m < 2; ++m) acc[rr][m] += chunk_dot(d[rr][m][c], xc);
    }
    float h[2];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const float gv = round_bf16(group_sum<64>(acc[rr][0]) * gsg);
      const float uv = round_bf16(group_sum<64>(acc[rr][1]) * gsu);
      h[rr] = round_bf16(silu_f32(gv)) * uv;
    }
    if ((lane >> 3) == j) {
      myword = pack_bf16x2(h[0], h[1]);
      mypair = pair ? pair[t] : t;
    }
  }
  if ((lane >> 3) < j)
    put_word(hw_all + (size_t)(lane & (kReplicas - 1)) * hrep + (size_t)mypair * hstride + p, epoch, myword);
}

struct DItem { uint4 raw[2]; uint32_t sc[2]; float gd; };

template <int NCH, int GD, int DW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fused_decode_bn_kernel(LayerArgs a, DecodeWs ws) {
  constexpr int GPW = 64 / GD;
  constexpr int DROWS = DW * GPW;                  // output rows per workgroup
  __shared__ float s_lp[4][kBT];
  __shared__ uint32_t s_emask[FLINT_MAX_EXPERTS];  // tokens that selected expert e
  __shared__ float s_ew[FLINT_MAX_EXPERTS][kBT];   // their combine weights
  __shared__ uint8_t s_ek[FLINT_MAX_EXPERTS][kBT]; // and the selection rank k
  __shared__ int s_cnt[4];
  __shared__ int s_nU;
  __shared__ int s_slot_e[kSlotsBn];
  __shared__ uint32_t s_slot_mask[kSlotsBn];
  __shared__ float s_slot_w[kSlotsBn][kBT];
  __shared__ uint8_t s_slot_pair[kSlotsBn][kBT];
  __shared__ double s_rms[kBT];
  __shared__ float s_red[4][DROWS][kBT];
  __shared__ uint32_t s_pool[kPoolWords];          // tokens [B][H/2], later h [pair][hstride]

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int G = gridDim.x, NWV = 4 * G, gw = blockIdx.x * 4 + wave;
  const int H = a.H, E = a.E, K = a.K, I = a.I, SI = a.SI, B = a.B;
  const bool has_sh = SI > 0;
  const int sh = has_sh ? 1 : 0;
  const bool norm = (a.flags & FLINT_PRE_RMSNORM) != 0;
  const int Hw = H / 2;
  const int hstride = (I > SI ? I : SI) / 2;
  const size_t hrep = (size_t)kPairStride * hstride;
  const size_t lrep = (size_t)kBT * E;
  uint64_t* lw_all = ws.logit_words;               // [kReplicas][kBT][E]
  uint64_t* hw_all = ws.h_words;                   // [kReplicas][pair][hstride]
  const int rep = blockIdx.x % kReplicas;
  const uint64_t* lw = lw_all + (size_t)rep * lrep;
  const uint64_t* hw = hw_all + (size_t)rep * hrep;
  uint32_t* s_x = s_pool;
  uint32_t* s_h = s_pool;

  // ---- tokens first (L2 hits), then the weights that need nothing ---------------
  // Loads complete in order: issuing the tokens before the HBM weight loads
  // lets the LDS staging wait for the tokens alone.
  constexpr int kXPer = kBT * 2048 * NCH / 8 / 256;   // 16-byte token chunks per thread, at most
  const int nxq = B * (H / 8);
  uint4 xv[kXPer];
#pragma unroll
  for (int i = 0; i < kXPer; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int qc = q < nxq ? q : 0;
    const int t = qc / (H / 8), c = 8 * (qc - t * (H / 8));
    xv[i] = *reinterpret_cast<const uint4*>(a.x + (size_t)t * H + c);
  }
  // the launch epoch (a vector load, so that waiting for it does not hold up
  // the kernel arguments), the first router row, then the shared expert
  const uint32_t epoch = __hip_atomic_load(ws.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  const int qlen = H / 4;                          // router columns per wave
  uint4 rw[NCH];
  const int e0 = (int)blockIdx.x < E ? (int)blockIdx.x : E - 1;   // workgroups past E own no row
#pragma unroll
  for (int c = 0; c < NCH; ++c)
    rw[c] = *reinterpret_cast<const uint4*>(a.router + (size_t)e0 * H + wave * qlen + 8 * lane + 512 * c);
  // shared expert: units (row pair, token group) on waves 1..3, so that no
  // wave carries all tokens of a row pair and wave 0 stays free for the logits
  const int nsh_items = has_sh ? SI / 2 : 0;
  int ngrp = nsh_items > 0 ? (3 * G) / nsh_items : 1;
  ngrp = ngrp < 1 ? 1 : (ngrp > B ? B : ngrp);
  const int tpg = (B + ngrp - 1) / ngrp;           // tokens per group
  ngrp = (B + tpg - 1) / tpg;
  const int nunits = nsh_items * ngrp;
  const int sw = wave == 0 ? -1 : (int)blockIdx.x * 3 + wave - 1;   // shared-unit worker index
  const bool my_sh = sw >= 0 && sw < nunits;
  GUItem<NCH> shit;
  const GURows Rsh = bn_rows(a, -1);
  float sh_gs[2] = {1.f, 1.f};
  if (my_sh) {
    gu_load<NCH>(shit, Rsh, sw / ngrp, H);
    sh_gs[0] = a.sh_gscale[0];
    sh_gs[1] = a.sh_gscale[1];
  }
  s_emask[threadIdx.x] = 0u;                       // 256 threads cover every expert

  // ---- phase 0: tokens -> LDS (then RMS-normalised in place when asked) -------
  // (unconditional stores: a thread past the end rewrites chunk 0 with the
  // value it holds, so no load is sunk into a branch and waited for there)
#pragma unroll
  for (int i = 0; i < kXPer; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int qc = q < nxq ? q : 0;
    const int t = qc / (H / 8), c = 8 * (qc - t * (H / 8));
    *reinterpret_cast<uint4*>(s_x + t * Hw + c / 2) = xv[i];
  }
  __syncthreads();
  announce_arrival(ws, E, epoch);
  if (norm) {
    for (int t = wave; t < B; t += 4) {
      double ss = 0.0;
      for (int c = 8 * lane; c < H; c += 512) {
        const uint4 v = *reinterpret_cast<const uint4*>(s_x + t * Hw + c / 2);
        const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const double lo = bf16_lo(q[m]), hi = bf16_hi(q[m]);
          ss = fma(lo, lo, ss);
          ss = fma(hi, hi, ss);
        }
      }
      ss = wave_sum_f64(ss);
      if (lane == 0) s_rms[t] = sqrt(ss / (double)H + (double)a.eps);
    }
    __syncthreads();
    uint4 gv[kXPer];
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int q = threadIdx.x + 256 * i;
      const int qc = q < nxq ? q : 0;
      gv[i] = *reinterpret_cast<const uint4*>(a.gamma + 8 * (qc % (H / 8)));
    }
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int q = threadIdx.x + 256 * i;
      if (q >= nxq) break;
      const int t = q / (H / 8), c = 8 * (q - t * (H / 8));
      uint4* px = reinterpret_cast<uint4*>(s_x + t * Hw + c / 2);
      const uint4 v = *px;
      const Rms rms = make_rms(s_rms[t]);
      *px = rms_norm_8(v, gv[i], rms);
    }
    __syncthreads();
  }

  // ---- phase 1: router logits of every token ----------------------------------
  for (int e = blockIdx.x; e < E; e += G) {
    if (e != blockIdx.x) {
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        rw[c] = *reinterpret_cast<const uint4*>(a.router + (size_t)e * H + wave * qlen + 8 * lane + 512 * c);
    }
    float part[kBT];
#pragma unroll
    for (int t = 0; t < kBT; ++t) {
      part[t] = 0.f;
      if (t < B) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const uint4 xq = *reinterpret_cast<const uint4*>(s_x + t * Hw + (wave * qlen + 8 * lane + 512 * c) / 2);
          part[t] = dot2_bf16(rw[c].x, xq.x, part[t]);
          part[t] = dot2_bf16(rw[c].y, xq.y, part[t]);
          part[t] = dot2_bf16(rw[c].z, xq.z, part[t]);
          part[t] = dot2_bf16(rw[c].w, xq.w, part[t]);
        }
        part[t] = group_sum<64>(part[t]);
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int t = 0; t < kBT; ++t) s_lp[wave][t] = part[t];
    }
    __syncthreads();
    if (wave == 0) {
      const int t = lane >> 3, r = lane & (kReplicas - 1);
      if (t < B) {
        const float l = s_lp[0][t] + s_lp[1][t] + s_lp[2][t] + s_lp[3][t];
        put_word(lw_all + (size_t)r * lrep + (size_t)t * E + e, epoch, __float_as_uint(l));
      }
    }
    __syncthreads();
  }

  // ---- phase 1: the shared expert's gate/up units ------------------------------
  {
    const uint32_t all = (1u << B) - 1u;
    auto group_mask = [&](int g) {
      const int lo = g * tpg, hi = lo + tpg < B ? lo + tpg : B;
      return (all >> lo << lo) & ((1u << hi) - 1u);
    };
    if (my_sh)
      gu_tokens<NCH>(shit, sh_gs[0], sh_gs[1], s_x, Hw, group_mask(sw % ngrp), nullptr, hw_all, hrep,
                     hstride, sw / ngrp, epoch);
    if (sw >= 0)
      for (int u = sw + 3 * G; u < nunits; u += 3 * G) {   // shared experts wider than the grid
        gu_load<NCH>(shit, Rsh, u / ngrp, H);
        gu_tokens<NCH>(shit, a.sh_gscale[0], a.sh_gscale[1], s_x, Hw, group_mask(u % ngrp), nullptr,
                       hw_all, hrep, hstride, u / ngrp, epoch);
      }
  }

  // ---- phase 2: top-k of tokens wave and wave + 4, then the slot table --------
  {
    uint64_t wd[12];
    const uint64_t* ptr[12];
    bool ok[12];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = wave + 4 * h;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ex = lane + 64 * q;
        ok[4 * h + q] = t < B && ex < E;
        ptr[4 * h + q] = lw + (size_t)(t < B ? t : 0) * E + (ex < E ? ex : 0);
      }
    }
    arrival_slots(ws, E, G, ptr + 8, ok + 8);     // workgroup 0 only
    poll_words<12>(wd, ptr, ok, epoch, ws.error);
    const bool renorm = (a.flags & FLINT_RENORM) != 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = wave + 4 * h;
      if (t >= B) break;                            // the same in every lane
      uint64_t key[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ex = lane + 64 * q;
        key[q] = ok[4 * h + q] ? (((uint64_t)float_order_key(__uint_as_float((uint32_t)wd[4 * h + q])) << 32) |
                                  (uint32_t)~(uint32_t)ex)
                               : 0ull;
      }
      const uint64_t my_key = select_topk(key, K);
      const int my_e = (int)~(uint32_t)my_key;
      const float my_s = lane < K ? 1.0f / (1.0f + expf(-float_from_order_key((uint32_t)(my_key >> 32)))) : 0.f;
      float ssum = 0.f;
      for (int k = 0; k < K; ++k)                   // selection order, like the split path
        ssum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), k));
      const float w = renorm ? my_s / ssum : my_s;
      if (lane < K) {
        atomicOr(&s_emask[my_e], 1u << t);
        s_ew[my_e][t] = w;
        s_ek[my_e][t] = (uint8_t)lane;
        if (blockIdx.x == 0) {
          a.topk_idx[t * K + lane] = my_e;
          a.topk_w[t * K + lane] = w;
        }
      }
    }
  }
  __syncthreads();
  {
    // routed slots: the selected experts in ascending index order; pair of
    // (token t, rank k) = B * sh + t * K + k, the shared pairs are 0..B-1
    const int e = threadIdx.x;
    const uint32_t m = e < E ? s_emask[e] : 0u;
    const unsigned long long bal = __ballot(m != 0u);
    if (lane == 0) s_cnt[wave] = __popcll(bal);
    __syncthreads();
    int base = sh;
    for (int w = 0; w < wave; ++w) base += s_cnt[w];
    if (m != 0u) {
      const int s = base + __popcll(bal & ((1ull << lane) - 1ull));
      s_slot_e[s] = e;
      s_slot_mask[s] = m;
#pragma unroll
      for (int t = 0; t < kBT; ++t) {
        const bool in = (m >> t) & 1u;
        s_slot_w[s][t] = in ? s_ew[e][t] : 0.f;
        s_slot_pair[s][t] = in ? (uint8_t)(B * sh + t * K + s_ek[e][t]) : (uint8_t)0;
      }
    }
    if (threadIdx.x == 0) {
      s_nU = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
      if (has_sh) {
        s_slot_e[0] = -1;
        s_slot_mask[0] = (1u << B) - 1u;
#pragma unroll
        for (int t = 0; t < kBT; ++t) {
          s_slot_w[0][t] = 1.f;
          s_slot_pair[0][t] = (uint8_t)t;
        }
      }
    }
    __syncthreads();
  }
  const int nU = s_nU, S = nU + sh;

  // ---- phase 3: routed gate/up row pairs, three in flight per wave -----------
  {
    const int ipw = I / 2;
    const int nitems = nU * ipw;
    if (gw < nitems) {
      GUItem<NCH> it0, it1, it2;
      float gs0[2], gs1[2], gs2[2];
      auto issue = [&](GUItem<NCH>& it, float (&gs)[2], int item) {
        const int ic = item < nitems ? item : 0;    // past the end: the first item, an L2 hit
        const int r = ic / ipw, p = ic - r * ipw;
        const int e = s_slot_e[sh + r];
        gu_load<NCH>(it, bn_rows(a, e), p, H);
        gs[0] = a.gscale[3 * e + 0];
        gs[1] = a.gscale[3 * e + 1];
      };
      auto finish = [&](const GUItem<NCH>& it, const float (&gs)[2], int item) {
        if (item >= nitems) return;                 // the same in every lane
        const int r = item / ipw, p = item - r * ipw, s = sh + r;
        gu_tokens<NCH>(it, gs[0], gs[1], s_x, Hw, s_slot_mask[s], s_slot_pair[s], hw_all, hrep, hstride, p,
                       epoch);
      };
      issue(it0, gs0, gw);
      issue(it1, gs1, gw + NWV);
      issue(it2, gs2, gw + 2 * NWV);
      for (int b0 = gw; b0 < nitems; b0 += 3 * NWV) {
        finish(it0, gs0, b0);
        issue(it0, gs0, b0 + 3 * NWV);
        finish(it1, gs1, b0 + NWV);
        issue(it1, gs1, b0 + 4 * NWV);
        finish(it2, gs2, b0 + 2 * NWV);
        issue(it2, gs2, b0 + 5 * NWV);
      }
    }
  }

  // ---- phase 4: down rows of this workgroup, for every slot and token --------
  const int n0 = blockIdx.x * DROWS;
  const int ncs = (I > SI ? I : SI) / 32;          // chunk steps of the widest slot
  const int dch = (ncs + GD - 1) / GD;
  const int grp = lane / GD, li = lane % GD;
  const int total = S * dch;                       // items (slot, chunk step), dealt to the waves
  const int nwi = wave < total ? (total - wave + 3) / 4 : 0;
  auto d_issue = [&](DItem& d, int u) {
    const int it = wave + 4 * u;
    const bool valid = it < total;
    const int s = valid ? it / dch : 0, c = valid ? it - s * dch : 0;
    const int e = s_slot_e[s];
    const int inter = e < 0 ? SI : I;
    const int j = li + GD * c;
    const bool ok = valid && j < inter / 32;
    const uint8_t* codes = e < 0 ? a.sh_d_codes : a.d_codes + (size_t)e * H * (inter / 2);
    const uint8_t* scales = e < 0 ? a.sh_d_scales : a.d_scales + (size_t)e * H * (inter / 16);
#pragma unroll
    for (int rw = 0; rw < DW; ++rw) {
      const int n = n0 + rw * GPW + grp;
      const bool okr = ok && n < H;
      const uint8_t* cp = okr ? codes + (size_t)n * (inter / 2) + 16 * j : a.d_codes;
      const uint8_t* sp = okr ? scales + (size_t)n * (inter / 16) + 2 * j : a.d_scales;
      d.raw[rw] = *reinterpret_cast<const uint4*>(cp);
      d.sc[rw] = *reinterpret_cast<const uint16_t*>(sp);
    }
    d.gd = e < 0 ? a.sh_gscale[2] : a.gscale[3 * e + 2];
  };
  DItem di[kDownSlots];
#pragma unroll
  for (int k = 0; k < kDownSlots; ++k) d_issue(di[k], k);

  // residual of the (row, token) this thread writes, fetched early
  const bool resid = (a.flags & FLINT_RESIDUAL) != 0;
  float xres = 0.f;
  if (resid && (int)threadIdx.x < DROWS * B) {
    const int rloc = threadIdx.x / B, t = threadIdx.x - rloc * B, n = n0 + rloc;
    if (n < H) xres = bf16_bits_to_f32(a.x[(size_t)t * H + n]);
  }
  __syncthreads();                                 // every wave is done with the tokens in LDS
  {
    // every (pair, word), kPollPer per thread in flight; words past a narrower
    // slot's width are never written and are skipped
    constexpr int kPollPer = 56;
    const int nw = B * (sh + K) * hstride;
    const bool ragged = has_sh && SI != I;
    for (int q0 = threadIdx.x; q0 < nw; q0 += 256 * kPollPer) {
      uint64_t wd[kPollPer];
      bool ok[kPollPer];
#pragma unroll
      for (int u = 0; u < kPollPer; ++u) {
        const int q = q0 + 256 * u;
        bool v = q < nw;
        if (ragged) {
          const int pr = q / hstride, wq = q - pr * hstride;
          v = v && wq < (pr < B ? SI : I) / 2;
        }
        ok[u] = v;
      }
#pragma unroll
      for (int u = 0; u < kPollPer; ++u)
        wd[u] = ok[u] ? __hip_atomic_load(hw + q0 + 256 * u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                      : ((uint64_t)epoch << 32);
      for (uint32_t spin = 0;; ++spin) {
        bool ready = true;
#pragma unroll
        for (int u = 0; u < kPollPer; ++u) ready = ready && (uint32_t)(wd[u] >> 32) == epoch;
        if (ready) break;
        if (spin >= kFusedSpin) { *ws.error = 1u; break; }
        __builtin_amdgcn_s_sleep(8);
#pragma unroll
        for (int u = 0; u < kPollPer; ++u)
          if ((uint32_t)(wd[u] >> 32) != epoch)
            wd[u] = __hip_atomic_load(hw + q0 + 256 * u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int u = 0; u < kPollPer; ++u)
        if (ok[u]) s_h[q0 + 256 * u] = (uint32_t)wd[u];
    }
  }
  __syncthreads();

  float acc[DW][kBT];
#pragma unroll
  for (int rw = 0; rw < DW; ++rw)
#pragma unroll
    for (int t = 0; t < kBT; ++t) acc[rw][t] = 0.f;
  auto d_use = [&](const DItem& d, int u) {
    const int it = wave + 4 * u;
    if (it >= total) return;                       // the same in every lane
    const int s = it / dch, c = it - s * dch;
    const int e = s_slot_e[s];
    const int inter = e < 0 ? SI : I;
    const int j = li + GD * c;
    if (j >= inter / 32) return;
    const uint32_t mask = s_slot_mask[s];
    const float gd = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(d.gd)));   // per slot
    DChunk<FMT_NVFP4> dd[DW];
#pragma unroll
    for (int rw = 0; rw < DW; ++rw) dd[rw] = decode_nvfp4(d.raw[rw], d.sc[rw]);
#pragma unroll 1
    for (uint32_t rest = mask; rest != 0u; rest &= rest - 1u) {
      const int t = __builtin_ctz(rest);           // the same in every lane
      XChunk<FMT_NVFP4> hx;
      const uint4* hp = reinterpret_cast<const uint4*>(s_h + (size_t)s_slot_pair[s][t] * hstride + 16 * j);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = hp[i];
        hx.v[4 * i + 0] = v.x; hx.v[4 * i + 1] = v.y; hx.v[4 * i + 2] = v.z; hx.v[4 * i + 3] = v.w;
      }
      const float f = s_slot_w[s][t] * gd;
#pragma unroll
      for (int rw = 0; rw < DW; ++rw) acc[rw][t] = fmaf(f, chunk_dot(dd[rw], hx), acc[rw][t]);
    }
  };
  for (int u0 = 0; u0 < nwi; u0 += kDownSlots) {
#pragma unroll
    for (int k = 0; k < kDownSlots; ++k) {
      d_use(di[k], u0 + k);
      d_issue(di[k], u0 + k + kDownSlots);
    }
  }
#pragma unroll
  for (int rw = 0; rw < DW; ++rw)
#pragma unroll
    for (int t = 0; t < kBT; ++t) {
      if (t >= B) break;
      const float v = group_sum<GD>(acc[rw][t]);
      if (li == 0) s_red[wave][rw * GPW + grp][t] = v;
    }
  __syncthreads();
  if ((int)threadIdx.x < DROWS * B) {
    const int rloc = threadIdx.x / B, t = threadIdx.x - rloc * B, n = n0 + rloc;
    if (n < H) {
      const float v = s_red[0][rloc][t] + s_red[1][rloc][t] + s_red[2][rloc][t] + s_red[3][rloc][t];
      float o = round_bf16(v);
      if (resid) o = xres + o;
      a.out[(size_t)t * H + n] = f32_to_bf16_bits(o);
    }
  }

  // ---- advance the epoch for the next launch -----------------------------------
  // As in the one-token kernel: workgroup 0 has seen a logit or an arrival
  // word from every workgroup, each written after that workgroup read the
  // epoch.
  if (blockIdx.x == 0 && threadIdx.x == 0) *ws.epoch = epoch;
}

struct BnConfig { int G, gd, dw, nch; };

bool bn_config(const LayerArgs& a, BnConfig& c) {
  if (a.B < 2 || a.B > kBT || (a.flags & FLINT_W_BF16)) return false;
  if (a.H % 2048 || a.H > 4096) return false;
  if (a.I > 2048 || a.SI > 2048 || a.K > kKM || a.E > FLINT_MAX_EXPERTS) return false;
  const int hstride = (a.I > a.SI ? a.I : a.SI) / 2;
  const int pairs = a.B * (a.K + (a.SI > 0 ? 1 : 0));
  if ((int64_t)pairs * hstride > kPoolWords || a.B * (a.H / 2) > kPoolWords) return false;
  c.nch = a.H / 2048;
  c.G = device_num_cu();
  const int need = (a.H + 7) / 8;
  if (c.G > need) c.G = need;
  if (c.G > a.E + kMaxArrivals) c.G = a.E + kMaxArrivals;
  const int rows_per_wg = (a.H + c.G - 1) / c.G;
  const int red = a.SI > 0 && a.SI < a.I ? a.SI : a.I;
  c.gd = 8;
  while (c.gd < red / 32 && c.gd < 64) c.gd <<= 1;
  c.dw = (rows_per_wg * c.gd + 63) / 64;
  if (c.dw > 2) return false;
  return true;
}

}  // namespace

bool fused_decode_bn_supported(const LayerArgs& a) {
  BnConfig c;
  return bn_config(a, c);
}

hipError_t launch_fused_decode_bn(const LayerArgs& a, const DecodeWs& ws, hipStream_t st) {
  BnConfig c;
  if (!bn_config(a, c)) return hipErrorInvalidConfiguration;
#define FLINT_BN(NCH_, GD_, DW_) \
  hipLaunchKernelGGL((fused_decode_bn_kernel<NCH_, GD_, DW_>), dim3(c.G), dim3(256), 0, st, a, ws)
#define FLINT_BN_GD(NCH_)                                                              \
  switch (c.gd) {                                                                      \
    case 8: if (c.dw <= 1) FLINT_BN(NCH_, 8, 1); else FLINT_BN(NCH_, 8, 2); break;     \
    case 16: if (c.dw <= 1) FLINT_BN(NCH_, 16, 1); else FLINT_BN(NCH_, 16, 2); break;  \
    case 32: if (c.dw <= 1) FLINT_BN(NCH_, 32, 1); else FLINT_BN(NCH_, 32, 2); break;  \
    default: if (c.dw <= 1) FLINT_BN(NCH_, 64, 1); else FLINT_BN(NCH_, 64, 2); break;  \
  }
  if (c.nch == 1) { FLINT_BN_GD(1) } else { FLINT_BN_GD(2) }
#undef FLINT_BN_GD
#undef FLINT_BN
  return hipGetLastError();
}

}  // namespace flint
