// Single-launch decode MoE layer for 2..8 tokens at the Flint shape (hidden
// 2048, 256 routed experts of intermediate 512, one shared expert of
// intermediate 512, top-k <= 8: "Day-0 Support for Flint on vLLM", "Model
// architecture"), on a GPU with at least 256 compute units; one workgroup of
// 8 waves per compute unit, all resident at once.
//
// The same arithmetic as the three-kernel path; the work is split so that
// every workgroup streams an equal share of the selected experts' weights
// and no kernel boundary stands between routing, gate/up and down:
//
//   1. Each workgroup copies the tokens, its router row (workgroup b owns
//      expert b) and gamma into LDS in the layout the gate/up dot products
//      read, and requests its share of the shared expert's gate/up rows
//      (rows 2b and 2b+1).  Wave t normalises token t (PRE_RMSNORM), takes
//      the logit of expert b and publishes it, then computes and publishes
//      the shared rows' h of token t while the other logits arrive.
//   2. Wave t polls the 256 logits of token t and selects its top-k in
//      registers; the selections go to LDS as an expert -> token mask, from
//      which wave 0 lists the routed slots (the selected experts, ascending).
//      Every workgroup does this itself, so the slot list never travels.
//   3. Gate/up: the routed slots' rows form units of 4 rows (128 per
//      expert); wave w takes every 8th of its workgroup's units from w, in a
//      pipeline two units deep.  A unit's h for each token routed to the
//      slot is published as tagged words (two BF16 per word).
//   4. Down: items of 8 output rows of one routed slot (256 per slot, in
//      slot-major order), and the shared expert's rows 8b..8b+7 on
//      workgroup b (wave t: token t).  Units and items are split over the
//      workgroups by cost (phase 3), so a workgroup needs the h of at most
//      two routed slots besides the shared expert's.  Each item's products
//      with its slot's tokens, times the combine weight, are published as
//      partial sums P[token][selection position][row] (position k_max for
//      the shared expert).
//   5. Workgroup b polls the partial sums of its output rows 8b..8b+7 and
//      adds them in a fixed order (selection order, then the shared
//      expert): one BF16 rounding (+ residual).
//
// Hand-offs are epoch-tagged 64-bit words (epoch << 32 | payload) with
// bounded waits; words every workgroup reads (logits, the shared expert's
// h) are published in one copy per XCD.
#include "flint_common.hpp"

namespace flint {
namespace {

constexpr int F8_BT = FLINT_MAX_DECODE_BATCH;      // token slots
constexpr int F8_Q = FL_H / 8;                     // 16-byte words of a token (256)
constexpr int F8_UPE = FL_I / 4;                   // gate/up units per expert (4 rows each)
constexpr int F8_TILES = FL_H / FL_ROWS;           // down row tiles per expert (256)
constexpr int F8_KS = FLINT_MAX_TOP_K;             // partial-sum position of the shared expert
constexpr int F8_PK = FLINT_MAX_TOP_K + 1;         // partial-sum positions per token
constexpr int F8_MAXSLOT = F8_BT * FLINT_MAX_TOP_K;  // routed slots, at most
constexpr int F8_MAXPAIR = 3 * F8_BT;              // h rows a workgroup takes: shared + two routed slots
constexpr size_t F8_MC = (size_t)FL_I * FL_H / 2, F8_MS = (size_t)FL_I * FL_H / 16;  // gate/up plane
constexpr size_t F8_DC = (size_t)FL_H * FL_I / 2, F8_DS = (size_t)FL_H * FL_I / 16;  // down plane
static_assert(F8_TILES == FL_G, "one shared down tile per workgroup");
static_assert(FL_G == 256, "unit and item ranges divide by 256 with shifts");

// A lane's part of a gate/up row: lane li of a 16-lane row group owns the
// 32-column chunks li, li + 16, li + 32, li + 48, so that each load of the
// group reads 256 contiguous bytes of the row.  Staged layout of a token
// (and of the router row and gamma): position q (16 bytes) holds columns
// col(q) .. col(q) + 7, so that lane li reads quad m of its chunk c as
// position (4 c + m) 16 + li: consecutive words.
__device__ __forceinline__ int staged_col(int q) { return 32 * (16 * (q >> 6) + (q & 15)) + 8 * ((q >> 4) & 3); }

// A lane's part of one gate/up unit: its four chunks of its row's gate and
// up rows, with their scales.
struct GU4 {
  uint4 g[4], u[4];
  uint32_t gs[4], us[4];
};

__device__ __forceinline__ void gu4_load(GU4& v, const uint8_t* codes, const uint8_t* scales, int row, int li) {
  const uint8_t* c = codes + (size_t)row * (FL_H / 2) + 16 * li;
  const uint8_t* s = scales + (size_t)row * (FL_H / 16) + 2 * li;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v.g[k] = ldg_nt(c + 256 * k);
    v.u[k] = ldg_nt(c + F8_MC + 256 * k);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v.gs[k] = ldg<uint16_t>(s + 32 * k);
    v.us[k] = ldg<uint16_t>(s + F8_MS + 32 * k);
  }
}

// h of the lane group's row for the staged token at xt (its 256 positions):
// BF16(BF16(SiLU(BF16(g gs_g))) * BF16(u gs_u)), valid in every lane of the
// group.  One token per call: the chunks are decoded again for each token
// of a slot (most slots have one), which keeps the code short.
__device__ __forceinline__ float gu4_h(const GU4& v, const uint4* xt, float gsg, float gsu, int li) {
  float ag = 0.f, au = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    XChunk<FMT_NVFP4> xc;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint4 w = xt[(4 * c + m) * 16 + li];
      xc.v[4 * m] = w.x; xc.v[4 * m + 1] = w.y; xc.v[4 * m + 2] = w.z; xc.v[4 * m + 3] = w.w;
    }
    // opaque copies: the decode stays inside the caller's token loop instead
    // of being hoisted out of it (eight decoded chunks would not fit in
    // registers beside the pipeline's loads)
    uint4 g = v.g[c], u = v.u[c];
    uint32_t gs = v.gs[c], us = v.us[c];
    asm volatile("" : "+v"(g.x), "+v"(g.y), "+v"(g.z), "+v"(g.w), "+v"(gs));
    asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w), "+v"(us));
    ag += chunk_dot(decode_nvfp4(g, gs), xc);
    au += chunk_dot(decode_nvfp4(u, us), xc);
  }
  const float gv = round_bf16(group_sum<16>(ag) * gsg);
  const float uv = round_bf16(group_sum<16>(au) * gsu);
  return round_bf16(silu_f32(gv)) * uv;
}

// The same for two staged tokens at once (one decode for both).
__device__ __forceinline__ void gu4_h2(const GU4& v, const uint4* xa, const uint4* xb, float gsg, float gsu, int li,
                                       float& ha, float& hb) {
  float ag = 0.f, au = 0.f, bg = 0.f, bu = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint4 g = v.g[c], u = v.u[c];
    uint32_t gs = v.gs[c], us = v.us[c];
    asm volatile("" : "+v"(g.x), "+v"(g.y), "+v"(g.z), "+v"(g.w), "+v"(gs));
    asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w), "+v"(us));
    const DChunk<FMT_NVFP4> dg = decode_nvfp4(g, gs), du = decode_nvfp4(u, us);
    XChunk<FMT_NVFP4> xc;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint4 w = xa[(4 * c + m) * 16 + li];
      xc.v[4 * m] = w.x; xc.v[4 * m + 1] = w.y; xc.v[4 * m + 2] = w.z; xc.v[4 * m + 3] = w.w;
    }
    ag += chunk_dot(dg, xc);
    au += chunk_dot(du, xc);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint4 w = xb[(4 * c + m) * 16 + li];
      xc.v[4 * m] = w.x; xc.v[4 * m + 1] = w.y; xc.v[4 * m + 2] = w.z; xc.v[4 * m + 3] = w.w;
    }
    bg += chunk_dot(dg, xc);
    bu += chunk_dot(du, xc);
    // chunk c is finished before chunk c + 1's opaque copies (volatile asm
    // keeps its order), so at most one chunk pair is decoded at a time
    asm volatile("" : "+v"(ag), "+v"(au), "+v"(bg), "+v"(bu));
  }
  ha = round_bf16(silu_f32(round_bf16(group_sum<16>(ag) * gsg))) * round_bf16(group_sum<16>(au) * gsu);
  hb = round_bf16(silu_f32(round_bf16(group_sum<16>(bg) * gsg))) * round_bf16(group_sum<16>(bu) * gsu);
}

// h of a unit's four rows (lanes 0, 16, 32, 48) for token t as two tagged
// words, kept in this wave's LDS queue (word index << 32 | payload) and
// published after the wave's last unit: a device-scope store issued between
// two units' loads holds back the later loads until it is acknowledged
// (loads and stores complete in order), which cost 0.8 us per layer.
__device__ __forceinline__ void stash_unit_h(uint64_t* q, int& n, int r, int t, int u, float h) {
  const int lane = threadIdx.x & 63;
  const float h0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(h), 0));
  const float h1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(h), 16));
  const float h2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(h), 32));
  const float h3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(h), 48));
  if (lane < 2)
    q[n + lane] = ((uint64_t)(((uint32_t)r * FLINT_MAX_DECODE_BATCH + t) * FL_IW + 2 * (u % (FL_I / 4)) + lane) << 32) |
                  (lane ? pack_bf16x2(h2, h3) : pack_bf16x2(h0, h1));
  n += 2;
}

// A lane's chunk li of down rows row0 + 2 grp and row0 + 2 grp + 1 (so that
// after the 16-lane sums lane 16 grp holds two consecutive output rows).
__device__ __forceinline__ void down_load_pairs(DownRows& d, const uint8_t* codes, const uint8_t* scales, int row0,
                                                int lane) {
  const int grp = lane >> 4, li = lane & 15;
#pragma unroll
  for (int rw = 0; rw < 2; ++rw) {
    const int n = row0 + 2 * grp + rw;
    d.c[rw] = ldg_nt(codes + (size_t)n * (FL_I / 2) + 16 * li);
    d.s[rw] = ldg<uint16_t>(scales + (size_t)n * (FL_I / 16) + 2 * li);
  }
}

// tokens of a slot mask, ascending, 4 bits each
__device__ __forceinline__ uint32_t mask_tokens(uint32_t m) {
  uint32_t tokp = 0;
#pragma unroll
  for (int i = 0; i < F8_BT; ++i)
    if (m) { tokp |= (uint32_t)(__ffs(m) - 1) << (4 * i); m &= m - 1u; }
  return tokp;
}

template <int KC>
__global__ __launch_bounds__(512) void flint_b8_kernel(LayerArgs a_arg, DecodeWs ws_arg) {
  // per-wave maxima (8 waves): with S <= 8 k routed slots and cost weights
  // w >= 5, a workgroup takes at most W / 10 + 1 = 4 k + 1 units and
  // W / 5 + 1 = 8 k + 1 down items (W = sum of the weights, see below)
  constexpr int KMAX = KC ? KC : FLINT_MAX_TOP_K;
  constexpr int U = (F8_BT * KMAX / 2 + 1 + FL_NW - 1) / FL_NW;
  constexpr int DI = (F8_BT * KMAX + 1 + FL_NW - 1) / FL_NW;
  constexpr int D1 = KC ? DI : (DI + 1) / 2;       // down items requested before the last unit is computed
  __shared__ __align__(16) uint4 s_x[F8_BT * F8_Q];
  __shared__ __align__(16) uint4 s_r[F8_Q];
  __shared__ __align__(16) uint4 s_g[F8_Q];
  __shared__ float s_gs[FL_E + 1][3];
  __shared__ __align__(16) uint32_t s_mask[FL_E];
  __shared__ uint8_t s_kpos[FL_E][F8_BT];
  __shared__ float s_wsel[F8_BT][FLINT_MAX_TOP_K];
  __shared__ int s_slot_e[F8_MAXSLOT];
  __shared__ uint32_t s_slot_m[F8_MAXSLOT];
  __shared__ int s_nslot;
  __shared__ int s_cw[F8_MAXSLOT + 1];
  __shared__ uint64_t s_pair[F8_MAXPAIR];
  __shared__ __align__(16) uint32_t s_h[F8_MAXPAIR][FL_IW];
  __shared__ float s_pp[F8_BT * F8_PK][FL_ROWS];
  __shared__ uint64_t s_hq[FL_NW][2 * F8_BT * ((F8_BT * FLINT_MAX_TOP_K / 2 + 1 + FL_NW - 1) / FL_NW)];   // h words per wave

  const LayerArgs a = pin_layer_args(a_arg);
  const DecodeWs ws = pin_decode_ws(ws_arg);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 4, li = lane & 15;
  const int b = blockIdx.x, rep = b % kReplicas;
  const int B = a.B;
  const int K = KC ? KC : a.K;
  const bool norm = (a.flags & FLINT_PRE_RMSNORM) != 0;
  const bool resid = (a.flags & FLINT_RESIDUAL) != 0;

  // ---- phase 0: everything that does not depend on the routing ------------
  // copies straight into LDS (global_load_lds: lane l of a wave writes the
  // l-th 16 bytes after the wave's base, i.e. position q = tid % 256)
  {
    const int q = tid & (F8_Q - 1), wb = q & ~63;
    const int col = staged_col(q);
#pragma unroll
    for (int j = 0; j < F8_BT / 2; ++j) {
      const int t = (tid >> 8) + 2 * j;            // the same in the whole wave
      if (t < B) __builtin_amdgcn_global_load_lds(a.x + (size_t)t * FL_H + col, s_x + t * F8_Q + wb, 16, 0, 0);
    }
    if (tid < F8_Q) __builtin_amdgcn_global_load_lds(a.router + (size_t)b * FL_H + col, s_r + wb, 16, 0, 0);
    else if (norm) __builtin_amdgcn_global_load_lds(a.gamma + col, s_g + wb, 16, 0, 0);
  }
  GsPre gsp;
  gs_prefetch(gsp, a.gscale, a.sh_gscale, FL_E);
  GU4 shu;                                         // shared rows 2b, 2b + 1 (groups 2, 3 repeat 0, 1)
  if (wave < B) gu4_load(shu, a.sh_gu_codes, a.sh_gu_scales, 2 * b + (grp & 1), li);
  // residual of output row 8b + (tid & 7), token tid / 8 (clamped, unconditional)
  const int xt = (tid >> 3) < B ? (tid >> 3) : 0;
  const float xres = bf16_bits_to_f32(ldg<uint16_t>(a.x + (size_t)xt * FL_H + FL_ROWS * b + (tid & 7)));
  const uint32_t epoch = __hip_atomic_load(ws.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  const uint32_t lim = wait_limit(ws);
  if (tid < FL_E) s_mask[tid] = 0u;
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);         // this wave's copies are in LDS
  gs_store(gsp, s_gs, FL_E);
  __syncthreads();

  // ---- phase 1: RMSNorm, logits, the shared expert's h -----------------------
  if (norm) {
    if (wave < B) {                                // wave t: token t
      uint32_t v[16], g[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 xv = s_x[wave * F8_Q + lane + 64 * j], gv = s_g[lane + 64 * j];
        v[4 * j] = xv.x; v[4 * j + 1] = xv.y; v[4 * j + 2] = xv.z; v[4 * j + 3] = xv.w;
        g[4 * j] = gv.x; g[4 * j + 1] = gv.y; g[4 * j + 2] = gv.z; g[4 * j + 3] = gv.w;
      }
      double ss = 0.0;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const double lo = bf16_lo(v[m]), hi = bf16_hi(v[m]);
        ss = fma(lo, lo, ss);
        ss = fma(hi, hi, ss);
      }
      ss = wave_sum_f64(ss);
      rms_norm_words<16>(v, g, make_rms(sqrt(ss / (double)FL_H + (double)a.eps)));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        s_x[wave * F8_Q + lane + 64 * j] = make_uint4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
    }
    __syncthreads();
  }
  if (wave < B) {                                  // logit of expert b for token `wave`
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 r = s_r[lane + 64 * j], xv = s_x[wave * F8_Q + lane + 64 * j];
      part = dot2_bf16(r.x, xv.x, part);
      part = dot2_bf16(r.y, xv.y, part);
      part = dot2_bf16(r.z, xv.z, part);
      part = dot2_bf16(r.w, xv.w, part);
    }
    put_word_all(ws.logit_words, (size_t)F8_BT * FL_E, (size_t)wave * FL_E + b, epoch,
                 __float_as_uint(group_sum<64>(part)));
    // the shared expert's rows 2b, 2b + 1 for this token, while the other
    // workgroups' logits are on their way (measured: 4.5 us per layer faster
    // than requesting the logits first and computing this while they travel)
    const float h = gu4_h(shu, s_x + wave * F8_Q, s_gs[FL_E][0], s_gs[FL_E][1], li);
    const float h0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(h), 0));
    const float h1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(h), 16));
    put_word_all(ws.h_words, (size_t)F8_BT * FL_IW, (size_t)wave * FL_IW + b, epoch, pack_bf16x2(h0, h1));
  }

  // ---- phase 2: top-k of token `wave`, expert -> token mask -------------------
  if (wave < B) {
    uint64_t wd[4], key[4];
    poll_lane_words4(wd, ws.logit_words + (size_t)rep * F8_BT * FL_E + (size_t)wave * FL_E, epoch, ws.error, lim);
    logit_keys(key, wd);
    const uint64_t my_key = topk_lane_key<KC>(key, K);   // lane k: the k-th selected key
    const int my_e = (int)~(uint32_t)my_key;
    const float my_s = lane < K ? 1.0f / (1.0f + expf(-float_from_order_key((uint32_t)(my_key >> 32)))) : 0.f;
    float ssum = 0.f;
#pragma unroll
    for (int k = 0; k < FLINT_MAX_TOP_K; ++k)     // selection order, like the split path
      if (k < K) ssum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), k));
    const float w = (a.flags & FLINT_RENORM) ? my_s / ssum : my_s;
    if (lane < K) {
      s_kpos[my_e][wave] = (uint8_t)lane;
      s_wsel[wave][lane] = w;
      atomicOr(&s_mask[my_e], 1u << wave);
      if (b == 0) {
        a.topk_idx[wave * K + lane] = my_e;
        a.topk_w[wave * K + lane] = w;
      }
    }
  }
  __syncthreads();
  if (wave == 0) {                                 // routed slots: selected experts, ascending
    // lane l holds experts 4l..4l+3; positions and cost prefixes from
    // ballots (no cross-lane scan): bit q of lane l's ballot q = expert 4l+q
    // selected, and the bits of each lane's token count
    const uint4 m4 = reinterpret_cast<const uint4*>(s_mask)[lane];
    const uint32_t mv[4] = {m4.x, m4.y, m4.z, m4.w};
    const unsigned long long below = (1ull << lane) - 1ull;
    int cnt_below = 0, nsl = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const unsigned long long bq = __ballot(mv[q] != 0u);
      cnt_below += __popcll(bq & below);
      nsl += __popcll(bq);
    }
    const int tk = __popc(mv[0]) + __popc(mv[1]) + __popc(mv[2]) + __popc(mv[3]);   // <= 32
    int tk_below = 0, tk_all = 0;
#pragma unroll
    for (int bit = 0; bit < 6; ++bit) {
      const unsigned long long bb = __ballot((tk >> bit) & 1);
      tk_below += __popcll(bb & below) << bit;
      tk_all += __popcll(bb) << bit;
    }
    // cost weight of a slot: 3 + 2 x its tokens (a unit or item of a slot
    // with two tokens took about 1.4 times as long as one with one token)
    int pos = cnt_below, cw = 3 * cnt_below + 2 * tk_below;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (mv[q]) {
        s_slot_e[pos] = 4 * lane + q; s_slot_m[pos] = mv[q]; s_cw[pos] = cw;
        cw += 3 + 2 * __popc(mv[q]); ++pos;
      }
    if (lane == 0) { s_nslot = nsl; s_cw[nsl] = 3 * nsl + 2 * tk_all; }
  }
  __syncthreads();

  // ---- phases 3, 4: gate/up units -> h words, down items requested ---------
  // A software pipeline two units deep: unit j + 2 (or, after the last
  // unit, the down items) is requested as soon as unit j is computed, so a
  // wave never has more than about sixteen 16-byte loads per lane in flight
  // (one-shot requests of all of a wave's rows streamed at 3.6 TB/s, a
  // pipeline of this depth at 5.8 TB/s).  The down items stay in registers
  // until their slot's h has arrived.
  //
  // The work is split by cost, not by count: every unit and item of routed
  // slot r weighs w_r = 3 + 2 n_r (n_r tokens).  On a scale where slot r
  // starts at 256 C_r (C_r = w_0 + .. + w_{r-1}, W = C_S), item t of slot r
  // sits at 256 C_r + t w_r and unit i at 256 C_r + 2 i w_r; workgroup b
  // takes the units and the items that start in [b W, (b + 1) W).
  const int nslot = __builtin_amdgcn_readfirstlane(s_nslot);
  const int wtot = __builtin_amdgcn_readfirstlane(s_cw[nslot]);
  // index (slot-major, `per` per slot) of the first unit or item at or after
  // position pos; `step` is 2 for units, 1 for items
  auto first_at = [&](int pos, int per, int step) {
    const unsigned long long bal = __ballot(lane < nslot && 256 * s_cw[lane < nslot ? lane : 0] <= pos);
    const int r = 63 - __clzll((long long)bal);
    const int w = step * (3 + 2 * __popc(s_slot_m[r]));
    return r * per + (pos - 256 * s_cw[r] + w - 1) / w;
  };
  const int u0 = __builtin_amdgcn_readfirstlane(first_at(b * wtot, F8_UPE, 2));
  const int u1 = __builtin_amdgcn_readfirstlane(first_at((b + 1) * wtot, F8_UPE, 2));
  const int i0 = __builtin_amdgcn_readfirstlane(first_at(b * wtot, F8_TILES, 1));
  const int i1 = __builtin_amdgcn_readfirstlane(first_at((b + 1) * wtot, F8_TILES, 1));
  const int nuw = u1 - u0 > wave ? (u1 - u0 - wave + FL_NW - 1) / FL_NW : 0;   // units of this wave
  GU4 gu[2];
  int ue[2];
  // Loads past a wave's list are skipped, not redirected: stand-in loads of
  // one common address from every compute unit made a cache hot spot.
  auto unit_load = [&](int j) {                    // unit j of this wave into buffer j & 1
    if (j < nuw) {
      const int u = u0 + wave + FL_NW * j;
      ue[j & 1] = __builtin_amdgcn_readfirstlane(s_slot_e[u / F8_UPE]);
      gu4_load(gu[j & 1], a.gu_codes + (size_t)(2 * ue[j & 1]) * F8_MC,
               a.gu_scales + (size_t)(2 * ue[j & 1]) * F8_MS, 4 * (u % F8_UPE) + grp, li);
    }
  };
  // down items: the shared expert's rows 8b..8b+7 (wave t takes token t),
  // and routed items i0 + i (slot (i0 + i) / 256, tile (i0 + i) % 256) for
  // i0 + i < i1 on wave i % 8
  DownRows dsh, dr[DI];
  int de[DI];
  auto item_load = [&](int m) {
    const int j = i0 + wave + FL_NW * m;
    if (j < i1) {
      const int e = __builtin_amdgcn_readfirstlane(s_slot_e[j >> 8]);
      de[m] = e;
      down_load_pairs(dr[m], a.d_codes + (size_t)e * F8_DC, a.d_scales + (size_t)e * F8_DS,
                      FL_ROWS * (j & (F8_TILES - 1)), lane);
    }
  };
  int n_hq = 0;                                    // words in this wave's h queue
  unit_load(0);
  if (U > 1) unit_load(1);
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int u = u0 + wave + FL_NW * j;
    if (j < nuw) {                                 // the same in the whole wave
      const int r = u / F8_UPE;
      const uint32_t m = s_slot_m[r];
      const int n = __popc(m);
      const uint32_t tokp = mask_tokens(m);
      const float gsg = s_gs[ue[j & 1]][0], gsu = s_gs[ue[j & 1]][1];
      int q = 0;
      for (; q + 1 < n; q += 2) {                  // tokens two at a time (one decode)
        const int ta = (tokp >> (4 * q)) & 15, tb = (tokp >> (4 * q + 4)) & 15;
        float ha, hb;
        gu4_h2(gu[j & 1], s_x + ta * F8_Q, s_x + tb * F8_Q, gsg, gsu, li, ha, hb);
        stash_unit_h(s_hq[wave], n_hq, r, ta, u, ha);
        stash_unit_h(s_hq[wave], n_hq, r, tb, u, hb);
      }
      if (q < n) {
        const int t = (tokp >> (4 * q)) & 15;
        stash_unit_h(s_hq[wave], n_hq, r, t, u, gu4_h(gu[j & 1], s_x + t * F8_Q, gsg, gsu, li));
      }
    }
    if (j + 2 < U) {
      unit_load(j + 2);
    } else if (j + 2 == U) {                       // the first down items
      if (wave < B) down_load_pairs(dsh, a.sh_d_codes, a.sh_d_scales, FL_ROWS * b, lane);
#pragma unroll
      for (int m = 0; m < D1; ++m) item_load(m);
    } else {
#pragma unroll
      for (int m = D1; m < DI; ++m) item_load(m);
    }
  }

  for (int k = lane; k < n_hq; k += 64) {          // the queued h words
    const uint64_t e = s_hq[wave][k];
    put_word(ws.hb_words + (e >> 32), epoch, (uint32_t)e);
  }

  // ---- phase 5: the shared expert's h, its down partial sums ------------------
  // (its h words were published in phase 1); wave 0 meanwhile lists the
  // routed (slot, token) rows the items need: the tokens of slot r_lo, then
  // those of r_hi (the slots of items i0 .. i1 - 1; i1 > i0 always, as a
  // workgroup's span W is at least any item's weight)
  const int r_lo = i0 >> 8, r_hi = (i1 - 1) >> 8;
  const uint32_t m_lo = s_slot_m[r_lo], m_hi = r_hi != r_lo ? s_slot_m[r_hi] : 0u;
  const int n_lo = __popc(m_lo);
  const int npair = n_lo + __popc(m_hi);
  if (wave == 0 && lane < npair) {
    const int r = lane < n_lo ? r_lo : r_hi;
    uint32_t m = lane < n_lo ? m_lo : m_hi;
    for (int k = lane < n_lo ? lane : lane - n_lo; k > 0; --k) m &= m - 1u;
    s_pair[lane] = reinterpret_cast<uint64_t>(ws.hb_words + ((size_t)r * F8_BT + (__ffs(m) - 1)) * FL_IW);
  }
  __syncthreads();                                 // every unit of this workgroup is out; s_pair
  {
    constexpr int NS = F8_BT * FL_IW / 512;        // shared-expert words per thread
    const uint64_t* hs = ws.h_words + (size_t)rep * F8_BT * FL_IW;
    uint64_t wd[NS];
    const uint64_t* ptr[NS];
    bool ok[NS];
#pragma unroll
    for (int v = 0; v < NS; ++v) {
      const int q = tid + 512 * v;
      ok[v] = q / FL_IW < B;
      ptr[v] = hs + (ok[v] ? q : 0);
    }
    poll_words<NS>(wd, ptr, ok, epoch, ws.error, lim);
#pragma unroll
    for (int v = 0; v < NS; ++v)
      if (ok[v]) (&s_h[0][0])[tid + 512 * v] = (uint32_t)wd[v];
  }
  __syncthreads();
  // rows 8 tile + 2 grp + rw of an item sit in lane 16 grp after the group
  // sums; that lane publishes both (when `store`)
  auto put_rows = [&](const DChunk<FMT_NVFP4>& d0, const DChunk<FMT_NVFP4>& d1, int pair, int t, int kp, int tile,
                      float f, bool store) {
    XChunk<FMT_NVFP4> hx;
    const uint4* hp = reinterpret_cast<const uint4*>(&s_h[pair][16 * li]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint4 v = hp[k];
      hx.v[4 * k] = v.x; hx.v[4 * k + 1] = v.y; hx.v[4 * k + 2] = v.z; hx.v[4 * k + 3] = v.w;
    }
    const float v0 = group_sum<16>(chunk_dot(d0, hx)), v1 = group_sum<16>(chunk_dot(d1, hx));
    if (store && li == 0) {
      uint64_t* p = ws.p_words + ((size_t)t * F8_PK + kp) * FL_H + FL_ROWS * tile + 2 * grp;
      put_word(p, epoch, __float_as_uint(f * v0));
      put_word(p + 1, epoch, __float_as_uint(f * v1));
    }
  };
  if (wave < B)                                    // the shared expert, token `wave`
    put_rows(decode_nvfp4(dsh.c[0], dsh.s[0]), decode_nvfp4(dsh.c[1], dsh.s[1]), wave, wave, F8_KS, b,
             s_gs[FL_E][2], true);

  // ---- phase 6: the routed h rows, then the routed items -> partial sums -------
  {
    constexpr int NR = 2 * F8_BT * FL_IW / 512;    // routed words per thread
    uint64_t wd[NR];
    const uint64_t* ptr[NR];
    bool ok[NR];
#pragma unroll
    for (int v = 0; v < NR; ++v) {
      const int q = tid + 512 * v, p = q / FL_IW;
      ok[v] = p < npair;
      ptr[v] = reinterpret_cast<const uint64_t*>(s_pair[ok[v] ? p : 0]) + (q % FL_IW);
    }
    poll_words<NR>(wd, ptr, ok, epoch, ws.error, lim);
#pragma unroll
    for (int v = 0; v < NR; ++v)
      if (ok[v]) (&s_h[F8_BT][0])[tid + 512 * v] = (uint32_t)wd[v];
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < DI; ++m) {
    const int j = i0 + wave + FL_NW * m;
    if (j >= i1) break;                            // the same in the whole wave
    const int e = de[m];
    const uint32_t mask = s_slot_m[j >> 8];
    const int pb = (j >> 8) == r_lo ? F8_BT : F8_BT + n_lo;
    const uint32_t tokp = mask_tokens(mask);
    const int n = __popc(mask);
    const float gsd = s_gs[e][2];
    const DChunk<FMT_NVFP4> d0 = decode_nvfp4(dr[m].c[0], dr[m].s[0]);
    const DChunk<FMT_NVFP4> d1 = decode_nvfp4(dr[m].c[1], dr[m].s[1]);
    for (int q = 0; q < n; ++q) {
      const int t = (tokp >> (4 * q)) & 15;
      const int kp = s_kpos[e][t];
      put_rows(d0, d1, pb + q, t, kp, j & (F8_TILES - 1), s_wsel[t][kp] * gsd, true);
    }
  }

  // ---- phase 7: this workgroup's output rows -------------------------------------
  {
    constexpr int NW2 = (F8_BT * F8_PK * FL_ROWS + 511) / 512;
    uint64_t wd[NW2];
    const uint64_t* ptr[NW2];
    bool ok[NW2];
#pragma unroll
    for (int v = 0; v < NW2; ++v) {
      const int q = tid + 512 * v, rest = q / FL_ROWS, t = rest / F8_PK, kp = rest % F8_PK;
      ok[v] = t < B && (kp < K || kp == F8_KS);
      ptr[v] = ws.p_words + (ok[v] ? ((size_t)t * F8_PK + kp) * FL_H + FL_ROWS * b + (q % FL_ROWS) : 0);
    }
    poll_words<NW2>(wd, ptr, ok, epoch, ws.error, lim);
#pragma unroll
    for (int v = 0; v < NW2; ++v) {
      const int q = tid + 512 * v;
      if (ok[v]) (&s_pp[0][0])[q] = __uint_as_float((uint32_t)wd[v]);
    }
  }
  __syncthreads();
  if (tid < B * FL_ROWS) {
    const int t = tid >> 3, r = tid & 7;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < FLINT_MAX_TOP_K; ++k)
      if (k < K) v += s_pp[t * F8_PK + k][r];
    v += s_pp[t * F8_PK + F8_KS][r];
    float o = round_bf16(v);
    if (resid) o = xres + o;
    a.out[(size_t)t * FL_H + FL_ROWS * b + r] = f32_to_bf16_bits(o);
  }
  // Every workgroup published its logits with the epoch it read at its start
  // and workgroup 0 saw all of them before its top-k: none of this launch can
  // still be about to read the old value.
  if (b == 0 && tid == 0) *ws.epoch = epoch;
}

}  // namespace

bool flint_b8_shape(const flint_moe_shape& s) {
  return s.hidden == FL_H && s.n_experts == FL_E && s.inter == FL_I && s.shared_inter == FL_I &&
         s.top_k >= 1 && s.top_k <= FLINT_MAX_TOP_K && !(s.flags & FLINT_W_BF16);
}

bool flint_b8_supported(const LayerArgs& a) {
  if (a.B < 2 || a.B > F8_BT || (a.flags & FLINT_W_BF16)) return false;
  if (a.H != FL_H || a.E != FL_E || a.I != FL_I || a.SI != FL_I || a.K < 1 || a.K > FLINT_MAX_TOP_K) return false;
  if (device_num_cu() < FL_G) return false;
  static int per_cu = -1;                          // co-residency of the grid (see fused.hip)
  if (per_cu == -1) {
    int ndev = 0, n = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0) per_cu = -2;
    else {
      int n6 = 0;
      const bool ok = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, flint_b8_kernel<0>, 512, 0) == hipSuccess &&
                      hipOccupancyMaxActiveBlocksPerMultiprocessor(&n6, flint_b8_kernel<6>, 512, 0) == hipSuccess;
      per_cu = ok ? (n < n6 ? n : n6) : -2;
    }
  }
  return per_cu == -2 || (int64_t)per_cu * device_num_cu() >= FL_G;
}

hipError_t launch_flint_b8(const LayerArgs& a, const DecodeWs& ws, hipStream_t st) {
  if (a.K == 6) hipLaunchKernelGGL(flint_b8_kernel<6>, dim3(FL_G), dim3(512), 0, st, a, ws);
  else hipLaunchKernelGGL(flint_b8_kernel<0>, dim3(FL_G), dim3(512), 0, st, a, ws);
  return hipGetLastError();
}

}  // namespace flint
