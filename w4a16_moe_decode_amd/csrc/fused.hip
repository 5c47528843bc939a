// Single-launch decode MoE layer for one token (batch 1), NVFP4 weights.
//
// The same layer as the three-kernel path (decode.hip) -- RMSNorm (opt.),
// router GEMV, sigmoid top-k, gate/up GEMV + SiLU*up, down GEMV + weighted
// combine + shared expert (+ residual) -- run by one persistent grid of
// workgroups so that the dependent steps overlap instead of paying a launch
// and a cold start each.  This is the low-latency decode path of "Day-0
// Support for Flint on vLLM" ("Optimizations", last bullet and the paragraph
// after the list: routing and the expert combine fused into neighbouring
// GEMV kernels, the next kernel's weight loads overlapping the previous
// one), built on one GPU without inter-kernel launches:
//
//   phase 1  router logits (one expert per workgroup, a quarter row per
//            wave) and the shared expert's gate/up rows, loaded together
//   phase 2  every workgroup waits for all logits, selects the top-k itself
//            and issues the loads of its own down rows of all selected
//            experts (they do not depend on h)
//   phase 3  routed gate/up rows (an equal share of row pairs per
//            workgroup, dealt round-robin over its waves)
//   phase 4  every workgroup waits for the h values it needs, then computes
//            its output rows: weighted combine of the selected experts and
//            the shared expert, one BF16 rounding (+ residual)
//
// Hand-offs between workgroups use 64-bit words (launch epoch << 32 |
// payload) written and read with agent-scope atomics: data and ready flag
// are one word, so no release fence (a whole-L2 write-back on this GPU) is
// needed.  Every wait is bounded: if a word does not arrive (it cannot while
// all workgroups are resident) the kernel records an error and still exits.
// The grid never exceeds the number of compute units, one workgroup each.
#include "fused_common.hpp"

namespace flint {
namespace {

template <int NCH>
__device__ __forceinline__ uint32_t gu_finish(const GUItem<NCH>& it, const GURows& R,
                                              const XChunk<FMT_NVFP4>* xc) {
  float acc[2][2];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr)
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) s += chunk_dot(decode_nvfp4(it.c[rr][m][c], it.s[rr][m][c]), xc[c]);
      acc[rr][m] = group_sum<64>(s);
    }
  float h[2];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const float gv = round_bf16(acc[rr][0] * R.g_scale);
    const float uv = round_bf16(acc[rr][1] * R.u_scale);
    h[rr] = round_bf16(silu_f32(gv)) * uv;
  }
  return pack_bf16x2(h[0], h[1]);
}

// One MoE layer for one token, run by every workgroup of the persistent grid.
// Down rows of one workgroup: GPW = 64/GD rows per wave-wide load, DW
// row-sets per workgroup (DW * GPW rows), chunk steps of GD lanes.  Layer
// `layer` of a launch tags its hand-off words with the stored epoch + 1 +
// layer; the epoch it used is returned.  a.x and a.out may point to LDS.
// A layer's first loads that do not depend on its input: this wave's
// quarter of gamma and of its first router row, and the launch epoch.  A
// stack of layers issues them for layer l + 1 while it waits for layer l's
// output rows.
template <int NCH>
struct LayerPre {
  uint4 gq[NCH], rq[NCH];
  GsPre gs;                                        // this thread's tensor-scale table entries
  uint32_t epoch0;                                 // the stored epoch
  uint32_t lim;                                    // bound of each wait
};

template <int NCH>
__device__ __forceinline__ void layer_prefetch(LayerPre<NCH>& p, const uint16_t* gamma, const uint16_t* router,
                                               const float* gscale, const float* sh_gscale, int H, int E) {
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int e0 = (int)blockIdx.x < E ? (int)blockIdx.x : 0;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int col = 32 * (lane + 64 * c) + 8 * wv;
    p.gq[c] = ldg<uint4>(gamma + col);
    p.rq[c] = ldg<uint4>(router + (size_t)e0 * H + col);
  }
  gs_prefetch(p.gs, gscale, sh_gscale, E);
}

template <int NCH, int GD, int DW, int MAXS, bool PRE>
__device__ __forceinline__ uint32_t fused_layer_b1(const LayerArgs& a, const DecodeWs& ws, int G, uint32_t layer,
                                                   const LayerPre<NCH>& pre) {
  constexpr int GPW = 64 / GD;
  constexpr int DROWS = DW * GPW;                 // output rows per workgroup
  constexpr int IMAXW = 2048 / 2;                 // h words per slot held in LDS (I <= 2048)
  __shared__ float s_logit_part[4];
  __shared__ int s_exp[MAXS];
  __shared__ float s_w[MAXS];
  __shared__ int s_nU;
  __shared__ uint64_t s_key[MAXS];
  __shared__ int s_sel_e[MAXS];
  __shared__ float s_sel_w[MAXS];
  __shared__ uint32_t s_h[MAXS][IMAXW];           // h of every slot, packed BF16 pairs
  __shared__ float s_red[4][DROWS];
  __shared__ float s_gs[FLINT_MAX_EXPERTS + 1][3]; // tensor scales: routed experts, then the shared one

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int NWV = 4 * G, gw = blockIdx.x * 4 + wave;
  const int H = a.H, E = a.E, K = a.K, I = a.I, SI = a.SI;
  const bool has_sh = SI > 0;
  const int sh = has_sh ? 1 : 0;
  const bool norm = (a.flags & FLINT_PRE_RMSNORM) != 0;
  const int hstride = (I > SI ? I : SI) / 2;
  const size_t lstride = E, hrep = (size_t)(FLINT_MAX_TOP_K + 1) * hstride;
  uint64_t* lw_all = ws.logit_words;              // [kReplicas][E]
  uint64_t* hw_all = ws.h_words;                  // [kReplicas][slot][hstride] tagged h pairs
  const int rep = blockIdx.x % kReplicas;
  const uint64_t* lw = lw_all + (size_t)rep * lstride;   // this workgroup's copies
  const uint64_t* hw = hw_all + (size_t)rep * hrep;

  // ---- the token --------------------------------------------------------------
  // Lane l holds chunks j = l + 64c (32 columns each) of x: every wave holds
  // the whole token.  Wave w owns the w-th quarter (8 columns) of each chunk:
  // it normalises that quarter and dots it with the same columns of its
  // router rows, so the router never waits on the other waves.  With
  // RMSNorm the four waves then swap their normalised quarters through LDS.
  // All loads are issued up front and unconditionally (loads complete in
  // order: a load issued on one path only would make the compiler wait for
  // it on the other path too): x, gamma, the first router row, epoch.
  __shared__ uint4 s_xn[4][64 * NCH];
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int e0 = (int)blockIdx.x < E ? (int)blockIdx.x : 0;
  const uint16_t* gsrc = norm ? a.gamma : a.x;
  XChunk<FMT_NVFP4> xc[NCH];
  uint4 xq[NCH], gq[NCH], rq[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {                  // this wave's quarter of each chunk
    const int col = 32 * (lane + 64 * c) + 8 * wv;
    xq[c] = *reinterpret_cast<const uint4*>(a.x + col);
    if constexpr (PRE) {
      gq[c] = pre.gq[c];
      rq[c] = pre.rq[c];
    } else {
      gq[c] = *reinterpret_cast<const uint4*>(gsrc + col);
      rq[c] = *reinterpret_cast<const uint4*>(a.router + (size_t)e0 * H + col);
    }
  }
#pragma unroll
  for (int c = 0; c < NCH; ++c) xc[c] = load_x<FMT_NVFP4>(a.x, lane + 64 * c);
  // The tensor-scale table goes to LDS, loaded with vector loads among the
  // first loads: a scalar load from memory shares its wait counter with LDS
  // accesses, so one still in flight would hold up every LDS access (and
  // barrier) behind it by a memory round trip.
  GsPre gsp;
  if constexpr (PRE) gsp = pre.gs;
  else gs_prefetch(gsp, a.gscale, SI > 0 ? a.sh_gscale : nullptr, E);
  // the launch epoch: a vector load, so that waiting for it holds up neither
  // the kernel arguments nor the loads above
  const uint32_t epoch =
      (PRE ? pre.epoch0 : __hip_atomic_load(ws.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) + 1u + layer;
  const uint32_t lim = PRE ? pre.lim : wait_limit(ws);
  __shared__ double s_ss[4];
  if (norm) {                                      // this wave's part of sum(x^2)
    double ss0 = 0.0, ss1 = 0.0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const uint32_t q[4] = {xq[c].x, xq[c].y, xq[c].z, xq[c].w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const double lo = bf16_lo(q[m]), hi = bf16_hi(q[m]);
        ss0 = fma(lo, lo, ss0);
        ss1 = fma(hi, hi, ss1);
      }
    }
    const double ssw = wave_sum_f64(ss0 + ss1);
    if (lane == 0) s_ss[wv] = ssw;
  }
  // wait for all first loads here (the epoch is the last of them), before
  // the loads below that only some waves issue
#pragma unroll
  for (int c = 0; c < NCH; ++c) asm volatile("" ::"v"(gq[c].x), "v"(rq[c].x));   // one register per load is enough
  asm volatile("" ::"v"(epoch), "v"(lim));
  gs_store(gsp, s_gs, E);

  // ---- phase 1: router quarter rows + shared expert gate/up ------------------
  // expert e is owned by workgroup e % G; its 4 waves take a quarter each
  const int nsh_items = has_sh ? SI / 2 : 0;
  // shared items are spread over all workgroups, one per sh_stride waves;
  // when there are fewer items than waves, wave 0 of each workgroup gets
  // none, so it can start polling the logits as soon as its router rows are
  // published
  const int sh_stride = nsh_items > 0 && nsh_items < NWV ? NWV / nsh_items : 1;
  const int sh_off = sh_stride > 1 ? 1 : 0;
  const int sh_first = (gw % sh_stride == sh_off) ? gw / sh_stride : nsh_items;
  GUItem<NCH> shit;
  const bool my_sh = sh_first < nsh_items;
  GURows Rsh;                                      // its tensor scales are read after the barrier below
  if (has_sh) Rsh = gu_rows(a, -1, nullptr);
  if (my_sh) gu_load<NCH>(shit, Rsh, sh_first, H);

  if (norm) {                                      // RMS, then this wave's normalised quarter
    __syncthreads();
    const double ss = (s_ss[0] + s_ss[1]) + (s_ss[2] + s_ss[3]);
    const Rms rms = make_rms(sqrt(ss / (double)H + (double)a.eps));
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      xq[c] = rms_norm_8(xq[c], gq[c], rms);
      s_xn[wv][lane + 64 * c] = xq[c];
    }
  }
  // This workgroup's router row, already in registers, then (grids smaller
  // than E only) further rows in a loop of their own: a load inside the
  // first row's code path would make the compiler wait for every load in
  // flight (wave 1's shared-expert rows among them) before the dot product.
#define FLINT_ROUTER_ROW(E_)                                                         \
  {                                                                                  \
    float part = 0.f;                                                                \
    _Pragma("unroll") for (int c = 0; c < NCH; ++c) {                                \
      part = dot2_bf16(rq[c].x, xq[c].x, part);                                      \
      part = dot2_bf16(rq[c].y, xq[c].y, part);                                      \
      part = dot2_bf16(rq[c].z, xq[c].z, part);                                      \
      part = dot2_bf16(rq[c].w, xq[c].w, part);                                      \
    }                                                                                \
    part = group_sum<64>(part);                                                      \
    if (lane == 0) s_logit_part[wave] = part;                                        \
    __syncthreads();                                                                 \
    if (wave == 0) {                                                                 \
      const float l = s_logit_part[0] + s_logit_part[1] + s_logit_part[2] + s_logit_part[3]; \
      put_word_all(lw_all, lstride, (E_), epoch, __float_as_uint(l));                \
    }                                                                                \
    __syncthreads();                                                                 \
  }
  if ((int)blockIdx.x < E) FLINT_ROUTER_ROW(blockIdx.x)
  for (int e = blockIdx.x + G; e < E; e += G) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) rq[c] = ldg<uint4>(a.router + (size_t)e * H + 32 * (lane + 64 * c) + 8 * wv);
    FLINT_ROUTER_ROW(e)
  }
#undef FLINT_ROUTER_ROW
  if ((int)blockIdx.x >= E) __syncthreads();      // the scale table (and xn) complete
  if (has_sh) { Rsh.g_scale = s_gs[E][0]; Rsh.u_scale = s_gs[E][1]; }
  if (norm) {                                      // the normalised token, from the four waves
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint4 v = s_xn[w][lane + 64 * c];
        xc[c].v[4 * w + 0] = v.x; xc[c].v[4 * w + 1] = v.y; xc[c].v[4 * w + 2] = v.z; xc[c].v[4 * w + 3] = v.w;
      }
  }
  announce_arrival(ws, E, epoch);
  if (my_sh) put_word_all(hw_all, hrep, sh_first, epoch, gu_finish<NCH>(shit, Rsh, xc));
  if (sh_stride == 1)
    for (int it = gw + NWV; it < nsh_items; it += NWV) {   // shared experts wider than the grid
      gu_load<NCH>(shit, Rsh, it, H);
      put_word_all(hw_all, hrep, it, epoch, gu_finish<NCH>(shit, Rsh, xc));
    }

  // ---- phase 2: top-k (every workgroup, wave 0) and down-row prefetch --------
  if (wave == 0) {
    uint64_t key[4];
    {
      uint64_t wd[8];
      const uint64_t* ptr[8];
      bool ok[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ex = lane + 64 * q;
        ok[q] = ex < E;
        ptr[q] = lw + (ex < E ? ex : 0);
      }
      arrival_slots(ws, E, G, ptr + 4, ok + 4);   // workgroup 0 only
      poll_words_pipelined<8, 1>(wd, ptr, ok, epoch, ws.error, lim);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ex = lane + 64 * q;
        key[q] = ok[q] ? (((uint64_t)float_order_key(__uint_as_float((uint32_t)wd[q])) << 32) |
                          (uint32_t)~(uint32_t)ex)
                       : 0ull;
      }
    }
    // the k-th selected key is the same in every lane (sel[k]); lane k
    // takes it over, so no LDS round trip and no readlane chain is needed
    uint64_t sel[FLINT_MAX_TOP_K];
    topk_keys_uniform(key, K, sel);
    uint64_t my_key = 0ull;
#pragma unroll
    for (int k = 0; k < FLINT_MAX_TOP_K; ++k) my_key = lane == k ? sel[k] : my_key;
    const int my_e = (int)~(uint32_t)my_key;
    const float my_s = lane < K ? 1.0f / (1.0f + expf(-float_from_order_key((uint32_t)(my_key >> 32)))) : 0.f;
    float ssum = 0.f;
#pragma unroll
    for (int k = 0; k < FLINT_MAX_TOP_K; ++k)     // selection order, like the split path
      if (k < K) ssum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), k));
    const float w = (a.flags & FLINT_RENORM) ? my_s / ssum : my_s;
    // routed slots in ascending expert order: rank of each selected expert
    int rank = 0;
#pragma unroll
    for (int k = 0; k < FLINT_MAX_TOP_K; ++k)
      if (k < K) rank += (int)~(uint32_t)sel[k] < my_e ? 1 : 0;
    if (lane < K) {
      s_exp[sh + rank] = my_e;
      s_w[sh + rank] = w;
      s_sel_e[lane] = my_e;                        // selection order, for the top-k outputs
      s_sel_w[lane] = w;
    }
    if (lane == 0) {
      s_nU = K;
      if (has_sh) { s_exp[0] = -1; s_w[0] = 1.f; }
    }
  }
  __syncthreads();
  // Nothing this wave loaded earlier is still in flight here (every earlier
  // load was consumed, every store long acknowledged), but loads issued on
  // one path only (the shared expert's rows and tensor scales) would leave
  // the compiler believing so: it then waits for the memory counter to drop
  // to a small number in the middle of the weight loads below, i.e. for the
  // first item's rows to arrive before the second item's and the down rows
  // are requested.  An explicit wait for zero clears that state for free.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  const int nU = s_nU, S = nU + sh;

  // ---- phase 3: routed gate/up items -----------------------------------------
  // Workgroup g takes items [g q, g q + q), q = ceil(items / workgroups), so
  // every workgroup streams the same number of rows (dealing the items
  // round-robin over all waves of the grid gave half of the workgroups twice
  // the rows of the others, and the last of them set the time of the h
  // exchange); its waves take them round-robin.  The first round's loads
  // (rounds 0 and 1) are issued before the down-row prefetch: loads complete
  // in order, so finishing these items then waits only on their own rows
  // while the prefetch stays in flight.
  const int ipw = I / 2;                           // items per routed slot
  const int nitems = nU * ipw;
  const int iq = (nitems + G - 1) / G;
  const int ibase = blockIdx.x * iq;
  const int iend = ibase + iq < nitems ? ibase + iq : nitems;
  GUItem<NCH> A, B;
  const int itA = ibase + wave, itB = itA + 4;
  const bool hasA = itA < iend, hasB = itB < iend;
  const int rA = hasA ? itA / ipw : 0, pA = hasA ? itA - rA * ipw : 0;
  const int rB = hasB ? itB / ipw : 0, pB = hasB ? itB - rB * ipw : 0;
  const GURows RA = gu_rows(a, __builtin_amdgcn_readfirstlane(s_exp[sh + rA]), s_gs);
  const GURows RB = gu_rows(a, __builtin_amdgcn_readfirstlane(s_exp[sh + rB]), s_gs);
  if (hasA) gu_load<NCH>(A, RA, pA, H);
  if (hasB) gu_load<NCH>(B, RB, pB, H);

  // this workgroup's output rows and their down-row loads (all slots)
  const int n0 = blockIdx.x * DROWS;
  const int ncs = (I > SI ? I : SI) / 32;          // chunk steps of the widest slot
  const int dch = (ncs + GD - 1) / GD;
  // items (slot, chunk step) dealt to the 4 waves; at most MAXI per wave
  constexpr int MAXI = (MAXS * 2 + 3) / 4;
  uint4 draw[MAXI][DW];
  uint32_t dsc[MAXI][DW];
  const int grp = lane / GD, li = lane % GD;
  const int total = S * dch;
#pragma unroll
  for (int u = 0; u < MAXI; ++u) {
    const int it = wave + 4 * u;
    const int s = it < total ? it / dch : 0, c = it - s * dch;
    const int e = __builtin_amdgcn_readfirstlane(s_exp[s < S ? s : 0]);
    const int inter = e < 0 ? SI : I;
    const int j = li + GD * c;
    const bool ok = it < total && j < inter / 32;
    const uint8_t* codes = e < 0 ? a.sh_d_codes : a.d_codes + (size_t)e * H * (inter / 2);
    const uint8_t* scales = e < 0 ? a.sh_d_scales : a.d_scales + (size_t)e * H * (inter / 16);
    // every lane loads: a masked-off lane reads the first chunk of routed
    // expert 0 (always present) and phase 4 skips its item, so no load is
    // conditional and the compiler need not wait on one to merge a default
#pragma unroll
    for (int rw = 0; rw < DW; ++rw) {
      const int n = n0 + rw * GPW + grp;
      const bool okr = ok && n < H;
      const uint8_t* cp = okr ? codes + (size_t)n * (inter / 2) + 16 * j : a.d_codes;
      const uint8_t* sp = okr ? scales + (size_t)n * (inter / 16) + 2 * j : a.d_scales;
      draw[u][rw] = ldg<uint4>(cp);
      dsc[u][rw] = ldg<uint16_t>(sp);
    }
  }

  if (hasA) put_word_all(hw_all, hrep, (size_t)(sh + rA) * hstride + pA, epoch, gu_finish<NCH>(A, RA, xc));
  if (hasB) put_word_all(hw_all, hrep, (size_t)(sh + rB) * hstride + pB, epoch, gu_finish<NCH>(B, RB, xc));
  // further rounds, for layers with more routed items than 8 per workgroup
  for (int it0 = itA + 8; it0 < iend; it0 += 8) {
    GUItem<NCH> C, D;
    const int itD = it0 + 4;
    const int rC = it0 / ipw, pC = it0 - rC * ipw;
    const GURows RC = gu_rows(a, __builtin_amdgcn_readfirstlane(s_exp[sh + rC]), s_gs);
    gu_load<NCH>(C, RC, pC, H);
    const bool hasD = itD < iend;
    const int rD = hasD ? itD / ipw : rC, pD = hasD ? itD - rD * ipw : pC;
    const GURows RD = gu_rows(a, __builtin_amdgcn_readfirstlane(s_exp[sh + rD]), s_gs);
    if (hasD) gu_load<NCH>(D, RD, pD, H);
    put_word_all(hw_all, hrep, (size_t)(sh + rC) * hstride + pC, epoch, gu_finish<NCH>(C, RC, xc));
    if (hasD)
      put_word_all(hw_all, hrep, (size_t)(sh + rD) * hstride + pD, epoch, gu_finish<NCH>(D, RD, xc));
  }

  // ---- phase 4: wait for h, down + combine -----------------------------------
  {
    // every (slot, word) pair, 8 per thread per batch
    const int per = hstride;                         // words per slot (widest slot)
    const int nw = S * per;
    for (int q0 = threadIdx.x; q0 < nw; q0 += 8 * 256) {
      uint64_t wd[8];
      const uint64_t* ptr[8];
      bool ok[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = q0 + 256 * u;
        const int sl = q / per, wq = q - sl * per;
        const int inter = (q < nw && s_exp[sl] < 0) ? SI : I;
        ok[u] = q < nw && wq < inter / 2;
        ptr[u] = hw + (ok[u] ? (size_t)sl * hstride + wq : 0);
      }
      poll_words<8>(wd, ptr, ok, epoch, ws.error, lim);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = q0 + 256 * u;
        if (ok[u]) s_h[q / per][q % per] = (uint32_t)wd[u];
      }
    }
  }
  // residual of this thread's output row, fetched early
  const bool resid = (a.flags & FLINT_RESIDUAL) != 0;
  float xres = 0.f;
  if (resid && threadIdx.x < DROWS && n0 + (int)threadIdx.x < H) xres = bf16_bits_to_f32(a.x[n0 + threadIdx.x]);
  __syncthreads();

  float acc[DW];
#pragma unroll
  for (int rw = 0; rw < DW; ++rw) acc[rw] = 0.f;
#pragma unroll
  for (int u = 0; u < MAXI; ++u) {
    const int it = wave + 4 * u;
    if (it >= total) break;
    const int s = it / dch, c = it - s * dch;
    const int e = __builtin_amdgcn_readfirstlane(s_exp[s]);
    const int inter = e < 0 ? SI : I;
    const int j = li + GD * c;
    if (j >= inter / 32) continue;
    XChunk<FMT_NVFP4> hx;
#pragma unroll
    for (int m = 0; m < 16; ++m) hx.v[m] = s_h[s][16 * j + m];
    const float f = s_w[s] * s_gs[e < 0 ? E : e][2];
#pragma unroll
    for (int rw = 0; rw < DW; ++rw) acc[rw] = fmaf(f, chunk_dot(decode_nvfp4(draw[u][rw], dsc[u][rw]), hx), acc[rw]);
  }
#pragma unroll
  for (int rw = 0; rw < DW; ++rw) {
    const float v = group_sum<GD>(acc[rw]);
    if (li == 0) s_red[wave][rw * GPW + grp] = v;
  }
  __syncthreads();
  if (threadIdx.x < DROWS) {
    const int n = n0 + threadIdx.x;
    if (n < H) {
      const float v = s_red[0][threadIdx.x] + s_red[1][threadIdx.x] + s_red[2][threadIdx.x] + s_red[3][threadIdx.x];
      float o = round_bf16(v);
      if (resid) o = xres + o;
      a.out[n] = f32_to_bf16_bits(o);
    }
  }
  if (blockIdx.x == 0 && (int)threadIdx.x < K) {  // the top-k outputs, off the critical path
    a.topk_idx[threadIdx.x] = s_sel_e[threadIdx.x];
    a.topk_w[threadIdx.x] = s_sel_w[threadIdx.x];
  }

  return epoch;
}

template <int NCH, int GD, int DW, int MAXS>
__global__ __launch_bounds__(256) void fused_decode_b1_kernel(LayerArgs a_arg, DecodeWs ws_arg, int G_arg) {
  const LayerArgs a = pin_layer_args(a_arg);
  const DecodeWs ws = pin_decode_ws(ws_arg);
  const int G = pin_sgpr(G_arg);                   // the grid size (gridDim.x would be another lazy load)
  const LayerPre<NCH> none{};
  const uint32_t epoch = fused_layer_b1<NCH, GD, DW, MAXS, false>(a, ws, G, 0, none);
  // ---- advance the epoch for the next launch -----------------------------------
  // Every workgroup published a router logit or an arrival word tagged with
  // the epoch it read at its start, and workgroup 0 has seen all of them
  // before its top-k: no workgroup of this launch can still be about to read
  // the old value.  No ticket round trip is needed.
  if (blockIdx.x == 0 && threadIdx.x == 0) *ws.epoch = epoch;
}

// A stack of L MoE layers for one token: layer l takes the residual x_l
// and leaves x_{l+1} = BF16(x_l + BF16(MoE_l(BF16(BF16(x_l / rms) * gamma_l))))
// (pre-norm residual sublayers, the decode step of "Day-0 Support for Flint
// on vLLM", "Model architecture").  The layers run back to back in one
// launch: each workgroup keeps the residual in LDS, computes its output rows
// of layer l, publishes them as epoch-tagged words (two BF16 per word,
// kReplicas copies) and polls every row before layer l + 1 starts.  No word
// can be overwritten while another workgroup still needs it: a workgroup
// moves on to layer l + 1's hand-offs only after it has seen layer l's
// logits (or arrival words) of every workgroup, each published after that
// workgroup finished reading layer l's inputs.
// A wave-uniform 64-bit value read from LDS, into scalar registers.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32) |
         (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
}

template <int NCH, int GD, int DW, int MAXS>
__global__ __launch_bounds__(256) void fused_stack_b1_kernel(StackArgs sa_arg, DecodeWs ws_arg, int G_arg) {
  StackArgs sa = sa_arg;
  sa.base.H = pin_sgpr(sa_arg.base.H); sa.base.E = pin_sgpr(sa_arg.base.E);
  sa.base.I = pin_sgpr(sa_arg.base.I); sa.base.SI = pin_sgpr(sa_arg.base.SI);
  sa.base.K = pin_sgpr(sa_arg.base.K); sa.base.flags = pin_sgpr(sa_arg.base.flags);
  sa.base.eps = pin_sgpr(sa_arg.base.eps);
  sa.layers = pin_sgpr(sa_arg.layers); sa.gammas = pin_sgpr(sa_arg.gammas);
  sa.x_in = pin_sgpr(sa_arg.x_in); sa.x_out = pin_sgpr(sa_arg.x_out);
  sa.topk_idx = pin_sgpr(sa_arg.topk_idx); sa.topk_w = pin_sgpr(sa_arg.topk_w);
  sa.layer_out = pin_sgpr(sa_arg.layer_out); sa.L = pin_sgpr(sa_arg.L);
  const DecodeWs ws = pin_decode_ws(ws_arg);
  const int G = pin_sgpr(G_arg);
  constexpr int DROWS = DW * (64 / GD);
  constexpr int NPTR = sizeof(flint_moe_weights) / sizeof(uint64_t);
  static_assert(NPTR <= 16, "pointer table");
  __shared__ __align__(16) uint16_t s_x[4096];      // the residual entering the layer
  __shared__ __align__(16) uint16_t s_xo[4096];     // this workgroup's rows of its output
  // Weight pointers of layer l in slot l & 1.  They are read with vector
  // loads one layer ahead (during the residual exchange before the layer
  // that precedes them), never with scalar loads: a scalar load from memory
  // in flight would hold up every LDS access behind it.
  __shared__ uint64_t s_lp[2][16];
  const int H = sa.base.H, K = sa.base.K, E = sa.base.E;
  const int n0 = blockIdx.x * DROWS;
  const int rep = blockIdx.x % kReplicas;
  const size_t xrep = (size_t)H / 2;
  const uint64_t* tab = reinterpret_cast<const uint64_t*>(sa.layers);
  for (int q = threadIdx.x; q < H / 8; q += 256)
    reinterpret_cast<uint4*>(s_x)[q] = reinterpret_cast<const uint4*>(sa.x_in)[q];
  if (threadIdx.x < NPTR) {
    s_lp[0][threadIdx.x] = ldg<uint64_t>(tab + threadIdx.x);
    s_lp[1][threadIdx.x] = ldg<uint64_t>(tab + (size_t)(sa.L > 1 ? 1 : 0) * NPTR + threadIdx.x);
  }
  __syncthreads();
  // layer 0's input-independent first loads (layer l + 1's are issued at the
  // end of layer l, before its output rows are exchanged)
  LayerPre<NCH> pre;
  pre.epoch0 = __hip_atomic_load(ws.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  pre.lim = wait_limit(ws);
  layer_prefetch<NCH>(pre, sa.gammas, reinterpret_cast<const uint16_t*>(uniform_u64(s_lp[0][0])),
                      reinterpret_cast<const float*>(uniform_u64(s_lp[0][5])),
                      sa.base.SI > 0 ? reinterpret_cast<const float*>(uniform_u64(s_lp[0][10])) : nullptr, H, E);
  uint64_t nxt = 0;                                // layer l + 2's pointer (lanes < NPTR of wave 0)
  uint32_t epoch = 0;
  for (int l = 0; l < sa.L; ++l) {
    // layer l + 1's pointers, loaded during the previous exchange, go to the
    // slot layer l - 1 used
    if (l >= 1 && l + 1 < sa.L && threadIdx.x < NPTR) s_lp[(l + 1) & 1][threadIdx.x] = nxt;
    const uint64_t* lp = s_lp[l & 1];
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
    a.gamma = sa.gammas + (size_t)l * H;
    a.x = s_x;
    a.out = s_xo;
    a.topk_idx = sa.topk_idx + (size_t)l * K;
    a.topk_w = sa.topk_w + (size_t)l * K;
    epoch = fused_layer_b1<NCH, GD, DW, MAXS, true>(a, ws, G, (uint32_t)l, pre);
    if (l + 1 < sa.L) {
      const uint64_t* ln = s_lp[(l + 1) & 1];
      layer_prefetch<NCH>(pre, sa.gammas + (size_t)(l + 1) * H, reinterpret_cast<const uint16_t*>(uniform_u64(ln[0])),
                          reinterpret_cast<const float*>(uniform_u64(ln[5])),
                          sa.base.SI > 0 ? reinterpret_cast<const float*>(uniform_u64(ln[10])) : nullptr, H, E);
      // unconditional (clamped): a conditional load merged with the old value
      // would be waited for at once
      const int l2 = l + 2 < sa.L ? l + 2 : sa.L - 1;
      const int f = (int)threadIdx.x < NPTR ? (int)threadIdx.x : NPTR - 1;
      nxt = ldg<uint64_t>(tab + (size_t)l2 * NPTR + f);
    }
    __syncthreads();                               // this workgroup's rows of x_{l+1} are in s_xo
    if (sa.layer_out)
      for (int r = threadIdx.x; r < DROWS; r += 256)
        if (n0 + r < H) sa.layer_out[(size_t)l * H + n0 + r] = s_xo[n0 + r];
    if (l + 1 == sa.L) {
      for (int r = threadIdx.x; r < DROWS; r += 256)
        if (n0 + r < H) sa.x_out[n0 + r] = s_xo[n0 + r];
      break;
    }
    // publish this workgroup's rows (pairs n, n+1), one replica per lane
    for (int q = threadIdx.x; q < (DROWS / 2) * kReplicas; q += 256) {
      const int wq = q / kReplicas, r = q % kReplicas, n = n0 + 2 * wq;
      if (n < H)
        put_word(ws.x_words + (size_t)r * xrep + n / 2, epoch,
                 (uint32_t)s_xo[n] | ((uint32_t)s_xo[n + 1] << 16));
    }
    // and take every row of x_{l+1}
    const uint64_t* xw = ws.x_words + (size_t)rep * xrep;
    for (int q0 = threadIdx.x; q0 < H / 2; q0 += 4 * 256) {
      uint64_t wd[4];
      const uint64_t* ptr[4];
      bool ok[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = q0 + 256 * u;
        ok[u] = q < H / 2;
        ptr[u] = xw + (ok[u] ? q : 0);
      }
      poll_words<4>(wd, ptr, ok, epoch, ws.error, pre.lim);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (ok[u]) reinterpret_cast<uint32_t*>(s_x)[q0 + 256 * u] = (uint32_t)wd[u];
    }
    __syncthreads();
  }
  // the last layer's epoch, seen by every workgroup as above
  if (blockIdx.x == 0 && threadIdx.x == 0) *ws.epoch = epoch;
}

struct FusedConfig { int G, gd, dw, nch; };

// Grid and tiling of the fused path for this shape; false when the shape is
// outside what the kernel holds (the three-kernel path then runs instead).
bool fused_config(const LayerArgs& a, FusedConfig& c) {
  if (a.B != 1 || (a.flags & FLINT_W_BF16)) return false;
  if (a.H % 2048 || a.H > 4096) return false;
  if (a.I > 2048 || a.SI > 2048 || a.K > FLINT_MAX_TOP_K) return false;
  c.nch = a.H / 2048;
  c.G = device_num_cu();
  const int need = (a.H + 7) / 8;             // at most 8 output rows per workgroup
  if (c.G > need) c.G = need;
  if (c.G > a.E + kMaxArrivals) c.G = a.E + kMaxArrivals;
  const int rows_per_wg = (a.H + c.G - 1) / c.G;
  const int red = a.SI > 0 && a.SI < a.I ? a.SI : a.I;
  c.gd = 8;
  while (c.gd < red / 32 && c.gd < 64) c.gd <<= 1;
  c.dw = (rows_per_wg * c.gd + 63) / 64;
  if (c.dw > 2) return false;
  // every (slot, chunk step) item of the down rows must fit the prefetch
  const int ncs = (a.I > a.SI ? a.I : a.SI) / 32;
  const int dch = (ncs + c.gd - 1) / c.gd;
  const int S = a.K + (a.SI > 0 ? 1 : 0);
  constexpr int MAXI = ((FLINT_MAX_TOP_K + 1) * 2 + 3) / 4;
  if (S * dch > 4 * MAXI) return false;
  return true;
}

// Calls f(kernel) with the instantiation of KERNEL (the single-launch layer
// or the layer stack) that matches the tiling c.
#define FLINT_FUSED_DISPATCH(KERNEL, c, f)                                              \
  do {                                                                                 \
    constexpr int MAXS_ = FLINT_MAX_TOP_K + 1;                                         \
    if ((c).nch == 1) {                                                                \
      switch ((c).gd) {                                                                \
        case 8: if ((c).dw <= 1) f(KERNEL<1, 8, 1, MAXS_>); else f(KERNEL<1, 8, 2, MAXS_>); break;    \
        case 16: if ((c).dw <= 1) f(KERNEL<1, 16, 1, MAXS_>); else f(KERNEL<1, 16, 2, MAXS_>); break; \
        case 32: if ((c).dw <= 1) f(KERNEL<1, 32, 1, MAXS_>); else f(KERNEL<1, 32, 2, MAXS_>); break; \
        default: if ((c).dw <= 1) f(KERNEL<1, 64, 1, MAXS_>); else f(KERNEL<1, 64, 2, MAXS_>); break; \
      }                                                                                \
    } else {                                                                           \
      switch ((c).gd) {                                                                \
        case 8: if ((c).dw <= 1) f(KERNEL<2, 8, 1, MAXS_>); else f(KERNEL<2, 8, 2, MAXS_>); break;    \
        case 16: if ((c).dw <= 1) f(KERNEL<2, 16, 1, MAXS_>); else f(KERNEL<2, 16, 2, MAXS_>); break; \
        case 32: if ((c).dw <= 1) f(KERNEL<2, 32, 1, MAXS_>); else f(KERNEL<2, 32, 2, MAXS_>); break; \
        default: if ((c).dw <= 1) f(KERNEL<2, 64, 1, MAXS_>); else f(KERNEL<2, 64, 2, MAXS_>); break; \
      }                                                                                \
    }                                                                                  \
  } while (0)

// Whether the device can hold all G workgroups of this kernel at once (each
// needs a compute unit's worth of registers and LDS; the persistent grid's
// hand-offs assume every workgroup runs concurrently).  Asked once per
// instantiation; where the runtime cannot answer (no device) the shape
// rules alone decide.
template <class K>
bool grid_resident(K kernel, int G) {
  static int per_cu = -1;                          // -1: not asked yet, -2: no answer
  if (per_cu == -1) {
    int ndev = 0, n = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0)
      per_cu = -2;
    else
      per_cu = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, 256, 0) == hipSuccess ? n : -2;
  }
  return per_cu == -2 || (int64_t)per_cu * device_num_cu() >= G;
}

bool fused_resident(const FusedConfig& c, bool stack) {
  bool ok = false;
  auto check = [&](auto kernel) { ok = grid_resident(kernel, c.G); };
  if (stack) FLINT_FUSED_DISPATCH(fused_stack_b1_kernel, c, check);
  else FLINT_FUSED_DISPATCH(fused_decode_b1_kernel, c, check);
  return ok;
}

}  // namespace

bool fused_stack_supported(const LayerArgs& a) {
  FusedConfig c;
  if (!fused_config(a, c)) return false;
  if ((c.dw * (64 / c.gd)) % 2) return false;      // rows are published in pairs
  return fused_resident(c, true);
}

hipError_t launch_fused_stack(const StackArgs& sa, const DecodeWs& ws, hipStream_t st) {
  FusedConfig c;
  if (!fused_config(sa.base, c) || (c.dw * (64 / c.gd)) % 2) return hipErrorInvalidConfiguration;
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, dim3(c.G), dim3(256), 0, st, sa, ws, c.G); };
  FLINT_FUSED_DISPATCH(fused_stack_b1_kernel, c, go);
  return hipGetLastError();
}

bool fused_decode_supported(const LayerArgs& a) {
  FusedConfig c;
  return fused_config(a, c) && fused_resident(c, false);
}

hipError_t launch_fused_decode(const LayerArgs& a, const DecodeWs& ws, hipStream_t st) {
  FusedConfig c;
  if (!fused_config(a, c)) return hipErrorInvalidConfiguration;
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, dim3(c.G), dim3(256), 0, st, a, ws, c.G); };
  FLINT_FUSED_DISPATCH(fused_decode_b1_kernel, c, go);
  return hipGetLastError();
}

}  // namespace flint
