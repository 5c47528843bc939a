// Small-batch (1..8 tokens) decode MoE layer for gfx950: three kernels.
//
//  route    RMSNorm (optional), router GEMV with fp32 accumulation, sigmoid
//           top-k and the expert set, done by the last workgroup to finish
//  gate_up  for every selected expert (and the shared one) and a tile of
//           rows: E2M1 x UE4M3 dequant in registers, BF16 dot products with
//           fp32 accumulation, DPP reductions, BF16(SiLU(g)) * u epilogue
//  down     per tile of output rows, every selected expert's down rows:
//           weighted combine, shared expert and optional residual, one
//           BF16 rounding of the sum
//
// What is computed follows "Day-0 Support for Flint on vLLM": "Model
// architecture" (256 experts, sigmoid top-6, a shared expert; W4A16 with
// BF16 activations, rounding where the reference rounds) and "Optimizations"
// (router and expert GEMVs that read only the selected experts' weights;
// routing and the combine fused into the neighbouring GEMV kernels on the
// path for up to 8 requests).  Each selected expert's weights are read once
// per call and applied to every token routed to it.
#include "fused_common.hpp"

namespace flint {
namespace {

constexpr int kMaxB = FLINT_MAX_DECODE_BATCH;

// ------------------------------------------------------------------ route --
// Router GEMV + top-k.  Each wave owns one routed expert and computes its
// logit for every token (all router and activation loads of a lane issued
// before the first use); with PRE_RMSNORM every wave normalises the tokens
// itself and workgroup 0 stores xn for the expert kernels.
//
// Hand-off without a cache-flushing fence: every logit is published as one
// 64-bit atomic word (call epoch << 32 | logit bits).  The workgroup that
// takes the last ticket polls the words, all of a wave's two tokens at once,
// until they carry this call's epoch (data and "ready" flag are the same
// word, so no store ordering is relied on), then selects the top-k of every
// token and writes the expert set.
// It finally advances the epoch and returns the ticket to zero; both are
// read again only by the next launch.  The poll is bounded: if a word never
// arrives (it cannot, short of a hardware fault) the kernel records an
// error word in the workspace and still exits.

template <int BT, int NIT, bool NORM>
__global__ __launch_bounds__(256) void route_kernel(LayerArgs a, DecodeWs ws) {
  __shared__ uint32_t s_mask[FLINT_MAX_EXPERTS];
  __shared__ float s_w[FLINT_MAX_EXPERTS][kMaxB];
  __shared__ int s_wcnt[4];
  __shared__ int s_last;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int H = a.H, B = a.B, E = a.E;
  constexpr bool norm = NORM;
  const int e = blockIdx.x * 4 + wave;
  const int er = e < E ? e : E - 1;          // surplus waves recompute the last expert
  const uint32_t epoch = *ws.epoch + 1u;

  // all tokens' activations are fetched up front when they fit in registers
  constexpr bool kHoist = NORM ? NIT * BT <= 16 : NIT <= 4;
  constexpr int XT = kHoist ? BT : 1;
  uint4 wv[NIT], gv[NIT], xv[XT][NIT];
  auto load_token = [&](uint4* dst, int t) {
    const int tt = t < B ? t : B - 1;        // rows past the batch re-read the last one
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
      const int col = 8 * (lane + 64 * i);
      dst[i] = col < H ? *reinterpret_cast<const uint4*>(a.x + (size_t)tt * H + col) : make_uint4(0, 0, 0, 0);
    }
  };
#pragma unroll
  for (int i = 0; i < NIT; ++i) {
    const int col = 8 * (lane + 64 * i);
    const bool ok = col < H;
    wv[i] = ok ? *reinterpret_cast<const uint4*>(a.router + (size_t)er * H + col) : make_uint4(0, 0, 0, 0);
    gv[i] = (ok && norm) ? *reinterpret_cast<const uint4*>(a.gamma + col) : make_uint4(0, 0, 0, 0);
  }
  if constexpr (kHoist) {
#pragma unroll
    for (int t = 0; t < BT; ++t) load_token(xv[t], t);
  }
  float acc[BT];
#pragma unroll
  for (int t = 0; t < BT; ++t) {
    uint4* xt = xv[kHoist ? t : 0];
    if constexpr (!kHoist) load_token(xt, t);
    if (norm) {
      double ss = 0.0;
#pragma unroll
      for (int i = 0; i < NIT; ++i) {
        const uint32_t q[4] = {xt[i].x, xt[i].y, xt[i].z, xt[i].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const double lo = bf16_lo(q[m]), hi = bf16_hi(q[m]);
          ss = fma(lo, lo, ss);
          ss = fma(hi, hi, ss);
        }
      }
      ss = wave_sum_f64(ss);
      const Rms rms = make_rms(sqrt(ss / (double)H + (double)a.eps));
#pragma unroll
      for (int i = 0; i < NIT; ++i) {
        uint32_t q[4] = {xt[i].x, xt[i].y, xt[i].z, xt[i].w};
        const uint32_t g4[4] = {gv[i].x, gv[i].y, gv[i].z, gv[i].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float lo = round_bf16(rms_scale_bf16(bf16_lo(q[m]), rms) * bf16_lo(g4[m]));
          const float hi = round_bf16(rms_scale_bf16(bf16_hi(q[m]), rms) * bf16_hi(g4[m]));
          q[m] = pack_bf16x2(lo, hi);
        }
        xt[i] = make_uint4(q[0], q[1], q[2], q[3]);
        const int col = 8 * (lane + 64 * i);
        if (e == 0 && t < B && col < H) *reinterpret_cast<uint4*>(ws.xn + (size_t)t * H + col) = xt[i];
      }
    }
    float sacc = 0.f;
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
      sacc = dot2_bf16(wv[i].x, xt[i].x, sacc);
      sacc = dot2_bf16(wv[i].y, xt[i].y, sacc);
      sacc = dot2_bf16(wv[i].z, xt[i].z, sacc);
      sacc = dot2_bf16(wv[i].w, xt[i].w, sacc);
    }
    acc[t] = sacc;
  }
#pragma unroll
  for (int t = 0; t < BT; ++t) {
    const float v = group_sum<64>(acc[t]);
    if (lane == 0 && t < B && e < E)
      __hip_atomic_store(ws.logit_words + t * E + e,
                         ((uint64_t)epoch << 32) | (uint64_t)__float_as_uint(v), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }

  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(ws.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;

  // ---- the last workgroup: top-k per token (tokens dealt to the waves)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    s_mask[threadIdx.x] = 0u;   // 256 threads cover the 256 experts
    s_w[threadIdx.x][j] = 0.f;
    s_w[threadIdx.x][j + 4] = 0.f;
  }
  __syncthreads();
  const bool renorm = (a.flags & FLINT_RENORM) != 0;
  {
    // tokens wave and wave + 4: all their logit words polled at once
    uint64_t wd[8];
    const uint64_t* ptr[8];
    bool ok[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = wave + 4 * h;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ex = lane + 64 * q;
        ok[4 * h + q] = t < B && ex < E;
        ptr[4 * h + q] = ws.logit_words + (size_t)(t < B ? t : 0) * E + (ex < E ? ex : 0);
      }
    }
    poll_words<8>(wd, ptr, ok, epoch, ws.error);
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
      const uint64_t my_key = select_topk(key, a.K);
      const int my_e = (int)~(uint32_t)my_key;
      const float my_s = lane < a.K ? 1.0f / (1.0f + expf(-float_from_order_key((uint32_t)(my_key >> 32)))) : 0.f;
      float ssum = 0.f;
      for (int k = 0; k < a.K; ++k)                 // selection order
        ssum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), k));
      if (lane < a.K) {
        const float w = renorm ? my_s / ssum : my_s;
        a.topk_idx[t * a.K + lane] = my_e;
        a.topk_w[t * a.K + lane] = w;
        atomicOr(&s_mask[my_e], 1u << t);
        s_w[my_e][t] = w;
      }
    }
  }
  __syncthreads();

  // routed slots = the selected experts in ascending index order
  const int ex = threadIdx.x;
  const uint32_t m = ex < E ? s_mask[ex] : 0u;
  const unsigned long long bal = __ballot(m != 0u);
  if (lane == 0) s_wcnt[wave] = __popcll(bal);
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += s_wcnt[w];
  if (m != 0u) {
    const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
    ws.slot_expert[pos] = ex;
    ws.slot_mask[pos] = m;
#pragma unroll
    for (int t = 0; t < kMaxB; ++t) ws.slot_w[pos * kMaxB + t] = s_w[ex][t];
  }
  if (threadIdx.x == 0) {
    *ws.nslot = s_wcnt[0] + s_wcnt[1] + s_wcnt[2] + s_wcnt[3];
    *ws.epoch = epoch;
    __hip_atomic_store(ws.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// -------------------------------------------------------------- weights ----

// Row pointers of one matrix of the selected expert.
template <int WF> struct MatRef {
  const uint8_t* codes;     // NVFP4 code plane of the matrix
  const uint8_t* scales;
  const uint16_t* wbf;      // BF16 matrix
  int cols;
};

template <int WF>
__device__ __forceinline__ uint4 load_chunk_raw(const MatRef<WF>& m, int row, int j, uint32_t& sc) {
  if constexpr (WF == FMT_NVFP4) {
    sc = reinterpret_cast<const uint16_t*>(m.scales + (size_t)row * (m.cols / 16))[j];
    return reinterpret_cast<const uint4*>(m.codes + (size_t)row * (m.cols / 2))[j];
  } else {
    sc = 0;
    return reinterpret_cast<const uint4*>(m.wbf + (size_t)row * m.cols)[j];
  }
}

template <int WF>
__device__ __forceinline__ DChunk<WF> decode_chunk(uint4 c, uint32_t sc) {
  if constexpr (WF == FMT_NVFP4) {
    return decode_nvfp4(c, sc);
  } else {
    DChunk<FMT_BF16> d;
    d.w[0] = c.x; d.w[1] = c.y; d.w[2] = c.z; d.w[3] = c.w;
    return d;
  }
}

// x chunk with RMSNorm applied on the fly: BF16(BF16(x / rms) * gamma)
template <int WF>
__device__ __forceinline__ XChunk<WF> load_x_norm(const uint16_t* row, const uint16_t* gamma, int j,
                                                  const Rms& rms) {
  XChunk<WF> x = load_x<WF>(row, j);
  const XChunk<WF> g = load_x<WF>(gamma, j);
#pragma unroll
  for (int m = 0; m < Fmt<WF>::VALS / 2; ++m) {
    const float lo = round_bf16(rms_scale_bf16(bf16_lo(x.v[m]), rms) * bf16_lo(g.v[m]));
    const float hi = round_bf16(rms_scale_bf16(bf16_hi(x.v[m]), rms) * bf16_hi(g.v[m]));
    x.v[m] = pack_bf16x2(lo, hi);
  }
  return x;
}

// ---------------------------------------------------------------- gate/up --
// Grid (row tiles, slots).  Slot 0 is the shared expert (when there is one):
// its workgroups start loading at once, with no routing to wait for.  Each
// wave owns P row sets of 64/G rows; lane group `grp` (G lanes) owns one row
// per set and walks its chunks.  The gate and the up row of the same index
// are computed by the same lanes, so SiLU(g) * u happens in registers.
template <int WF, int G, int P, int NW, int BT, bool NORM>
__global__ __launch_bounds__(64 * NW) void gate_up_kernel(LayerArgs a, DecodeWs ws, int dense,
                                                          uint16_t* hout, int h_slot_stride,
                                                          int h_tok_stride) {
  constexpr int GPW = 64 / G;           // rows per wave-wide load
  constexpr int RPW = P * GPW;          // rows per wave
  const int slot = blockIdx.y;
  const bool has_sh = a.SI > 0;
  const bool shared = has_sh && slot == 0;
  const int inter = shared ? a.SI : a.I;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int grp = lane / G, li = lane % G;
  const int row0 = (blockIdx.x * NW + wave) * RPW;
  if (row0 >= inter) return;
  const int H = a.H;
  const int cpr = H / Fmt<WF>::VALS;

  MatRef<WF> mg, mu;
  float gs_g = 1.f, gs_u = 1.f;
  mg.cols = mu.cols = H;
  uint32_t mask;
  if (shared) {
    mask = (1u << a.B) - 1u;
    if constexpr (WF == FMT_NVFP4) {
      mg.codes = a.sh_gu_codes;  mu.codes = a.sh_gu_codes + (size_t)inter * H / 2;
      mg.scales = a.sh_gu_scales; mu.scales = a.sh_gu_scales + (size_t)inter * H / 16;
      gs_g = a.sh_gscale[0]; gs_u = a.sh_gscale[1];
    } else {
      mg.wbf = a.sh_gu_bf16; mu.wbf = a.sh_gu_bf16 + (size_t)inter * H;
    }
  } else {
    const int r = slot - (has_sh ? 1 : 0);
    if (dense || r >= *ws.nslot) return;
    const int e = ws.slot_expert[r];
    mask = ws.slot_mask[r];
    if constexpr (WF == FMT_NVFP4) {
      const size_t mc = (size_t)inter * H / 2, ms = (size_t)inter * H / 16;
      mg.codes = a.gu_codes + (size_t)(2 * e) * mc;  mu.codes = mg.codes + mc;
      mg.scales = a.gu_scales + (size_t)(2 * e) * ms; mu.scales = mg.scales + ms;
      gs_g = a.gscale[3 * e + 0]; gs_u = a.gscale[3 * e + 1];
    } else {
      const size_t mb = (size_t)inter * H;
      mg.wbf = a.gu_bf16 + (size_t)(2 * e) * mb; mu.wbf = mg.wbf + mb;
    }
  }
  const uint16_t* xsrc = NORM ? a.x : ((a.flags & FLINT_PRE_RMSNORM) && !dense ? ws.xn : a.x);

  Rms rinv[BT];         // RMS of each token (only with NORM)
#pragma unroll
  for (int t = 0; t < BT; ++t) rinv[t] = Rms{1.0, 1.0};
  if constexpr (NORM) {
    const int niter = (H + 511) / 512;
#pragma unroll
    for (int t = 0; t < BT; ++t) {
      if ((mask >> t) & 1u) {
        double ss = 0.0;
        for (int i = 0; i < niter; ++i) {
          const int col = 8 * (lane + 64 * i);
          if (col < H) {
            const uint4 v = *reinterpret_cast<const uint4*>(a.x + (size_t)t * H + col);
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const double lo = bf16_lo(w4[q]), hi = bf16_hi(w4[q]);
              ss = fma(lo, lo, ss);
              ss = fma(hi, hi, ss);
            }
          }
        }
        ss = wave_sum_f64(ss);
        rinv[t] = make_rms(sqrt(ss / (double)H + (double)a.eps));
      }
    }
  }

  float acc[P][2][BT];
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int t = 0; t < BT; ++t) acc[p][0][t] = acc[p][1][t] = 0.f;

  const int nch = (cpr + G - 1) / G;
  for (int c = 0; c < nch; ++c) {
    const int j = li + G * c;
    const bool jv = j < cpr;
    uint4 rg[P], ru[P];
    uint32_t sg[P], su[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int r = row0 + p * GPW + grp;
      rg[p] = ru[p] = make_uint4(0, 0, 0, 0);
      sg[p] = su[p] = 0;
      if (jv && r < inter) {
        rg[p] = load_chunk_raw<WF>(mg, r, j, sg[p]);
        ru[p] = load_chunk_raw<WF>(mu, r, j, su[p]);
      }
    }
    // the first token's activations are fetched together with the weights
    XChunk<WF> x0;
    int t0 = -1;
#pragma unroll
    for (int t = BT - 1; t >= 0; --t)
      if ((mask >> t) & 1u) t0 = t;
    if (jv && t0 >= 0) {
      if constexpr (NORM) x0 = load_x_norm<WF>(xsrc + (size_t)t0 * H, a.gamma, j, rinv[t0]);
      else x0 = load_x<WF>(xsrc + (size_t)t0 * H, j);
    }
    DChunk<WF> dg[P], du[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      dg[p] = decode_chunk<WF>(rg[p], sg[p]);
      du[p] = decode_chunk<WF>(ru[p], su[p]);
    }
#pragma unroll
    for (int t = 0; t < BT; ++t) {
      if (((mask >> t) & 1u) && jv) {
        XChunk<WF> xc;
        if (t == t0) xc = x0;
        else if constexpr (NORM) xc = load_x_norm<WF>(xsrc + (size_t)t * H, a.gamma, j, rinv[t]);
        else xc = load_x<WF>(xsrc + (size_t)t * H, j);
#pragma unroll
        for (int p = 0; p < P; ++p) {
          acc[p][0][t] += chunk_dot(dg[p], xc);
          acc[p][1][t] += chunk_dot(du[p], xc);
        }
      }
    }
  }

#pragma unroll
  for (int t = 0; t < BT; ++t) {
    if ((mask >> t) & 1u) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const float g = group_sum<G>(acc[p][0][t]);
        const float u = group_sum<G>(acc[p][1][t]);
        const int r = row0 + p * GPW + grp;
        if (li == 0 && r < inter) {
          const float gv = round_bf16(g * gs_g);
          const float uv = round_bf16(u * gs_u);
          const float av = round_bf16(silu_f32(gv));
          hout[(size_t)slot * h_slot_stride + (size_t)t * h_tok_stride + r] =
              f32_to_bf16_bits(av * uv);
        }
      }
    }
  }
}

// ------------------------------------------------------------ down+combine --
// Grid: tiles of RPW output rows.  The slot table is staged in LDS once; the
// work items (slot, chunk step) are dealt to the NW waves, U items per wave
// with all their weight (and, at batch 1, activation) loads in flight
// together.  Every wave accumulates weight * W_d h for its items, the waves'
// partial sums are added in a fixed order through LDS, and the sum is
// rounded once (then the residual is added and rounded, if asked).
constexpr int kMaxSlots = FLINT_MAX_DECODE_BATCH * FLINT_MAX_TOP_K + 1;

template <int WF, int G, int RW, int NW, int U, int BT>
__global__ __launch_bounds__(64 * NW) void down_kernel(LayerArgs a, DecodeWs ws, int dense, int epi,
                                                       const uint16_t* hin, int h_slot_stride,
                                                       int h_tok_stride, int dense_cols,
                                                       const uint16_t* aux) {
  constexpr int GPW = 64 / G;
  constexpr int RPW = RW * GPW;
  __shared__ float s_red[NW][RPW][BT];
  __shared__ int s_exp[kMaxSlots];
  __shared__ uint32_t s_msk[kMaxSlots];
  __shared__ float s_wt[kMaxSlots][BT];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int grp = lane / G, li = lane % G;
  const int H = a.H;          // output rows
  const int n0 = blockIdx.x * RPW;
  const bool has_sh = dense || a.SI > 0;
  const int sh = has_sh ? 1 : 0;
  const int nU = dense ? 0 : *ws.nslot;
  const int S = nU + sh;
  const int I = dense ? dense_cols : a.I;
  const int SI = dense ? dense_cols : a.SI;
  const int cpr_max = (I > SI ? I : SI) / Fmt<WF>::VALS;
  const int nch = (cpr_max + G - 1) / G;
  const bool resid = dense ? (epi == FLINT_EPI_RESIDUAL) : ((a.flags & FLINT_RESIDUAL) != 0);
  const uint16_t* xr = dense ? aux : a.x;

  // slot table -> LDS (slot s: 0 = shared, s >= sh = routed slot s - sh)
  for (int q = threadIdx.x; q < S; q += 64 * NW) {
    if (has_sh && q == 0) {
      s_exp[0] = -1;
      s_msk[0] = (1u << a.B) - 1u;
#pragma unroll
      for (int t = 0; t < BT; ++t) s_wt[0][t] = 1.f;
    } else {
      const int r = q - sh;
      s_exp[q] = ws.slot_expert[r];
      s_msk[q] = ws.slot_mask[r];
#pragma unroll
      for (int t = 0; t < BT; ++t) s_wt[q][t] = ws.slot_w[r * kMaxB + t];
    }
  }
  // the residual of the rows this thread will write, fetched early
  float xres = 0.f;
  {
    const int q = threadIdx.x;
    if (resid && q < RPW * BT) {
      const int rloc = q / BT, t = q - rloc * BT, n = n0 + rloc;
      if (t < a.B && n < H) xres = bf16_bits_to_f32(xr[(size_t)t * H + n]);
    }
  }
  __syncthreads();

  float acc[RW][BT];
#pragma unroll
  for (int rw = 0; rw < RW; ++rw)
#pragma unroll
    for (int t = 0; t < BT; ++t) acc[rw][t] = 0.f;

  const int total = S * nch;
  for (int it0 = wave; it0 < total; it0 += NW * U) {
    uint4 raw[U][RW];
    uint32_t sc[U][RW];
    XChunk<WF> h0[U];
    bool jv[U];
    int sl[U], jj[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = it0 + u * NW;
      const int s = it < total ? it / nch : 0;
      const int c = it - s * nch;
      sl[u] = s;
      const int e = s_exp[s];
      const int inter = e < 0 ? SI : I;
      const int cpr = inter / Fmt<WF>::VALS;
      const int j = li + G * c;
      jj[u] = j;
      jv[u] = it < total && j < cpr;
      MatRef<WF> md;
      md.cols = inter;
      if (e < 0) {
        if constexpr (WF == FMT_NVFP4) { md.codes = a.sh_d_codes; md.scales = a.sh_d_scales; }
        else md.wbf = a.sh_d_bf16;
      } else {
        if constexpr (WF == FMT_NVFP4) {
          md.codes = a.d_codes + (size_t)e * H * (inter / 2);
          md.scales = a.d_scales + (size_t)e * H * (inter / 16);
        } else {
          md.wbf = a.d_bf16 + (size_t)e * H * inter;
        }
      }
#pragma unroll
      for (int rw = 0; rw < RW; ++rw) {
        const int n = n0 + rw * GPW + grp;
        raw[u][rw] = make_uint4(0, 0, 0, 0);
        sc[u][rw] = 0;
        if (jv[u] && n < H) raw[u][rw] = load_chunk_raw<WF>(md, n, j, sc[u][rw]);
      }
      if constexpr (BT == 1) {
        if (jv[u]) h0[u] = load_x<WF>(hin + (size_t)(dense ? 0 : s) * h_slot_stride, j);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!jv[u]) continue;
      const int s = sl[u];
      const int e = s_exp[s];
      const uint32_t mask = s_msk[s];
      float gd = 1.f;
      if constexpr (WF == FMT_NVFP4) gd = e < 0 ? a.sh_gscale[dense ? 0 : 2] : a.gscale[3 * e + 2];
      DChunk<WF> d[RW];
#pragma unroll
      for (int rw = 0; rw < RW; ++rw) d[rw] = decode_chunk<WF>(raw[u][rw], sc[u][rw]);
      const uint16_t* hs = hin + (size_t)(dense ? 0 : s) * h_slot_stride;
#pragma unroll
      for (int t = 0; t < BT; ++t) {
        if ((mask >> t) & 1u) {
          XChunk<WF> hx;
          if constexpr (BT == 1) hx = h0[u];
          else hx = load_x<WF>(hs + (size_t)t * h_tok_stride, jj[u]);
          const float f = s_wt[s][t] * gd;
#pragma unroll
          for (int rw = 0; rw < RW; ++rw) acc[rw][t] = fmaf(f, chunk_dot(d[rw], hx), acc[rw][t]);
        }
      }
    }
  }

#pragma unroll
  for (int rw = 0; rw < RW; ++rw)
#pragma unroll
    for (int t = 0; t < BT; ++t) {
      const float v = group_sum<G>(acc[rw][t]);
      if (li == 0) s_red[wave][rw * GPW + grp][t] = v;
    }
  __syncthreads();

  const int q = threadIdx.x;
  if (q < RPW * BT) {
    const int rloc = q / BT, t = q - rloc * BT;
    const int n = n0 + rloc;
    if (t < a.B && n < H) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += s_red[w][rloc][t];
      float o = round_bf16(v);
      if (resid) o = xres + o;
      a.out[(size_t)t * H + n] = f32_to_bf16_bits(o);
    }
  }
}

// ------------------------------------------------------------ dispatch ----

inline int pow2ceil(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

inline int lanes_per_row(int cpr) { return cpr >= 64 ? 64 : (pow2ceil(cpr) < 8 ? 8 : pow2ceil(cpr)); }

template <int WF, int G, int BT>
hipError_t gate_up_dispatch_norm(const LayerArgs& a, const DecodeWs& ws, bool dense, bool norm,
                                 uint16_t* hout, int hs, int ht, int rows, hipStream_t st) {
  constexpr int NW = 4;
  constexpr int P = (G == 64) ? 2 : 1;
  constexpr int RPW = P * (64 / G);
  const int tiles = (rows + NW * RPW - 1) / (NW * RPW);
  const int slots = dense ? 1 : decode_max_slots({a.H, a.E, a.I, a.SI, a.K, 0, 0.f}, a.B);
  dim3 grid(tiles, slots);
  if (norm)
    hipLaunchKernelGGL((gate_up_kernel<WF, G, P, NW, BT, true>), grid, dim3(64 * NW), 0, st, a, ws,
                       dense ? 1 : 0, hout, hs, ht);
  else
    hipLaunchKernelGGL((gate_up_kernel<WF, G, P, NW, BT, false>), grid, dim3(64 * NW), 0, st, a, ws,
                       dense ? 1 : 0, hout, hs, ht);
  return hipGetLastError();
}

template <int WF, int BT>
hipError_t gate_up_dispatch_g(const LayerArgs& a, const DecodeWs& ws, bool dense, bool norm,
                              uint16_t* hout, int hs, int ht, int rows, hipStream_t st) {
  switch (lanes_per_row(a.H / Fmt<WF>::VALS)) {
    case 8: return gate_up_dispatch_norm<WF, 8, BT>(a, ws, dense, norm, hout, hs, ht, rows, st);
    case 16: return gate_up_dispatch_norm<WF, 16, BT>(a, ws, dense, norm, hout, hs, ht, rows, st);
    case 32: return gate_up_dispatch_norm<WF, 32, BT>(a, ws, dense, norm, hout, hs, ht, rows, st);
    default: return gate_up_dispatch_norm<WF, 64, BT>(a, ws, dense, norm, hout, hs, ht, rows, st);
  }
}

template <int WF, int G, int BT>
hipError_t down_dispatch_rw(const LayerArgs& a, const DecodeWs& ws, bool dense, int epi,
                            const uint16_t* hin, int hs, int ht, int dense_cols,
                            const uint16_t* aux, hipStream_t st) {
  constexpr int NW = 4;
  constexpr int RW = (G == 64) ? 4 : (BT == 1 ? 1 : 2);
  constexpr int U = BT == 1 ? 2 : 4;
  constexpr int RPW = RW * (64 / G);
  const int tiles = (a.H + RPW - 1) / RPW;
  hipLaunchKernelGGL((down_kernel<WF, G, RW, NW, U, BT>), dim3(tiles), dim3(64 * NW), 0, st, a, ws,
                     dense ? 1 : 0, epi, hin, hs, ht, dense_cols, aux);
  return hipGetLastError();
}

template <int WF, int BT>
hipError_t down_dispatch_g(const LayerArgs& a, const DecodeWs& ws, bool dense, int epi,
                           const uint16_t* hin, int hs, int ht, int dense_cols,
                           const uint16_t* aux, hipStream_t st) {
  int red = dense ? dense_cols : a.I;
  if (!dense && a.SI > 0 && a.SI < red) red = a.SI;
  switch (lanes_per_row(red / Fmt<WF>::VALS)) {
    case 8: return down_dispatch_rw<WF, 8, BT>(a, ws, dense, epi, hin, hs, ht, dense_cols, aux, st);
    case 16: return down_dispatch_rw<WF, 16, BT>(a, ws, dense, epi, hin, hs, ht, dense_cols, aux, st);
    case 32: return down_dispatch_rw<WF, 32, BT>(a, ws, dense, epi, hin, hs, ht, dense_cols, aux, st);
    default: return down_dispatch_rw<WF, 64, BT>(a, ws, dense, epi, hin, hs, ht, dense_cols, aux, st);
  }
}

template <int BT, bool NORM>
hipError_t route_dispatch_n(const LayerArgs& a, const DecodeWs& ws, hipStream_t st) {
  const int nit = (a.H + 511) / 512;
  dim3 grid((a.E + 3) / 4), block(256);
  switch (nit) {
    case 1: hipLaunchKernelGGL((route_kernel<BT, 1, NORM>), grid, block, 0, st, a, ws); break;
    case 2: hipLaunchKernelGGL((route_kernel<BT, 2, NORM>), grid, block, 0, st, a, ws); break;
    case 3: hipLaunchKernelGGL((route_kernel<BT, 3, NORM>), grid, block, 0, st, a, ws); break;
    case 4: hipLaunchKernelGGL((route_kernel<BT, 4, NORM>), grid, block, 0, st, a, ws); break;
    default: hipLaunchKernelGGL((route_kernel<BT, 8, NORM>), grid, block, 0, st, a, ws); break;
  }
  return hipGetLastError();
}

template <int BT>
hipError_t route_dispatch(const LayerArgs& a, const DecodeWs& ws, hipStream_t st) {
  return (a.flags & FLINT_PRE_RMSNORM) ? route_dispatch_n<BT, true>(a, ws, st)
                                       : route_dispatch_n<BT, false>(a, ws, st);
}

}  // namespace

int decode_max_slots(const flint_moe_shape& s, int batch) {
  int u = batch * s.top_k;
  if (u > s.n_experts) u = s.n_experts;
  return u + (s.shared_inter > 0 ? 1 : 0);
}

hipError_t launch_route(const LayerArgs& a, const DecodeWs& ws, hipStream_t st) {
  return a.B == 1 ? route_dispatch<1>(a, ws, st) : route_dispatch<kMaxB>(a, ws, st);
}

hipError_t launch_gate_up(const LayerArgs& a, const DecodeWs& ws, bool dense, bool norm,
                          hipStream_t st) {
  // decode: h[slot][t][Imax]; dense: y[t][rows] with rows = SI
  const int imax = a.I > a.SI ? a.I : a.SI;
  uint16_t* hout = dense ? a.out : ws.h;
  const int hs = dense ? 0 : kMaxB * imax;
  const int ht = dense ? a.SI : imax;
  const bool bf = (a.flags & FLINT_W_BF16) != 0;
  if (a.B == 1)
    return bf ? gate_up_dispatch_g<FMT_BF16, 1>(a, ws, dense, norm, hout, hs, ht, imax, st)
              : gate_up_dispatch_g<FMT_NVFP4, 1>(a, ws, dense, norm, hout, hs, ht, imax, st);
  return bf ? gate_up_dispatch_g<FMT_BF16, kMaxB>(a, ws, dense, norm, hout, hs, ht, imax, st)
            : gate_up_dispatch_g<FMT_NVFP4, kMaxB>(a, ws, dense, norm, hout, hs, ht, imax, st);
}

hipError_t launch_down(const LayerArgs& a, const DecodeWs& ws, bool dense, int dense_epilogue,
                       const uint16_t* dense_in, const uint16_t* aux, hipStream_t st) {
  const int imax = a.I > a.SI ? a.I : a.SI;
  const uint16_t* hin = dense ? dense_in : ws.h;
  const int hs = dense ? 0 : kMaxB * imax;
  const int ht = dense ? a.SI : imax;
  const int dcols = dense ? a.SI : 0;
  const bool bf = (a.flags & FLINT_W_BF16) != 0;
  if (a.B == 1)
    return bf ? down_dispatch_g<FMT_BF16, 1>(a, ws, dense, dense_epilogue, hin, hs, ht, dcols, aux, st)
              : down_dispatch_g<FMT_NVFP4, 1>(a, ws, dense, dense_epilogue, hin, hs, ht, dcols, aux, st);
  return bf ? down_dispatch_g<FMT_BF16, kMaxB>(a, ws, dense, dense_epilogue, hin, hs, ht, dcols, aux, st)
            : down_dispatch_g<FMT_NVFP4, kMaxB>(a, ws, dense, dense_epilogue, hin, hs, ht, dcols, aux, st);
}

}  // namespace flint
