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
        xt[i] = rms_norm_8(xt[i], gv[i], rms);
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
    poll_words<8>(wd, ptr, ok, epoch, ws.error, wait_limit(ws));
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

// ------------------------------------------------------ route, batch 2..8 --
// One workgroup per routed expert; wave w takes the w-th quarter of the row
// (8 columns per lane), so every load of the kernel -- its router quarter,
// every token's matching quarter, γ -- is one 16-byte load per lane, all
// issued at once and unconditionally (tokens past the batch re-read token
// 0).  With RMSNorm each wave adds its quarter's squares (float64) and the
// four are combined through LDS.  A logit is the sum of the four quarter
// sums in wave order, with the same per-lane order as the single-launch
// batch kernel, so both produce the same logits bit for bit.  Workgroup 0
// then polls every logit word (no ticket: the other workgroups' words carry
// this call's epoch, read before they were written), selects the top-k of
// every token, writes the expert set and advances the epoch.
template <int NQ, bool NORM>
__global__ __launch_bounds__(256) void route_batch_kernel(LayerArgs a, DecodeWs ws) {
  constexpr int BT = kMaxB;
  __shared__ float s_part[4][BT];
  __shared__ double s_ss[4][BT];
  __shared__ uint32_t s_mask[FLINT_MAX_EXPERTS];
  __shared__ float s_w[FLINT_MAX_EXPERTS][kMaxB];
  __shared__ int s_wcnt[4];
  __shared__ uint64_t s_key[4][FLINT_MAX_TOP_K];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int H = a.H, B = a.B, E = a.E;
  const int e = blockIdx.x;
  const int qlen = H / 4, q0 = wave * qlen;
  uint4 rv[NQ], gv[NQ], xv[BT][NQ];
  bool okc[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int off = 8 * lane + 512 * i;
    okc[i] = off < qlen;
    const int col = q0 + (okc[i] ? off : 0);
    rv[i] = *reinterpret_cast<const uint4*>(a.router + (size_t)e * H + col);
    if constexpr (NORM) gv[i] = *reinterpret_cast<const uint4*>(a.gamma + col);
#pragma unroll
    for (int t = 0; t < BT; ++t) xv[t][i] = *reinterpret_cast<const uint4*>(a.x + (size_t)(t < B ? t : 0) * H + col);
  }
  // the launch epoch (a vector load behind the others)
  const uint32_t epoch = __hip_atomic_load(ws.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  if constexpr (NORM) {
#pragma unroll
    for (int t = 0; t < BT; ++t) {
      double ss0 = 0.0, ss1 = 0.0;
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        if (!okc[i]) continue;
        const uint32_t q[4] = {xv[t][i].x, xv[t][i].y, xv[t][i].z, xv[t][i].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const double lo = bf16_lo(q[m]), hi = bf16_hi(q[m]);
          ss0 = fma(lo, lo, ss0);
          ss1 = fma(hi, hi, ss1);
        }
      }
      const double ssw = wave_sum_f64(ss0 + ss1);
      if (lane == 0) s_ss[wave][t] = ssw;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < BT; ++t) {
      const double ss = (s_ss[0][t] + s_ss[1][t]) + (s_ss[2][t] + s_ss[3][t]);
      const Rms rms = make_rms(sqrt(ss / (double)H + (double)a.eps));
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        xv[t][i] = rms_norm_8(xv[t][i], gv[i], rms);
        if (e == 0 && t < B && okc[i])
          *reinterpret_cast<uint4*>(ws.xn + (size_t)t * H + q0 + 8 * lane + 512 * i) = xv[t][i];
      }
    }
  }
  float part[BT];
#pragma unroll
  for (int t = 0; t < BT; ++t) {
    float p = 0.f;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      if (!okc[i]) continue;
      p = dot2_bf16(rv[i].x, xv[t][i].x, p);
      p = dot2_bf16(rv[i].y, xv[t][i].y, p);
      p = dot2_bf16(rv[i].z, xv[t][i].z, p);
      p = dot2_bf16(rv[i].w, xv[t][i].w, p);
    }
    part[t] = group_sum<64>(p);
  }
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < BT; ++t) s_part[wave][t] = part[t];
  }
  __syncthreads();
  if (wave == 0 && lane < B) {
    const float l = s_part[0][lane] + s_part[1][lane] + s_part[2][lane] + s_part[3][lane];
    __hip_atomic_store(ws.logit_words + (size_t)lane * E + e, ((uint64_t)epoch << 32) | (uint64_t)__float_as_uint(l),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (blockIdx.x != 0) return;

  // ---- workgroup 0: top-k per token (tokens w and w + 4 on wave w)
  for (int q = threadIdx.x; q < FLINT_MAX_EXPERTS; q += 256) {
    s_mask[q] = 0u;
#pragma unroll
    for (int t = 0; t < kMaxB; ++t) s_w[q][t] = 0.f;
  }
  __syncthreads();
  const bool renorm = (a.flags & FLINT_RENORM) != 0;
  {
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
    poll_words_pipelined<8, 1>(wd, ptr, ok, epoch, ws.error, wait_limit(ws));
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
      topk_keys_to_lds(key, a.K, s_key[wave]);
      const uint64_t my_key = lane < a.K ? s_key[wave][lane] : 0ull;   // lane k: the k-th selected key
      const int my_e = (int)~(uint32_t)my_key;
      const float my_s = lane < a.K ? 1.0f / (1.0f + expf(-float_from_order_key((uint32_t)(my_key >> 32)))) : 0.f;
      float ssum = 0.f;
#pragma unroll
      for (int k = 0; k < FLINT_MAX_TOP_K; ++k)     // selection order
        if (k < a.K) ssum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), k));
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
  rms_norm_words<Fmt<WF>::VALS / 2>(x.v, g.v, rms);
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
  for (int t = 0; t < BT; ++t) rinv[t] = make_rms(1.0);
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

// routed + shared slots a decode of this batch can fill (decode_max_slots)
__device__ __forceinline__ int decode_max_slots_dev(const LayerArgs& a) {
  const int u = a.B * a.K;
  return (u < a.E ? u : a.E) + (a.SI > 0 ? 1 : 0);
}

// q / d and q % d for 0 <= q < 2^22 and d >= 1 (inv = 1.0f / d): a float
// estimate corrected by one step either way, instead of an integer division.
__device__ __forceinline__ int div_small(int q, int d, float inv, int& rem) {
  int p = (int)((float)q * inv);
  int r = q - p * d;
  if (r >= d) { ++p; r -= d; }
  if (r < 0) { --p; r += d; }
  rem = r;
  return p;
}

// ----------------------------------------------------- gate/up, batch 2..8 --
// The rows of gate_up_kernel for a batch of tokens, 64 lanes per row.  The
// workgroup issues its weight loads, then stages the activations of the
// tokens routed to its slot in LDS (one copy per workgroup; every load of
// the workgroup is in flight at once, so the whole prologue costs one HBM
// round trip).  Each lane then decodes its NCH weight chunks once and walks
// the staged tokens,
// finishing one token (reduction, SiLU * up, store) before the next.  LDS
// layout: staged token i, 16-byte quad m of chunk j at
// s_x[(i * QPC + m) * cpr + j], so a wave reads consecutive words.
template <int WF, int P, int NW, int NCH, int KQ>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(KQ > 1 ? 2 : 4, KQ > 1 ? 2 : 4)))
void gate_up_batch_kernel(LayerArgs a, DecodeWs ws, uint16_t* hout,
                                                                int h_slot_stride, int h_tok_stride) {
  constexpr int BT = kMaxB, NT = 64 * NW;
  constexpr int VALS = Fmt<WF>::VALS, QPC = VALS / 8;
  extern __shared__ uint4 s_x[];
  const int slot = blockIdx.y;
  const bool has_sh = a.SI > 0;
  const bool shared = has_sh && slot == 0;
  const int inter = shared ? a.SI : a.I;
  if ((int)blockIdx.x * NW * P >= inter) return;    // the whole workgroup
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row0 = (blockIdx.x * NW + wave) * P;
  const int H = a.H, cpr = H / VALS, q8 = H / 8;

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
    if (r >= *ws.nslot) return;
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
  const uint16_t* xsrc = (a.flags & FLINT_PRE_RMSNORM) ? ws.xn : a.x;
  const int n = __popc(mask);
  uint32_t tokp = 0;                               // token of staged position i, 4 bits each
  {
    uint32_t m = mask;
#pragma unroll
    for (int i = 0; i < BT; ++i)
      if (m) { tokp |= (uint32_t)(__ffs(m) - 1) << (4 * i); m &= m - 1u; }
  }

  // weights: chunks j = lane + 64 c of P gate rows and P up rows, every load
  // unconditional (rows and chunks out of range read row 0, chunk 0)
  uint4 rg[NCH][P], ru[NCH][P];
  uint32_t sg[NCH][P], su[NCH][P];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int j = lane + 64 * c;
    const int jc = j < cpr ? j : 0;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int r = row0 + p;
      const int rc = r < inter ? r : 0;
      rg[c][p] = load_chunk_raw<WF>(mg, rc, jc, sg[c][p]);
      ru[c][p] = load_chunk_raw<WF>(mu, rc, jc, su[c][p]);
    }
  }
  // activations: quad q (chunk j, quad m) of every staged token, q8 <= KQ * NT
  uint4 xv[KQ][BT];
  int qv[KQ];
  const float inv_cpr = 1.0f / (float)cpr;
#pragma unroll
  for (int kq = 0; kq < KQ; ++kq) {
    const int q = threadIdx.x + NT * kq;
    qv[kq] = q;
    int j;
    const int m = div_small(q, cpr, inv_cpr, j);
    // every load is issued; positions out of range all read the first quad,
    // so their lanes share one address
#pragma unroll
    for (int i = 0; i < BT; ++i) {
      const int t = (tokp >> (4 * i)) & 15;
      const bool ok = q < q8 && i < n;
      const uint16_t* src = ok ? xsrc + (size_t)t * H + j * VALS + 8 * m : xsrc;
      xv[kq][i] = *reinterpret_cast<const uint4*>(src);
    }
  }

  // every store is made too (a conditional one would draw its load into the
  // branch, behind a full wait): positions out of range go to this thread's
  // slot past the staged tokens
#pragma unroll
  for (int kq = 0; kq < KQ; ++kq)
#pragma unroll
    for (int i = 0; i < BT; ++i)
      s_x[qv[kq] < q8 && i < n ? i * q8 + qv[kq] : a.B * q8 + (int)threadIdx.x] = xv[kq][i];
  __syncthreads();

  DChunk<WF> dg[NCH][P], du[NCH][P];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int p = 0; p < P; ++p) {
      dg[c][p] = decode_chunk<WF>(rg[c][p], sg[c][p]);
      du[c][p] = decode_chunk<WF>(ru[c][p], su[c][p]);
    }
  for (int i = 0; i < n; ++i) {
    float acc[P][2];
#pragma unroll
    for (int p = 0; p < P; ++p) acc[p][0] = acc[p][1] = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int j = lane + 64 * c;
      if (j < cpr) {
        XChunk<WF> xc;
#pragma unroll
        for (int m = 0; m < QPC; ++m) {
          const uint4 v = s_x[(i * QPC + m) * cpr + j];
          xc.v[4 * m + 0] = v.x; xc.v[4 * m + 1] = v.y; xc.v[4 * m + 2] = v.z; xc.v[4 * m + 3] = v.w;
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
          acc[p][0] += chunk_dot(dg[c][p], xc);
          acc[p][1] += chunk_dot(du[c][p], xc);
        }
      }
    }
    const int t = (tokp >> (4 * i)) & 15;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const float g = group_sum<64>(acc[p][0]);
      const float u = group_sum<64>(acc[p][1]);
      const int r = row0 + p;
      if (lane == 0 && r < inter) {
        const float gv = round_bf16(g * gs_g);
        const float uv = round_bf16(u * gs_u);
        const float av = round_bf16(silu_f32(gv));
        hout[(size_t)slot * h_slot_stride + (size_t)t * h_tok_stride + r] = f32_to_bf16_bits(av * uv);
      }
    }
  }
}

// ------------------------------------------- gate/up, batch 2..8, NVFP4 ----
// The NVFP4 rows of gate_up_kernel for a batch, 16 lanes per row: lane li of
// a row group owns the CPL consecutive chunks li * CPL .. li * CPL + CPL - 1
// (64 * CPL bytes of codes, 2 * CPL of scales), so a row's cross-lane sum is
// four steps, paid once per CPL chunks.  A wave holds 4 rows, a workgroup
// NW * 4 (small workgroups: the grid of ~45 slots x 32 row tiles then
// streams through the CUs instead of running as one full round and a
// latency-bound second round).  The slot table entry is read first (scalar
// loads, one round trip); the weight loads follow, then the activations of
// the slot's tokens are copied into LDS (every load of the workgroup in
// flight at once; the copies complete after the weights, as loads complete
// in order).  The expert
// and the matrix bases are wave-uniform; each lane adds a 32-bit offset of
// its row and chunks, taken once.  LDS layout: staged token i, quad m of the
// lane's chunk c at s_x[i * q8 + (c * 4 + m) * 16 + li], so the 16 lanes of
// a row group read consecutive words.
template <int NW, int CPL>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(CPL > 4 ? 2 : 4, CPL > 4 ? 2 : 4)))
void gate_up_nv_batch_kernel(LayerArgs a, DecodeWs ws, uint16_t* hout, int h_slot_stride, int h_tok_stride) {
  constexpr int BT = kMaxB, NT = 64 * NW;
  constexpr int G = 16, QPC = 4;
  extern __shared__ uint4 s_x[];
  const int slot = blockIdx.y;
  const bool has_sh = a.SI > 0;
  const bool shared = has_sh && slot == 0;
  const int inter = shared ? a.SI : a.I;
  if ((int)blockIdx.x * NW * 4 >= inter) return;    // the whole workgroup
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int grp = lane / G, li = lane % G;
  const int r = (blockIdx.x * NW + wave) * 4 + grp;  // this lane's row
  const int H = a.H, q8 = H / 8;

  // the slot table entry (read before the slot count, which the table always
  // exceeds, so that the three loads make one round trip)
  const int rr = slot - (has_sh ? 1 : 0);
  const int e = shared ? 0 : ws.slot_expert[rr];
  const uint32_t mask = shared ? (1u << a.B) - 1u : ws.slot_mask[rr];
  if (!shared && rr >= *ws.nslot) return;
  const size_t mc = (size_t)inter * H / 2, ms = (size_t)inter * H / 16;
  const uint8_t* gc = shared ? a.sh_gu_codes : a.gu_codes + (size_t)(2 * e) * mc;
  const uint8_t* gsb = shared ? a.sh_gu_scales : a.gu_scales + (size_t)(2 * e) * ms;
  const uint8_t* uc = gc + mc;
  const uint8_t* usb = gsb + ms;
  const float gs_g = shared ? a.sh_gscale[0] : a.gscale[3 * e + 0];
  const float gs_u = shared ? a.sh_gscale[1] : a.gscale[3 * e + 1];

  // weights: this lane's CPL chunks of its gate and up rows (rows past the
  // matrix read row 0 and are not stored)
  const uint32_t rc = r < inter ? (uint32_t)r : 0u;
  const uint32_t oc = rc * ((uint32_t)H / 2) + (uint32_t)li * 16u * CPL;
  const uint32_t os = rc * ((uint32_t)H / 16) + (uint32_t)li * 2u * CPL;
  uint4 wg[CPL], wu[CPL];
  uint32_t sg2[CPL / 2], su2[CPL / 2];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    wg[c] = reinterpret_cast<const uint4*>(gc + oc)[c];
    wu[c] = reinterpret_cast<const uint4*>(uc + oc)[c];
  }
#pragma unroll
  for (int c = 0; c < CPL; c += 2) {
    sg2[c / 2] = reinterpret_cast<const uint32_t*>(gsb + os)[c / 2];
    su2[c / 2] = reinterpret_cast<const uint32_t*>(usb + os)[c / 2];
  }

  const uint16_t* xsrc = (a.flags & FLINT_PRE_RMSNORM) ? ws.xn : a.x;
  const int n = __popc(mask);
  uint32_t tokp = 0;                               // token of staged position i, 4 bits each
  {
    uint32_t m = mask;
#pragma unroll
    for (int i = 0; i < BT; ++i)
      if (m) { tokp |= (uint32_t)(__ffs(m) - 1) << (4 * i); m &= m - 1u; }
  }
  // activations: LDS position q of staged token i holds columns
  // 32 * (CPL * (q % 16) + (q / 16) / 4) + 8 * ((q / 16) % 4), q < q8 = H / 8.
  // They are copied by the load units straight into LDS (global_load_lds:
  // lane l of a wave writes the l-th 16 bytes after the wave's base, and
  // positions q = threadIdx.x + NT * kq are consecutive within a wave), so
  // no registers hold them and a workgroup of any width stages all q8
  // positions; positions of tokens past the slot's are not copied.
  {
    constexpr int KQ = CPL * 64 / NT;              // positions per thread (H = 512 * CPL)
    static_assert(KQ >= 1 && KQ * NT == CPL * 64, "staging layout");
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) {
      const int q = threadIdx.x + NT * kq;
      const int qli = q % G, qcm = q / G;
      const int col = 32 * (CPL * qli + qcm / QPC) + 8 * (qcm % QPC);
#pragma unroll
      for (int i = 0; i < BT; ++i) {
        const int t = (tokp >> (4 * i)) & 15;
        uint4* dst = s_x + i * q8 + NT * kq + (threadIdx.x & ~63);
        if (i < n) __builtin_amdgcn_global_load_lds(xsrc + (size_t)t * H + col, dst, 16, 0, 0);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);         // this wave's copies (and weights) are in
  __syncthreads();

  float ag[BT], au[BT];
#pragma unroll
  for (int i = 0; i < BT; ++i) ag[i] = au[i] = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const uint32_t sgc = c % 2 ? sg2[c / 2] >> 16 : sg2[c / 2] & 0xffffu;
    const uint32_t suc = c % 2 ? su2[c / 2] >> 16 : su2[c / 2] & 0xffffu;
    const DChunk<FMT_NVFP4> dg = decode_nvfp4(wg[c], sgc);
    const DChunk<FMT_NVFP4> du = decode_nvfp4(wu[c], suc);
#pragma unroll
    for (int i = 0; i < BT; ++i) {
      if (i >= n) break;
      XChunk<FMT_NVFP4> xc;
#pragma unroll
      for (int m = 0; m < QPC; ++m) {
        const uint4 v = s_x[i * q8 + (c * QPC + m) * G + li];
        xc.v[4 * m + 0] = v.x; xc.v[4 * m + 1] = v.y; xc.v[4 * m + 2] = v.z; xc.v[4 * m + 3] = v.w;
      }
      ag[i] += chunk_dot(dg, xc);
      au[i] += chunk_dot(du, xc);
    }
  }
#pragma unroll
  for (int i = 0; i < BT; ++i) {
    if (i >= n) break;
    const float g = group_sum<G>(ag[i]);
    const float u = group_sum<G>(au[i]);
    if (li == 0 && r < inter) {
      const int t = (tokp >> (4 * i)) & 15;
      const float gv = round_bf16(g * gs_g);
      const float uv = round_bf16(u * gs_u);
      const float av = round_bf16(silu_f32(gv));
      hout[(size_t)slot * h_slot_stride + (size_t)t * h_tok_stride + r] = f32_to_bf16_bits(av * uv);
    }
  }
}

// ------------------------------------------------ down+combine, batch 2..8 --
// down_kernel for a batch.  Every (slot, token) pair of the layer has its h
// row staged in LDS once per workgroup: wave 0 reads the slot table (one
// round trip: every entry a lane may need is loaded at once) and builds the
// pair list with a prefix sum of the slots' token counts; all threads then
// issue the loads of the h rows, then the weight loads, and only then store
// h to LDS: vector loads complete in order, so h issued first is waited for
// alone, and the weights are already in flight meanwhile; weights issued
// last let each item be computed as soon as its own rows arrive.  LDS
// layout as in
// gate_up_batch_kernel: pair p, quad m of chunk j at
// s_h[(p * QPC + m) * cmax + j].
template <int WF, int G, int RW, int NW, int U>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 2))) void down_batch_kernel(LayerArgs a, DecodeWs ws, const uint16_t* hin,
                                                             int h_slot_stride, int h_tok_stride) {
  constexpr int BT = kMaxB, NT = 64 * NW;
  constexpr int GPW = 64 / G, RPW = RW * GPW;
  constexpr int VALS = Fmt<WF>::VALS, QPC = VALS / 8;
  constexpr int NHL = 8;                           // h loads per thread issued together
  extern __shared__ uint4 s_h[];
  __shared__ float s_red[NW][RPW][BT];
  __shared__ int s_exp[kMaxSlots];
  __shared__ uint32_t s_msk[kMaxSlots];
  __shared__ int s_pb[kMaxSlots];
  __shared__ float s_wt[kMaxSlots][BT];
  __shared__ uint16_t s_pair[kMaxSlots * BT];      // pair -> slot << 3 | token
  __shared__ int s_np;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int grp = lane / G, li = lane % G;
  const int H = a.H;
  const int n0 = blockIdx.x * RPW;
  const int sh = a.SI > 0 ? 1 : 0;
  const int I = a.I, SI = a.SI;
  const int imax = I > SI ? I : SI;
  const int cmax = imax / VALS, qmax = imax / 8;
  const int nch = (cmax + G - 1) / G;
  const bool resid = (a.flags & FLINT_RESIDUAL) != 0;
  const int nmax = decode_max_slots_dev(a) - sh;   // routed slots the table can hold

  // slot table and pair list (wave 0, two slots per lane, S <= 128)
  if (wave == 0) {
    const int S = *ws.nslot + sh;
    uint32_t mraw[2];
    int eraw[2];
    float wraw[2][BT];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {             // every load at once, clamped to the table
      const int r = 2 * lane + h2 - sh;
      const int rc = r < 0 ? 0 : (r < nmax ? r : nmax - 1);
      eraw[h2] = ws.slot_expert[rc];
      mraw[h2] = ws.slot_mask[rc];
#pragma unroll
      for (int t = 0; t < BT; ++t) wraw[h2][t] = ws.slot_w[rc * kMaxB + t];
    }
    uint32_t msk[2];
    int cnt[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int s = 2 * lane + h2;
      const bool is_sh = sh && s == 0;
      const uint32_t m = s < S ? (is_sh ? (1u << a.B) - 1u : mraw[h2]) : 0u;
      if (s < S) {
        s_exp[s] = is_sh ? -1 : eraw[h2];
        s_msk[s] = m;
#pragma unroll
        for (int t = 0; t < BT; ++t) s_wt[s][t] = is_sh ? 1.f : wraw[h2][t];
      }
      msk[h2] = m;
      cnt[h2] = __popc(m);
    }
    int incl = cnt[0] + cnt[1];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    int base = incl - cnt[0] - cnt[1];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int s = 2 * lane + h2;
      if (s < S) s_pb[s] = base;
      uint32_t m = msk[h2];
      for (int k = 0; m; ++k, m &= m - 1u) s_pair[base + k] = (uint16_t)((s << 3) | (__ffs(m) - 1));
      base += cnt[h2];
    }
    if (lane == 63) s_np = incl;
  }
  // the residual of the rows this thread will write, fetched early (always:
  // threads without a row read x[0])
  uint16_t xres_bits;
  {
    const int q = threadIdx.x;
    const int rloc = q / BT, t = q - rloc * BT, n = n0 + rloc;
    const bool ok = q < RPW * BT && t < a.B && n < H;
    xres_bits = a.x[ok ? (size_t)t * H + n : 0];
  }
  __syncthreads();
  const int S = *ws.nslot + sh;

  // h rows into LDS, copied by the load units straight from memory
  // (global_load_lds: no registers).  Thread t copies quad (m, j) = t % qmax
  // of pairs t / qmax + ppp * k (ppp = NT / qmax pairs per pass,
  // qmax <= NT) to s_h[t + ppp * k * qmax], so each wave's 64 quads land in
  // consecutive LDS words.  The first pass is issued before the weight loads
  // below: loads complete in order, so waiting for the copies does not wait
  // for the weights, and the weights' latency runs under the copies' instead
  // of after them.  (Layers with more than ppp * NHL pairs copy the rest
  // after the weights.)
  const int np = s_np;
  const int ppp = NT / qmax;
  int hrem, hj;
  const int hp0 = div_small(threadIdx.x, qmax, 1.0f / (float)qmax, hrem);
  const int hm = div_small(hrem, cmax, 1.0f / (float)cmax, hj);
  const size_t hoff = (size_t)hj * VALS + 8 * hm;
#define FLINT_H_COPY(PB0)                                                                              \
  _Pragma("unroll") for (int k = 0; k < NHL; ++k) {                                                   \
    const int p = hp0 + (PB0) + ppp * k;                                                                \
    const bool ok = p < np;                                                                             \
    const int pr = s_pair[ok ? p : 0];                                                                  \
    const uint16_t* src = hin + (size_t)(pr >> 3) * h_slot_stride + (size_t)(pr & 7) * h_tok_stride + hoff; \
    uint4* dst = s_h + ((PB0) + ppp * k) * qmax + (threadIdx.x & ~63);                                  \
    if (ok) __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);                                       \
  }
  FLINT_H_COPY(0)
  asm volatile("" ::: "memory");                   // the weight loads stay behind the copies

  // Weights of U items (slot, chunk step) per wave.  The item, its expert and
  // the matrix bases are wave-uniform (scalar); each lane adds fixed 32-bit
  // offsets of its rows and chunk, taken once.  Every load is made: an item
  // out of range reads slot 0's first chunk, a chunk past a narrower slot
  // reads the row's first chunk, and neither is used.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int total = S * nch;
  uint32_t oc[2][RW], osc[2][RW];                 // [routed, shared] code / scale offsets
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int inter = k == 0 ? I : SI;
    const uint32_t rowc = WF == FMT_NVFP4 ? (uint32_t)inter / 2 : (uint32_t)inter * 2;
#pragma unroll
    for (int rw = 0; rw < RW; ++rw) {
      const int n = n0 + rw * GPW + grp;
      const uint32_t nc = n < H ? (uint32_t)n : 0u;
      oc[k][rw] = nc * rowc + 16u * (uint32_t)li;
      osc[k][rw] = nc * ((uint32_t)inter / 16) + 2u * (uint32_t)li;
    }
  }
  uint4 raw[U][RW];
  uint32_t sc[U][RW];
  int ie[U];
  float igd[U];
  auto load_items = [&](int it0) {
    int sl[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = it0 + u * NW;
      sl[u] = it < total ? (nch == 1 ? it : it / nch) : 0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) ie[u] = __builtin_amdgcn_readfirstlane(s_exp[sl[u]]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = it0 + u * NW;
      const int c = it < total ? it - sl[u] * nch : 0;
      const int e = ie[u];
      const bool shd = e < 0;
      const int inter = shd ? SI : I;
      igd[u] = 1.f;
      if constexpr (WF == FMT_NVFP4) igd[u] = shd ? a.sh_gscale[2] : a.gscale[3 * e + 2];
      const bool jok = li + G * c < inter / VALS;
      const uint8_t* cb;
      const uint8_t* sb = nullptr;
      if constexpr (WF == FMT_NVFP4) {
        cb = shd ? a.sh_d_codes : a.d_codes + (size_t)e * H * (inter / 2);
        sb = shd ? a.sh_d_scales : a.d_scales + (size_t)e * H * (inter / 16);
      } else {
        cb = reinterpret_cast<const uint8_t*>(shd ? a.sh_d_bf16 : a.d_bf16 + (size_t)e * H * inter);
      }
      cb += (size_t)16 * G * c;
      if constexpr (WF == FMT_NVFP4) sb += (size_t)2 * G * c;
#pragma unroll
      for (int rw = 0; rw < RW; ++rw) {
        const uint32_t o = jok ? (shd ? oc[1][rw] : oc[0][rw]) : 0u;
        raw[u][rw] = *reinterpret_cast<const uint4*>(cb + o);
        if constexpr (WF == FMT_NVFP4) {
          const uint32_t os = jok ? (shd ? osc[1][rw] : osc[0][rw]) : 0u;
          sc[u][rw] = *reinterpret_cast<const uint16_t*>(sb + os);
        } else {
          sc[u][rw] = 0;
        }
      }
    }
  };
  load_items(wv);

  // This wave's copies are complete once at most the weight loads issued
  // after them are outstanding; then the barrier makes every wave's copies
  // visible.  Only the 16-byte code loads are counted (every one is made,
  // and no two can merge; scale loads may be merged into fewer), so the
  // count never exceeds the loads actually issued after the copies.
  constexpr int kWeightLoads = U * RW;
  static_assert(kWeightLoads < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0 | (kWeightLoads & 15) | ((kWeightLoads & 48) << 10));
  if (np > ppp * NHL) {
    for (int pb0 = ppp * NHL; pb0 < np; pb0 += ppp * NHL) { FLINT_H_COPY(pb0) }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }
#undef FLINT_H_COPY
  __syncthreads();

  float acc[RW][BT];
#pragma unroll
  for (int rw = 0; rw < RW; ++rw)
#pragma unroll
    for (int t = 0; t < BT; ++t) acc[rw][t] = 0.f;
  // The first round of items is straight-line code: inside a loop, the
  // registers the last weight loads write were reused at the loop head,
  // which made every item wait for all of them.
#define FLINT_DOWN_ITEMS(IT0)                                                 \
  {                                                                           \
    const int it0 = (IT0);                                                    \
  _Pragma("unroll")                                                      \
    for (int u = 0; u < U; ++u) {                                             \
      const int it = it0 + u * NW;                                            \
      if (it >= total) break;                                                 \
      const int s = nch == 1 ? it : it / nch, c = it - s * nch;               \
      const int e = ie[u];                                                    \
      const int inter = e < 0 ? SI : I;                                       \
      const int j = li + G * c;                                               \
      if (j >= inter / VALS) continue;                                        \
      const uint32_t mask = s_msk[s];                                         \
      const int pb = s_pb[s];                                                 \
      const float gd = igd[u];                                                \
      DChunk<WF> d[RW];                                                       \
  _Pragma("unroll")                                                      \
      for (int rw = 0; rw < RW; ++rw) d[rw] = decode_chunk<WF>(raw[u][rw], sc[u][rw]); \
  _Pragma("unroll")                                                      \
      for (int t = 0; t < BT; ++t) {                                          \
        if ((mask >> t) & 1u) {                                               \
          const int p = pb + __popc(mask & ((1u << t) - 1u));                 \
          XChunk<WF> hx;                                                      \
  _Pragma("unroll")                                                      \
          for (int m = 0; m < QPC; ++m) {                                     \
            const uint4 v = s_h[(p * QPC + m) * cmax + j];                    \
            hx.v[4 * m + 0] = v.x; hx.v[4 * m + 1] = v.y; hx.v[4 * m + 2] = v.z; hx.v[4 * m + 3] = v.w; \
          }                                                                   \
          const float f = s_wt[s][t] * gd;                                    \
  _Pragma("unroll")                                                      \
          for (int rw = 0; rw < RW; ++rw) acc[rw][t] = fmaf(f, chunk_dot(d[rw], hx), acc[rw][t]); \
        }                                                                     \
      }                                                                       \
    }                                                                         \
  }
  FLINT_DOWN_ITEMS(wv)
  for (int it1 = wv + NW * U; it1 < total; it1 += NW * U) {   // layers with more items than U per wave
    load_items(it1);
    FLINT_DOWN_ITEMS(it1)
  }
#undef FLINT_DOWN_ITEMS

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
      if (resid) o = bf16_bits_to_f32(xres_bits) + o;
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

// Batch kernels: the LDS they stage (activations of up to 8 tokens; h rows
// of every (slot, token) pair) must fit these bounds, else the per-wave
// kernels above run.
constexpr int kBatchXBytes = 64 * 1024;
constexpr int kBatchHBytes = 96 * 1024;

// Raises a kernel's dynamic LDS limit to the largest size it may be given;
// each launch template below calls it once, from a function-local static.
template <typename K>
bool allow_dynamic_lds(K kernel, int bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             bytes) == hipSuccess;
}

// chunk steps of the batch gate/up kernel (64 lanes per row); 0 = not covered
template <int WF>
int gate_up_batch_nch(const LayerArgs& a) {
  const int cpr = a.H / Fmt<WF>::VALS;
  if (a.B < 2 || cpr < 64 || a.H / 8 > 2 * 256 || a.B * a.H * 2 > kBatchXBytes) return 0;
  const int nch = (cpr + 63) / 64;
  return (WF == FMT_NVFP4 ? (nch <= 2) : (nch == 4)) ? nch : 0;
}

int down_batch_lds(const LayerArgs& a) {
  const int imax = a.I > a.SI ? a.I : a.SI;
  const int pairs = a.B * (a.K < a.E ? a.K : a.E) + (a.SI > 0 ? a.B : 0);
  return pairs * imax * 2;
}

template <int WF, int NCH, int KQ>
hipError_t gate_up_batch_launch(const LayerArgs& a, const DecodeWs& ws, uint16_t* hout, int hs, int ht,
                                int rows, hipStream_t st) {
  constexpr int NW = 4, P = 2;
  const int tiles = (rows + NW * P - 1) / (NW * P);
  const int slots = decode_max_slots({a.H, a.E, a.I, a.SI, a.K, 0, 0.f}, a.B);
  auto k = gate_up_batch_kernel<WF, P, NW, NCH, KQ>;
  static const bool lds_ok = allow_dynamic_lds(k, kBatchXBytes + 64 * NW * 16);
  (void)lds_ok;
  hipLaunchKernelGGL(k, dim3(tiles, slots), dim3(64 * NW), a.B * a.H * 2 + 64 * NW * 16, st, a, ws, hout, hs,
                     ht);
  return hipGetLastError();
}

template <int CPL>
hipError_t gate_up_nv_batch_launch(const LayerArgs& a, const DecodeWs& ws, uint16_t* hout, int hs, int ht,
                                   int rows, hipStream_t st) {
  constexpr int NW = 4;                           // 16 rows per workgroup (8 waves: +2.6 us at batch 8)
  const int tiles = (rows + NW * 4 - 1) / (NW * 4);
  const int slots = decode_max_slots({a.H, a.E, a.I, a.SI, a.K, 0, 0.f}, a.B);
  auto k = gate_up_nv_batch_kernel<NW, CPL>;
  static const bool lds_ok = allow_dynamic_lds(k, kBatchXBytes + 64 * NW * 16);
  (void)lds_ok;
  hipLaunchKernelGGL(k, dim3(tiles, slots), dim3(64 * NW), a.B * a.H * 2 + 64 * NW * 16, st, a, ws, hout, hs,
                     ht);
  return hipGetLastError();
}

template <int WF, int G>
hipError_t down_batch_dispatch(const LayerArgs& a, const DecodeWs& ws, const uint16_t* hin, int hs, int ht,
                               hipStream_t st) {
  constexpr int NW = 8, U = 6;
  // 4 output rows per workgroup at 16 lanes per row (two workgroups per CU:
  // -0.7 us per batch-8 Flint layer against 8 rows and one workgroup)
  constexpr int RW = (G == 64) ? 4 : (G == 16 ? 1 : 2);
  constexpr int RPW = RW * (64 / G);
  const int tiles = (a.H + RPW - 1) / RPW;
  auto k = down_batch_kernel<WF, G, RW, NW, U>;
  static const bool lds_ok = allow_dynamic_lds(k, kBatchHBytes + 64 * NW * 16);
  (void)lds_ok;
  hipLaunchKernelGGL(k, dim3(tiles), dim3(64 * NW), down_batch_lds(a) + 64 * NW * 16, st, a, ws, hin, hs, ht);
  return hipGetLastError();
}

template <int WF>
hipError_t down_batch_g(const LayerArgs& a, const DecodeWs& ws, const uint16_t* hin, int hs, int ht,
                        hipStream_t st) {
  int red = a.I;
  if (a.SI > 0 && a.SI < red) red = a.SI;
  switch (lanes_per_row(red / Fmt<WF>::VALS)) {
    case 8: return down_batch_dispatch<WF, 8>(a, ws, hin, hs, ht, st);
    case 16: return down_batch_dispatch<WF, 16>(a, ws, hin, hs, ht, st);
    case 32: return down_batch_dispatch<WF, 32>(a, ws, hin, hs, ht, st);
    default: return down_batch_dispatch<WF, 64>(a, ws, hin, hs, ht, st);
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
  if (a.B == 1) return route_dispatch<1>(a, ws, st);
  const bool norm = (a.flags & FLINT_PRE_RMSNORM) != 0;
  const int nq = (a.H / 4 + 511) / 512;            // 16-byte loads per lane per quarter row
  if (a.E <= FLINT_MAX_EXPERTS && nq <= 2) {
    if (nq == 1) {
      if (norm) hipLaunchKernelGGL((route_batch_kernel<1, true>), dim3(a.E), dim3(256), 0, st, a, ws);
      else hipLaunchKernelGGL((route_batch_kernel<1, false>), dim3(a.E), dim3(256), 0, st, a, ws);
    } else {
      if (norm) hipLaunchKernelGGL((route_batch_kernel<2, true>), dim3(a.E), dim3(256), 0, st, a, ws);
      else hipLaunchKernelGGL((route_batch_kernel<2, false>), dim3(a.E), dim3(256), 0, st, a, ws);
    }
    return hipGetLastError();
  }
  return route_dispatch<kMaxB>(a, ws, st);
}

namespace {

// ------------------------------------- dense NVFP4 projection, tall matrix --
// y[t][r] = BF16(g * sum_c W[r][c] x[t][c]), or BF16(aux[t][r] + that), for a
// packed NVFP4 matrix W [rows][cols] with many rows and 1..8 tokens: the
// plain and residual projections of flint_dense_gemv (the small-batch dense
// GEMV on the same packed weights of "Day-0 Support for Flint on vLLM",
// "Optimizations"; the same call serves an NVFP4 LM head).  16 lanes per
// row, lane li owning the CPL consecutive chunks li * CPL .. li * CPL +
// CPL - 1, so a row's cross-lane sum is four DPP steps; a wave holds RPL
// sets of 4 rows, a workgroup NW * 4 * RPL rows (NW = 1 for one token).  Every weight load of the
// workgroup is issued first, then the tokens are staged in LDS in the layout
// of gate_up_nv_batch_kernel (position q of token i holds columns
// 32 * (CPL * (q % 16) + (q / 16) / 4) + 8 * ((q / 16) % 4), so the 16 lanes
// of a row group read consecutive words), and each decoded chunk is applied
// to every token.  Every load and LDS store is made (rows past the matrix
// read row 0 and are not stored; token positions past the batch read token
// 0 and are stored past the staged tokens).  BT is the token capacity (1 for
// the one-token variant, so that its staging registers stay few).  With SW
// the matrix is the SwiGLU pair [2][rows][cols]: lane group g of a wave takes
// the gate row (row set 0) and the up row (set 1) of the same index, and
// writes h = BF16(BF16(SiLU(BF16(g))) * BF16(u)); with NORM every workgroup
// first RMS-normalises the tokens it stages (float64 mean of squares,
// BF16(BF16(x / rms) * gamma), as the other kernels do).
template <int NW, int CPL, int RPL, int BT, bool SW, bool NORM>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(4, 4)))
void dense_nv_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                     const float* __restrict__ gscale, const uint16_t* __restrict__ x, int B, int rows, int cols,
                     uint16_t* y, const uint16_t* aux, int resid, const uint16_t* __restrict__ gamma, float eps) {
  constexpr int G = 16, QPC = 4, NT = 64 * NW;
  constexpr int KQ = CPL / NW;                     // staged positions per thread: cols / 8 = KQ * NT
  static_assert(CPL % NW == 0, "staging layout");
  static_assert(!SW || RPL == 2, "the SwiGLU pair takes row set 0 from gate, 1 from up");
  extern __shared__ uint4 s_x[];
  __shared__ double s_ss[NW][BT];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int grp = lane / G, li = lane % G;
  // output row of row set p (SW: row r of the gate (p = 0) and up (p = 1)
  // matrices, stacked as [2][rows][cols])
  const int r0 = SW ? (blockIdx.x * NW + wave) * 4 + grp : (blockIdx.x * NW + wave) * 4 * RPL + grp;
  auto out_row = [&](int p) { return SW ? r0 : r0 + 4 * p; };
  const int q8 = cols / 8;

  uint4 wc[RPL][CPL];
  uint32_t sc2[RPL][CPL / 2];
#pragma unroll
  for (int p = 0; p < RPL; ++p) {
    const int r = out_row(p);
    const uint32_t rc = (r < rows ? (uint32_t)r : 0u) + (SW && p == 1 ? (uint32_t)rows : 0u);
    const uint32_t oc = rc * ((uint32_t)cols / 2) + (uint32_t)li * 16u * CPL;
    const uint32_t os = rc * ((uint32_t)cols / 16) + (uint32_t)li * 2u * CPL;
#pragma unroll
    for (int c = 0; c < CPL; ++c) wc[p][c] = reinterpret_cast<const uint4*>(codes + oc)[c];
#pragma unroll
    for (int c = 0; c < CPL; c += 2) sc2[p][c / 2] = reinterpret_cast<const uint32_t*>(scales + os)[c / 2];
  }
  const float g0 = gscale[0], g1 = SW ? gscale[1] : 0.f;
  // residual values of this lane's rows, fetched early (always: without a
  // residual, or past the batch or the matrix, they read y's first element)
  uint16_t xr[RPL][BT];
  const uint16_t* ab = resid ? aux : y;
#pragma unroll
  for (int p = 0; p < RPL; ++p)
#pragma unroll
    for (int i = 0; i < BT; ++i) {
      const int r = out_row(p);
      const bool ok = resid && i < B && r < rows;
      xr[p][i] = ab[ok ? (size_t)i * rows + r : 0];
    }
  // tokens (and gamma) into LDS; with NORM each thread first adds the
  // squares of its positions, and the tokens are normalised in LDS after the
  // barrier (gamma staged at s_x[(B + 1) * q8 + q]), so no staged value
  // stays in a register across it
  {
    uint4 xv[KQ][BT], gv[KQ];
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) {
      const int q = threadIdx.x + NT * kq;
      const int col = 32 * (CPL * (q % G) + (q / G) / QPC) + 8 * ((q / G) % QPC);
#pragma unroll
      for (int i = 0; i < BT; ++i) xv[kq][i] = *reinterpret_cast<const uint4*>(x + (size_t)(i < B ? i : 0) * cols + col);
      if constexpr (NORM) gv[kq] = *reinterpret_cast<const uint4*>(gamma + col);
    }
    if constexpr (NORM) {
#pragma unroll
      for (int i = 0; i < BT; ++i) {
        double ss0 = 0.0, ss1 = 0.0;
#pragma unroll
        for (int kq = 0; kq < KQ; ++kq) {
          const uint32_t w4[4] = {xv[kq][i].x, xv[kq][i].y, xv[kq][i].z, xv[kq][i].w};
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const double lo = bf16_lo(w4[m]), hi = bf16_hi(w4[m]);
            ss0 = fma(lo, lo, ss0);
            ss1 = fma(hi, hi, ss1);
          }
        }
        const double ssw = wave_sum_f64(ss0 + ss1);
        if (lane == 0) s_ss[wave][i] = ssw;
      }
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq) s_x[(B + 1) * q8 + threadIdx.x + NT * kq] = gv[kq];
    }
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) {
      const int q = threadIdx.x + NT * kq;
#pragma unroll
      for (int i = 0; i < BT; ++i) s_x[(i < B ? i : B) * q8 + q] = xv[kq][i];
    }
  }
  __syncthreads();
  if constexpr (NORM) {
    // RMSNorm of every token, as in the other decode kernels: the mean of
    // squares and the square root in float64, BF16(BF16(x / rms) * gamma)
#pragma unroll
    for (int i = 0; i < BT; ++i) {
      if (i >= B) break;
      double ss = 0.0;
#pragma unroll
      for (int w = 0; w < NW; ++w) ss += s_ss[w][i];
      const Rms rms = make_rms(sqrt(ss / (double)cols + (double)eps));
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq) {
        const int q = threadIdx.x + NT * kq;
        s_x[i * q8 + q] = rms_norm_8(s_x[i * q8 + q], s_x[(B + 1) * q8 + q], rms);
      }
    }
    __syncthreads();
  }

  float acc[RPL][BT];
#pragma unroll
  for (int p = 0; p < RPL; ++p)
#pragma unroll
    for (int i = 0; i < BT; ++i) acc[p][i] = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    DChunk<FMT_NVFP4> d[RPL];
#pragma unroll
    for (int p = 0; p < RPL; ++p)
      d[p] = decode_nvfp4(wc[p][c], c % 2 ? sc2[p][c / 2] >> 16 : sc2[p][c / 2] & 0xffffu);
#pragma unroll
    for (int i = 0; i < BT; ++i) {
      if (i >= B) break;
      XChunk<FMT_NVFP4> xc;
#pragma unroll
      for (int m = 0; m < QPC; ++m) {
        const uint4 v = s_x[i * q8 + (c * QPC + m) * G + li];
        xc.v[4 * m + 0] = v.x; xc.v[4 * m + 1] = v.y; xc.v[4 * m + 2] = v.z; xc.v[4 * m + 3] = v.w;
      }
#pragma unroll
      for (int p = 0; p < RPL; ++p) acc[p][i] += chunk_dot(d[p], xc);
    }
  }
  if constexpr (SW) {
    // h = BF16(BF16(SiLU(BF16(g)))  * BF16(u)), the SwiGLU rounding points
#pragma unroll
    for (int i = 0; i < BT; ++i) {
      if (i >= B) break;
      const float gsum = group_sum<G>(acc[0][i]);
      const float usum = group_sum<G>(acc[1][i]);
      if (li == 0 && r0 < rows) {
        const float gv = round_bf16(gsum * g0);
        const float uv = round_bf16(usum * g1);
        const float av = round_bf16(silu_f32(gv));
        y[(size_t)i * rows + r0] = f32_to_bf16_bits(av * uv);
      }
    }
  } else {
#pragma unroll
    for (int p = 0; p < RPL; ++p) {
      const int r = out_row(p);
#pragma unroll
      for (int i = 0; i < BT; ++i) {
        if (i >= B) break;
        const float v = group_sum<G>(acc[p][i]);
        if (li == 0 && r < rows) {
          float o = round_bf16(v * g0);
          if (resid) o = bf16_bits_to_f32(xr[p][i]) + o;
          y[(size_t)i * rows + r] = f32_to_bf16_bits(o);
        }
      }
    }
  }
}

// Dense NVFP4 GEMV for 2..8 tokens at 2048 columns on MFMA 16x16x32 BF16:
// y[t][r] = BF16(g . sum_c W[r][c] x[t][c]) (+ residual, rounded again), the
// same definition as dense_nv_kernel.  There each weight value costs about
// five VALU instructions at batch 8 (a dot product per token); here the
// tokens are the B operand (16 columns, those past the batch zero) and only
// the exact BF16 decode of the weights (E2M1 x UE4M3 has at most 6
// significant bits) stays on the VALU.
// A wave takes DM_TILES tiles of 16 rows (A: lane (q, r) = (lane / 16, lane %
// 16) holds row r), all of their loads issued first.  K steps of 128
// columns: lane (q, r) loads the 16 code bytes (32 codes) of row r at column
// 128 j + 32 q and their 2 scale bytes; MFMA i of step j takes columns
// 128 j + 32 q + 8 i .. + 7 from lane group q, for A and B alike.  The tokens
// sit in LDS as [8][2048] BF16, 16-byte chunk c of token t at slot c ^ (t &
// 15), so that the 16 lanes of a group, one token each, read 16 different
// bank groups.  (One 8-wave workgroup per CU, each wave taking five tiles
// with two in registers at a time, ran slower: 61 against 56 us.)
constexpr int DM_TILES = 2;

// s_waitcnt immediate (gfx9 encoding) that waits for lgkmcnt 0 and leaves
// vmcnt and expcnt at their maxima.
constexpr int kWaitLgkmcnt0 = 0xC07F;

template <int NW>
__global__ __launch_bounds__(64 * NW) void dense_nv_mfma_kernel(const uint8_t* __restrict__ codes,
                                                                const uint8_t* __restrict__ scales,
                                                                const float* __restrict__ gscale,
                                                                const uint16_t* __restrict__ x, int B, int rows,
                                                                uint16_t* y, const uint16_t* aux, int resid) {
  constexpr int C = 2048, CH = C / 8, NT = 64 * NW;
  __shared__ uint4 s_x[kMaxB * CH];                // 32 KB
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int q = lane >> 4, r = lane & 15;
  const int rbase = (blockIdx.x * NW + wave) * 16 * DM_TILES;
  // The tokens' loads go out first and the weights' after them, in the
  // order the K steps use them: the staging then waits for the token loads
  // only, and each step for its own weight loads, so the decode of the first
  // steps runs while the later steps' rows are still arriving.
  static_assert((kMaxB * CH) % NT == 0, "whole token loads per thread");
  uint4 xs[kMaxB * CH / NT];
#pragma unroll
  for (int i = 0; i < kMaxB * CH / NT; ++i) {      // tokens past the batch read token 0
    const int k = threadIdx.x + NT * i, t = k / CH, c = k - t * CH;
    xs[i] = *reinterpret_cast<const uint4*>(x + (size_t)(t < B ? t : 0) * C + 8 * c);
  }
  // every load is made: rows past the matrix read row 0 and are not stored
  uint4 wc[DM_TILES][16];
  uint32_t ws[DM_TILES][16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
#pragma unroll
    for (int tt = 0; tt < DM_TILES; ++tt) {
      const int row = rbase + 16 * tt + r;
      const size_t rr = row < rows ? (size_t)row : 0;
      wc[tt][j] = ldg<uint4>(codes + rr * (C / 2) + 64 * j + 16 * q);
      ws[tt][j] = ldg<uint16_t>(scales + rr * (C / 16) + 8 * j + 2 * q);
    }
  }
#pragma unroll
  for (int i = 0; i < kMaxB * CH / NT; ++i) {
    const int k = threadIdx.x + NT * i, t = k / CH, c = k - t * CH;
    s_x[t * CH + (c ^ (t & 15))] = xs[i];
  }
  __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);       // the staged tokens are in LDS (no wait on the weights)
  __builtin_amdgcn_s_barrier();
  const float g0 = gscale[0];
  const int tx = r < kMaxB ? r : 0;                // this lane's token slot as B column
  const bool live = r < B;
  f32x4_t acc[DM_TILES];
#pragma unroll
  for (int tt = 0; tt < DM_TILES; ++tt) acc[tt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 16 * j + 4 * q + i;
      uint4 xv = s_x[tx * CH + (c ^ (tx & 15))];
      if (!live) xv = make_uint4(0u, 0u, 0u, 0u);
      const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, xv);
#pragma unroll
      for (int tt = 0; tt < DM_TILES; ++tt) {
        const uint32_t w = i == 0 ? wc[tt][j].x : i == 1 ? wc[tt][j].y : i == 2 ? wc[tt][j].z : wc[tt][j].w;
        const float sc = i < 2 ? e4m3_to_f32<0>(ws[tt][j]) : e4m3_to_f32<1>(ws[tt][j]);
        const f32x2_t f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
        const f32x2_t f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
        const f32x2_t f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
        const f32x2_t f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, make_uint4(pack_bf16x2_rne(f0.x * sc, f0.y * sc),
                                                                    pack_bf16x2_rne(f1.x * sc, f1.y * sc),
                                                                    pack_bf16x2_rne(f2.x * sc, f2.y * sc),
                                                                    pack_bf16x2_rne(f3.x * sc, f3.y * sc)));
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[tt], 0, 0, 0);
      }
    }
  }
  // lane (q, t) holds rows 4 q .. 4 q + 3 of each tile for token t = r
  if (live) {
#pragma unroll
    for (int tt = 0; tt < DM_TILES; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rbase + 16 * tt + 4 * q + i;
        if (row < rows) {
          const size_t o = (size_t)r * rows + row;
          float v = round_bf16(acc[tt][i] * g0);
          if (resid) v = bf16_bits_to_f32(aux[o]) + v;
          y[o] = f32_to_bf16_bits(v);
        }
      }
  }
}

// the tall-matrix kernel covers NVFP4 weights with 2048 or 4096 columns
bool dense_nv_supported(int cols, int batch) {
  return (cols == 2048 || cols == 4096) && batch >= 1 && batch <= kMaxB;
}

template <int NW, int CPL, int RPL, int BT, bool SW, bool NORM>
hipError_t dense_nv_launch(const uint8_t* codes, const uint8_t* scales, const float* gscale, const uint16_t* x,
                           int B, int rows, int cols, uint16_t* y, const uint16_t* aux, int resid,
                           const uint16_t* gamma, float eps, hipStream_t st) {
  auto k = dense_nv_kernel<NW, CPL, RPL, BT, SW, NORM>;
  // the staged tokens, one slot for positions past them, gamma
  const int lds = (B + 2) * (cols / 8) * 16;
  static const bool lds_ok = allow_dynamic_lds(k, (BT + 2) * (CPL * 64) * 16);
  (void)lds_ok;
  const int per = SW ? NW * 4 : NW * 4 * RPL;
  hipLaunchKernelGGL(k, dim3((rows + per - 1) / per), dim3(64 * NW), lds, st, codes, scales, gscale, x, B, rows,
                     cols, y, aux, resid, gamma, eps);
  return hipGetLastError();
}

// SwiGLU pair [2][rows][cols] -> h [B][rows], with the RMSNorm of x fused
// when asked; one-wave workgroups for one token, four waves for a batch
hipError_t dense_nv_swiglu(const LayerArgs& a, bool norm, hipStream_t st) {
#define FLINT_DNV_SW(NW_, CPL_, BT_, N_)                                                                     \
  dense_nv_launch<NW_, CPL_, 2, BT_, true, N_>(a.sh_gu_codes, a.sh_gu_scales, a.sh_gscale, a.x, a.B, a.SI, a.H, \
                                               a.out, nullptr, 0, a.gamma, a.eps, st)
  if (a.H == 2048) {
    if (norm) return a.B == 1 ? FLINT_DNV_SW(1, 4, 1, true) : FLINT_DNV_SW(4, 4, kMaxB, true);
    return a.B == 1 ? FLINT_DNV_SW(1, 4, 1, false) : FLINT_DNV_SW(4, 4, kMaxB, false);
  }
  return norm ? FLINT_DNV_SW(1, 8, 1, true) : FLINT_DNV_SW(1, 8, 1, false);   // 4096 columns, one token
#undef FLINT_DNV_SW
}
// shapes of the SwiGLU pair this path takes (4096 columns for a batch would
// not fit the registers of four waves per SIMD)
bool dense_nv_swiglu_supported(int cols, int batch) {
  return dense_nv_supported(cols, batch) && (cols == 2048 || batch == 1);
}

}  // namespace

hipError_t launch_gate_up(const LayerArgs& a, const DecodeWs& ws, bool dense, bool norm,
                          hipStream_t st) {
  // decode: h[slot][t][Imax]; dense: y[t][rows] with rows = SI
  const int imax = a.I > a.SI ? a.I : a.SI;
  uint16_t* hout = dense ? a.out : ws.h;
  const int hs = dense ? 0 : kMaxB * imax;
  const int ht = dense ? a.SI : imax;
  const bool bf = (a.flags & FLINT_W_BF16) != 0;
  if (dense && !bf && dense_nv_swiglu_supported(a.H, a.B)) return dense_nv_swiglu(a, norm, st);
  if (a.B == 1)
    return bf ? gate_up_dispatch_g<FMT_BF16, 1>(a, ws, dense, norm, hout, hs, ht, imax, st)
              : gate_up_dispatch_g<FMT_NVFP4, 1>(a, ws, dense, norm, hout, hs, ht, imax, st);
  if (!dense && !norm) {
    const int kq = a.H / 8 > 256 ? 2 : 1;
    if (bf && gate_up_batch_nch<FMT_BF16>(a) == 4 && kq == 1)
      return gate_up_batch_launch<FMT_BF16, 4, 1>(a, ws, hout, hs, ht, imax, st);
    if (!bf && a.B > 1 && a.B * a.H * 2 <= kBatchXBytes && (a.H == 2048 || a.H == 4096))
      return a.H == 2048 ? gate_up_nv_batch_launch<4>(a, ws, hout, hs, ht, imax, st)
                         : gate_up_nv_batch_launch<8>(a, ws, hout, hs, ht, imax, st);
  }
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
  if (dense && !bf && dense_nv_supported(a.SI, a.B)) {      // W [H][SI] . x[B][SI]
    // one-wave workgroups for one token (more of them resident per CU: a
    // 2048-column LM head ran at 67 % of HBM peak against 57 % with 8
    // waves); four waves for a batch, whose 8 staged tokens each workgroup
    // would otherwise read again
    const int resid = dense_epilogue == FLINT_EPI_RESIDUAL ? 1 : 0;
#define FLINT_DENSE_NV(NW_, CPL_, RPL_, BT_)                                                                   \
  dense_nv_launch<NW_, CPL_, RPL_, BT_, false, false>(a.sh_d_codes, a.sh_d_scales, a.sh_gscale, hin, a.B, a.H,  \
                                                      a.SI, a.out, aux, resid, nullptr, 0.f, st)
    if (a.SI == 2048 && a.B > 1) {                 // the MFMA form (see dense_nv_mfma_kernel)
      constexpr int NW = 4, per = NW * 16 * DM_TILES;
      hipLaunchKernelGGL(dense_nv_mfma_kernel<NW>, dim3((a.H + per - 1) / per), dim3(64 * NW), 0, st, a.sh_d_codes,
                         a.sh_d_scales, a.sh_gscale, hin, a.B, a.H, a.out, aux, resid);
      return hipGetLastError();
    }
    if (a.SI == 2048) return FLINT_DENSE_NV(1, 4, 2, 1);
    return a.B == 1 ? FLINT_DENSE_NV(1, 8, 1, 1) : FLINT_DENSE_NV(4, 8, 1, kMaxB);
#undef FLINT_DENSE_NV
  }
  if (a.B == 1)
    return bf ? down_dispatch_g<FMT_BF16, 1>(a, ws, dense, dense_epilogue, hin, hs, ht, dcols, aux, st)
              : down_dispatch_g<FMT_NVFP4, 1>(a, ws, dense, dense_epilogue, hin, hs, ht, dcols, aux, st);
  if (!dense && down_batch_lds(a) <= kBatchHBytes && (a.I > a.SI ? a.I : a.SI) / 8 <= 512)
    return bf ? down_batch_g<FMT_BF16>(a, ws, hin, hs, ht, st) : down_batch_g<FMT_NVFP4>(a, ws, hin, hs, ht, st);
  return bf ? down_dispatch_g<FMT_BF16, kMaxB>(a, ws, dense, dense_epilogue, hin, hs, ht, dcols, aux, st)
            : down_dispatch_g<FMT_NVFP4, kMaxB>(a, ws, dense, dense_epilogue, hin, hs, ht, dcols, aux, st);
}

}  // namespace flint
