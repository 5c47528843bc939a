// flint_decode_attention: one decode token per sequence attends, with GQA,
// to its sliding window or to its whole context in a BF16 KV cache, with a
// learned sink logit per query head ("Day-0 Support for Flint on vLLM",
// "Model architecture": 35 layers see the current token and the 512 before
// it, 14 layers the whole context; GQA with 32 query and 4 KV heads of
// dimension 128; learned attention sinks.  "Optimizations": a decode
// attention kernel with sinks and sliding windows).
//
// Split over the context (flash decoding): workgroup (b, chunk, g) takes
// chunk `chunk` of sequence b's attended positions for KV head g, i.e. the
// `group` query heads that read it.  Each wave works in steps of 32
// positions; per step
//   S = K Q^T      16 positions x 16 heads per MFMA 16x16x32 (K rows from
//                  HBM straight into the A operand; heads past the group
//                  are zero columns), two tiles;
//   online softmax in the base-2 domain (scores pre-scaled by
//                  scale * log2 e), one running max per head;
//   O^T += V^T P^T 16 head-dim rows x 16 heads per MFMA, eight of them;
//                  MFMA db takes dims 8 m + db (m = 0..15), so that the A
//                  operand of lane (q4, hh) is chunk hh (dims 8 hh .. + 7)
//                  of the eight V rows its P^T entries weight: the lane
//                  loads exactly those 16-byte chunks (a wave reads four
//                  whole 256-byte rows per load) and builds the transposed
//                  operands of all eight MFMAs with byte permutes, so V
//                  needs no LDS.
// The GQA group shares every K and V byte, which is what makes the two
// products real matrix products; the kernel is bound by the KV bytes.
// Steps are double-buffered in registers.  The four waves' results merge
// in LDS; with one chunk per sequence the workgroup writes
// the output, otherwise each chunk leaves (max, sum, unnormalised O) and a
// second kernel folds the chunks and the sink.
#include <hip/hip_runtime.h>

#include "common.hpp"

namespace flint {
namespace {


constexpr int AD_D = 128;                  // head dimension
constexpr int AD_STEP = 32;                // positions per wave step
constexpr int AD_PART = 32 + 16 * AD_D;    // floats per chunk result: m[16], l[16], o[16][128]
constexpr int AD_TARGET_WGS = 512;         // workgroups the context split aims for (2 per CU)
constexpr int AD_CMB_CAP = 16;             // chunks per combine lane group per pass
constexpr float AD_LOG2E = 1.4426950408889634f;

struct AdArgs {
  const uint16_t* q;         // [B][n_q][128]
  const uint16_t* k_cache;   // [n_rows][n_kv][128]
  const uint16_t* v_cache;
  const int32_t* seq_base;
  const int32_t* seq_len;
  const float* sinks;        // [n_q]
  uint16_t* out;             // [B][n_q][128]
  float* part;               // [B][n_kv][n_chunks][AD_PART]
  int32_t* error;
  int n_q, n_kv, group, window, ring, n_rows, max_len, n_chunks, chunk;   // chunk: positions per workgroup
  float scale_log2;          // scale * log2(e)
};

// The attended positions of sequence b: lo .. lo + span - 1, in rows
// base + (p mod ring).  False when the sequence's description is invalid.
__device__ __forceinline__ bool seq_span(const AdArgs& a, int b, int& base, int& lo, int& span) {
  base = a.seq_base[b];
  const int len = a.seq_len[b];
  lo = (a.window > 0 && len > a.window) ? len - a.window : 0;
  span = len - lo;
  return len >= 1 && len <= a.max_len && base >= 0 && (int64_t)base + a.ring <= a.n_rows && span <= a.ring;
}

__device__ __forceinline__ float max_rows(float v) {      // over lanes l, l^16, l^32, l^48
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_rows(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// The rows of one step: lane (q4, hh) needs the element offsets of the K
// rows of positions 16 i + hh (i = 0, 1) and of the V rows of positions
// tau(q4, j) = 4 q4 + j (j < 4) and 16 + 4 q4 + j - 4 (j >= 4), the order
// of its P^T entries.  Positions past the span read the last attended row
// (finite; their weights are zero).
struct StepRows {
  uint32_t k[2];
  uint32_t v[8];
};

__device__ __forceinline__ int tau(int q4, int j) { return j < 4 ? 4 * q4 + j : 16 + 4 * q4 + (j - 4); }

__device__ __forceinline__ void step_rows(StepRows& r, const AdArgs& a, int base, int lo, int span, int g,
                                          int tb, int q4, int hh) {
  const int t0 = tb < span ? tb : span - 1;       // first position of the step, clamped
  const int r0 = (lo + t0) % a.ring;               // its row in the ring
  auto row = [&](int o) -> uint32_t {
    const int t = tb + o < span ? tb + o : span - 1;
    int rr = r0 + (t - t0);                        // t - t0 < ring, so one wrap at most
    if (rr >= a.ring) rr -= a.ring;
    return ((uint32_t)(base + rr) * a.n_kv + g) * AD_D;
  };
  r.k[0] = row(hh);
  r.k[1] = row(16 + hh);
#pragma unroll
  for (int j = 0; j < 8; ++j) r.v[j] = row(tau(q4, j));
}

struct StepData {
  uint4 k[8];          // K: tile i, dims 32 s + 8 q4 .. + 7 at [4 i + s]
  uint4 v[8];          // V: row tau(q4, j), dims 8 hh .. + 7 at [j]
};

__device__ __forceinline__ void step_load(StepData& d, const AdArgs& a, const StepRows& r, int q4, int hh) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int s = 0; s < 4; ++s) d.k[4 * i + s] = ldg_nt(a.k_cache + r.k[i] + 32 * s + 8 * q4);
#pragma unroll
  for (int j = 0; j < 8; ++j) d.v[j] = ldg_nt(a.v_cache + r.v[j] + 8 * hh);
}

struct Online {
  float m;             // running max of head hh (base-2 scores), the same in its four lanes
  float l;             // this lane's part of the running sum
  f32x4_t o[8];        // O^T: element e of block db is head hh, dim 8 (4 q4 + e) + db
};

// One step of 32 positions (tb: the first one's index in the attended span).
__device__ __forceinline__ void step_compute(Online& st, const StepData& sd, const bf16x8_t (&qf)[4], int tb,
                                             int span, float scale_log2, int q4) {
  f32x4_t s[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    s[i] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      s[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(sd.k[4 * i + k]), qf[k], s[i], 0, 0, 0);
  }
  // s[i][e]: position tb + 16 i + 4 q4 + e, head hh
  float x[2][4];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = tb + 16 * i + 4 * q4 + e < span;
      x[i][e] = ok ? s[i][e] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, x[i][e]);
    }
  mx = max_rows(mx);
  const float mn = fmaxf(st.m, mx);
  const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(st.m - mn);
  st.m = mn;
  float p[2][4];
  float ps = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[i][e] = x[i][e] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x[i][e] - mn);
      ps += p[i][e];
    }
  st.l = st.l * alpha + ps;
  // P^T operand: k index 8 q4 + j is position 4 q4 + j (j < 4) or 16 + 4 q4 + j - 4
  const uint4 pw = make_uint4(pack_bf16x2_rne(p[0][0], p[0][1]), pack_bf16x2_rne(p[0][2], p[0][3]),
                              pack_bf16x2_rne(p[1][0], p[1][1]), pack_bf16x2_rne(p[1][2], p[1][3]));
  const bf16x8_t pb = as_bf16x8(pw);
  // V^T operands: element db of each V chunk is dword db / 2, half db % 2
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const uint32_t sel = (db & 1) ? 0x07060302u : 0x05040100u;
    uint32_t w[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint4 ra = sd.v[2 * jj], rb = sd.v[2 * jj + 1];
      const uint32_t da = (db >> 1) == 0 ? ra.x : (db >> 1) == 1 ? ra.y : (db >> 1) == 2 ? ra.z : ra.w;
      const uint32_t dbw = (db >> 1) == 0 ? rb.x : (db >> 1) == 1 ? rb.y : (db >> 1) == 2 ? rb.z : rb.w;
      w[jj] = __builtin_amdgcn_perm(dbw, da, sel);
    }
    st.o[db] *= alpha;
    st.o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(make_uint4(w[0], w[1], w[2], w[3])), pb,
                                                       st.o[db], 0, 0, 0);
  }
}

template <int NW, int NS>
__global__ __launch_bounds__(64 * NW) void attn_decode_part_kernel(AdArgs a) {
  constexpr int NT = 64 * NW;
  __shared__ float s_o[NW * 16 * AD_D];           // the waves' O for the merge
  __shared__ float s_mw[NW][16], s_lw[NW][16];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int q4 = lane >> 4, hh = lane & 15;
  const int g = blockIdx.x % a.n_kv;
  const int bc = blockIdx.x / a.n_kv;
  const int c = bc % a.n_chunks, b = bc / a.n_chunks;
  const bool single = a.n_chunks == 1;
  int base, lo, span;
  if (!seq_span(a, b, base, lo, span)) {           // the combine (or the zeros below) answers
    if (single)
      for (int e = tid; e < a.group * AD_D; e += NT)
        a.out[((size_t)b * a.n_q + g * a.group) * AD_D + e] = 0;
    if (tid == 0 && c == 0 && g == 0 && a.error) *a.error = 1;
    return;
  }
  const int ch = NS * NW * AD_STEP;
  if (c * ch >= span) return;                      // past this sequence's last chunk

  // Q^T operand: head hh of the group (zero past it), dims 32 k + 8 q4 .. + 7
  bf16x8_t qf[4];
  {
    const int hq = g * a.group + (hh < a.group ? hh : 0);
    const uint16_t* qp = a.q + ((size_t)b * a.n_q + hq) * AD_D + 8 * q4;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint4 v = ldg<uint4>(qp + 32 * k);
      qf[k] = as_bf16x8(hh < a.group ? v : make_uint4(0u, 0u, 0u, 0u));
    }
  }
  Online st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int db = 0; db < 8; ++db) st.o[db] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  // wave w's step s covers positions c ch + (NW s + w) 32 .. + 31; the steps
  // are straight-line code: step s + 1's loads go out before step s waits
  // for its own (the scheduling barriers keep that order), so two steps of
  // K and V are in flight per wave
  auto tb_of = [&](int s) { return c * ch + (NW * s + wave) * AD_STEP; };
  StepData sd[2];
  StepRows rows;
  step_rows(rows, a, base, lo, span, g, tb_of(0), q4, hh);
  step_load(sd[0], a, rows, q4, hh);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s + 1 < NS) {
      step_rows(rows, a, base, lo, span, g, tb_of(s + 1), q4, hh);
      step_load(sd[(s + 1) & 1], a, rows, q4, hh);
    }
    __builtin_amdgcn_sched_barrier(0);
    step_compute(st, sd[s & 1], qf, tb_of(s), span, a.scale_log2, q4);
    __builtin_amdgcn_sched_barrier(0);
  }
  const float lsum = sum_rows(st.l);

  // merge the four waves
  if (q4 == 0) {
    s_mw[wave][hh] = st.m;
    s_lw[wave][hh] = lsum;
  }
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_o[(wave * 16 + hh) * AD_D + 8 * (4 * q4 + e) + db] = st.o[db][e];
  __syncthreads();
  for (int e = tid; e < a.group * AD_D; e += NT) {
    const int h = e / AD_D, d = e % AD_D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, s_mw[w][h]);
    float l = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = s_mw[w][h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_mw[w][h] - mx);
      l += f * s_lw[w][h];
      o += f * s_o[(w * 16 + h) * AD_D + d];
    }
    if (single) {
      const float sk = a.sinks[g * a.group + h] * AD_LOG2E;
      const float m2 = fmaxf(mx, sk);
      const float f = __builtin_amdgcn_exp2f(mx - m2);
      const float z = l * f + __builtin_amdgcn_exp2f(sk - m2);
      a.out[((size_t)b * a.n_q + g * a.group + h) * AD_D + d] = f32_to_bf16_bits(o * f / z);
    } else {
      float* pp = a.part + (((size_t)b * a.n_kv + g) * a.n_chunks + c) * AD_PART;
      if (d == 0) {
        pp[h] = mx;
        pp[16 + h] = l;
      }
      pp[32 + h * AD_D + d] = o;
    }
  }
}

// Folds the chunks of one (sequence, query head) and the sink for 32 of the
// 128 output dimensions (blockIdx = (b h) 4 + quarter).  Lane group k (32
// lanes, dimension 32 quarter + lane) takes chunks c = k (mod 8), and every
// chunk's loads go out before any is used (up to AD_CMB_CAP per group per
// pass): the fold costs two memory round trips, not one per chunk.
__global__ __launch_bounds__(256) void attn_decode_combine_kernel(AdArgs a) {
  __shared__ float s_red[4];
  __shared__ float s_o[8][32];
  __shared__ float s_z[8];
  const int bh = blockIdx.x >> 2, qd = blockIdx.x & 3;
  const int b = bh / a.n_q, h = bh % a.n_q;
  const int g = h / a.group, hh = h % a.group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, k = tid >> 5, d = 32 * qd + (tid & 31);
  uint16_t* dst = a.out + ((size_t)b * a.n_q + h) * AD_D;
  int base, lo, span;
  if (!seq_span(a, b, base, lo, span)) {
    if (tid < 32) dst[d] = 0;
    return;
  }
  const int nc = (span + a.chunk - 1) / a.chunk;
  const float* pp = a.part + ((size_t)b * a.n_kv + g) * a.n_chunks * AD_PART;
  const float sk = a.sinks[h] * AD_LOG2E;
  // the largest chunk maximum (and the sink)
  float mx = -INFINITY;
  for (int c = tid; c < nc; c += 256) mx = fmaxf(mx, pp[(size_t)c * AD_PART + hh]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) s_red[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(sk, s_red[0]), fmaxf(fmaxf(s_red[1], s_red[2]), s_red[3]));
  float o = 0.f, z = 0.f;
  for (int c0 = 0; c0 < nc; c0 += 8 * AD_CMB_CAP) {
    float ov[AD_CMB_CAP], mv[AD_CMB_CAP], lv[AD_CMB_CAP];
#pragma unroll
    for (int i = 0; i < AD_CMB_CAP; ++i) {         // clamped, unconditional loads
      const int c = c0 + k + 8 * i;
      const float* q = pp + (size_t)(c < nc ? c : nc - 1) * AD_PART;
      ov[i] = q[32 + hh * AD_D + d];
      mv[i] = q[hh];
      lv[i] = q[16 + hh];
    }
#pragma unroll
    for (int i = 0; i < AD_CMB_CAP; ++i) {
      const float f = c0 + k + 8 * i < nc ? __builtin_amdgcn_exp2f(mv[i] - mx) : 0.f;
      o += f * ov[i];
      z += f * lv[i];
    }
  }
  s_o[k][tid & 31] = o;
  if ((tid & 31) == 0) s_z[k] = z;
  __syncthreads();
  if (tid < 32) {
    float os = 0.f, zs = __builtin_amdgcn_exp2f(sk - mx);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      os += s_o[j][tid];
      zs += s_z[j];
    }
    dst[d] = f32_to_bf16_bits(os / zs);
  }
}

// Context split: chunks of 64, 128, 256, 512 or 1024 positions (2 or 4
// waves of 1, 2, 4 or 8 steps), one size above the smallest that keeps the
// batch's (sequence, KV head, chunk) workgroups at or under AD_TARGET_WGS
// (else 1024 and more workgroups): the combine reads every chunk's
// partial, so short reads gain from fewer, longer chunks (a 513-position
// window: 9.5 -> 9.1 us at batch 1, 12.0 -> 11.4 us at batch 8).  Small reads spread over many CUs: one CU keeps only
// enough misses in flight for its share of the chip's bandwidth, so 1 MB
// read by 4 workgroups takes several times longer than by 68.  Long reads
// take chunks large enough that every workgroup is resident from the start
// (a second, partly empty round of workgroups is the slowest part).
struct AdPlan {
  int waves, steps, n_chunks;
};

AdPlan ad_plan(int n_kv, int window, int batch, int max_len) {
  const int span = window > 0 && window < max_len ? window : max_len;
  const int64_t per_wg = ((int64_t)span * batch * n_kv + AD_TARGET_WGS - 1) / AD_TARGET_WGS;
  AdPlan p;
  if (per_wg <= 32) p = {2, 1, 0};
  else if (per_wg <= 128) p = {4, 1, 0};
  else if (per_wg <= 256) p = {4, 2, 0};
  else if (per_wg <= 512) p = {4, 4, 0};
  else p = {4, 8, 0};
  const int chunk = p.waves * p.steps * AD_STEP;
  p.n_chunks = (span + chunk - 1) / chunk;
  return p;
}

int32_t ad_check_shape(const flint_attn_shape* shape, int32_t window, int32_t batch, int32_t max_len) {
  if (!shape || batch <= 0 || max_len <= 0 || window < 0) return FLINT_ERR_INVALID_ARG;
  if (shape->head_dim != AD_D || shape->n_q_heads <= 0 || shape->n_kv_heads <= 0 ||
      shape->n_q_heads % shape->n_kv_heads || shape->n_q_heads / shape->n_kv_heads > 16 || shape->flags)
    return FLINT_ERR_UNSUPPORTED;
  return FLINT_OK;
}

}  // namespace
}  // namespace flint

extern "C" int64_t flint_decode_attention_workspace_bytes(const flint_attn_shape* shape, int32_t window,
                                                          int32_t batch, int32_t max_len) {
  using namespace flint;
  if (ad_check_shape(shape, window, batch, max_len) != FLINT_OK) return -1;
  const AdPlan p = ad_plan(shape->n_kv_heads, window, batch, max_len);
  if (p.n_chunks == 1) return 0;
  return (int64_t)batch * shape->n_kv_heads * p.n_chunks * AD_PART * (int64_t)sizeof(float);
}

extern "C" int32_t flint_decode_attention(const flint_attn_shape* shape, int32_t window, int32_t ring, float scale,
                                          const void* q, int32_t batch, const void* k_cache, const void* v_cache,
                                          int32_t n_rows, const int32_t* seq_base, const int32_t* seq_len,
                                          int32_t max_len, const float* sinks, void* out, void* workspace,
                                          int64_t workspace_bytes, int32_t* error, void* stream) {
  using namespace flint;
  const int32_t st = ad_check_shape(shape, window, batch, max_len);
  if (st != FLINT_OK) return st;
  if (!q || !k_cache || !v_cache || !seq_base || !seq_len || !sinks || !out || ring <= 0 || n_rows <= 0 ||
      !(scale > 0.f) || !(scale < INFINITY))
    return FLINT_ERR_INVALID_ARG;
  if ((uint64_t)n_rows * shape->n_kv_heads * AD_D > 0xffffffffull) return FLINT_ERR_UNSUPPORTED;
  auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  auto a4 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; };
  if (!a16(q) || !a16(k_cache) || !a16(v_cache) || !a16(out) || !a4(seq_base) || !a4(seq_len) || !a4(sinks) ||
      (error && !a4(error)) || (workspace && !a16(workspace)))
    return FLINT_ERR_ALIGNMENT;
  AdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.seq_base = seq_base;
  a.seq_len = seq_len;
  a.sinks = sinks;
  a.out = static_cast<uint16_t*>(out);
  a.part = static_cast<float*>(workspace);
  a.error = error;
  a.n_q = shape->n_q_heads;
  a.n_kv = shape->n_kv_heads;
  a.group = a.n_q / a.n_kv;
  a.window = window;
  a.ring = ring;
  a.n_rows = n_rows;
  a.max_len = max_len;
  const AdPlan p = ad_plan(a.n_kv, window, batch, max_len);
  a.n_chunks = p.n_chunks;
  a.chunk = p.waves * p.steps * AD_STEP;
  a.scale_log2 = scale * AD_LOG2E;
  if (a.n_chunks > 1) {
    const int64_t need = (int64_t)batch * a.n_kv * a.n_chunks * AD_PART * (int64_t)sizeof(float);
    if (!workspace || workspace_bytes < need) return FLINT_ERR_WORKSPACE;
  }
  const int64_t wgs = (int64_t)batch * a.n_chunks * a.n_kv;
  if (wgs > 0x7fffffff) return FLINT_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)wgs);
#define AD_LAUNCH(W, S) hipLaunchKernelGGL((attn_decode_part_kernel<W, S>), grid, dim3(64 * W), 0, s, a)
  if (p.waves == 2) AD_LAUNCH(2, 1);
  else if (p.steps == 1) AD_LAUNCH(4, 1);
  else if (p.steps == 2) AD_LAUNCH(4, 2);
  else if (p.steps == 4) AD_LAUNCH(4, 4);
  else AD_LAUNCH(4, 8);
#undef AD_LAUNCH
  if (a.n_chunks > 1)
    hipLaunchKernelGGL(attn_decode_combine_kernel, dim3((unsigned)(batch * a.n_q * 4)), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? FLINT_OK : FLINT_ERR_DEVICE;
}
