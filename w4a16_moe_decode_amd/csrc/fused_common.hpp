// Pieces of the single-launch decode kernels (fused.hip): the epoch-tagged
// hand-off words, the gate/up
// row pairs of a selected expert and their loads, and the CU count.
#pragma once
#include "common.hpp"

namespace flint {
namespace {

// A kernel argument the compiler must hold in scalar registers from here on.
// Kernel arguments are otherwise loaded lazily, each with a scalar load
// where it is first needed, and the wait for such a load (its counter is
// shared with LDS accesses) stalls the next LDS access or barrier by a
// memory round trip; pinning every argument a kernel uses at its start
// makes all of them one batch of loads and one wait.
template <class T>
__device__ __forceinline__ T pin_sgpr(T v) {
  asm volatile("" : "+s"(v));
  return v;
}
// Pointers are pinned as global-memory pointers, so the compiler still knows
// that loads through them are global loads (a generic pointer of unknown
// origin would make them flat loads, which count against the LDS counter).
template <class T>
__device__ __forceinline__ T* pin_sgpr(T* p) {
  typedef __attribute__((address_space(1))) T GT;
  GT* g = (GT*)p;
  asm volatile("" : "+s"(g));
  return (T*)g;
}

// The fields of the layer arguments the single-launch kernels use, pinned.
__device__ __forceinline__ LayerArgs pin_layer_args(const LayerArgs& in) {
  LayerArgs a = in;
  a.H = pin_sgpr(in.H); a.E = pin_sgpr(in.E); a.I = pin_sgpr(in.I); a.SI = pin_sgpr(in.SI);
  a.K = pin_sgpr(in.K); a.flags = pin_sgpr(in.flags); a.eps = pin_sgpr(in.eps);
  a.router = pin_sgpr(in.router);
  a.gu_codes = pin_sgpr(in.gu_codes); a.gu_scales = pin_sgpr(in.gu_scales);
  a.d_codes = pin_sgpr(in.d_codes); a.d_scales = pin_sgpr(in.d_scales); a.gscale = pin_sgpr(in.gscale);
  a.sh_gu_codes = pin_sgpr(in.sh_gu_codes); a.sh_gu_scales = pin_sgpr(in.sh_gu_scales);
  a.sh_d_codes = pin_sgpr(in.sh_d_codes); a.sh_d_scales = pin_sgpr(in.sh_d_scales);
  a.sh_gscale = pin_sgpr(in.sh_gscale);
  a.x = pin_sgpr(in.x); a.gamma = pin_sgpr(in.gamma); a.out = pin_sgpr(in.out);
  a.topk_idx = pin_sgpr(in.topk_idx); a.topk_w = pin_sgpr(in.topk_w);
  return a;
}
__device__ __forceinline__ DecodeWs pin_decode_ws(const DecodeWs& in) {
  DecodeWs w = in;
  w.epoch = pin_sgpr(in.epoch); w.error = pin_sgpr(in.error); w.wait_limit = pin_sgpr(in.wait_limit);
  w.logit_words = pin_sgpr(in.logit_words); w.h_words = pin_sgpr(in.h_words);
  w.x_words = pin_sgpr(in.x_words); w.hb_words = pin_sgpr(in.hb_words); w.p_words = pin_sgpr(in.p_words);
  return w;
}

// Default bound of every wait for a hand-off word (reloads of one batch of
// words); the workspace's wait-limit word, when not zero, replaces it.
constexpr uint32_t kFusedSpin = 1u << 20;

// A vector load: a scalar load from memory would share its wait counter
// with every LDS access that follows it.
__device__ __forceinline__ uint32_t wait_limit(const DecodeWs& ws) {
  const uint32_t v = __hip_atomic_load(ws.wait_limit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v ? v : kFusedSpin;
}

__device__ __forceinline__ uint64_t poll_word(const uint64_t* p, uint32_t epoch, uint32_t* err, uint32_t lim) {
  uint64_t w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (uint32_t spin = 0; (uint32_t)(w >> 32) != epoch && spin < lim; ++spin) {
    __builtin_amdgcn_s_sleep(1);
    w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if ((uint32_t)(w >> 32) != epoch) *err = 1u;
  return w;
}

// Batched wait: all U words are loaded at once, then only the ones that do
// not carry the epoch yet are loaded again.  Entries with ok[u] false are
// skipped; their pointers must still be valid: the first loads are made
// unconditionally (a load made on one path only can leave the compiler
// believing it may still be in flight, and waiting for the memory counter
// to drain in the middle of the next batch of loads).
template <int U>
__device__ __forceinline__ void poll_words(uint64_t (&w)[U], const uint64_t* const (&p)[U],
                                           const bool (&ok)[U], uint32_t epoch, uint32_t* err, uint32_t lim) {
#pragma unroll
  for (int u = 0; u < U; ++u) w[u] = __hip_atomic_load(p[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (!ok[u]) w[u] = (uint64_t)epoch << 32;
  for (uint32_t spin = 0; spin < lim; ++spin) {
    bool ready = true;
#pragma unroll
    for (int u = 0; u < U; ++u) ready = ready && (uint32_t)(w[u] >> 32) == epoch;
    if (ready) return;
    __builtin_amdgcn_s_sleep(1);     // a short back-off: a reload takes a round trip anyway
#pragma unroll
    for (int u = 0; u < U; ++u)
      if ((uint32_t)(w[u] >> 32) != epoch)
        w[u] = __hip_atomic_load(p[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  *err = 1u;
}

// Pipelined wait for small sets of words: a new batch of loads of all U
// words is issued every SLEEP x 64 cycles, and each batch is checked while
// the next is in flight (loads complete in order, so checking one batch
// waits only for it).  A word that lands just after a batch passed it is
// then seen about one issue interval later instead of one round trip later.
// Entries with ok[u] false are skipped; their pointers must still be valid.
template <int U, int SLEEP>
__device__ __forceinline__ void poll_words_pipelined(uint64_t (&w)[U], const uint64_t* const (&p)[U],
                                                     const bool (&ok)[U], uint32_t epoch, uint32_t* err,
                                                     uint32_t lim) {
  uint64_t a[U], b[U];
  auto ready = [&](const uint64_t (&v)[U]) {
    bool r = true;
#pragma unroll
    for (int u = 0; u < U; ++u) r = r && (!ok[u] || (uint32_t)(v[u] >> 32) == epoch);
    return r;
  };
#pragma unroll
  for (int u = 0; u < U; ++u) a[u] = __hip_atomic_load(p[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (uint32_t spin = 0; spin < lim; spin += 2) {
    __builtin_amdgcn_s_sleep(SLEEP);
#pragma unroll
    for (int u = 0; u < U; ++u) b[u] = __hip_atomic_load(p[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (ready(a)) {
#pragma unroll
      for (int u = 0; u < U; ++u) w[u] = ok[u] ? a[u] : (uint64_t)epoch << 32;
      return;
    }
    __builtin_amdgcn_s_sleep(SLEEP);
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = __hip_atomic_load(p[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (ready(b)) {
#pragma unroll
      for (int u = 0; u < U; ++u) w[u] = ok[u] ? b[u] : (uint64_t)epoch << 32;
      return;
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) w[u] = ok[u] ? a[u] : (uint64_t)epoch << 32;
  *err = 1u;
}

__device__ __forceinline__ void put_word(uint64_t* p, uint32_t epoch, uint32_t payload) {
  __hip_atomic_store(p, ((uint64_t)epoch << 32) | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Hand-off words are published in kReplicas copies (lanes 0..kReplicas-1 of
// the writing wave each store one); workgroup g reads copy g % kReplicas.
// Every workgroup needs every word: one copy per XCD keeps the readers of a
// line to the workgroups of one XCD without multiplying the stores much.
constexpr int kReplicas = 8;

__device__ __forceinline__ void put_word_all(uint64_t* base, size_t stride, size_t idx, uint32_t epoch,
                                             uint32_t payload) {
  const int lane = threadIdx.x & 63;
  if (lane < kReplicas) put_word(base + (size_t)lane * stride + idx, epoch, payload);
}

struct GURows {            // gate and up rows of one selected expert
  const uint8_t* gc; const uint8_t* gs;
  const uint8_t* uc; const uint8_t* us;
  float g_scale, u_scale;
  int inter;
};

// Rows of a selected expert (-1 = the shared one); the tensor scales come
// from the LDS table `gs` ([E][3] routed, then the shared expert's), or are
// left for the caller to fill when gs is null.
__device__ __forceinline__ GURows gu_rows(const LayerArgs& a, int expert, const float (*gs)[3]) {
  GURows r;
  const int H = a.H;
  if (expert < 0) {
    r.inter = a.SI;
    const size_t mc = (size_t)a.SI * H / 2, ms = (size_t)a.SI * H / 16;
    r.gc = a.sh_gu_codes; r.uc = a.sh_gu_codes + mc;
    r.gs = a.sh_gu_scales; r.us = a.sh_gu_scales + ms;
    r.g_scale = gs ? gs[a.E][0] : 0.f; r.u_scale = gs ? gs[a.E][1] : 0.f;
  } else {
    r.inter = a.I;
    const size_t mc = (size_t)a.I * H / 2, ms = (size_t)a.I * H / 16;
    r.gc = a.gu_codes + (size_t)(2 * expert) * mc; r.uc = r.gc + mc;
    r.gs = a.gu_scales + (size_t)(2 * expert) * ms; r.us = r.gs + ms;
    r.g_scale = gs[expert][0]; r.u_scale = gs[expert][1];
  }
  return r;
}

// This thread's entries (threadIdx.x and threadIdx.x + 256) of the tensor
// scale table: routed experts 0..E-1, then the shared expert at E.  Vector
// loads (the addresses differ per lane), unconditional (clamped pointers).
struct GsPre { float v[2][3]; };
__device__ __forceinline__ void gs_prefetch(GsPre& g, const float* gscale, const float* sh_gscale, int E) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = threadIdx.x + 256 * q;
    const float* p = i < E ? gscale + 3 * i : (i == E && sh_gscale ? sh_gscale : gscale);
#pragma unroll
    for (int j = 0; j < 3; ++j) g.v[q][j] = ldg<float>(p + j);
  }
}
__device__ __forceinline__ void gs_store(const GsPre& g, float (*gs)[3], int E) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = threadIdx.x + 256 * q;
    if (i <= E)
#pragma unroll
      for (int j = 0; j < 3; ++j) gs[i][j] = g.v[q][j];
  }
}

// One gate/up item: rows 2p and 2p+1 of a selected expert, a whole wave per
// row (H/32 chunks of 32 columns per row, NCH per lane).  Returns the packed
// BF16 pair h[2p], h[2p+1] (valid in every lane).
template <int NCH>
struct GUItem {
  uint4 c[2][2][NCH];       // [row][gate|up][chunk]
  uint32_t s[2][2][NCH];
};

template <int NCH>
__device__ __forceinline__ void gu_load(GUItem<NCH>& it, const GURows& R, int p, int H) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int row = 2 * p + rr;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int j = lane + 64 * c;
      it.c[rr][0][c] = ldg<uint4>(R.gc + (size_t)row * (H / 2) + 16 * j);
      it.s[rr][0][c] = ldg<uint16_t>(R.gs + (size_t)row * (H / 16) + 2 * j);
      it.c[rr][1][c] = ldg<uint4>(R.uc + (size_t)row * (H / 2) + 16 * j);
      it.s[rr][1][c] = ldg<uint16_t>(R.us + (size_t)row * (H / 16) + 2 * j);
    }
  }
}

// Workgroups that own no router row (a grid wider than E) announce with a
// word of their own that they have read the launch epoch; workgroup 0 waits
// for these words (with the logits) before it may advance the epoch at its
// end.  They sit after the logit words of 8 tokens x kReplicas copies.
constexpr int kMaxArrivals = 256;               // grid width - E is capped to this
__device__ __forceinline__ uint64_t* arrival_words(const DecodeWs& ws, int E) {
  return ws.logit_words + (size_t)FLINT_MAX_DECODE_BATCH * kReplicas * E;
}
__device__ __forceinline__ void announce_arrival(const DecodeWs& ws, int E, uint32_t epoch) {
  if ((int)blockIdx.x >= E && threadIdx.x == 0) put_word(arrival_words(ws, E) + (blockIdx.x - E), epoch, 0u);
}
// the four arrival words lane `lane` polls in workgroup 0 (none elsewhere)
__device__ __forceinline__ void arrival_slots(const DecodeWs& ws, int E, int G, const uint64_t** p, bool* ok) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int b = lane + 64 * q;
    ok[q] = blockIdx.x == 0 && b < G - E;
    p[q] = arrival_words(ws, E) + (ok[q] ? b : 0);
  }
}

// top-k of one token from its four logit words per lane: lane k < K returns
// the k-th selected key (descending logit, ties to the lower index)
__device__ __forceinline__ uint64_t select_topk(uint64_t (&key)[4], int K) {
  const int lane = threadIdx.x & 63;
#define FLINT_CSWAP(i, j) { const uint64_t hi_ = key[i] > key[j] ? key[i] : key[j]; \
                            const uint64_t lo_ = key[i] > key[j] ? key[j] : key[i]; key[i] = hi_; key[j] = lo_; }
  FLINT_CSWAP(0, 1) FLINT_CSWAP(2, 3) FLINT_CSWAP(0, 2) FLINT_CSWAP(1, 3) FLINT_CSWAP(1, 2)
#undef FLINT_CSWAP
  uint64_t mine = 0ull;
  for (int k = 0; k < K; ++k) {
    const uint64_t m = wave_max_key(key[0]);
    if (key[0] == m) { key[0] = key[1]; key[1] = key[2]; key[2] = key[3]; key[3] = 0ull; }
    if (lane == k) mine = m;
  }
  return mine;
}

// Maximum over the wave of a 32-bit value, in every lane: DPP steps within
// rows of 16 lanes, then the four row maxima combined with the permlane
// swaps, so that no value makes a round trip through a scalar register.
__device__ __forceinline__ uint32_t wave_max_u32_all(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));                   // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));                   // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141>(v));                  // row_half_mirror
  v = max(v, dpp_u32<0x140>(v));                  // row_mirror
  { const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false); v = max(r[0], r[1]); }
  { const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false); v = max(r[0], r[1]); }
  return v;
}

// top-k of one token from its four keys per lane (order key of the logit
// << 32 | inverted expert index; 0 for no entry): the k-th selected key
// (descending logit, equal logits to the lower index) is written to
// s_key[k].  Each lane sorts its keys, then every round takes the wave
// maximum of the lanes' heads on the 32-bit logit key alone and the winning
// lane stores and pops its head; only when several lanes hold the maximal
// logit (equal logits) is the index half compared too.
__device__ __forceinline__ void topk_keys_to_lds(uint64_t (&key)[4], int K, uint64_t* s_key) {
#define FLINT_CSWAP(i, j) { const uint64_t hi_ = key[i] > key[j] ? key[i] : key[j]; \
                            const uint64_t lo_ = key[i] > key[j] ? key[j] : key[i]; key[i] = hi_; key[j] = lo_; }
  FLINT_CSWAP(0, 1) FLINT_CSWAP(2, 3) FLINT_CSWAP(0, 2) FLINT_CSWAP(1, 3) FLINT_CSWAP(1, 2)
#undef FLINT_CSWAP
#pragma unroll
  for (int k = 0; k < FLINT_MAX_TOP_K; ++k) {
    if (k >= K) break;                            // the same in every lane
    const uint32_t hi = (uint32_t)(key[0] >> 32), lo = (uint32_t)key[0];
    const uint32_t mhi = wave_max_u32_all(hi);
    const bool at = hi == mhi;
    bool win = at;
    if (__popcll(__ballot(at)) != 1) {            // equal logits: the lower index wins
      const uint32_t mlo = wave_max_u32_all(at ? lo : 0u);
      win = at && lo == mlo;
    }
    if (win) {
      s_key[k] = key[0];
      key[0] = key[1]; key[1] = key[2]; key[2] = key[3]; key[3] = 0ull;
    }
  }
}

// The same selection with the result in registers: sel[k] (equal in every
// lane) is the k-th selected key for k < K, 0 beyond.
__device__ __forceinline__ void topk_keys_uniform(uint64_t (&key)[4], int K, uint64_t (&sel)[FLINT_MAX_TOP_K]) {
#define FLINT_CSWAP(i, j) { const uint64_t hi_ = key[i] > key[j] ? key[i] : key[j]; \
                            const uint64_t lo_ = key[i] > key[j] ? key[j] : key[i]; key[i] = hi_; key[j] = lo_; }
  FLINT_CSWAP(0, 1) FLINT_CSWAP(2, 3) FLINT_CSWAP(0, 2) FLINT_CSWAP(1, 3) FLINT_CSWAP(1, 2)
#undef FLINT_CSWAP
#pragma unroll
  for (int k = 0; k < FLINT_MAX_TOP_K; ++k) {
    sel[k] = 0ull;
    if (k >= K) continue;                         // the same in every lane
    const uint32_t hi = (uint32_t)(key[0] >> 32), lo = (uint32_t)key[0];
    const uint32_t mhi = wave_max_u32_all(hi);
    const bool at = hi == mhi;
    const unsigned long long bal = __ballot(at);
    uint32_t mlo;
    if (__popcll(bal) == 1)
      mlo = __builtin_amdgcn_readlane(lo, __ffsll((long long)bal) - 1);
    else                                          // equal logits: the lower index wins
      mlo = wave_max_u32_all(at ? lo : 0u);
    sel[k] = ((uint64_t)mhi << 32) | mlo;
    if (key[0] == sel[k]) { key[0] = key[1]; key[1] = key[2]; key[2] = key[3]; key[3] = 0ull; }
  }
}

inline int device_num_cu() {
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    n_cu = n;
  }
  return n_cu;
}

}  // namespace
}  // namespace flint
