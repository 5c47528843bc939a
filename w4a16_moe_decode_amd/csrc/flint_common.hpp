// Pieces of the single-launch kernels specialised to the Flint layer shape
// ("Day-0 Support for Flint on vLLM", "Model architecture": hidden 2048,
// 256 routed experts, sigmoid top-6 plus one always-on shared expert; the
// expert intermediate 512 is this library's reading): the compile-time
// sizes, a lane's part of eight down rows, and the register top-k.
#pragma once
#include "fused_common.hpp"

namespace flint {
namespace {

constexpr int FL_H = 2048, FL_E = 256, FL_I = 512;
constexpr int FL_G = 256;                          // workgroups (one per compute unit)
constexpr int FL_NW = 8;                           // waves per workgroup
constexpr int FL_ROWS = FL_H / FL_G;               // output rows per workgroup
constexpr int FL_IW = FL_I / 2;                    // h words (BF16 pairs) per slot

static_assert(FL_G == FL_E, "one router row per workgroup");
static_assert(FL_I / 32 == 16 && FL_ROWS == 8, "down rows: 16 lanes per row, 4 rows per load, 2 loads");

// The 16 bytes of codes and 2 scale bytes of a lane's chunk of two down rows
// (rows row0 + grp and row0 + 4 + grp, chunk li) of one expert.
struct DownRows {
  uint4 c[2];
  uint32_t s[2];
};

__device__ __forceinline__ void down_load(DownRows& d, const uint8_t* codes, const uint8_t* scales, int row0,
                                          int lane) {
  const int grp = lane >> 4, li = lane & 15;
#pragma unroll
  for (int rw = 0; rw < 2; ++rw) {
    const int n = row0 + 4 * rw + grp;
    d.c[rw] = ldg_nt(codes + (size_t)n * (FL_I / 2) + 16 * li);
    d.s[rw] = ldg<uint16_t>(scales + (size_t)n * (FL_I / 16) + 2 * li);
  }
}

// Top-k of one token held by a wave, lane l holding the keys of experts
// 4l..4l+3 (order key of the logit << 32 | inverted expert index).  Returns
// in lane k < K the k-th selected key (descending logit).  Each round takes
// the wave maximum of the lanes' best 32-bit logit keys; among the lanes
// holding it the lowest lane has the lowest expert index (experts rise with
// the lane), so it wins and pops its key: equal logits go to the lower
// index with no second reduction and no branch.  KC > 0 makes K a
// compile-time constant (straight-line rounds).
template <int KC>
__device__ __forceinline__ uint64_t topk_lane_key(uint64_t (&key)[4], int K) {
  const int lane = threadIdx.x & 63;
#define FLINT_CSWAP(i, j) { const uint64_t hi_ = key[i] > key[j] ? key[i] : key[j]; \
                            const uint64_t lo_ = key[i] > key[j] ? key[j] : key[i]; key[i] = hi_; key[j] = lo_; }
  FLINT_CSWAP(0, 1) FLINT_CSWAP(2, 3) FLINT_CSWAP(0, 2) FLINT_CSWAP(1, 3) FLINT_CSWAP(1, 2)
#undef FLINT_CSWAP
  uint64_t my_key = 0ull;
#pragma unroll
  for (int k = 0; k < (KC ? KC : FLINT_MAX_TOP_K); ++k) {
    if (!KC && k >= K) break;                      // the same in every lane
    const uint32_t hi = (uint32_t)(key[0] >> 32);
    const uint32_t mhi = wave_max_u32_all(hi);
    const int wl = __ffsll((long long)__ballot(hi == mhi)) - 1;
    const uint32_t mlo = __builtin_amdgcn_readlane((uint32_t)key[0], wl);
    const uint64_t sk = ((uint64_t)mhi << 32) | mlo;
    my_key = lane == k ? sk : my_key;
    const bool win = lane == wl;
    key[0] = win ? key[1] : key[0]; key[1] = win ? key[2] : key[1];
    key[2] = win ? key[3] : key[2]; key[3] = win ? 0ull : key[3];
  }
  return my_key;
}

// Bounded wait until the four tagged words of lane l (lw + 4l .. 4l + 3)
// carry the epoch; every lane of the wave reloads until all of them do.
__device__ __forceinline__ void poll_lane_words4(uint64_t (&wd)[4], const uint64_t* lw, uint32_t epoch,
                                                 uint32_t* err, uint32_t lim) {
  const uint64_t* p = lw + 4 * (threadIdx.x & 63);
  for (uint32_t spin = 0;; ++spin) {
#pragma unroll
    for (int q = 0; q < 4; ++q) wd[q] = __hip_atomic_load(p + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool ok = true;
#pragma unroll
    for (int q = 0; q < 4; ++q) ok = ok && (uint32_t)(wd[q] >> 32) == epoch;
    if (__all(ok)) break;
    if (spin >= lim) { *err = 1u; break; }
  }
}

// The four logit keys of lane l (experts 4l..4l+3) from their tagged words.
__device__ __forceinline__ void logit_keys(uint64_t (&key)[4], const uint64_t (&wd)[4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    key[q] = ((uint64_t)float_order_key(__uint_as_float((uint32_t)wd[q])) << 32) | (uint32_t)~(uint32_t)(4 * lane + q);
}

}  // namespace
}  // namespace flint
