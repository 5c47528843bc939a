// Prefill MoE layer (any number of tokens) for gfx950.
//
// "Day-0 Support for Flint on vLLM", "Optimizations": the small-batch MoE
// change is also the largest gain for an 8,192-token prefill, running on the
// same packed NVFP4 weights as the large-batch kernel.  Per token the result
// is the decode layer's: out_t = BF16(sum_k w_tk E_idx(xn_t) + E_shared(xn_t)),
// with the same rounding points (g, u, SiLU(g), SiLU(g)*u, the output).
// Grouping tokens by expert only changes the fp32 summation order.
//
// Stages (one kernel each):
//   norm      xn = BF16(BF16(x * rsqrt(mean x^2 + eps)) * gamma)   (optional)
//   router    logits[T][E] = xn . W_r^T, BF16 MFMA with fp32 accumulation
//   topk      per token: top-k by descending logit (ties: lower index),
//             sigmoid weights; per 64-token chunk a token bitmask per expert
//   scan      per-expert counts -> offsets; per (chunk, expert) bases;
//             the tile list (group, first row) of the grouped GEMMs
//   scatter   stable permutation of (token, slot) pairs by (expert, token)
//   gate_up   grouped GEMM per expert (shared expert = last group, all
//             tokens): rows gathered from xn, NVFP4 weight tiles decoded
//             into LDS as exact BF16, MFMA, then SiLU(g) * u -> h (BF16);
//             all column tiles of a row tile on one XCD (its L2 serves
//             the gathered rows)
//   down      grouped GEMM h . W_d^T -> y (fp32, tensor scale applied)
//   combine   out_t = BF16(sum_k w_tk y[pos(t,k)] + y[shared row of t])
//             (+ residual)
#include "common.hpp"
#include "prefill_ws.hpp"

namespace flint {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_STRIDE = BK + 8;        // bf16 per LDS row (16 B of padding)
constexpr int CHUNK = 64;                 // tokens per top-k / scatter chunk

// ---------------------------------------------------------- tile loaders --

// A tile: BM rows x BK columns of BF16, one row pointer per tile row.  256
// threads, 8 per row (16 B each), 4 passes of 32 rows.
struct ARegs { uint4 v[4]; };
struct Rows { const uint16_t* p[4]; };   // source row of each of this thread's 4 segments

__device__ __forceinline__ void load_a(ARegs& r, const Rows& rows, int k0) {
  const int seg = threadIdx.x & 7;
  r.v[0] = *reinterpret_cast<const uint4*>(rows.p[0] + k0 + seg * 8);
  r.v[1] = *reinterpret_cast<const uint4*>(rows.p[1] + k0 + seg * 8);
  r.v[2] = *reinterpret_cast<const uint4*>(rows.p[2] + k0 + seg * 8);
  r.v[3] = *reinterpret_cast<const uint4*>(rows.p[3] + k0 + seg * 8);
}
__device__ __forceinline__ void store_a(const ARegs& r, uint16_t* lds) {
  const int t = threadIdx.x, seg = t & 7;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int row = p * 32 + (t >> 3);
    *reinterpret_cast<uint4*>(lds + row * LDS_STRIDE + seg * 8) = r.v[p];
  }
}

// B tile from NVFP4: BN weight rows x BK columns; two threads per row, each
// 32 codes (16 B) and their two scale bytes, decoded to exact BF16
// (E2M1 x UE4M3 has at most 6 significant bits).
struct BRegsNv { uint4 c; uint32_t s; };

__device__ __forceinline__ void load_b_nv(BRegsNv& r, const uint8_t* codes_row, const uint8_t* scales_row,
                                          int k0) {
  const int half = threadIdx.x & 1;
  r.c = *reinterpret_cast<const uint4*>(codes_row + k0 / 2 + half * 16);
  r.s = *reinterpret_cast<const uint16_t*>(scales_row + k0 / 16 + half * 2);
}
__device__ __forceinline__ void store_b_nv(const BRegsNv& r, uint16_t* lds) {
  const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
  // two codes -> two exact fp32 values, times the UE4M3 scale of their 16
  // columns (exact: at most 6 significant bits), packed to BF16 with round to
  // nearest even (exact as well)
  const float s0 = e4m3_to_f32<0>(r.s), s1 = e4m3_to_f32<1>(r.s);
  const uint32_t q[4] = {r.c.x, r.c.y, r.c.z, r.c.w};
  uint32_t o[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float s = i < 2 ? s0 : s1;               // columns 0..15, then 16..31
    const f32x2_t f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[i], 1.0f, 0);
    const f32x2_t f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[i], 1.0f, 1);
    const f32x2_t f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[i], 1.0f, 2);
    const f32x2_t f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[i], 1.0f, 3);
    o[4 * i + 0] = pack_bf16x2_rne(f0.x * s, f0.y * s);
    o[4 * i + 1] = pack_bf16x2_rne(f1.x * s, f1.y * s);
    o[4 * i + 2] = pack_bf16x2_rne(f2.x * s, f2.y * s);
    o[4 * i + 3] = pack_bf16x2_rne(f3.x * s, f3.y * s);
  }
  uint4* dst = reinterpret_cast<uint4*>(lds + row * LDS_STRIDE + half * 32);
  dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
  dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
  dst[2] = make_uint4(o[8], o[9], o[10], o[11]);
  dst[3] = make_uint4(o[12], o[13], o[14], o[15]);
}

// B tile from BF16 weights (router; W16A16): same pattern as the A tile.
__device__ __forceinline__ void load_b_bf(ARegs& r, const Rows& rows, int k0) { load_a(r, rows, k0); }

// ------------------------------------------------------------- MFMA core --
// 4 waves in 2 x 2; wave (wm, wn) owns rows 64wm..64wm+63 and columns
// 64wn..64wn+63 of the tile as 2 x 2 MFMA 32x32x16 blocks.  Operand layout
// (measured on gfx950): A lane l holds A[l%32][8(l/32) .. +7], B lane l holds
// B[8(l/32) .. +7][l%32]; result element i of lane l is C[8(i/4) + 4(l/32) +
// i%4][l%32].
struct Acc { f32x16 c[2][2]; };

__device__ __forceinline__ void mfma_tile(Acc& acc, const uint16_t* la, const uint16_t* lb) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    bf16x8_t a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 64 * wm + 32 * i + (lane & 31);
      a[i] = *reinterpret_cast<const bf16x8_t*>(la + row * LDS_STRIDE + kk * 16 + 8 * (lane >> 5));
      const int col = 64 * wn + 32 * i + (lane & 31);
      b[i] = *reinterpret_cast<const bf16x8_t*>(lb + col * LDS_STRIDE + kk * 16 + 8 * (lane >> 5));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc.c[i][j], 0, 0, 0);
  }
}

__device__ __forceinline__ void acc_zero(Acc& acc) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc.c[i][j][e] = 0.f;
}

// tile-local (row, col) of result element e of block (i, j) for this lane
__device__ __forceinline__ int acc_row(int i, int e) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  return 64 * (wave >> 1) + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}
__device__ __forceinline__ int acc_col(int j) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  return 64 * (wave & 1) + 32 * j + (lane & 31);
}

// ------------------------------------------------------------- K loop ---
// Software pipeline: a ring of kStages register sets, the loads of step
// kt + kStages issued at step kt, so a load has kStages - 1 MFMA steps to
// arrive; LDS is double-buffered (the tile of step kt + 1 is stored while
// step kt is multiplied).  Every load is unconditional (rows and steps past
// the end are clamped to valid ones), so each store waits for its own set.
constexpr int kStages = 4;

// Register ring of one GEMM's operands: A rows of BF16, B rows of NVFP4
// (WF = FMT_NVFP4) or of BF16.
template <int WF>
struct TileRing {
  Rows arow, bbf;
  const uint8_t* bcodes;
  const uint8_t* bscales;
  ARegs ra[kStages];
  ARegs rbb[kStages];
  BRegsNv rbn[kStages];
  template <int S>
  __device__ __forceinline__ void load(int k0) {
    load_a(ra[S], arow, k0);
    if constexpr (WF == FMT_NVFP4) load_b_nv(rbn[S], bcodes, bscales, k0);
    else load_b_bf(rbb[S], bbf, k0);
  }
  template <int S>
  __device__ __forceinline__ void store(uint16_t* la, uint16_t* lb) {
    store_a(ra[S], la);
    if constexpr (WF == FMT_NVFP4) store_b_nv(rbn[S], lb);
    else store_a(rbb[S], lb);
  }
};

template <int U, int WF>
__device__ __forceinline__ void k_step(Acc& acc, uint16_t (&la)[2][BM * LDS_STRIDE],
                                       uint16_t (&lb)[2][BN * LDS_STRIDE], TileRing<WF>& ring, int kt,
                                       int nk) {
  if (kt < nk) mfma_tile(acc, la[U & 1], lb[U & 1]);            // same in every lane
  ring.template store<(U + 1) % kStages>(la[(U + 1) & 1], lb[(U + 1) & 1]);
  const int kl = kt + kStages < nk ? kt + kStages : nk - 1;
  ring.template load<U>(kl * BK);
  __syncthreads();
}

template <int WF>
__device__ __forceinline__ void gemm_k_loop(Acc& acc, uint16_t (&la)[2][BM * LDS_STRIDE],
                                            uint16_t (&lb)[2][BN * LDS_STRIDE], TileRing<WF>& ring, int nk) {
  static_assert(kStages == 4, "the ring is unrolled for four stages");
  ring.template load<0>(0);
  ring.template load<1>((1 < nk ? 1 : nk - 1) * BK);
  ring.template load<2>((2 < nk ? 2 : nk - 1) * BK);
  ring.template load<3>((3 < nk ? 3 : nk - 1) * BK);
  ring.template store<0>(la[0], lb[0]);
  __syncthreads();
  for (int kt0 = 0; kt0 < nk; kt0 += kStages) {
    k_step<0>(acc, la, lb, ring, kt0 + 0, nk);
    k_step<1>(acc, la, lb, ring, kt0 + 1, nk);
    k_step<2>(acc, la, lb, ring, kt0 + 2, nk);
    k_step<3>(acc, la, lb, ring, kt0 + 3, nk);
  }
}

// --------------------------------------------------- XCD-aware tile order --
// Workgroup i of a launch runs on XCD i mod 8, and each XCD has its own L2.
// The grouped GEMMs take a 1-D grid in which workgroup i computes row tile
// 8 (i / 8 / ntn) + i mod 8 and column tile (i / 8) mod ntn: all column
// tiles of a row tile run on one XCD, one after the other, so its gathered
// A rows are fetched from memory once per XCD and then served from that
// L2, instead of being fetched by every column tile on all eight XCDs.
struct TileIdx { int m, n; };
__device__ __forceinline__ TileIdx tile_of_block(int ntn) {
  const int id = blockIdx.x, xcd = id & 7, slot = id >> 3;
  const int mg = slot / ntn;
  return TileIdx{mg * 8 + xcd, slot - mg * ntn};
}
inline unsigned grouped_grid(int max_tiles, int ntn) { return (unsigned)(((max_tiles + 7) / 8) * 8 * ntn); }
// The same with runs of FG consecutive M tiles per XCD, N-major inside a
// run: N tile n of tiles FG q .. FG q + FG - 1 (mostly one expert's) runs
// back to back on one XCD, so its weight rows come from that XCD's L2 after
// the first tile, as the run's A rows do for the other N tiles.  (The
// gate/up GEMM gains from it; the down GEMM, with 8 N tiles and a quarter of
// the weights per tile, does not and keeps the plain mapping.)
constexpr int FG = 4;
__device__ __forceinline__ TileIdx tile_of_block_runs(int ntn) {
  const int id = blockIdx.x, xcd = id & 7, slot = id >> 3;
  const int lg = slot / (FG * ntn), w = slot - lg * (FG * ntn);
  return TileIdx{(lg * 8 + xcd) * FG + w % FG, w / FG};
}
inline unsigned grouped_grid_runs(int max_tiles, int ntn) {
  return (unsigned)(((max_tiles + 8 * FG - 1) / (8 * FG)) * 8 * FG * ntn);
}

// ---------------------------------------------------------- workspaces ----
}  // namespace



int prefill_max_tiles(const flint_moe_shape& s, int T) {
  const int pairs = T * s.top_k;
  return (pairs + BM - 1) / BM + s.n_experts + (s.shared_inter > 0 ? (T + BM - 1) / BM + 1 : 0);
}

PrefillWs carve_prefill_ws(void* base, const flint_moe_shape& s, int T) {
  auto up = [](int64_t v) { return (v + 255) / 256 * 256; };
  const int E = s.n_experts, K = s.top_k, H = s.hidden;
  const int C = (T + CHUNK - 1) / CHUNK;
  const int imax = s.inter > s.shared_inter ? s.inter : s.shared_inter;
  const int64_t rows = (int64_t)T * K + (s.shared_inter > 0 ? T : 0);
  char* b = static_cast<char*>(base);
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    char* p = b ? b + off : nullptr;
    off = up(off + bytes);
    return p;
  };
  PrefillWs w;
  w.max_tiles = prefill_max_tiles(s, T);
  w.xn = reinterpret_cast<uint16_t*>(take((int64_t)T * H * 2));
  w.logits = reinterpret_cast<float*>(take((int64_t)T * E * 4));
  w.idx = reinterpret_cast<int32_t*>(take((int64_t)T * K * 4));
  w.wgt = reinterpret_cast<float*>(take((int64_t)T * K * 4));
  w.cmask = reinterpret_cast<uint64_t*>(take((int64_t)C * E * 8));
  w.cbase = reinterpret_cast<int32_t*>(take((int64_t)C * E * 4));
  w.counts = reinterpret_cast<int32_t*>(take((int64_t)(E + 1) * 4));
  w.offsets = reinterpret_cast<int32_t*>(take((int64_t)(E + 2) * 4));
  w.ntiles = reinterpret_cast<int32_t*>(take(4));
  w.tiles = reinterpret_cast<int2*>(take((int64_t)w.max_tiles * 8));
  w.perm_tok = reinterpret_cast<int32_t*>(take((int64_t)T * K * 4));
  w.perm_w = reinterpret_cast<float*>(take((int64_t)T * K * 4));
  w.pos = reinterpret_cast<int32_t*>(take((int64_t)T * K * 4));
  w.h = reinterpret_cast<uint16_t*>(take(rows * imax * 2));
  w.y = reinterpret_cast<float*>(take(rows * H * 4));
  w.router_f = (H == 2048 && E == 256) ? reinterpret_cast<uint16_t*>(take((int64_t)E * H * 2)) : nullptr;
  w.bytes = off;
  return w;
}

namespace {

// ------------------------------------------------------------------ norm --
// One wave per token; the mean of squares, its square root and x / rms are
// taken in float64, x / rms is rounded to BF16 once from float64.
__global__ __launch_bounds__(256) void prefill_norm_kernel(LayerArgs a, PrefillWs ws, int T) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const int H = a.H;
  const uint16_t* xr = a.x + (size_t)t * H;
  double ss = 0.0;
  for (int c = 8 * lane; c < H; c += 512) {
    const uint4 v = *reinterpret_cast<const uint4*>(xr + c);
    const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const double lo = bf16_lo(q[m]), hi = bf16_hi(q[m]);
      ss = fma(lo, lo, ss);
      ss = fma(hi, hi, ss);
    }
  }
  ss = wave_sum_f64(ss);
  const Rms rms = make_rms(sqrt(ss / (double)H + (double)a.eps));
  for (int c = 8 * lane; c < H; c += 512) {
    const uint4 v = *reinterpret_cast<const uint4*>(xr + c);
    const uint4 g = *reinterpret_cast<const uint4*>(a.gamma + c);
    *reinterpret_cast<uint4*>(ws.xn + (size_t)t * H + c) = rms_norm_8(v, g, rms);
  }
}

// ---------------------------------------------------------------- router --
// logits[T][E] = xn . W_r^T.  Grid (token tiles, expert tiles).
__global__ __launch_bounds__(256) void prefill_router_kernel(LayerArgs a, PrefillWs ws, int T,
                                                             const uint16_t* xin) {
  __shared__ uint16_t la[2][BM * LDS_STRIDE];
  __shared__ uint16_t lb[2][BN * LDS_STRIDE];
  const int H = a.H, E = a.E;
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
  const int t = threadIdx.x;
  TileRing<FMT_BF16> ring;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = p * 32 + (t >> 3);
    const int tok = m0 + r < T ? m0 + r : T - 1;
    ring.arow.p[p] = xin + (size_t)tok * H;
    const int e = n0 + r < E ? n0 + r : E - 1;
    ring.bbf.p[p] = a.router + (size_t)e * H;
  }
  Acc acc;
  acc_zero(acc);
  gemm_k_loop(acc, la, lb, ring, H / BK);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = m0 + acc_row(i, e), c = n0 + acc_col(j);
        if (r < T && c < E) ws.logits[(size_t)r * E + c] = acc.c[i][j][e];
      }
}

// Router at hidden 2048 (expert count a multiple of 128).  Tile: 64 tokens x
// 128 experts, 4 waves; wave w owns experts 32 w .. 32 w + 31 of the tile for
// all 64 tokens (two 32x32 blocks of MFMA 32x32x16).  K chunks of 512, the
// next chunk's loads issued before the current chunk's 64 MFMAs per wave:
//   A  the token rows go straight into LDS (global_load_lds), two stages of
//      64 rows x 1 KB; 16-byte segment g of tile row r sits at slot
//      g ^ (r & 31), so a wave's operand reads of 32 rows hit 32 slots;
//   B  the router rows go straight into registers: for MFMA s of a chunk,
//      lane (h, n) holds the 8 values at k = 16 s + 8 h .. + 7 of expert row
//      n, so the two lanes of a row read 32 contiguous bytes per load, and A
//      is read in the same k order.
// The router weights (1 MB) stay in L2; every workgroup reads a quarter of
// them, against 64 token rows.
constexpr int RTM = 64, RTN = 128, RKC = 512, RH = 2048;

struct RtB { uint4 v[RKC / 16]; };

__global__ __launch_bounds__(256, 1) void prefill_router_f_kernel(LayerArgs a, PrefillWs ws, int T,
                                                               const uint16_t* xin) {
  __shared__ __attribute__((aligned(16))) uint8_t s_x[2][RTM * RKC * 2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5, n = lane & 31;
  const int E = a.E;
  const int m0 = blockIdx.x * RTM, e = blockIdx.y * RTN + 32 * wave + n;
  // copy i of wave w fills tile row 16 w + i, slot `lane` <- segment lane ^ (row & 31)
  uint32_t off[RTM / 4];
#pragma unroll
  for (int i = 0; i < RTM / 4; ++i) {
    const int r = 16 * wave + i;
    const int tok = m0 + r < T ? m0 + r : T - 1;
    off[i] = 2u * ((uint32_t)tok * RH + 8u * (uint32_t)(lane ^ (r & 31)));
  }
  const uint8_t* x_base = reinterpret_cast<const uint8_t*>(xin);
  auto copy_x = [&](int c, int buf) {
    uint64_t sb = reinterpret_cast<uint64_t>(x_base + (size_t)c * RKC * 2);
    asm volatile("" : "+s"(sb));             // keep the base scalar (offsets stay 32-bit)
    const uint8_t* src = reinterpret_cast<const uint8_t*>(sb);
#pragma unroll
    for (int i = 0; i < RTM / 4; ++i)
      __builtin_amdgcn_global_load_lds(src + (uint64_t)off[i], &s_x[buf][(16 * wave + i) * 1024], 16, 0, 0);
  };
  const uint16_t* wrow = a.router + (size_t)e * RH + 8 * h;
  auto load_b = [&](RtB& b, int c) {
#pragma unroll
    for (int s = 0; s < RKC / 16; ++s) b.v[s] = ldg<uint4>(wrow + c * RKC + 16 * s);
  };
  f32x16 acc[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
  auto step = [&](int c, const RtB& cur, RtB& nxt, int buf) {
    // everything of chunk c (issued one chunk earlier) has landed; no wave
    // still reads the stage chunk c + 1 overwrites
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (c + 1 < RH / RKC) {
      copy_x(c + 1, buf ^ 1);
      load_b(nxt, c + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* la = s_x[buf];
#pragma unroll
    for (int s = 0; s < RKC / 16; ++s) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int r = 32 * mb + n;
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(la + r * 1024 + 16 * ((2 * s + h) ^ (r & 31)));
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8_t, cur.v[s]), acc[mb], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  RtB b0, b1;
  load_b(b0, 0);
  copy_x(0, 0);
  static_assert((RH / RKC) % 2 == 0, "chunks go in pairs");
#pragma unroll 1
  for (int c = 0; c < RH / RKC; c += 2) {
    step(c, b0, b1, 0);
    step(c + 1, b1, b0, 1);
  }
  // element i of block mb: token 32 mb + 8 (i / 4) + 4 h + i % 4, expert e
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = m0 + 32 * mb + 8 * (i >> 2) + 4 * h + (i & 3);
      if (t < T) ws.logits[(size_t)t * E + e] = acc[mb][i];
    }
}

// ------------------------------------------------------------------ topk --
// The selection of one half chunk (32 tokens) by 8 waves, 4 tokens per wave.
// A round of a token takes the wave maximum of the 32-bit order keys and
// finds the lowest expert that holds it with ballots (lane l holds experts
// l + 64 q, so q = 0 is searched first, then the lowest lane), then removes
// that key.  Key 0 (below every order key) marks an expert past E or already
// taken.  The TPW tokens of a wave take their K rounds together (independent
// chains of wave reductions, so their latencies overlap).  Lane k ends with
// selection k of each token: its order key and its expert.
constexpr int HT = CHUNK / 2, TPW = HT / 8;
__device__ __forceinline__ void select_topk(uint32_t (&key)[TPW][4], int K, uint32_t (&my_m)[TPW],
                                            int (&my_e)[TPW], int lane) {
#pragma unroll
  for (int u = 0; u < TPW; ++u) { my_m[u] = 0u; my_e[u] = 0; }
  for (int k = 0; k < K; ++k) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const uint32_t m = wave_max_u32(max(max(key[u][0], key[u][1]), max(key[u][2], key[u][3])));
      int win = -1;                                // workgroup-uniform
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (win < 0) {
          const unsigned long long b = __ballot(key[u][q] == m);
          if (b != 0ull) {
            const int w = __ffsll((long long)b) - 1;
            win = w + 64 * q;
            if (lane == w) key[u][q] = 0u;
          }
        }
      }
      if (lane == k) { my_m[u] = m; my_e[u] = win; }
    }
  }
}

// Writes the selections of the wave's tokens (token t0 + 4 wave + u): each
// selection's sigmoid once (lane k), summed in selection order for the
// renormalised weights; and sets bit j of the token in its experts' half
// chunk masks in LDS.
__device__ __forceinline__ void emit_topk(const LayerArgs& a, int T, int t0, int wave, int lane,
                                          const uint32_t (&my_m)[TPW], const int (&my_e)[TPW], uint32_t* s_mask) {
  const int K = a.K;
  const bool renorm = (a.flags & FLINT_RENORM) != 0;
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int j = wave * TPW + u;
    const int t = t0 + j;
    const float sg = 1.0f / (1.0f + expf(-float_from_order_key(my_m[u])));
    float ssum = 0.f;
    for (int k = 0; k < K; ++k) ssum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sg), k));
    if (t < T && lane < K) {
      a.topk_idx[(size_t)t * K + lane] = my_e[u];
      a.topk_w[(size_t)t * K + lane] = renorm ? sg / ssum : sg;
      atomicOr(&s_mask[my_e[u]], 1u << j);
    }
  }
}

// The half chunk's token bitmask per expert: its own 32-bit half of the
// chunk's 64-bit mask, so no two workgroups write the same word, and the
// half's count beside it (little-endian: half h of word w is subword 2 w + h).
__device__ __forceinline__ void write_half_masks(const PrefillWs& ws, int E, int c, int half, const uint32_t* s_mask) {
  if (threadIdx.x < E) {
    const uint32_t m = s_mask[threadIdx.x];
    const size_t w = (size_t)c * E + threadIdx.x;
    reinterpret_cast<uint32_t*>(ws.cmask)[2 * w + half] = m;
    reinterpret_cast<uint16_t*>(ws.cbase)[2 * w + half] = (uint16_t)__popc(m);
  }
}

// One workgroup per half chunk, all its logits fetched before the selection.
__global__ __launch_bounds__(512) void prefill_topk_kernel(LayerArgs a, PrefillWs ws, int T) {
  __shared__ uint32_t s_mask[FLINT_MAX_EXPERTS];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int E = a.E;
  const int c = blockIdx.x >> 1, half = blockIdx.x & 1;
  const int t0 = c * CHUNK + half * HT;
  if (threadIdx.x < FLINT_MAX_EXPERTS) s_mask[threadIdx.x] = 0u;
  __syncthreads();
  uint32_t key[TPW][4];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int t = t0 + wave * TPW + u;
    const int tt = t < T ? t : T - 1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ex = lane + 64 * q;
      key[u][q] = ex < E ? float_order_key(ws.logits[(size_t)tt * E + ex]) : 0u;
    }
  }
  uint32_t my_m[TPW];
  int my_e[TPW];
  select_topk(key, a.K, my_m, my_e, lane);
  emit_topk(a, T, t0, wave, lane, my_m, my_e, s_mask);
  __syncthreads();
  write_half_masks(ws, E, c, half, s_mask);
}

// ------------------------------------------------- router + top-k, fused --
// At hidden 2048 and 256 experts, one workgroup of 8 waves per half chunk
// (32 tokens) computes all 256 logits of its tokens and selects their top-k,
// so the logits never go to memory.  Wave w computes experts 32 w .. + 31
// for the 32 tokens: one MFMA 32x32x16 block over K = 2048, with the same
// operand layout and k order as prefill_router_f_kernel (identical logits).
//   A  the 32 token rows (128 KB) are copied straight into LDS
//      (global_load_lds), in 4 groups of 512 columns; slot p of row r holds
//      the row's 16-byte segment p ^ (r & 31), so the 32 rows that one A
//      read touches spread over the banks.  The first group goes out with
//      the first router chunk, the other three with the second.
//   B  the router rows stream from L2 straight into registers in chunks of
//      256 columns, one chunk ahead, from a copy in fragment order
//      (prefill_router_frag_kernel): each load instruction reads 1 KB in one
//      piece.  Read from the row-major router, the 32 rows of a load are
//      4 KB apart, and the kernel took 45 us at 8,192 tokens.
// Each token's x row is read from memory once (the two-kernel path reads it
// once per expert tile), and the router (1 MB) once per workgroup from L2.
constexpr int RFK = 256;
struct RfB { uint4 v[RFK / 16]; };

// The router in fragment order: 1 KB piece f = 8 (16 ck + s) + w holds, at
// lane (h, n), row 32 w + n, columns 256 ck + 16 s + 8 h .. + 7.  One thread
// per 16 bytes, E H / 8 of them.
__global__ __launch_bounds__(256) void prefill_router_frag_kernel(const uint16_t* router, uint16_t* out) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  const int lane = p & 63, f = p >> 6;
  const int w = f & 7, s = (f >> 3) & 15, ck = f >> 7;
  const int h = lane >> 5, n = lane & 31;
  const uint4 v = ldg<uint4>(router + (size_t)(32 * w + n) * RH + RFK * ck + 16 * s + 8 * h);
  *reinterpret_cast<uint4*>(out + (size_t)p * 8) = v;
}

__global__ __launch_bounds__(512, 1) void prefill_route_f_kernel(LayerArgs a, PrefillWs ws, int T,
                                                              const uint16_t* xin) {
  __shared__ __attribute__((aligned(16))) uint8_t s_x[HT * RH * 2];
  __shared__ uint32_t s_mask[FLINT_MAX_EXPERTS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5, n = lane & 31;
  const int c = blockIdx.x >> 1, half = blockIdx.x & 1;
  const int t0 = c * CHUNK + half * HT;
  const int e = 32 * wave + n;
  if (threadIdx.x < FLINT_MAX_EXPERTS) s_mask[threadIdx.x] = 0u;
  // copy i of wave w fills row 4 w + i of group g: 1 KB, slot 64 g + lane
  uint32_t off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * wave + i;
    const int tok = t0 + r < T ? t0 + r : T - 1;
    off[i] = 2u * ((uint32_t)tok * RH + 8u * (uint32_t)(lane ^ (r & 31)));
  }
  const uint8_t* x_base = reinterpret_cast<const uint8_t*>(xin);
  auto copy_x = [&](int g) {
    uint64_t sb = reinterpret_cast<uint64_t>(x_base + (size_t)g * 1024);
    asm volatile("" : "+s"(sb));             // keep the base scalar (offsets stay 32-bit)
    const uint8_t* src = reinterpret_cast<const uint8_t*>(sb);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(src + (uint64_t)off[i], &s_x[(4 * wave + i) * (RH * 2) + g * 1024], 16, 0, 0);
  };
  const uint8_t* wfrag = reinterpret_cast<const uint8_t*>(ws.router_f) + 1024 * wave + 16 * lane;
  auto load_b = [&](RfB& b, int ck) {
#pragma unroll
    for (int s = 0; s < RFK / 16; ++s) b.v[s] = ldg<uint4>(wfrag + (size_t)(8 * (16 * ck + s)) * 1024);
  };
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  // MFMA s of chunk ck: lane (h, n) takes row n's segment 32 ck + 2 s + h
  auto mfmas = [&](int ck, const RfB& b) {
    const uint8_t* row = s_x + n * (RH * 2);
#pragma unroll
    for (int s = 0; s < RFK / 16; ++s) {
      const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(row + 16 * ((32 * ck + 2 * s + h) ^ n));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8_t, b.v[s]), acc, 0, 0, 0);
    }
  };
  RfB b0, b1;
  copy_x(0);
  load_b(b0, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();                                 // x group 0 and the masks' zeros visible
  // Chunk 0's A fragments are read before the other groups' copies go out:
  // an LDS read issued behind a pending copy into LDS waits for the copy.
  bf16x8_t a0[RFK / 16];
  {
    const uint8_t* row = s_x + n * (RH * 2);
#pragma unroll
    for (int s = 0; s < RFK / 16; ++s) a0[s] = *reinterpret_cast<const bf16x8_t*>(row + 16 * ((2 * s + h) ^ n));
  }
  __builtin_amdgcn_sched_barrier(0);
  copy_x(1);
  copy_x(2);
  copy_x(3);
  load_b(b1, 1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < RFK / 16; ++s)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[s], __builtin_bit_cast(bf16x8_t, b0.v[s]), acc, 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __builtin_amdgcn_s_barrier();                    // every group of x in LDS
  __builtin_amdgcn_sched_barrier(0);
  static_assert(RH / RFK == 8, "eight router chunks");
#pragma unroll
  for (int ck = 1; ck < RH / RFK - 1; ck += 2) {   // chunks 1 .. 6 in pairs; b1 holds chunk ck
    load_b(b0, ck + 1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(ck, b1);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    load_b(b1, ck + 2);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(ck + 1, b0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }
  mfmas(RH / RFK - 1, b1);
  // the logits, [32 tokens][256 experts] fp32, over the x rows
  __syncthreads();                                 // every wave is done with x
  float* s_l = reinterpret_cast<float*>(s_x);
  // element i: token 8 (i / 4) + 4 h + i % 4, expert e
#pragma unroll
  for (int i = 0; i < 16; ++i) s_l[(8 * (i >> 2) + 4 * h + (i & 3)) * 256 + e] = acc[i];
  __syncthreads();
  uint32_t key[TPW][4];
#pragma unroll
  for (int u = 0; u < TPW; ++u)
#pragma unroll
    for (int q = 0; q < 4; ++q) key[u][q] = float_order_key(s_l[(wave * TPW + u) * 256 + lane + 64 * q]);
  uint32_t my_m[TPW];
  int my_e[TPW];
  select_topk(key, a.K, my_m, my_e, lane);
  emit_topk(a, T, t0, wave, lane, my_m, my_e, s_mask);
  __syncthreads();
  write_half_masks(ws, a.E, c, half, s_mask);
}

// ------------------------------------------------------------------ scan --
// One workgroup of 1024 threads: thread (part, e) sums the counts of expert e
// over its quarter of the chunks (all loads of a pass in flight together),
// the parts and then the experts are scanned through LDS and wave prefix
// sums, and a second pass writes every chunk's base over its count (the two
// 16-bit half-chunk counts the top-k kernel left in cbase).  Then the tile
// list.
__global__ __launch_bounds__(1024) void prefill_scan_kernel(LayerArgs a, PrefillWs ws, int T) {
  constexpr int NB = 32;                           // chunk loads per thread per batch
  __shared__ int s_cnt[4][FLINT_MAX_EXPERTS];
  __shared__ int s_part[4];
  const int E = a.E, C = (T + CHUNK - 1) / CHUNK;
  const int e = threadIdx.x & 255, part = threadIdx.x >> 8;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool has_sh = a.SI > 0;
  const int cpp = (C + 3) / 4, c_lo = part * cpp, c_hi = min(C, c_lo + cpp);
  int cnt = 0;
  if (e < E) {
    for (int c0 = c_lo; c0 < c_hi; c0 += NB) {
      int cw[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) cw[u] = ws.cbase[(size_t)(c0 + u < c_hi ? c0 + u : c_lo) * E + e];
#pragma unroll
      for (int u = 0; u < NB; ++u) cnt += c0 + u < c_hi ? (cw[u] & 0xffff) + (cw[u] >> 16) : 0;
    }
  }
  s_cnt[part][e] = cnt;
  __syncthreads();
  // expert totals and the exclusive scan over experts (first 256 threads)
  int total_e = 0, before_part = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int v = s_cnt[q][e];
    if (q < part) before_part += v;
    total_e += v;
  }
  if (e >= E) total_e = 0;
  int incl = total_e;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (part == 0 && lane == 63) s_part[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < (wave & 3); ++w) before += s_part[w];
  const int offset = before + incl - total_e;     // expert e's first permuted position
  const int total = s_part[0] + s_part[1] + s_part[2] + s_part[3];
  if (e < E) {
    if (part == 0) {
      ws.counts[e] = total_e;
      ws.offsets[e] = offset;
    }
    int run = offset + before_part;
    for (int c0 = c_lo; c0 < c_hi; c0 += NB) {
      int cw[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) cw[u] = ws.cbase[(size_t)(c0 + u < c_hi ? c0 + u : c_lo) * E + e];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        if (c0 + u < c_hi) {
          ws.cbase[(size_t)(c0 + u) * E + e] = run;
          run += (cw[u] & 0xffff) + (cw[u] >> 16);
        }
      }
    }
  }
  if (threadIdx.x == 0) {
    ws.offsets[E] = total;
    ws.counts[E] = has_sh ? T : 0;
  }
  // tile list: routed groups in expert order, then the shared group
  const int nt = (part == 0 && e < E) ? (total_e + BM - 1) / BM : 0;
  int tincl = nt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(tincl, off, 64);
    if (lane >= off) tincl += v;
  }
  __syncthreads();
  if (part == 0 && lane == 63) s_part[wave] = tincl;
  __syncthreads();
  int tbefore = 0;
  for (int w = 0; w < (wave & 3); ++w) tbefore += s_part[w];
  const int tfirst = tbefore + tincl - nt;
  for (int i = 0; i < nt; ++i) ws.tiles[tfirst + i] = make_int2(e, i * BM);
  const int routed_tiles = s_part[0] + s_part[1] + s_part[2] + s_part[3];
  const int sh_tiles = has_sh ? (T + BM - 1) / BM : 0;
  for (int i = threadIdx.x; i < sh_tiles; i += 1024) ws.tiles[routed_tiles + i] = make_int2(E, i * BM);
  if (threadIdx.x == 0) *ws.ntiles = routed_tiles + sh_tiles;
}

// --------------------------------------------------------------- scatter --
// Permuted position of pair (t, k) with expert e: the expert's offset, plus
// the pairs of e in earlier chunks, plus the earlier tokens of this chunk
// routed to e.  Stable by (expert, token).
__global__ __launch_bounds__(256) void prefill_scatter_kernel(LayerArgs a, PrefillWs ws, int T) {
  const int E = a.E, K = a.K;
  const int c = blockIdx.x;
  for (int q = threadIdx.x; q < CHUNK * K; q += 256) {
    const int j = q / K, k = q - j * K;
    const int t = c * CHUNK + j;
    if (t >= T) continue;
    const int e = a.topk_idx[(size_t)t * K + k];
    const uint64_t before = ws.cmask[(size_t)c * E + e] & ((1ull << j) - 1ull);
    const int p = ws.cbase[(size_t)c * E + e] + __popcll(before);
    ws.perm_tok[p] = t;
    ws.perm_w[p] = a.topk_w[(size_t)t * K + k];
    ws.pos[(size_t)t * K + k] = p;
  }
}

// --------------------------------------------------------------- gate/up --
// Grouped GEMM, grid (tiles, column tiles).  A tile rows are the tile's
// tokens (gathered xn rows); the B tile interleaves gate and up rows
// (tile row 2i = gate row i0+i, 2i+1 = up row i0+i), so the result columns
// alternate g and u and each lane's partner lane (lane ^ 1) holds the other
// half of its pair.
template <int WF>
__global__ __launch_bounds__(256) void prefill_gate_up_kernel(LayerArgs a, PrefillWs ws, int T,
                                                              const uint16_t* xin) {
  __shared__ uint16_t la[2][BM * LDS_STRIDE];
  __shared__ uint16_t lb[2][BN * LDS_STRIDE];
  const int imax0 = a.I > a.SI ? a.I : a.SI;
  const TileIdx ti = tile_of_block((imax0 + BN / 2 - 1) / (BN / 2));
  if (ti.m >= *ws.ntiles) return;
  const int2 tile = ws.tiles[ti.m];
  const int g = tile.x, m0 = tile.y;
  const int E = a.E, K = a.K, H = a.H;
  const bool shared = g == E;
  const int inter = shared ? a.SI : a.I;
  const int i0 = ti.n * (BN / 2);
  if (i0 >= inter) return;
  const int cnt = shared ? T : ws.counts[g];
  const int base = shared ? 0 : ws.offsets[g];
  const int imax = a.I > a.SI ? a.I : a.SI;
  const int t = threadIdx.x;

  TileRing<WF> ring;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = m0 + p * 32 + (t >> 3);
    const int rr = r < cnt ? r : cnt - 1;
    const int tok = shared ? rr : ws.perm_tok[base + rr];
    ring.arow.p[p] = xin + (size_t)tok * H;
  }
  // this thread's B row: tile row t/2 (NVFP4: two threads per row)
  const int brow_t = t >> 1;
  const int bi = i0 + (brow_t >> 1), bup = brow_t & 1;
  const int bic = bi < inter ? bi : inter - 1;
  ring.bcodes = nullptr;
  ring.bscales = nullptr;
  float gs_g = 1.f, gs_u = 1.f;
  if constexpr (WF == FMT_NVFP4) {
    const size_t mc = (size_t)inter * H / 2, ms = (size_t)inter * H / 16;
    const uint8_t* c0 = shared ? a.sh_gu_codes : a.gu_codes + (size_t)(2 * g) * mc;
    const uint8_t* s0 = shared ? a.sh_gu_scales : a.gu_scales + (size_t)(2 * g) * ms;
    ring.bcodes = c0 + bup * mc + (size_t)bic * (H / 2);
    ring.bscales = s0 + bup * ms + (size_t)bic * (H / 16);
    const float* gsp = shared ? a.sh_gscale : a.gscale + 3 * g;
    gs_g = gsp[0];
    gs_u = gsp[1];
  } else {
    const size_t mb = (size_t)inter * H;
    const uint16_t* w0 = shared ? a.sh_gu_bf16 : a.gu_bf16 + (size_t)(2 * g) * mb;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = p * 32 + (t >> 3);           // tile row of this thread's 16-B segment
      const int ii = i0 + (r >> 1);
      const int iic = ii < inter ? ii : inter - 1;
      ring.bbf.p[p] = w0 + (r & 1) * mb + (size_t)iic * H;
    }
  }

  Acc acc;
  acc_zero(acc);
  gemm_k_loop(acc, la, lb, ring, H / BK);
  // Even columns hold gate rows, odd columns the matching up rows, in
  // neighbouring lanes.  The lanes of a pair swap half of their results, so
  // that the even lane finishes the elements of block row 0 and the odd lane
  // those of block row 1: every lane does useful epilogue work.
  const int lane = threadIdx.x & 63;
  const bool even = (lane & 1) == 0;
  const int ih = even ? 0 : 1;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float a0 = acc.c[0][j][e], a1 = acc.c[1][j][e];
      const float recv = dpp_f<0xB1>(even ? a1 : a0);   // partner lane ^ 1
      const float gacc = even ? a0 : recv;
      const float uacc = even ? recv : a1;
      const int r = m0 + acc_row(ih, e);
      const int ii = i0 + (acc_col(j) >> 1);
      if (r < cnt && ii < inter) {
        const float gv = round_bf16(gacc * gs_g);
        const float uv = round_bf16(uacc * gs_u);
        const float av = round_bf16(silu_f32(gv));
        const size_t row = shared ? (size_t)T * K + r : (size_t)base + r;
        ws.h[row * imax + ii] = f32_to_bf16_bits(av * uv);
      }
    }
}

// ------------------------------------------------------------------ down --
// Grouped GEMM h . W_d^T -> y (fp32), grid (tiles, column tiles of H).
template <int WF>
__global__ __launch_bounds__(256) void prefill_down_kernel(LayerArgs a, PrefillWs ws, int T) {
  __shared__ uint16_t la[2][BM * LDS_STRIDE];
  __shared__ uint16_t lb[2][BN * LDS_STRIDE];
  const TileIdx ti = tile_of_block((a.H + BN - 1) / BN);
  if (ti.m >= *ws.ntiles) return;
  const int2 tile = ws.tiles[ti.m];
  const int g = tile.x, m0 = tile.y;
  const int E = a.E, K = a.K, H = a.H;
  const bool shared = g == E;
  const int inter = shared ? a.SI : a.I;
  const int n0 = ti.n * BN;
  const int cnt = shared ? T : ws.counts[g];
  const size_t base = shared ? (size_t)T * K : (size_t)ws.offsets[g];
  const int imax = a.I > a.SI ? a.I : a.SI;
  const int t = threadIdx.x;

  TileRing<WF> ring;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = m0 + p * 32 + (t >> 3);
    const int rr = r < cnt ? r : cnt - 1;
    ring.arow.p[p] = ws.h + (base + rr) * imax;
  }
  const int bn = n0 + (t >> 1);
  const int bnc = bn < H ? bn : H - 1;
  ring.bcodes = nullptr;
  ring.bscales = nullptr;
  float gd = 1.f;
  if constexpr (WF == FMT_NVFP4) {
    const uint8_t* c0 = shared ? a.sh_d_codes : a.d_codes + (size_t)g * H * (inter / 2);
    const uint8_t* s0 = shared ? a.sh_d_scales : a.d_scales + (size_t)g * H * (inter / 16);
    ring.bcodes = c0 + (size_t)bnc * (inter / 2);
    ring.bscales = s0 + (size_t)bnc * (inter / 16);
    gd = shared ? a.sh_gscale[2] : a.gscale[3 * g + 2];
  } else {
    const uint16_t* w0 = shared ? a.sh_d_bf16 : a.d_bf16 + (size_t)g * H * inter;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = n0 + p * 32 + (t >> 3);
      ring.bbf.p[p] = w0 + (size_t)(r < H ? r : H - 1) * inter;
    }
  }
  Acc acc;
  acc_zero(acc);
  gemm_k_loop(acc, la, lb, ring, inter / BK);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = m0 + acc_row(i, e), c = n0 + acc_col(j);
        if (r < cnt && c < H) ws.y[(base + r) * H + c] = acc.c[i][j][e] * gd;
      }
}

// ------------------------------------ Flint-shape NVFP4 grouped GEMMs --
// Hidden 2048, intermediate 512 (routed and shared), NVFP4 weights.  Tile:
// 128 rows (tokens of one group) x 256 output columns, 4 waves; wave w owns
// columns 64 w .. 64 w + 63 of all 128 rows as 4 x 2 blocks of MFMA
// 32x32x16.  K steps of 128:
//   A  the gathered BF16 rows go straight into LDS (global_load_lds: no
//      registers), double-buffered; 16-byte chunk c of tile row r sits at
//      slot c ^ (r & 15), so the operand reads of 16 consecutive rows hit
//      16 different bank groups.  Each lane copies the same 8 (row, chunk)
//      pairs every step: its 32-bit offsets are fixed and only the
//      workgroup-uniform base advances.
//   B  the NVFP4 weights never pass through LDS.  Within a step, MFMA j's
//      k index 8 h + e (lane half h) stands for column 64 h + 8 j + e (the
//      same order for A and B), so lane (h, n) needs 64 consecutive codes
//      (32 bytes) and their 4 scale bytes of weight row n per step: loaded
//      one step ahead into the second of two register buffers, decoded to
//      exact BF16 (E2M1 x UE4M3 has at most 6 significant bits) just before
//      each MFMA.
// A tile's M blocks past its last row get no copies and no MFMAs.
// Each B value is decoded once per 128 rows: 2 VALU per value against 16
// MFMA rows, and LDS carries only A.
constexpr int FBM = 128, FBN = 256, FBK = 128;
constexpr int FH = 2048, FI = 512;

struct FBRaw {
  uint4 c[2][2];     // [N block][first, second 16 bytes of the lane's 32]
  uint32_t s[2];     // [N block] 4 scale bytes
};

template <int NK>
struct FbRows {      // this lane's weight rows (codes, scales) of its two N blocks
  const uint8_t* c[2];
  const uint8_t* s[2];
};

// TL: the weights in the prefill layout, where the lane's pointers already
// hold its place in a 32-row block and a step is one block (2 KB of codes,
// 256 B of scales); else the packed planes, row by row.
template <int NK, bool TL>
__device__ __forceinline__ void fb_load(FBRaw& r, const FbRows<NK>& b, int t, int h) {
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    if constexpr (TL) {
      // the down GEMMs' rows as non-temporal loads (down 163.5 -> 157.3 us;
      // gate/up, whose rows a second M tile re-reads from L2, lost 3 us)
      r.c[nb][0] = NK == FI / FBK ? ldg_nt(b.c[nb] + 2048 * t) : ldg<uint4>(b.c[nb] + 2048 * t);
      r.c[nb][1] = NK == FI / FBK ? ldg_nt(b.c[nb] + 2048 * t + 1024) : ldg<uint4>(b.c[nb] + 2048 * t + 1024);
      r.s[nb] = ldg<uint32_t>(b.s[nb] + 256 * t);
    } else {
      r.c[nb][0] = ldg<uint4>(b.c[nb] + 64 * t + 32 * h);
      r.c[nb][1] = ldg<uint4>(b.c[nb] + 64 * t + 32 * h + 16);
      r.s[nb] = ldg<uint32_t>(b.s[nb] + 8 * t + 4 * h);
    }
  }
}

// the lane's B pointers for N block nb in the prefill layout: virtual row
// block vb of a set whose blocks start at codes / scales, nkb K steps per
// block row; lane (h, n) at 16 (2 n + h) / 4 (2 n + h)
template <int NKB>
__device__ __forceinline__ void fb_tiled_rows(const uint8_t*& c, const uint8_t*& sc, const uint8_t* codes,
                                              const uint8_t* scales, int vb, int lane) {
  const int ln = 2 * (lane & 31) + (lane >> 5);
  c = codes + (size_t)vb * NKB * 2048 + 16 * ln;
  sc = scales + (size_t)vb * NKB * 256 + 4 * ln;
}

// the 8 codes of word j (columns 64 h + 8 j .. + 7) times their UE4M3 scale
template <int J>
__device__ __forceinline__ bf16x8_t fb_decode(const FBRaw& r, int nb) {
  const uint4 q = r.c[nb][J / 4];
  const uint32_t w = (J % 4) == 0 ? q.x : (J % 4) == 1 ? q.y : (J % 4) == 2 ? q.z : q.w;
  const float sc = e4m3_to_f32<J / 2>(r.s[nb]);
  const f32x2_t f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const f32x2_t f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const f32x2_t f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const f32x2_t f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  return __builtin_bit_cast(bf16x8_t, make_uint4(pack_bf16x2_rne(f0.x * sc, f0.y * sc),
                                                 pack_bf16x2_rne(f1.x * sc, f1.y * sc),
                                                 pack_bf16x2_rne(f2.x * sc, f2.y * sc),
                                                 pack_bf16x2_rne(f3.x * sc, f3.y * sc)));
}

struct FAcc { f32x16 c[4][2]; };   // [M block][N block]

// One K step on A stage `la` (128 rows x 256 bytes, swizzled) and B ring
// entry r, for the tile's first NMB M blocks (the rest hold no rows).
template <int NMB>
__device__ __forceinline__ void fb_step(FAcc& acc, const uint8_t* la, const FBRaw& r, int lane) {
  const int h = lane >> 5, m = lane & 31;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    bf16x8_t av[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      const int row = 32 * mb + m;
      av[mb] = *reinterpret_cast<const bf16x8_t*>(la + row * 256 + 16 * ((8 * h + j) ^ (m & 15)));
    }
    bf16x8_t bv[2];
#define FB_DEC(JJ) { bv[0] = fb_decode<JJ>(r, 0); bv[1] = fb_decode<JJ>(r, 1); }
    switch (j) {
      case 0: FB_DEC(0) break; case 1: FB_DEC(1) break; case 2: FB_DEC(2) break; case 3: FB_DEC(3) break;
      case 4: FB_DEC(4) break; case 5: FB_DEC(5) break; case 6: FB_DEC(6) break; default: FB_DEC(7) break;
    }
#undef FB_DEC
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc.c[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mb], bv[nb], acc.c[mb][nb], 0, 0, 0);
  }
}

// The K loop: NK steps (even), A stages double-buffered in s_a, B rows
// double-buffered in registers; NMB M blocks hold rows.  a_src: workgroup-
// uniform base of step 0's A elements; a_off[i]: this lane's byte offset of
// its i-th copy; each step advances by FBK.
template <int NK, int NMB, bool TL>
__device__ __forceinline__ void fb_gemm(FAcc& acc, uint8_t (&s_a)[2][FBM * 256], const uint16_t* a_src,
                                        const uint32_t (&a_off)[8], const FbRows<NK>& brows) {
  static_assert(NK % 2 == 0, "steps go in pairs");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5;
  // byte offsets on a workgroup-uniform base: the copies take the scalar
  // base + 32-bit offset form, so no address register of a copy in flight is
  // ever rewritten (the compiler would wait for the copy first)
  const uint8_t* a_base = reinterpret_cast<const uint8_t*>(a_src);
  auto copy_a = [&](int t, int buf) {
    // wave w copies exactly M block w: an empty block is neither copied nor read
    if (wave >= NMB) return;
    // the step's base as an opaque scalar pair: folded into the per-lane
    // offsets it would make 64-bit addresses again
    uint64_t sb = reinterpret_cast<uint64_t>(a_base + (size_t)t * FBK * 2);
    asm volatile("" : "+s"(sb));
    const uint8_t* src = reinterpret_cast<const uint8_t*>(sb);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_global_load_lds(src + (uint64_t)a_off[i], &s_a[buf][(8 * wave + i) * 1024], 16, 0, 0);
  };
  // Per step t: wait for everything in flight (the copies and B rows of step
  // t, issued one step earlier), barrier, issue copies(t + 1) and B rows(t + 1),
  // then multiply.  Waiting for everything leaves the compiler no wait of its
  // own to add: with a copy into LDS in flight it could only wait for all
  // loads (it cannot tell the copies' memory counts from the loads').  One
  // step of latency is covered by the other workgroup on the CU.  The loop
  // runs a pair of steps per iteration (static register buffers) and is not
  // unrolled further, so four instances of it fit the instruction cache.
  auto step = [&](int t, const FBRaw& cur, FBRaw& nxt, int buf) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    // a bare barrier: a workgroup fence would add nothing here
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < NK) {
      copy_a(t + 1, buf ^ 1);
      fb_load<NK, TL>(nxt, brows, t + 1, h);
    }
    __builtin_amdgcn_sched_barrier(0);
    fb_step<NMB>(acc, s_a[buf], cur, lane);
    __builtin_amdgcn_sched_barrier(0);
  };
  FBRaw r0, r1;
  fb_load<NK, TL>(r0, brows, 0, h);
  copy_a(0, 0);
#pragma unroll 1
  for (int t = 0; t < NK; t += 2) {
    step(t, r0, r1, 0);
    step(t + 1, r1, r0, 1);
  }
}

// fb_gemm for a tile holding `rows` (1 .. FBM) rows
template <int NK, bool TL>
__device__ __forceinline__ void fb_gemm_rows(FAcc& acc, uint8_t (&s_a)[2][FBM * 256], const uint16_t* a_src,
                                             const uint32_t (&a_off)[8], const FbRows<NK>& brows, int rows) {
  switch ((rows + 31) >> 5) {
    case 1: fb_gemm<NK, 1, TL>(acc, s_a, a_src, a_off, brows); break;
    case 2: fb_gemm<NK, 2, TL>(acc, s_a, a_src, a_off, brows); break;
    case 3: fb_gemm<NK, 3, TL>(acc, s_a, a_src, a_off, brows); break;
    default: fb_gemm<NK, 4, TL>(acc, s_a, a_src, a_off, brows); break;
  }
}

// the lane's 8 A copies (byte offsets): copy i of wave w fills tile row
// 32 w + 4 i + lane / 16, slot lane % 16 <- chunk (lane % 16) ^ (row & 15);
// row_off(r) is the element offset of tile row r's source row
template <typename RowOff>
__device__ __forceinline__ void fb_a_offsets(uint32_t (&off)[8], RowOff row_off) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 32 * wave + 4 * i + (lane >> 4);
    off[i] = 2u * (row_off(r) + 8u * (uint32_t)((lane & 15) ^ (r & 15)));   // bytes
  }
}

__device__ __forceinline__ void facc_zero(FAcc& acc) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc.c[mb][nb][e] = 0.f;
}

// gate/up at the Flint shape: tile columns interleave gate and up rows of
// pairs i0 .. i0 + 127 (column 2 i gate row i0 + i, 2 i + 1 up row i0 + i)
template <bool TL>
__global__ __launch_bounds__(256, 2) void prefill_gate_up_f_kernel(LayerArgs a, PrefillWs ws, int T,
                                                                const uint16_t* xin) {
  __shared__ __attribute__((aligned(16))) uint8_t s_a[2][FBM * 256];
  const TileIdx ti = tile_of_block_runs(2 * FI / FBN);
  if (ti.m >= *ws.ntiles) return;
  const int2 tile = ws.tiles[ti.m];
  const int g = tile.x, m0 = tile.y;
  const int E = a.E, K = a.K;
  const bool shared = g == E;
  const int cnt = shared ? T : ws.counts[g];
  const int base = shared ? 0 : ws.offsets[g];
  const int i0 = ti.n * (FBN / 2);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  uint32_t a_off[8];
  fb_a_offsets(a_off, [&](int r) {
    const int rr = m0 + r < cnt ? m0 + r : cnt - 1;
    const int tok = shared ? rr : ws.perm_tok[base + rr];
    return (uint32_t)tok * FH;
  });
  constexpr size_t MC = (size_t)FI * FH / 2, MS = (size_t)FI * FH / 16;
  const uint8_t* c0 = shared ? a.sh_gu_codes : a.gu_codes + (size_t)(2 * g) * MC;
  const uint8_t* s0 = shared ? a.sh_gu_scales : a.gu_scales + (size_t)(2 * g) * MS;
  FbRows<FH / FBK> br;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    if constexpr (TL) {                            // column 2 i + u is virtual row 2 i + u of the pair set
      const uint8_t* tc = shared ? a.pf_sh_gu_codes : a.pf_gu_codes + (size_t)(2 * g) * MC;
      const uint8_t* ts = shared ? a.pf_sh_gu_scales : a.pf_gu_scales + (size_t)(2 * g) * MS;
      fb_tiled_rows<FH / FBK>(br.c[nb], br.s[nb], tc, ts, ti.n * (FBN / 32) + 2 * wave + nb, lane);
    } else {
      const int col = 64 * wave + 32 * nb + (lane & 31);
      const int wrow = i0 + (col >> 1), up = col & 1;
      br.c[nb] = c0 + up * MC + (size_t)wrow * (FH / 2);
      br.s[nb] = s0 + up * MS + (size_t)wrow * (FH / 16);
    }
  }
  const float* gsp = shared ? a.sh_gscale : a.gscale + 3 * g;
  const float gs_g = gsp[0], gs_u = gsp[1];

  FAcc acc;
  facc_zero(acc);
  fb_gemm_rows<FH / FBK, TL>(acc, s_a, xin, a_off, br, cnt - m0);

  // even lanes hold gate columns, odd lanes the matching up columns: the
  // lanes of a pair swap half of their blocks so that the even lane
  // finishes M blocks 0, 2 and the odd lane M blocks 1, 3.  h goes to LDS
  // (the A stages are free once every wave is past its last MFMA), then to
  // memory as whole 256-byte rows.
  __builtin_amdgcn_s_barrier();
  uint16_t* s_h = reinterpret_cast<uint16_t*>(&s_a[0][0]);   // [128 rows][128 pairs]
  const bool even = (lane & 1) == 0;
  const int h = lane >> 5;
#pragma unroll
  for (int pr = 0; pr < 2; ++pr)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        float gacc[2], uacc[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float a0 = acc.c[2 * pr][nb][e + q], a1 = acc.c[2 * pr + 1][nb][e + q];
          const float recv = dpp_f<0xB1>(even ? a1 : a0);
          gacc[q] = even ? a0 : recv;
          uacc[q] = even ? recv : a1;
        }
        // rows r and r + 1 (elements e, e + 1), the same pair column
        const uint32_t gw = pack_bf16x2_rne(gacc[0] * gs_g, gacc[1] * gs_g);
        const uint32_t uw = pack_bf16x2_rne(uacc[0] * gs_u, uacc[1] * gs_u);
        const uint32_t aw = pack_bf16x2_rne(silu_fast(bf16_lo(gw)), silu_fast(bf16_hi(gw)));
        const uint32_t hw = pack_bf16x2_rne(bf16_lo(aw) * bf16_lo(uw), bf16_hi(aw) * bf16_hi(uw));
        const int mb = 2 * pr + (even ? 0 : 1);
        const int r = 32 * mb + 8 * (e >> 2) + 4 * h + (e & 3);
        const int c = (64 * wave + 32 * nb + (lane & 31)) >> 1;
        s_h[r * 128 + c] = (uint16_t)(hw & 0xffffu);
        s_h[(r + 1) * 128 + c] = (uint16_t)(hw >> 16);
      }
  __syncthreads();
  {
    const int tid = threadIdx.x;
#pragma unroll
    for (int k = 0; k < 8; ++k) {                  // 2048 segments of 16 bytes
      const int q = tid + 256 * k, r = q >> 4, seg = q & 15;
      if (m0 + r < cnt) {
        const size_t row = shared ? (size_t)T * K + m0 + r : (size_t)base + m0 + r;
        *reinterpret_cast<uint4*>(ws.h + row * FI + i0 + 8 * seg) =
            *reinterpret_cast<const uint4*>(s_h + r * 128 + 8 * seg);
      }
    }
  }
}

// down at the Flint shape: y = h . W_d^T (fp32, tensor scale applied) for
// the routed groups (the shared expert's tiles are left to the fused
// kernel below)
template <bool TL>
__global__ __launch_bounds__(256, 2) void prefill_down_f_kernel(LayerArgs a, PrefillWs ws, int T) {
  __shared__ __attribute__((aligned(16))) uint8_t s_a[2][FBM * 256];
  const TileIdx ti = tile_of_block(FH / FBN);
  if (ti.m >= *ws.ntiles) return;
  const int2 tile = ws.tiles[ti.m];
  const int g = tile.x, m0 = tile.y;
  const int E = a.E, K = a.K;
  const bool shared = g == E;
  if (shared) return;
  const int cnt = shared ? T : ws.counts[g];
  const size_t base = shared ? (size_t)T * K : (size_t)ws.offsets[g];
  const int n0 = ti.n * FBN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  uint32_t a_off[8];
  fb_a_offsets(a_off, [&](int r) {
    const int rr = m0 + r < cnt ? m0 + r : cnt - 1;
    return (uint32_t)((base + rr) * FI);
  });
  const uint8_t* c0 = shared ? a.sh_d_codes : a.d_codes + (size_t)g * FH * (FI / 2);
  const uint8_t* s0 = shared ? a.sh_d_scales : a.d_scales + (size_t)g * FH * (FI / 16);
  FbRows<FI / FBK> br;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    if constexpr (TL) {
      fb_tiled_rows<FI / FBK>(br.c[nb], br.s[nb], a.pf_d_codes + (size_t)g * FH * (FI / 2),
                              a.pf_d_scales + (size_t)g * FH * (FI / 16), ti.n * (FBN / 32) + 2 * wave + nb, lane);
    } else {
      const int n = n0 + 64 * wave + 32 * nb + (lane & 31);
      br.c[nb] = c0 + (size_t)n * (FI / 2);
      br.s[nb] = s0 + (size_t)n * (FI / 16);
    }
  }
  const float gd = shared ? a.sh_gscale[2] : a.gscale[3 * g + 2];

  FAcc acc;
  facc_zero(acc);
  fb_gemm_rows<FI / FBK, TL>(acc, s_a, ws.h, a_off, br, cnt - m0);
  // y goes through LDS in two halves of 64 rows x 256 fp32 columns and out
  // as whole 1 KB rows, 16 bytes a lane.  The stores are non-temporal: with
  // them the combine kernel that reads y back ran 12 % faster at 8,192 tokens.  Column c of row r sits at
  // c ^ (32 ((r >> 2) & 1)): the two lane halves of a write (rows 4 apart)
  // then fill the two different halves of the 64 banks.
  float* s_y = reinterpret_cast<float*>(&s_a[0][0]);   // [64][256]
  const int h = lane >> 5, tid = threadIdx.x;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    __syncthreads();                               // the A stages, then the previous half, are free
#pragma unroll
    for (int mq = 0; mq < 2; ++mq)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = 32 * mq + 8 * (e >> 2) + 4 * h + (e & 3);
          const int c = 64 * wave + 32 * nb + (lane & 31);
          s_y[r * FBN + (c ^ (32 * ((r >> 2) & 1)))] = acc.c[2 * hf + mq][nb][e] * gd;
        }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {                 // 4096 segments of 16 bytes
      const int q = tid + 256 * k, r = q >> 6, g = q & 63;
      const int row = m0 + 64 * hf + r;
      if (row < cnt)
        __builtin_nontemporal_store(*reinterpret_cast<const f32x4_t*>(s_y + r * FBN + 4 * (g ^ (8 * ((r >> 2) & 1)))),
                                    reinterpret_cast<f32x4_t*>(ws.y + (base + row) * FH + n0 + 4 * g));
    }
  }
}

// The shared expert's down GEMM fused with the combine, at the Flint shape:
// workgroup (token tile mt, column tile nt) computes the shared expert's
// y for tokens 128 mt .. + 127 and columns 256 nt .. + 255 in registers,
// then, for each of them, out = BF16(sum_k w_k y[pos(t, k)] + y_shared) (+
// residual, rounded again): the routed rows in selection order, then the
// shared one, as in prefill_combine_kernel.  The routed y rows were written
// by prefill_down_f_kernel (the previous launch); the shared expert's y
// never goes to memory, and no separate combine pass reads any of it.
// KC: the top-k as a compile-time constant (straight-line epilogue), or 0.
template <int KC, bool TL>
__global__ __launch_bounds__(256, 2) void prefill_down_shared_combine_f_kernel(LayerArgs a, PrefillWs ws, int T) {
  __shared__ __attribute__((aligned(16))) uint8_t s_a[2][FBM * 256];
  __shared__ int s_pos[FBM][FLINT_MAX_TOP_K];
  __shared__ float s_w[FBM][FLINT_MAX_TOP_K];
  const TileIdx ti = tile_of_block(FH / FBN);
  const int m0 = ti.m * FBM;
  if (m0 >= T) return;
  const int K = KC ? KC : a.K;
  constexpr int KM = KC ? KC : FLINT_MAX_TOP_K;   // unrolled selections
  const size_t base = (size_t)T * K;
  const int n0 = ti.n * FBN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool resid = (a.flags & FLINT_RESIDUAL) != 0;

  for (int q = tid; q < FBM * FLINT_MAX_TOP_K; q += 256) {   // the tile's tokens' positions and weights
    const int r = q / FLINT_MAX_TOP_K, k = q % FLINT_MAX_TOP_K;
    const bool ok = m0 + r < T && k < K;
    s_pos[r][k] = ok ? ws.pos[(size_t)(m0 + r) * K + k] : 0;
    s_w[r][k] = ok ? a.topk_w[(size_t)(m0 + r) * K + k] : 0.f;
  }
  uint32_t a_off[8];
  fb_a_offsets(a_off, [&](int r) {
    const int rr = m0 + r < T ? m0 + r : T - 1;
    return (uint32_t)((base + rr) * FI);
  });
  FbRows<FI / FBK> br;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    if constexpr (TL) {
      fb_tiled_rows<FI / FBK>(br.c[nb], br.s[nb], a.pf_sh_d_codes, a.pf_sh_d_scales,
                              ti.n * (FBN / 32) + 2 * wave + nb, lane);
    } else {
      const int n = n0 + 64 * wave + 32 * nb + (lane & 31);
      br.c[nb] = a.sh_d_codes + (size_t)n * (FI / 2);
      br.s[nb] = a.sh_d_scales + (size_t)n * (FI / 16);
    }
  }
  const float gd = a.sh_gscale[2];

  FAcc acc;
  facc_zero(acc);
  fb_gemm_rows<FI / FBK, TL>(acc, s_a, ws.h, a_off, br, T - m0);
  __syncthreads();                                 // A stages free, s_pos / s_w visible

  // the weighted sum of each (token, column) of the lane into LDS as BF16
  uint16_t* s_o = reinterpret_cast<uint16_t*>(&s_a[0][0]);   // [128 rows][256 columns]
  const int h = lane >> 5;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int c = 64 * wave + 32 * nb + (lane & 31);
#pragma unroll
      for (int e0 = 0; e0 < 16; e0 += 4) {       // four rows' routed values in flight together (y is
                                                 // read once: non-temporal loads, 94.8 -> 87.7 us)
        float yv[4][KM];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = 32 * mb + 8 * (e0 >> 2) + 4 * h + q;
#pragma unroll
          for (int k = 0; k < KM; ++k)
            yv[q][k] = k < K ? __builtin_nontemporal_load(&ws.y[(size_t)s_pos[r][k] * FH + n0 + c]) : 0.f;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = 32 * mb + 8 * (e0 >> 2) + 4 * h + q;
          float sum = 0.f;
#pragma unroll
          for (int k = 0; k < KM; ++k)
            if (k < K) sum = fmaf(s_w[r][k], yv[q][k], sum);
          sum += acc.c[mb][nb][e0 + q] * gd;
          s_o[r * 256 + c] = f32_to_bf16_bits(sum);
        }
      }
    }
  }
  __syncthreads();
#pragma unroll 4
  for (int k = 0; k < 16; ++k) {                   // 4096 segments of 16 bytes: + residual, to memory
    const int q = tid + 256 * k, r = q >> 5, seg = q & 31;
    if (m0 + r < T) {
      const size_t o = (size_t)(m0 + r) * FH + n0 + 8 * seg;
      uint4 v = *reinterpret_cast<const uint4*>(s_o + r * 256 + 8 * seg);
      if (resid) {
        const uint4 xv = *reinterpret_cast<const uint4*>(a.x + o);
        const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
        uint32_t vs[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) vs[i] = pack_bf16x2(bf16_lo(xs[i]) + bf16_lo(vs[i]), bf16_hi(xs[i]) + bf16_hi(vs[i]));
        v = make_uint4(vs[0], vs[1], vs[2], vs[3]);
      }
      *reinterpret_cast<uint4*>(a.out + o) = v;
    }
  }
}

// --------------------------------------------------------------- combine --
// One workgroup per token; 8 columns per thread per pass.
__global__ __launch_bounds__(256) void prefill_combine_kernel(LayerArgs a, PrefillWs ws, int T) {
  const int t = blockIdx.x;
  const int H = a.H, K = a.K;
  const bool has_sh = a.SI > 0;
  const bool resid = (a.flags & FLINT_RESIDUAL) != 0;
  int p[FLINT_MAX_TOP_K];
  float w[FLINT_MAX_TOP_K];
#pragma unroll
  for (int k = 0; k < FLINT_MAX_TOP_K; ++k) {
    p[k] = k < K ? ws.pos[(size_t)t * K + k] : 0;
    w[k] = k < K ? a.topk_w[(size_t)t * K + k] : 0.f;
  }
  for (int c = 8 * threadIdx.x; c < H; c += 8 * 256) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
#pragma unroll
    for (int k = 0; k < FLINT_MAX_TOP_K; ++k) {
      if (k < K) {
        const float4* yr = reinterpret_cast<const float4*>(ws.y + (size_t)p[k] * H + c);
        const float4 v0 = yr[0], v1 = yr[1];
        acc[0] = fmaf(w[k], v0.x, acc[0]); acc[1] = fmaf(w[k], v0.y, acc[1]);
        acc[2] = fmaf(w[k], v0.z, acc[2]); acc[3] = fmaf(w[k], v0.w, acc[3]);
        acc[4] = fmaf(w[k], v1.x, acc[4]); acc[5] = fmaf(w[k], v1.y, acc[5]);
        acc[6] = fmaf(w[k], v1.z, acc[6]); acc[7] = fmaf(w[k], v1.w, acc[7]);
      }
    }
    if (has_sh) {
      const float4* yr = reinterpret_cast<const float4*>(ws.y + ((size_t)T * K + t) * H + c);
      const float4 v0 = yr[0], v1 = yr[1];
      acc[0] += v0.x; acc[1] += v0.y; acc[2] += v0.z; acc[3] += v0.w;
      acc[4] += v1.x; acc[5] += v1.y; acc[6] += v1.z; acc[7] += v1.w;
    }
    uint32_t xr[4] = {0, 0, 0, 0};
    if (resid) {
      const uint4 xv = *reinterpret_cast<const uint4*>(a.x + (size_t)t * H + c);
      xr[0] = xv.x; xr[1] = xv.y; xr[2] = xv.z; xr[3] = xv.w;
    }
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float lo = round_bf16(acc[2 * q]), hi = round_bf16(acc[2 * q + 1]);
      if (resid) {
        lo = bf16_lo(xr[q]) + lo;
        hi = bf16_hi(xr[q]) + hi;
      }
      o[q] = pack_bf16x2(lo, hi);
    }
    *reinterpret_cast<uint4*>(a.out + (size_t)t * H + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace

hipError_t launch_prefill(const LayerArgs& a, const PrefillWs& ws, int T, hipStream_t st) {
  const bool norm = (a.flags & FLINT_PRE_RMSNORM) != 0;
  const bool bf = (a.flags & FLINT_W_BF16) != 0;
  const uint16_t* xin = norm ? ws.xn : a.x;
  const int C = (T + CHUNK - 1) / CHUNK;
  const int imax = a.I > a.SI ? a.I : a.SI;
  if (norm) hipLaunchKernelGGL(prefill_norm_kernel, dim3((T + 3) / 4), dim3(256), 0, st, a, ws, T);
  if (a.H == RH && a.E == 256 && (int64_t)T * RH * 2 < (1ll << 32)) {
    hipLaunchKernelGGL(prefill_router_frag_kernel, dim3(a.E * RH / 8 / 256), dim3(256), 0, st, a.router, ws.router_f);
    hipLaunchKernelGGL(prefill_route_f_kernel, dim3(2 * C), dim3(512), 0, st, a, ws, T, xin);
  } else {
    if (a.H == RH && a.E % RTN == 0 && (int64_t)T * RH * 2 < (1ll << 32))
      hipLaunchKernelGGL(prefill_router_f_kernel, dim3((T + RTM - 1) / RTM, a.E / RTN), dim3(256), 0, st, a, ws, T,
                         xin);
    else
      hipLaunchKernelGGL(prefill_router_kernel, dim3((T + BM - 1) / BM, (a.E + BN - 1) / BN), dim3(256), 0,
                         st, a, ws, T, xin);
    hipLaunchKernelGGL(prefill_topk_kernel, dim3(2 * C), dim3(512), 0, st, a, ws, T);
  }
  hipLaunchKernelGGL(prefill_scan_kernel, dim3(1), dim3(1024), 0, st, a, ws, T);
  hipLaunchKernelGGL(prefill_scatter_kernel, dim3(C), dim3(256), 0, st, a, ws, T);
  const dim3 ggu(grouped_grid(ws.max_tiles, (imax + BN / 2 - 1) / (BN / 2)));
  const dim3 gdn(grouped_grid(ws.max_tiles, (a.H + BN - 1) / BN));
  // the Flint-shape GEMMs address A with 32-bit byte offsets
  const bool flint = !bf && a.H == FH && a.I == FI && a.SI == FI && FBM == BM &&
                     (int64_t)T * FH * 2 < (1ll << 32) && ((int64_t)T * a.K + T) * FI * 2 < (1ll << 32);
  if (bf) {
    hipLaunchKernelGGL(prefill_gate_up_kernel<FMT_BF16>, ggu, dim3(256), 0, st, a, ws, T, xin);
    hipLaunchKernelGGL(prefill_down_kernel<FMT_BF16>, gdn, dim3(256), 0, st, a, ws, T);
  } else if (flint) {
    const dim3 ggu(grouped_grid_runs(ws.max_tiles, 2 * FI / FBN)), gdn(grouped_grid(ws.max_tiles, FH / FBN));
    const dim3 gsc(grouped_grid((T + FBM - 1) / FBM, FH / FBN));
    if (a.pf_gu_codes) {                           // the weights in the prefill layout
      hipLaunchKernelGGL(prefill_gate_up_f_kernel<true>, ggu, dim3(256), 0, st, a, ws, T, xin);
      hipLaunchKernelGGL(prefill_down_f_kernel<true>, gdn, dim3(256), 0, st, a, ws, T);
      if (a.K == 6) hipLaunchKernelGGL((prefill_down_shared_combine_f_kernel<6, true>), gsc, dim3(256), 0, st, a, ws, T);
      else hipLaunchKernelGGL((prefill_down_shared_combine_f_kernel<0, true>), gsc, dim3(256), 0, st, a, ws, T);
    } else {
      hipLaunchKernelGGL(prefill_gate_up_f_kernel<false>, ggu, dim3(256), 0, st, a, ws, T, xin);
      hipLaunchKernelGGL(prefill_down_f_kernel<false>, gdn, dim3(256), 0, st, a, ws, T);
      if (a.K == 6) hipLaunchKernelGGL((prefill_down_shared_combine_f_kernel<6, false>), gsc, dim3(256), 0, st, a, ws, T);
      else hipLaunchKernelGGL((prefill_down_shared_combine_f_kernel<0, false>), gsc, dim3(256), 0, st, a, ws, T);
    }
    return hipGetLastError();
  } else {
    hipLaunchKernelGGL(prefill_gate_up_kernel<FMT_NVFP4>, ggu, dim3(256), 0, st, a, ws, T, xin);
    hipLaunchKernelGGL(prefill_down_kernel<FMT_NVFP4>, gdn, dim3(256), 0, st, a, ws, T);
  }
  hipLaunchKernelGGL(prefill_combine_kernel, dim3(T), dim3(256), 0, st, a, ws, T);
  return hipGetLastError();
}

}  // namespace flint
