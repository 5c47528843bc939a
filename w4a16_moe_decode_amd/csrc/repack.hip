// Load-time repack of source NVFP4 super-blocks into the packed gfx950
// planes, its exact inverse, and a float32 dequantiser exposing the GEMV
// kernels' decode.
//
// Source format ("Day-0 Support for Flint on vLLM", "Model architecture":
// the checkpoint's NVFP4 blocks come in another byte order and are repacked
// losslessly at load; arex-research Flint write-up, section
// "七个内核的依赖链", second paragraph: a 64-value super-block is four groups
// of one UE4M3 scale and 16 E2M1 codes).  The byte order inside the
// 36-byte super-block is not printed; both readings are accepted:
//   FLINT_SRC_INTERLEAVED   byte 9j = scale of group j, 9j+1..9j+8 its codes
//   FLINT_SRC_SCALES_FIRST  bytes 0..3 = scales, 4..35 = codes in order
// Packed planes: codes [R][C/2] (column 2i low nibble), scales [R][C/16].
#include "common.hpp"

namespace flint {
namespace {

// position in the source super-block of packed code byte p (0..31)
__device__ __forceinline__ int src_code_pos(int layout, int p) {
  return layout == FLINT_SRC_INTERLEAVED ? 9 * (p >> 3) + 1 + (p & 7) : 4 + p;
}
__device__ __forceinline__ int src_scale_pos(int layout, int j) {
  return layout == FLINT_SRC_INTERLEAVED ? 9 * j : j;
}

__device__ __forceinline__ uint32_t byte_of(const uint32_t* w, int pos) {
  return (w[pos >> 2] >> (8 * (pos & 3))) & 0xffu;
}

template <int LAYOUT>
__global__ __launch_bounds__(256) void repack_kernel(const uint8_t* __restrict__ src,
                                                     int64_t n_blocks, int64_t blocks_per_mat,
                                                     int64_t mat_stride, uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_blocks;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t* s = reinterpret_cast<const uint32_t*>(src + 36 * i);
    uint32_t w[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) w[k] = s[k];
    uint32_t c[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) v |= byte_of(w, src_code_pos(LAYOUT, 4 * k + b)) << (8 * b);
      c[k] = v;
    }
    uint32_t sc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) sc |= byte_of(w, src_scale_pos(LAYOUT, j)) << (8 * j);
    const int64_t m = i / blocks_per_mat, r = i - m * blocks_per_mat;
    const int64_t dst = m * mat_stride * blocks_per_mat + r;   // super-block index in the planes
    uint4* cd = reinterpret_cast<uint4*>(codes + 32 * dst);
    cd[0] = make_uint4(c[0], c[1], c[2], c[3]);
    cd[1] = make_uint4(c[4], c[5], c[6], c[7]);
    reinterpret_cast<uint32_t*>(scales)[dst] = sc;
  }
}

template <int LAYOUT>
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales,
                                                     int64_t n_blocks, int64_t blocks_per_mat,
                                                     int64_t mat_stride, uint8_t* __restrict__ dst) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_blocks;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / blocks_per_mat, r = i - m * blocks_per_mat;
    const int64_t srcb = m * mat_stride * blocks_per_mat + r;
    const uint4* cp = reinterpret_cast<const uint4*>(codes + 32 * srcb);
    const uint4 a = cp[0], b = cp[1];
    const uint32_t c[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    const uint32_t sc = reinterpret_cast<const uint32_t*>(scales)[srcb];
    uint32_t w[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) w[k] = 0;
#pragma unroll
    for (int p = 0; p < 32; ++p) {
      const int pos = src_code_pos(LAYOUT, p);
      w[pos >> 2] |= byte_of(c, p) << (8 * (pos & 3));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pos = src_scale_pos(LAYOUT, j);
      w[pos >> 2] |= ((sc >> (8 * j)) & 0xffu) << (8 * (pos & 3));
    }
    uint32_t* d = reinterpret_cast<uint32_t*>(dst + 36 * i);
#pragma unroll
    for (int k = 0; k < 9; ++k) d[k] = w[k];
  }
}

// one thread per 32-column chunk of a packed row
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      int64_t n_chunks, int64_t chunks_per_mat,
                                                      const float* __restrict__ tscale,
                                                      float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_chunks;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint4 c = reinterpret_cast<const uint4*>(codes)[i];
    const uint32_t sc = reinterpret_cast<const uint16_t*>(scales)[i];
    const DChunk<FMT_NVFP4> d = decode_nvfp4(c, sc);
    const float g = tscale ? tscale[i / chunks_per_mat] : 1.0f;
    float4* o = reinterpret_cast<float4*>(out + 32 * i);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float s = q < 4 ? d.s0 : d.s1;
      const bf16x2_t a = d.w[2 * q], b = d.w[2 * q + 1];
      o[q] = make_float4((float)a.x * s * g, (float)a.y * s * g, (float)b.x * s * g,
                         (float)b.y * s * g);
    }
  }
}

inline unsigned grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  return (unsigned)(g < 65536 ? (g < 1 ? 1 : g) : 65536);
}

// Prefill layout: one thread per 16 code bytes of the output.  Output unit
// w (0..127) of block (set, vb, kb) is piece p = w / 64 of half h = w & 1
// of virtual row n = (w & 63) / 2: code bytes 64 kb + 32 h + 16 p .. + 15 of
// that row; the unit with p = 0 also moves the row's scale bytes 8 kb + 4 h
// .. + 3.  Virtual row v of a set is row v of its matrix, or (interleave)
// row v / 2 of matrix v & 1 of its pair.
__global__ __launch_bounds__(256) void prefill_layout_kernel(const uint8_t* __restrict__ codes,
                                                             const uint8_t* __restrict__ scales, int64_t n_sets,
                                                             int rows, int cols, int interleave,
                                                             uint8_t* __restrict__ oc, uint8_t* __restrict__ os) {
  const int64_t nkb = cols / 128, nvb = (int64_t)rows * (1 + interleave) / 32;
  const int64_t blocks = n_sets * nvb * nkb, units = blocks * 128;
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units; u += (int64_t)gridDim.x * 256) {
    const int64_t blk = u >> 7;                    // global block index (set, vb, kb)
    const int w = (int)(u & 127), p = w >> 6, nh = w & 63, n = nh >> 1, h = nh & 1;
    const int64_t set = blk / (nvb * nkb), rest = blk - set * nvb * nkb;
    const int64_t vb = rest / nkb, kb = rest - vb * nkb;
    const int64_t v = vb * 32 + n;
    const int64_t mat = interleave ? 2 * set + (v & 1) : set, row = interleave ? v >> 1 : v;
    const int64_t r = mat * rows + row;            // row of the packed planes
    *reinterpret_cast<uint4*>(oc + blk * 2048 + 16 * w) =
        *reinterpret_cast<const uint4*>(codes + r * (cols / 2) + kb * 64 + 32 * h + 16 * p);
    if (p == 0)
      *reinterpret_cast<uint32_t*>(os + blk * 256 + 4 * nh) =
          *reinterpret_cast<const uint32_t*>(scales + r * (cols / 16) + kb * 8 + 4 * h);
  }
}

}  // namespace

hipError_t launch_repack(const uint8_t* src, int64_t n_mats, int rows, int cols, int layout,
                         uint8_t* codes, uint8_t* scales, int64_t mat_stride, hipStream_t st) {
  const int64_t bpm = (int64_t)rows * (cols / 64);
  const int64_t n = n_mats * bpm;
  if (layout == FLINT_SRC_INTERLEAVED)
    hipLaunchKernelGGL(repack_kernel<FLINT_SRC_INTERLEAVED>, dim3(grid_for(n)), dim3(256), 0, st,
                       src, n, bpm, mat_stride, codes, scales);
  else
    hipLaunchKernelGGL(repack_kernel<FLINT_SRC_SCALES_FIRST>, dim3(grid_for(n)), dim3(256), 0, st,
                       src, n, bpm, mat_stride, codes, scales);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* codes, const uint8_t* scales, int64_t n_mats, int rows,
                         int cols, int layout, int64_t mat_stride, uint8_t* dst, hipStream_t st) {
  const int64_t bpm = (int64_t)rows * (cols / 64);
  const int64_t n = n_mats * bpm;
  if (layout == FLINT_SRC_INTERLEAVED)
    hipLaunchKernelGGL(unpack_kernel<FLINT_SRC_INTERLEAVED>, dim3(grid_for(n)), dim3(256), 0, st,
                       codes, scales, n, bpm, mat_stride, dst);
  else
    hipLaunchKernelGGL(unpack_kernel<FLINT_SRC_SCALES_FIRST>, dim3(grid_for(n)), dim3(256), 0, st,
                       codes, scales, n, bpm, mat_stride, dst);
  return hipGetLastError();
}

hipError_t launch_prefill_layout(const uint8_t* codes, const uint8_t* scales, int64_t n_mats, int rows, int cols,
                                 int interleave, uint8_t* out_codes, uint8_t* out_scales, hipStream_t st) {
  const int64_t units = n_mats * rows * (int64_t)(cols / 128) * 4;   // 16-byte code units
  const int64_t blocks = (units + 255) / 256;
  hipLaunchKernelGGL(prefill_layout_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0, st,
                     codes, scales, n_mats / (1 + interleave), rows, cols, interleave, out_codes, out_scales);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, int64_t n_mats, int rows,
                          int cols, const float* tscale, float* out, hipStream_t st) {
  const int64_t cpm = (int64_t)rows * (cols / 32);
  const int64_t n = n_mats * cpm;
  hipLaunchKernelGGL(dequant_kernel, dim3(grid_for(n)), dim3(256), 0, st, codes, scales, n, cpm,
                     tscale, out);
  return hipGetLastError();
}

}  // namespace flint
