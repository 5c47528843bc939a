// flint_stream_read: a plain streaming read of a device buffer, the
// measurement utility against which the decode kernels' HBM rates are
// compared.  Every thread reads `loads` 16-byte words per pass (all issued
// before any is used) in a grid-stride loop and folds them into one word;
// the fold is written only if it equals a value no buffer of the library's
// tests produces, so the reads cannot be dropped and nothing is written.
#include <hip/hip_runtime.h>

#include "common.hpp"

namespace flint {
namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

template <int U>
__global__ void stream_read_kernel(const v4u* __restrict__ src, int64_t n16, uint32_t* sink) {
  const int64_t nt = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i0 < n16; i0 += nt * U) {
    v4u v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + nt * u;
      v[u] = i < n16 ? src[i] : (v4u){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace
}  // namespace flint

extern "C" int32_t flint_stream_read(const void* src, int64_t bytes, int32_t threads, int32_t loads,
                                     int32_t blocks, void* sink, void* stream) {
  using namespace flint;
  if (!src || !sink || bytes <= 0 || (bytes & 15) || blocks <= 0) return FLINT_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(sink) & 3)) return FLINT_ERR_ALIGNMENT;
  if (threads < 64 || threads > 1024 || threads % 64) return FLINT_ERR_UNSUPPORTED;
  const int64_t n16 = bytes / 16;
  const auto* s = static_cast<const v4u*>(src);
  auto* k = static_cast<uint32_t*>(sink);
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (loads) {
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(blocks), dim3(threads), 0, st, s, n16, k); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(blocks), dim3(threads), 0, st, s, n16, k); break;
    case 16: hipLaunchKernelGGL(stream_read_kernel<16>, dim3(blocks), dim3(threads), 0, st, s, n16, k); break;
    case 27: hipLaunchKernelGGL(stream_read_kernel<27>, dim3(blocks), dim3(threads), 0, st, s, n16, k); break;
    default: return FLINT_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? FLINT_OK : FLINT_ERR_DEVICE;
}
