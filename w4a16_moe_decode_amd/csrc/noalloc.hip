// flint_moe_decode_noalloc: the decode MoE layer with the library's own
// device scratch in place of a caller-allocated workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).  Same kernels and results as
// flint_moe_decode; no allocation, no host synchronisation.
#include <hip/hip_runtime.h>

#include <mutex>

#include "common.hpp"

namespace flint {
namespace {

// The decode workspace of every no-alloc call on a device: header (launch
// counters, epoch, error word), hand-off words, slot table and h buffers.
// Zero at load, like a freshly zero-filled workspace; every call leaves it
// ready for the next (counters reset, hand-off words tagged with a launch
// epoch).  Each device holds its own copy until the process ends.
static __device__ __align__(256) uint8_t scratch[FLINT_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of `scratch` per device (host code must not use the
// symbol's name as an address: in host code it is only a stand-in).
void* g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

// The scratch address on the current device, looked up once per device with
// that device current; nullptr if the runtime cannot give it.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace
}  // namespace flint

extern "C" int32_t flint_moe_decode_noalloc(const flint_moe_shape* shape, const flint_moe_weights* weights,
                                            const void* x, int32_t batch, void* out, int32_t* topk_idx,
                                            float* topk_w, const void* gamma, void* stream) {
  // every argument check first (with no workspace given, a valid call stops
  // at the workspace check), then the scratch's capacity, then its address
  const int32_t st = flint::decode_common(-1, shape, weights, x, batch, out, topk_idx, topk_w, gamma,
                                          nullptr, 0, stream);
  if (st != FLINT_ERR_WORKSPACE) return st;
  if (flint::decode_ws_bytes(*shape, FLINT_MAX_DECODE_BATCH) > FLINT_NOALLOC_SCRATCH_BYTES)
    return FLINT_ERR_WORKSPACE;
  void* ws = flint::scratch_on_current_device();
  if (!ws) return FLINT_ERR_DEVICE;
  return flint::decode_common(-1, shape, weights, x, batch, out, topk_idx, topk_w, gamma, ws,
                              FLINT_NOALLOC_SCRATCH_BYTES, stream);
}
