// noalloc.hip -- int8_gemm_noalloc: int8_gemm_ws with a workspace that the
// library holds in a static device array, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops).
//
// `scratch` is a file-scope device array: the code object's loader reserves it
// on every GPU the library is loaded on, and it stays there until the process
// ends.  Host code never passes its name to a kernel (on the host the name is a
// stand-in, not a device address); the device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and kept.
//
// The split-K partials it holds are written in full by the gemm launch before
// the summing launch reads them, so nothing in it has to start at zero and no
// call clears it.  Every call on one GPU uses the same array: calls that can
// overlap on that GPU (several streams, several host threads) race.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "int8w.h"
#include "launch.h"

namespace int8w {
namespace {

static_assert(INT8W_NOALLOC_SCRATCH_BYTES % 256u == 0, "scratch size is a whole number of 256-byte blocks");

static __device__ __align__(256) uint8_t scratch[INT8W_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on device `dev`; nullptr (and the error
// recorded) when it cannot be had.
void *scratch_on(int dev) {
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p) return p;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) {
    report_error(INT8W_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) {
    report_error(INT8W_ERR_HIP, "hipSetDevice(%d) failed: %s", dev, hipGetErrorString(e));
    return nullptr;
  }
  void *q = nullptr;
  e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess || q == nullptr) {
    report_error(INT8W_ERR_HIP, "hipGetSymbolAddress of the gemm scratch on device %d failed: %s", dev,
                 hipGetErrorString(e));
    return nullptr;
  }
  g_scratch_ptr[dev].store(q, std::memory_order_release);
  return q;
}

}  // namespace
}  // namespace int8w

using namespace int8w;

extern "C" int int8_gemm_noalloc(const int8w_weight *w, const uint16_t *x, uint16_t *y, uint32_t m,
                                 uint64_t stream) {
  // int8_gemm_workspace_bytes validates w (0 for an invalid weight, whose
  // error gemm_common then reports)
  const uint64_t need = int8_gemm_workspace_bytes(w, m);
  if (need > INT8W_NOALLOC_SCRATCH_BYTES)
    return report_error(INT8W_ERR_SHAPE,
                        "m=%u on this weight splits K over a workspace of %llu bytes, more than the %llu bytes "
                        "of int8_gemm_noalloc's scratch (int8_gemm_ws takes a workspace of any size)",
                        m, (unsigned long long)need, (unsigned long long)INT8W_NOALLOC_SCRATCH_BYTES);
  if (need == 0) return gemm_common(w, x, y, m, nullptr, 0, stream);
  hipStream_t s = reinterpret_cast<hipStream_t>(static_cast<uintptr_t>(stream));
  int dev = -1;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return report_error(INT8W_ERR_HIP, "device of the stream: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return report_error(INT8W_ERR_HIP, "device %d out of range", dev);
  void *ws = scratch_on(dev);
  if (!ws) return INT8W_ERR_HIP;
  return gemm_common(w, x, y, m, ws, INT8W_NOALLOC_SCRATCH_BYTES, stream);
}
