// fs4_quantize_noalloc: the quantizer for callers that cannot allocate.
//
// fs4_quantize takes its scratch (the amax pass's per-workgroup partial
// maxima) from a caller-provided workspace.  This entry point takes it from a
// file-scope device array instead, so the caller allocates nothing beyond the
// input and the output views: it suits code under HIP graph capture, tight
// loops and harnesses that forbid allocation.
//
// The array exists once per GPU for the life of the process.  Host code never
// uses its name as a device address: the address is asked of the runtime
// (hipGetSymbolAddress, with the device current) on the first call on each
// device and kept per device.  Every call on one GPU shares that GPU's array;
// the amax pass writes every partial the encode pass then reads, so nothing
// needs clearing between calls, and calls that overlap on one GPU race.
#include <atomic>

#include "fs4_common.h"

namespace fs4 {
namespace {

// the quantizer's scratch: kAmaxPartials uint32 partial maxima (4 KB), the
// same for every input size
constexpr size_t kScratchBytes = 4096;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// This device's address of `scratch`, asked of the runtime once per device.
fs4_status device_scratch(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FS4_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FS4_ERR_ARG;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FS4_ERR_HIP;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return FS4_OK;
}

}  // namespace
}  // namespace fs4

using namespace fs4;

extern "C" size_t fs4_quantize_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" fs4_status fs4_quantize_noalloc(const void *x, fs4_dtype dt, int64_t rows, int64_t cols,
                                           const fs4_nvfp4 *rowwise, const fs4_nvfp4 *colwise, void *stream) {
  const fs4_status st = check_quantize_args(x, dt, rows, cols, rowwise, colwise);
  if (st != FS4_OK) return st;
  if (quantize_ws_bytes() > kScratchBytes) return FS4_ERR_WORKSPACE;
  void *ws = nullptr;
  const fs4_status sp = device_scratch(&ws);
  if (sp != FS4_OK) return sp;
  return launch_quantize(x, dt, rows, cols, rowwise, colwise, ws, (hipStream_t)stream);
}
