// qlinear_int8_noalloc: the INT8 quantized linear with its workspace in a
// device array of the library's own, for callers that cannot allocate
// device memory (code under stream capture, serving loops, harnesses that
// forbid hipMalloc).  The kernels are qlinear_int8's; only the scratch
// differs.
//
// The array lives in this file's code object: every GPU the library runs
// on holds one copy, at its own address, until the process ends.  Its
// name is a host-side stand-in in host code, so the device address is
// looked up once per device (hipGetSymbolAddress with that device current)
// and only that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <stdint.h>

#include "qact.h"
#include "qact_internal.h"

namespace {

constexpr size_t kScratchBytes = QA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "the scratch holds whole 256-byte lines");

// K-split partial sums (and, for the fp16-MFMA kernel, the per-tile scale
// copies) of one qlinear_int8_noalloc call.  No word of it needs to start
// at zero: every word a kernel reads was written earlier in the same call.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on device `dev`, which must be current.
int scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return QA_EHIP;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QA_EHIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return QA_OK;
}

}  // namespace

extern "C" int qlinear_int8_noalloc(const int8_t* a_q, const float* a_s, const uint8_t* w_q,
                                    const uint8_t* w_s, const float* w_ts, const void* w8,
                                    int64_t M, int64_t N, int64_t K, const uint16_t* bias, void* y,
                                    int64_t ldy, qa_out out, qa_epi epi, hipStream_t stream) {
  if (int s = qact::int8_linear_status(a_q, a_s, w_q, w_s, w_ts, w8, M, N, K, y, ldy, out, epi))
    return s;
  if (qlinear_workspace(QA_INT8, M, N, K) > kScratchBytes) return QA_ESCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return QA_EHIP;
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return QA_EHIP;
    if (sdev != dev) return QA_EINVAL;
  }
  void* ws = nullptr;
  if (int s = scratch_address(dev, &ws)) return s;
  return qlinear_int8(a_q, a_s, w_q, w_s, w_ts, w8, M, N, K, bias, y, ldy, out, epi, ws,
                      kScratchBytes, stream);
}
