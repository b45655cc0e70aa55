// Test-only entry point: the element conversions the quantization kernels
// are built on, applied to a range of float32 bit patterns, so that a test
// can compare them with the NVFP4 format's rounding rules on every input
// (6Bit-Diffusion, abstract: E2M1 elements with E4M3 group scales; the
// bf16 rounding of the GEMM epilogues and the TDC kernels).  Not used by any
// other call.
#include "qact_device.h"
#include "qact_internal.h"

namespace qact {

// pattern p = first + i for i < count; one output per pattern
template <int OP>
__global__ void __launch_bounds__(256)
convert_kernel(uint32_t first, int64_t count, void* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += stride) {
    const float x = __uint_as_float(first + (uint32_t)i);
    if constexpr (OP == 0) {
      // the E2M1 conversion of the NVFP4 encoders (unit scale)
      static_cast<uint8_t*>(out)[i] = (uint8_t)(QACT_E2M1_PK(0u, x, 0.0f, 0) & 15u);
    } else if constexpr (OP == 1) {
      // the E4M3 group-scale encoder (non-negative finite inputs)
      static_cast<uint8_t*>(out)[i] = (uint8_t)e4m3_encode(x);
    } else {
      // the packed float32 -> bf16 conversion of the epilogues
      static_cast<uint16_t*>(out)[i] = (uint16_t)(bf16_pack(x, 0.0f) & 0xFFFFu);
    }
  }
}

hipError_t launch_convert(int op, uint32_t first, int64_t count, void* out, hipStream_t stream) {
  int64_t blocks = (count + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  const dim3 g((unsigned)blocks), t(256);
  if (op == 0)
    hipLaunchKernelGGL(convert_kernel<0>, g, t, 0, stream, first, count, out);
  else if (op == 1)
    hipLaunchKernelGGL(convert_kernel<1>, g, t, 0, stream, first, count, out);
  else
    hipLaunchKernelGGL(convert_kernel<2>, g, t, 0, stream, first, count, out);
  return hipGetLastError();
}

}  // namespace qact
