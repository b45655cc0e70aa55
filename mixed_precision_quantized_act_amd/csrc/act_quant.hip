// Activation quantization kernels for gfx950: NVFP4 (E2M1 + E4M3 per 16 +
// float32 tensor scale) and per-token symmetric INT8.  6Bit-Diffusion,
// abstract: activations of each linear are quantized at inference time to
// NVFP4 or INT8; Fig. 2 caption: the choice is per linear layer.
//
// Both kernels stream bf16 rows with 16-byte loads.  NVFP4 runs two passes:
// a tensor |x| max (per-workgroup partial maxima into scratch) and the
// encoder, whose workgroups each fold the partial maxima into s_T before
// encoding one 16-element group per thread.  INT8 gives each token row to
// one wave: a row max by wave shuffles, then the encode of the same row.
#include "qact_device.h"
#include "qact_internal.h"

namespace qact {

// ---------------------------------------------------------------- NVFP4 --

// Partial tensor amax: group-strided over 16-element groups.
__global__ void __launch_bounds__(256)
nvfp4_amax_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
                  float* __restrict__ partial) {
  const int64_t gpr = K / 16;
  const int64_t groups = M * gpr;
  uint32_t mx = 0;                                  // max of |bf16| bit patterns
  for (int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gi < groups;
       gi += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = gi / gpr, g = gi - m * gpr;
    const u32x4* p = reinterpret_cast<const u32x4*>(x + m * ldx + g * 16);
    u32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mx = max(mx, max(a[i] & 0x7FFFu, (a[i] >> 16) & 0x7FFFu));
      mx = max(mx, max(b[i] & 0x7FFFu, (b[i] >> 16) & 0x7FFFu));
    }
  }
  float v = wave_max(__uint_as_float(mx << 16));
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0)
    partial[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Encoder: one 16-element group per thread.  s_T from the partial maxima
// (or *tscale when given); workgroup 0 publishes s_T.
__global__ void __launch_bounds__(256)
nvfp4_encode_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
                    uint8_t* __restrict__ q, uint8_t* __restrict__ scales,
                    float* __restrict__ tscale, const float* __restrict__ partial,
                    int nparts, int given) {
  __shared__ float red[4];
  float s_t;
  if (given) {
    s_t = *tscale;
  } else {
    float v = 0.0f;
    for (int i = threadIdx.x; i < nparts; i += blockDim.x) v = fmaxf(v, partial[i]);
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    s_t = amax / 2688.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0) *tscale = s_t;
  }
  const float g = recip0(6.0f * s_t);
  const int64_t gpr = K / 16;
  const int64_t groups = M * gpr;
  for (int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gi < groups;
       gi += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = gi / gpr, gg = gi - m * gpr;
    const u32x4* p = reinterpret_cast<const u32x4*>(x + m * ldx + gg * 16);
    u32x4 a = p[0], b = p[1];
    uint32_t w[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) mx = max(mx, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
    const float amax_g = __uint_as_float(mx << 16);
    const uint32_t enc = e4m3_encode(amax_g * g);
    const float inv = recip0(e4m3_decode(enc) * s_t);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t c0 = e2m1_encode(bf16_lo(w[i]) * inv);
      const uint32_t c1 = e2m1_encode(bf16_hi(w[i]) * inv);
      lo |= (c0 | (c1 << 4)) << (8 * i);
      const uint32_t c2 = e2m1_encode(bf16_lo(w[i + 4]) * inv);
      const uint32_t c3 = e2m1_encode(bf16_hi(w[i + 4]) * inv);
      hi |= (c2 | (c3 << 4)) << (8 * i);
    }
    u32x2 out = {lo, hi};
    *reinterpret_cast<u32x2*>(q + m * (K / 2) + gg * 8) = out;
    scales[m * gpr + gg] = (uint8_t)enc;
  }
}

// ----------------------------------------------------------------- INT8 --

// One wave per token row: row |x| max, then q = clamp(rint(x * inv)).
__global__ void __launch_bounds__(256)
int8_encode_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
                   int8_t* __restrict__ q, float* __restrict__ scale) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const uint16_t* xr = x + row * ldx;
  const int64_t nvec = K / 8;                       // 8 bf16 per 16-byte vector
  uint32_t mx = 0;
  for (int64_t v = lane; v < nvec; v += 64) {
    u32x4 a = reinterpret_cast<const u32x4*>(xr)[v];
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = max(mx, max(a[i] & 0x7FFFu, (a[i] >> 16) & 0x7FFFu));
  }
  const float amax = wave_max(__uint_as_float(mx << 16));
  const float s = amax / 127.0f;
  const float inv = recip0(s);
  int8_t* qr = q + row * K;
  for (int64_t v = lane; v < nvec; v += 64) {
    u32x4 a = reinterpret_cast<const u32x4*>(xr)[v];
    uint32_t packed[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float f0 = fminf(fmaxf(rintf(bf16_lo(a[i]) * inv), -127.0f), 127.0f);
      float f1 = fminf(fmaxf(rintf(bf16_hi(a[i]) * inv), -127.0f), 127.0f);
      uint32_t b = ((uint32_t)(int32_t)f0 & 0xFFu) | (((uint32_t)(int32_t)f1 & 0xFFu) << 8);
      packed[i >> 1] |= b << (16 * (i & 1));
    }
    u32x2 o = {packed[0], packed[1]};
    reinterpret_cast<u32x2*>(qr)[v] = o;
  }
  if (lane == 0) scale[row] = s;
}

// ----------------------------------------------------------------- host --

static constexpr int kAmaxBlocks = 1024;

size_t nvfp4_quant_ws_bytes(int64_t, int64_t) { return kAmaxBlocks * sizeof(float); }

hipError_t launch_nvfp4_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                              uint8_t* q, uint8_t* scales, float* tscale, bool given,
                              void* ws, hipStream_t stream) {
  const int64_t groups = M * (K / 16);
  int64_t want = (groups + 255) / 256;
  int nblk = (int)(want < kAmaxBlocks ? (want < 1 ? 1 : want) : kAmaxBlocks);
  float* partial = static_cast<float*>(ws);
  if (!given) {
    hipLaunchKernelGGL(nvfp4_amax_kernel, dim3(nblk), dim3(256), 0, stream, x, M, K, ldx,
                       partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  int64_t eblk = (groups + 255) / 256;
  if (eblk > 8192) eblk = 8192;
  if (eblk < 1) eblk = 1;
  hipLaunchKernelGGL(nvfp4_encode_kernel, dim3((unsigned)eblk), dim3(256), 0, stream, x, M,
                     K, ldx, q, scales, tscale, partial, nblk, given ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_int8_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                             float* scale, hipStream_t stream) {
  const int64_t blocks = (M + 3) / 4;
  hipLaunchKernelGGL(int8_encode_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, M, K,
                     ldx, q, scale);
  return hipGetLastError();
}

}  // namespace qact
