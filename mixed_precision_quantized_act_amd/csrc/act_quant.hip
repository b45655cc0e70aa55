// Activation quantization kernels for gfx950: NVFP4 (E2M1 + E4M3 per 16 +
// float32 tensor scale) and per-token symmetric INT8.  6Bit-Diffusion,
// abstract: activations of each linear are quantized at inference time to
// NVFP4 or INT8; Fig. 2 caption: the choice is per linear layer.
//
// All kernels stream bf16 with 16-byte loads.  NVFP4 runs two passes: a
// tensor |x| max (per-workgroup partial maxima into scratch) and the
// encoder, whose workgroups each fold the partial maxima into s_T before
// encoding four 16-element groups per thread.  INT8 gives each token row
// to one wave: the row stays in registers between the row max (wave
// shuffles) and the encode, so it is read from memory once.
#include "qact_device.h"
#include "qact_internal.h"

namespace qact {

// ---------------------------------------------------------------- NVFP4 --

static constexpr int kUnroll = 4;

__device__ __forceinline__ uint32_t abs_max8(u32x4 a, uint32_t mx) {
  return max(mx, fold_max(abs_max8_pk(a, u16x2{0, 0})));
}

__device__ __forceinline__ void block_max_to(float v, float* dst) {
  __shared__ float red[4];
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) *dst = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Partial tensor amax.  CONTIG (ldx == K): one flat sweep of 16-byte
// vectors, kUnroll per thread in flight; otherwise row by row.
template <bool CONTIG>
__global__ void __launch_bounds__(256)
nvfp4_amax_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
                  float* __restrict__ partial) {
  uint32_t mx = 0;
  if (CONTIG) {
    const int64_t nvec = M * K / 8;
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    for (int64_t v0 = (int64_t)blockIdx.x * 256 * kUnroll + threadIdx.x; v0 < nvec;
         v0 += (int64_t)gridDim.x * 256 * kUnroll) {
      u32x4 r[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t v = v0 + u * 256;
        r[u] = v < nvec ? xv[v] : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) mx = abs_max8(r[u], mx);
    }
  } else {
    for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
      const u32x4* xv = reinterpret_cast<const u32x4*>(x + row * ldx);
      for (int64_t v = threadIdx.x; v < K / 8; v += 256) mx = abs_max8(xv[v], mx);
    }
  }
  block_max_to(__uint_as_float(mx << 16), partial + blockIdx.x);
}

// Encoder: G consecutive 16-element groups of one row per thread (G = 4
// when K % 64 == 0: 128 bytes read, 32 bytes of codes and one 32-bit word
// of scales written).  s_T from the partial maxima (or *tscale when
// given); workgroup 0 publishes s_T.
template <int G>
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
  const uint32_t cpr = (uint32_t)(K / (16 * G));          // thread chunks per row
  const uint64_t total = (uint64_t)M * cpr;
  for (uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (uint64_t)gridDim.x * blockDim.x) {
    const uint64_t row = total < 0xFFFFFFFFull ? (uint32_t)t / cpr : t / cpr;
    const uint32_t c = (uint32_t)(t - row * cpr);
    const u32x4* p = reinterpret_cast<const u32x4*>(x + row * ldx + (int64_t)c * 16 * G);
    u32x4 w[2 * G];
#pragma unroll
    for (int i = 0; i < 2 * G; ++i) w[i] = p[i];
    uint32_t sc_word = 0;
    u32x2 codes[G];
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      const uint32_t mx = fold_max(abs_max8_pk(w[2 * gg + 1], abs_max8_pk(w[2 * gg], u16x2{0, 0})));
      const uint32_t enc = e4m3_encode(__uint_as_float(mx << 16) * g);
      const float inv = recip0(e4m3_decode(enc) * s_t);
      codes[gg] = u32x2{e2m1_pack8(w[2 * gg], inv), e2m1_pack8(w[2 * gg + 1], inv)};
      sc_word |= enc << (8 * gg);
    }
    uint8_t* qp = q + row * (K / 2) + (int64_t)c * 8 * G;
    if (G == 4) {
      reinterpret_cast<u32x4*>(qp)[0] = u32x4{codes[0][0], codes[0][1], codes[1][0], codes[1][1]};
      reinterpret_cast<u32x4*>(qp)[1] = u32x4{codes[2][0], codes[2][1], codes[3][0], codes[3][1]};
      *reinterpret_cast<uint32_t*>(scales + row * (K / 16) + c * G) = sc_word;
    } else {
#pragma unroll
      for (int gg = 0; gg < G; ++gg) {
        reinterpret_cast<u32x2*>(qp)[gg] = codes[gg];
        scales[row * (K / 16) + c * G + gg] = (uint8_t)(sc_word >> (8 * gg));
      }
    }
  }
}

// ----------------------------------------------------------------- INT8 --

__device__ __forceinline__ u32x2 int8_pack8(u32x4 a, float inv) {
  uint32_t packed[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float f0 = fminf(fmaxf(rintf(bf16_lo(a[i]) * inv), -127.0f), 127.0f);
    const float f1 = fminf(fmaxf(rintf(bf16_hi(a[i]) * inv), -127.0f), 127.0f);
    const uint32_t b = ((uint32_t)(int32_t)f0 & 0xFFu) | (((uint32_t)(int32_t)f1 & 0xFFu) << 8);
    packed[i >> 1] |= b << (16 * (i & 1));
  }
  return u32x2{packed[0], packed[1]};
}

// One wave per token row.  VPL > 0: the row (at most VPL 16-byte vectors
// per lane) is held in registers between the row max and the encode, so
// it is read once; VPL == 0: any K, the row is read twice.
template <int VPL>
__global__ void __launch_bounds__(256)
int8_encode_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
                   int8_t* __restrict__ q, float* __restrict__ scale) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + row * ldx);
  u32x2* qr = reinterpret_cast<u32x2*>(q + row * K);
  const int64_t nvec = K / 8;
  uint32_t mx = 0;
  if (VPL > 0) {
    u32x4 r[VPL > 0 ? VPL : 1];
#pragma unroll
    for (int u = 0; u < VPL; ++u) {
      const int64_t v = lane + u * 64;
      r[u] = v < nvec ? xr[v] : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < VPL; ++u) mx = abs_max8(r[u], mx);
    const float s = wave_max(__uint_as_float(mx << 16)) / 127.0f;
    const float inv = recip0(s);
#pragma unroll
    for (int u = 0; u < VPL; ++u) {
      const int64_t v = lane + u * 64;
      if (v < nvec) qr[v] = int8_pack8(r[u], inv);
    }
    if (lane == 0) scale[row] = s;
  } else {
    for (int64_t v = lane; v < nvec; v += 64) mx = abs_max8(xr[v], mx);
    const float s = wave_max(__uint_as_float(mx << 16)) / 127.0f;
    const float inv = recip0(s);
    for (int64_t v = lane; v < nvec; v += 64) qr[v] = int8_pack8(xr[v], inv);
    if (lane == 0) scale[row] = s;
  }
}

// ----------------------------------------------------------------- host --

static constexpr int kAmaxBlocks = 1024;

size_t nvfp4_quant_ws_bytes(int64_t, int64_t) { return kAmaxBlocks * sizeof(float); }

hipError_t launch_nvfp4_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                              uint8_t* q, uint8_t* scales, float* tscale, bool given,
                              void* ws, hipStream_t stream) {
  float* partial = static_cast<float*>(ws);
  int nblk = 1;
  if (!given) {
    const bool contig = ldx == K;
    const int64_t work = contig ? (M * K / 8 + 256 * kUnroll - 1) / (256 * kUnroll) : M;
    nblk = (int)(work < kAmaxBlocks ? (work < 1 ? 1 : work) : kAmaxBlocks);
    if (contig)
      hipLaunchKernelGGL(nvfp4_amax_kernel<true>, dim3(nblk), dim3(256), 0, stream, x, M, K,
                         ldx, partial);
    else
      hipLaunchKernelGGL(nvfp4_amax_kernel<false>, dim3(nblk), dim3(256), 0, stream, x, M, K,
                         ldx, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const bool g4 = K % 64 == 0 && (reinterpret_cast<uintptr_t>(scales) & 3u) == 0;
  const int64_t chunks = M * (K / (g4 ? 64 : 16));
  int64_t eblk = (chunks + 255) / 256;
  if (eblk > 8192) eblk = 8192;
  if (eblk < 1) eblk = 1;
  if (g4)
    hipLaunchKernelGGL(nvfp4_encode_kernel<4>, dim3((unsigned)eblk), dim3(256), 0, stream, x, M,
                       K, ldx, q, scales, tscale, partial, nblk, given ? 1 : 0);
  else
    hipLaunchKernelGGL(nvfp4_encode_kernel<1>, dim3((unsigned)eblk), dim3(256), 0, stream, x, M,
                       K, ldx, q, scales, tscale, partial, nblk, given ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_int8_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                             float* scale, hipStream_t stream) {
  const dim3 g((unsigned)((M + 3) / 4)), t(256);
  const int64_t vpl = (K / 8 + 63) / 64;
  if (vpl <= 1)
    hipLaunchKernelGGL(int8_encode_kernel<1>, g, t, 0, stream, x, M, K, ldx, q, scale);
  else if (vpl <= 2)
    hipLaunchKernelGGL(int8_encode_kernel<2>, g, t, 0, stream, x, M, K, ldx, q, scale);
  else if (vpl <= 4)
    hipLaunchKernelGGL(int8_encode_kernel<4>, g, t, 0, stream, x, M, K, ldx, q, scale);
  else if (vpl <= 8)
    hipLaunchKernelGGL(int8_encode_kernel<8>, g, t, 0, stream, x, M, K, ldx, q, scale);
  else if (vpl <= 16)
    hipLaunchKernelGGL(int8_encode_kernel<16>, g, t, 0, stream, x, M, K, ldx, q, scale);
  else
    hipLaunchKernelGGL(int8_encode_kernel<0>, g, t, 0, stream, x, M, K, ldx, q, scale);
  return hipGetLastError();
}

}  // namespace qact
