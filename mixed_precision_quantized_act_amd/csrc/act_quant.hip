// Activation quantization kernels for gfx950: NVFP4 (E2M1 + E4M3 per 16 +
// float32 tensor scale) and per-token symmetric INT8.  6Bit-Diffusion,
// abstract: activations of each linear are quantized at inference time to
// NVFP4 or INT8; Fig. 2 caption: the choice is per linear layer.
//
// All kernels stream bf16 with 16-byte loads.  NVFP4 runs two passes: a
// tensor |x| max (per-workgroup partial maxima into scratch) and the
// encoder.  The encoder gives each lane one 16-byte vector (half a
// 16-element group) per load, so that a wave's load covers 1 KB of
// consecutive memory; the two halves of a group sit in neighbouring lanes,
// which exchange their maxima through one DPP move.  Its first loads are
// issued before its workgroup folds the partial maxima into s_T.  INT8 gives each token row
// to one wave: the row stays in registers between the row max (wave
// shuffles) and the encode, so it is read from memory once.
#include "qact_device.h"
#include "qact_internal.h"

namespace qact {

// ---------------------------------------------------------------- NVFP4 --

static constexpr int kUnroll = 4;
static constexpr int kPartsMax = 1024;          // partial maxima of the amax pass, at most

__device__ __forceinline__ uint32_t abs_max8(u32x4 a, uint32_t mx) {
  return max(mx, fold_max(abs_max8_pk(a, u16x2{0, 0})));
}

// Max over the workgroup (at most 16 waves), written by thread 0.
__device__ __forceinline__ void block_max_to(float v, float* dst) {
  __shared__ float red[16];
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = red[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i) m = fmaxf(m, red[i]);
    *dst = m;
  }
}

// Partial tensor amax.  CONTIG (ldx == K): one flat sweep of 16-byte
// vectors, kUnroll per thread in flight; otherwise row by row.
template <bool CONTIG>
__global__ void __launch_bounds__(256)
nvfp4_amax_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
                  float* __restrict__ partial, Gate gate, Gate route) {
  if (gated_off(gate) || gated_off(route)) return;
  uint32_t mx = 0;
  if (CONTIG) {
    const int64_t nvec = M * K / 8;
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    const int64_t bs = blockDim.x;
    for (int64_t v0 = (int64_t)blockIdx.x * bs * kUnroll + threadIdx.x; v0 < nvec;
         v0 += (int64_t)gridDim.x * bs * kUnroll) {
      u32x4 r[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t v = v0 + u * bs;
        r[u] = v < nvec ? xv[v] : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) mx = abs_max8(r[u], mx);
    }
  } else {
    for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
      const u32x4* xv = reinterpret_cast<const u32x4*>(x + row * ldx);
      for (int64_t v = threadIdx.x; v < K / 8; v += blockDim.x) mx = abs_max8(xv[v], mx);
    }
  }
  block_max_to(__uint_as_float(mx << 16), partial + blockIdx.x);
}

// Encoder: vector v (8 bf16 of row v / (K/8), column 8 (v % (K/8))) goes
// to lane v % 256 of the workgroup's sweep, U vectors per lane in flight;
// s_T = amax / (6 * 448) unless given, then the steps of the NVFP4 encode
// per group (6Bit-Diffusion, abstract: one E4M3 scale per 16 elements and
// one float32 tensor scale).  K % 16 == 0, so a group is the even vector v and v + 1, held
// by lanes 2j and 2j+1.  Outputs are indexed by v alone: code word v of
// the [M][K/2] code array and scale byte v / 2 of the [M][K/16] scales.
// (run by workgroup `bid` of `nblk`; CONTIG: ldx == K, one flat index)
template <int U, bool CONTIG>
__device__ __forceinline__ void nvfp4_encode_body(const uint16_t* __restrict__ x, int64_t M,
                                                  int64_t K, int64_t ldx, uint8_t* __restrict__ q,
                                                  uint8_t* __restrict__ scales,
                                                  float* __restrict__ tscale,
                                                  const float* __restrict__ partial, int nparts,
                                                  int given, int bid, int nblk) {
  const int64_t vpr = K / 8;                               // vectors per row
  const int64_t nvec = M * vpr;
  const bool small = nvec <= 0xFFFFFFFFll;
  const int64_t sweep = (int64_t)nblk * 256 * U;
  const int64_t start = (int64_t)bid * 256 * U + threadIdx.x;
  auto load = [&](int64_t v0, u32x4 (&w)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + u * 256;
      int64_t off = v * 8;
      if constexpr (!CONTIG) {
        const int64_t row = small ? (int64_t)((uint32_t)v / (uint32_t)vpr) : v / vpr;
        off = row * ldx + (v - row * vpr) * 8;
      }
      w[u] = v < nvec ? *reinterpret_cast<const u32x4*>(x + off) : u32x4{0, 0, 0, 0};
    }
  };
  // s_T first -- given, or the tensor max folded from the amax pass's
  // partial maxima (measured faster than issuing the first loads ahead of
  // the fold) -- then the sweeps
  __shared__ float red[4];
  float s_t;
  if (given) {
    s_t = *tscale;
  } else {
    // at most kPartsMax partial maxima: all loads issued at once
    float pv[kPartsMax / 256];
#pragma unroll
    for (int j = 0; j < kPartsMax / 256; ++j) {
      const int i = threadIdx.x + 256 * j;
      pv[j] = i < nparts ? partial[i] : 0.0f;
    }
    float v = 0.0f;
#pragma unroll
    for (int j = 0; j < kPartsMax / 256; ++j) v = fmaxf(v, pv[j]);
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    s_t = amax / 2688.0f;
    if (bid == 0 && threadIdx.x == 0) *tscale = s_t;
  }
  const float g = recip0(6.0f * s_t);
  uint32_t* const q32 = reinterpret_cast<uint32_t*>(q);
  for (int64_t v0 = start; v0 < nvec; v0 += sweep) {
    u32x4 w[U];
    load(v0, w);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + u * 256;
      const uint32_t own = fold_max(abs_max8_pk(w[u], u16x2{0, 0}));
      // the partner lane's maximum: quad_perm [1, 0, 3, 2] swaps lanes 2j, 2j+1
      const uint32_t other = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)own, 0xB1, 0xF, 0xF, false);
      const uint32_t mx = max(own, other);
      const uint32_t enc = e4m3_encode(__uint_as_float(mx << 16) * g);
      const float inv = recip0(e4m3_decode(enc) * s_t);
      const uint32_t codes = e2m1_pack8(w[u], inv);
      if (v < nvec) {
        q32[v] = codes;
        if ((v & 1) == 0) scales[v >> 1] = (uint8_t)enc;
      }
    }
  }
}

template <int U, bool CONTIG>
__global__ void __launch_bounds__(256)
nvfp4_encode_vec_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
                        uint8_t* __restrict__ q, uint8_t* __restrict__ scales,
                        float* __restrict__ tscale, const float* __restrict__ partial,
                        int nparts, int given, Gate gate) {
  if (gated_off(gate)) return;
  nvfp4_encode_body<U, CONTIG>(x, M, K, ldx, q, scales, tscale, partial, nparts, given,
                               (int)blockIdx.x, (int)gridDim.x);
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
__device__ __forceinline__ void int8_encode_row(const uint16_t* __restrict__ x, int64_t row,
                                                int64_t K, int64_t ldx, int8_t* __restrict__ q,
                                                float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
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

template <int VPL>
__global__ void __launch_bounds__(256)
int8_encode_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
                   int8_t* __restrict__ q, float* __restrict__ scale, Gate gate) {
  if (gated_off(gate)) return;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row < M) int8_encode_row<VPL>(x, row, K, ldx, q, scale);
}

// ---------------------------------------------------------------- routed --

// One launch for either format, the format read from the device byte
// *route (kRouteNvfp4: the NVFP4 encoder on its first nvfp4_blocks
// workgroups, with a given tensor scale or the partial maxima in `partial`;
// kRouteInt8: every workgroup takes token rows 4 b + wave, 4 (b + grid) +
// wave, ...; neither: nothing).  6Bit-Diffusion, Fig. 2 caption: the format
// of each linear's activations is chosen per timestep.
template <int U, int VPL>
__global__ void __launch_bounds__(256)
act_quant_routed_kernel(const uint8_t* __restrict__ route, const uint16_t* __restrict__ x,
                        int64_t M, int64_t K, int64_t ldx, uint8_t* __restrict__ q4,
                        uint8_t* __restrict__ s4, float* __restrict__ ts4,
                        const float* __restrict__ partial, int nparts, int given,
                        int nvfp4_blocks, int8_t* __restrict__ q8, float* __restrict__ s8,
                        Gate gate) {
  if (gated_off(gate)) return;
  const uint32_t r = *route;
  if (r & kRouteNvfp4) {
    if ((int)blockIdx.x < nvfp4_blocks) {
      if (ldx == K)
        nvfp4_encode_body<U, true>(x, M, K, ldx, q4, s4, ts4, partial, nparts, given,
                                   (int)blockIdx.x, nvfp4_blocks);
      else
        nvfp4_encode_body<U, false>(x, M, K, ldx, q4, s4, ts4, partial, nparts, given,
                                    (int)blockIdx.x, nvfp4_blocks);
    }
  } else if (r & kRouteInt8) {
    for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < M;
         row += (int64_t)gridDim.x * 4)
      int8_encode_row<VPL>(x, row, K, ldx, q8, s8);
  }
}

// ----------------------------------------------------------------- host --

static constexpr int kAmaxBlocks = 1024;
static_assert(kAmaxBlocks <= kPartsMax && kAmaxSlots <= kPartsMax,
              "encoder folds at most kPartsMax partial maxima");
static_assert(kAmaxSlots <= kAmaxBlocks, "the workspace holds the producer's slots");
// encoder: vectors in flight per lane, and at most this many workgroups
// (one resident round; measured against 2 vectors per lane and an uncapped
// grid, which pay the s_T fold again in every later workgroup)
static constexpr int kEncU = 4;
static constexpr int kEncBlocks = 2048;

size_t nvfp4_quant_ws_bytes(int64_t, int64_t) { return kAmaxBlocks * sizeof(float); }

hipError_t launch_nvfp4_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                              uint8_t* q, uint8_t* scales, float* tscale, bool given,
                              bool amax_given, void* ws, hipStream_t stream) {
  const Gate gt = current_gate();
  float* partial = static_cast<float*>(ws);
  int nblk = kAmaxSlots;         // amax_given: the producer's partial maxima in ws
  if (!given && !amax_given) {
    const bool contig = ldx == K;
    const int64_t work = contig ? (M * K / 8 + 256 * kUnroll - 1) / (256 * kUnroll) : M;
    nblk = (int)(work < kAmaxBlocks ? (work < 1 ? 1 : work) : kAmaxBlocks);
    if (contig)
      hipLaunchKernelGGL(nvfp4_amax_kernel<true>, dim3(nblk), dim3(256), 0, stream, x, M, K,
                         ldx, partial, gt, Gate{nullptr, 0u});
    else
      hipLaunchKernelGGL(nvfp4_amax_kernel<false>, dim3(nblk), dim3(256), 0, stream, x, M, K,
                         ldx, partial, gt, Gate{nullptr, 0u});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  int64_t eblk = (M * (K / 8) + 256 * kEncU - 1) / (256 * kEncU);
  if (eblk > kEncBlocks) eblk = kEncBlocks;
  if (eblk < 1) eblk = 1;
  if (ldx == K)
    hipLaunchKernelGGL((nvfp4_encode_vec_kernel<kEncU, true>), dim3((unsigned)eblk), dim3(256), 0,
                       stream, x, M, K, ldx, q, scales, tscale, partial, nblk, given ? 1 : 0, gt);
  else
    hipLaunchKernelGGL((nvfp4_encode_vec_kernel<kEncU, false>), dim3((unsigned)eblk), dim3(256),
                       0, stream, x, M, K, ldx, q, scales, tscale, partial, nblk, given ? 1 : 0,
                       gt);
  return hipGetLastError();
}

hipError_t launch_int8_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                             float* scale, hipStream_t stream) {
  const Gate gt = current_gate();
  const dim3 g((unsigned)((M + 3) / 4)), t(256);
  const int64_t vpl = (K / 8 + 63) / 64;
  if (vpl <= 1)
    hipLaunchKernelGGL(int8_encode_kernel<1>, g, t, 0, stream, x, M, K, ldx, q, scale, gt);
  else if (vpl <= 2)
    hipLaunchKernelGGL(int8_encode_kernel<2>, g, t, 0, stream, x, M, K, ldx, q, scale, gt);
  else if (vpl <= 4)
    hipLaunchKernelGGL(int8_encode_kernel<4>, g, t, 0, stream, x, M, K, ldx, q, scale, gt);
  else if (vpl <= 8)
    hipLaunchKernelGGL(int8_encode_kernel<8>, g, t, 0, stream, x, M, K, ldx, q, scale, gt);
  else if (vpl <= 16)
    hipLaunchKernelGGL(int8_encode_kernel<16>, g, t, 0, stream, x, M, K, ldx, q, scale, gt);
  else
    hipLaunchKernelGGL(int8_encode_kernel<0>, g, t, 0, stream, x, M, K, ldx, q, scale, gt);
  return hipGetLastError();
}

// the INT8 rows per wave held in registers: 16-byte vectors per lane
static int int8_vpl(int64_t K) {
  const int64_t vpl = (K / 8 + 63) / 64;
  return vpl <= 1 ? 1 : vpl <= 2 ? 2 : vpl <= 4 ? 4 : vpl <= 8 ? 8 : vpl <= 16 ? 16 : 0;
}

hipError_t launch_act_quant_routed(const uint8_t* route, const uint16_t* x, int64_t M, int64_t K,
                                   int64_t ldx, uint8_t* q4, uint8_t* s4, float* ts4, bool given,
                                   bool amax_given, void* ws, int8_t* q8, float* s8,
                                   hipStream_t stream) {
  const Gate gt = current_gate();
  float* partial = static_cast<float*>(ws);
  int nblk = kAmaxSlots;
  if (!given && !amax_given) {
    // the tensor-max pass, run only when the route byte selects NVFP4
    const Gate rg = {route, kRouteNvfp4};
    const bool contig = ldx == K;
    const int64_t work = contig ? (M * K / 8 + 256 * kUnroll - 1) / (256 * kUnroll) : M;
    nblk = (int)(work < kAmaxBlocks ? (work < 1 ? 1 : work) : kAmaxBlocks);
    if (contig)
      hipLaunchKernelGGL(nvfp4_amax_kernel<true>, dim3(nblk), dim3(256), 0, stream, x, M, K, ldx,
                         partial, gt, rg);
    else
      hipLaunchKernelGGL(nvfp4_amax_kernel<false>, dim3(nblk), dim3(256), 0, stream, x, M, K,
                         ldx, partial, gt, rg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  int64_t eblk = (M * (K / 8) + 256 * kEncU - 1) / (256 * kEncU);
  if (eblk > kEncBlocks) eblk = kEncBlocks;
  if (eblk < 1) eblk = 1;
  const int64_t rows_blk = (M + 3) / 4;
  const int64_t grid = rows_blk > eblk ? (rows_blk < 65535 ? rows_blk : 65535) : eblk;
  const dim3 g((unsigned)grid), t(256);
#define QACT_ROUTED(V)                                                                          \
  hipLaunchKernelGGL((act_quant_routed_kernel<kEncU, V>), g, t, 0, stream, route, x, M, K, ldx, \
                     q4, s4, ts4, partial, nblk, given ? 1 : 0, (int)eblk, q8, s8, gt)
  switch (int8_vpl(K)) {
    case 1: QACT_ROUTED(1); break;
    case 2: QACT_ROUTED(2); break;
    case 4: QACT_ROUTED(4); break;
    case 8: QACT_ROUTED(8); break;
    case 16: QACT_ROUTED(16); break;
    default: QACT_ROUTED(0); break;
  }
#undef QACT_ROUTED
  return hipGetLastError();
}

}  // namespace qact
