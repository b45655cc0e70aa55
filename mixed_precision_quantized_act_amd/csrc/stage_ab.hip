// Test and benchmark only: the compute stage of three designs of the
// NVFP4 x NVFP4 linear on gfx950, on register-resident operands, so that
// their MFMA + VALU cost per multiply-accumulate can be compared without
// the memory side (which reads the same 4-bit codes and E4M3 scales in all
// three).  6Bit-Diffusion, abstract: NVFP4 activations against NVFP4
// weights, one E4M3 scale per 16 elements.
//
// One iteration is one 16-element scale group of K for a wave's tile:
//   design 0 (D, the library's): both operands expanded exactly to fp16
//     with their group scales (E2M1 x E4M3 is exact in fp16), then
//     v_mfma_f32_32x32x16_f16 accumulating across groups; 4 x 4 tiles of
//     32 x 32 per wave, accumulators in AGPRs;
//   design 1 (S): the codes as fp8 (E2M1 values are exact in E4M3), one
//     v_mfma_f32_32x32x16_fp8_fp8 per group from zero, and the group's
//     partial product rescaled into the accumulators by s_a s_w per output
//     (a multiply and an FMA per output); 2 x 4 tiles, accumulators in VGPRs;
//   design 2 (S'): activations expanded with their scale to fp16 as in D,
//     weight codes to fp16 without scale, v_mfma_f32_32x32x16_f16 per group
//     from zero, rescaled by s_w per output (one FMA); 2 x 4 tiles.
// Operand layout (per lane l, MFMA issued as W x A^T): an operand holds row
// l % 32 of its 32-row tile, K elements 8 (l / 32) .. +7 of the group;
// accumulator r of tile (i, j) is output (W row 8 (r / 4) + 4 (l / 32) +
// r % 4 of tile j, A row l % 32 of tile i).
#include "qgemm_common.h"

namespace qact {

namespace {

typedef __attribute__((ext_vector_type(2))) _Float16 h2;

// 8 E2M1 codes -> 8 fp16 times the fp16 scale pair (exact)
__device__ __forceinline__ f16x8 fp4x8_f16(uint32_t w, h2 sc) {
  const h2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sc;
  const h2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sc;
  const h2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sc;
  const h2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sc;
  return f16x8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

__device__ __forceinline__ h2 e4m3_h2(uint32_t byte) {
  const h2 two = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(byte, 1.0f, false);
  return h2{two[0], two[0]};
}

template <typename T>
__device__ __forceinline__ void opaque(T& v) {
  asm volatile("" : "+v"(v));
}

// Per-lane input block (64 words), by design:
//   D:  words 0-3 A codes (tiles 0-3), 4-7 W codes, 8-11 A scale bytes,
//       12-15 W scale bytes (in the low byte);
//   S:  words 0-3 A fp8 (tiles 0, 1: 8 bytes each), 4-11 W fp8 (tiles
//       0-3), 12-13 s_a (float bits, tiles 0, 1);
//   S': words 0-1 A codes (tiles 0, 1), 2 A scale bytes (byte i for tile
//       i), 4-7 W codes;
//   S and S': s_w of accumulator r of W tile j at word 16 + 16 (j % 3) + r
//       (float bits; tile 3 reuses tile 0's).
template <int DESIGN>
__global__ void __launch_bounds__(256)
stage_kernel(const uint32_t* __restrict__ in, float* __restrict__ out, int iters) {
  const int gtid = (int)(blockIdx.x * 256 + threadIdx.x);
  const uint32_t* blk = in + (size_t)(gtid % 1024) * 64;
  float* dst = out + (size_t)(gtid % 1024) * 256;
  if constexpr (DESIGN == 0) {
    uint32_t ac[4], wc[4], as[4], ws[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ac[i] = blk[i];
      wc[i] = blk[4 + i];
      as[i] = blk[8 + i];
      ws[i] = blk[12 + i];
    }
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        opaque(ac[i]);
        opaque(wc[i]);
        opaque(as[i]);
        opaque(ws[i]);
      }
      f16x8 a[4], w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = fp4x8_f16(ac[i], e4m3_h2(as[i]));
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = fp4x8_f16(wc[j], e4m3_h2(ws[j]));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(w[j], a[i], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[(i * 4 + j) * 16 + r] = acc[i][j][r];
  } else {
    float sw[4][16];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) sw[j][r] = __uint_as_float(blk[16 + 16 * (j % 3) + r]);
    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    f32x16 zero;
#pragma unroll
    for (int r = 0; r < 16; ++r) zero[r] = 0.0f;
    if constexpr (DESIGN == 1) {
      long a8[2], w8[4];
      float sa[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a8[i] = (long)(((uint64_t)blk[2 * i + 1] << 32) | blk[2 * i]);
        sa[i] = __uint_as_float(blk[12 + i]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) w8[j] = (long)(((uint64_t)blk[4 + 2 * j + 1] << 32) | blk[4 + 2 * j]);
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          opaque(a8[i]);
          opaque(sa[i]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          opaque(w8[j]);
#pragma unroll
          for (int r = 0; r < 16; ++r) opaque(sw[j][r]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x16 p = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(w8[j], a8[i], zero, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(p[r], sa[i] * sw[j][r], acc[i][j][r]);
          }
      }
    } else {
      uint32_t ac[2], wc[4], as = blk[2];
      ac[0] = blk[0];
      ac[1] = blk[1];
#pragma unroll
      for (int j = 0; j < 4; ++j) wc[j] = blk[4 + j];
      const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
      for (int it = 0; it < iters; ++it) {
        opaque(ac[0]);
        opaque(ac[1]);
        opaque(as);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          opaque(wc[j]);
#pragma unroll
          for (int r = 0; r < 16; ++r) opaque(sw[j][r]);
        }
        f16x8 a[2], w[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) a[i] = fp4x8_f16(ac[i], e4m3_h2((as >> (8 * i)) & 0xFFu));
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = fp4x8_f16(wc[j], one);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x16 p = __builtin_amdgcn_mfma_f32_32x32x16_f16(w[j], a[i], zero, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(p[r], sw[j][r], acc[i][j][r]);
          }
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[(i * 4 + j) * 16 + r] = acc[i][j][r];
  }
}

}  // namespace

hipError_t launch_stage_ab(int design, int iters, int blocks, const uint32_t* in, float* out,
                           hipStream_t stream) {
  const dim3 g((unsigned)blocks), t(256);
  if (design == 0)
    hipLaunchKernelGGL(stage_kernel<0>, g, t, 0, stream, in, out, iters);
  else if (design == 1)
    hipLaunchKernelGGL(stage_kernel<1>, g, t, 0, stream, in, out, iters);
  else
    hipLaunchKernelGGL(stage_kernel<2>, g, t, 0, stream, in, out, iters);
  return hipGetLastError();
}

}  // namespace qact
