// Pieces shared by the two GEMM kernels of libqact (the fp16-MFMA kernel
// for NVFP4 or INT8 activations and the i8-MFMA kernel of the INT8 path):
// raw buffer loads into LDS, the output epilogues and their arguments.
#pragma once

#include <type_traits>

#include "qact_device.h"
#include "qact_internal.h"
#include "tile_order.h"

namespace qact {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(16))) int i32x16;

#ifndef QACT_EPI_ROWS
#define QACT_EPI_ROWS 32
#endif
// rows of a wave's output staged per pass of the bf16 epilogue
static constexpr int kPassTiles = QACT_EPI_ROWS / 32;

// Raw buffer (stride 0) over [base, base + bytes): loads at offsets >=
// bytes return zero.  Both values must be wave-uniform; they are passed
// through readfirstlane so that the descriptor lives in scalar registers
// (a descriptor the compiler cannot prove uniform turns every load into a
// loop over the distinct descriptors of the wave).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, (int)n, 0x00020000);
}

// 16 (or 4) bytes per lane from a buffer straight into LDS: lane l's bytes
// land at lds + 16 l (4 l); the LDS address is wave-uniform, through M0.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds, 16, (int)off, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds, 4, (int)off, 0, 0, 0);
}

// Wait until at most n vector-memory operations of this wave are in flight.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// GELU, tanh form: 0.5 v (1 + tanh u) = v / (1 + exp(-2u)) with
// u = sqrt(2/pi) (v + 0.044715 v^3); exp and the reciprocal are the
// hardware's (about 1 ulp each in float32).  Large negative v gives
// 1/inf = 0, large positive v gives v.
__device__ __forceinline__ float gelu_tanh(float v) {
  const float u = 0.7978845608028654f * (v + 0.044715f * v * v * v);
  const float ex = __builtin_amdgcn_exp2f(-2.0f * 1.4426950408889634f * u);
  return v * __builtin_amdgcn_rcpf(1.0f + ex);
}

struct EpiArgs {
  void* y;
  int64_t ldy;
  int out_f32;
  int gelu;
  const uint16_t* bias;
  int64_t M, N;
  int vec_ok;            // y 16-byte aligned and ldy % 4 == 0: vector stores
  uint8_t* yq;           // NVFP4 output: codes [M][N/2], scales [M][N/16],
  uint8_t* ys;           // with the given tensor scale *y_ts
  const float* y_ts;
  uint32_t* amax;        // bf16 staged output: |max| of the stored values (float bits), atomic max
};

// Epilogue kinds (one kernel each, so that the executed epilogue code stays
// compact): bf16 output with 16-byte aligned rows staged through LDS (no
// bias or GELU, bias, GELU, both); any output stored from registers;
// NVFP4-quantized output.
enum {
  kEpiPlain = 0,
  kEpiGeneral = 1,
  kEpiQuant = 2,
  kEpiStagedBias = 3,
  kEpiStagedGelu = 4,
  kEpiStagedBiasGelu = 5,
  // the staged kinds plus the |max| of the stored outputs: kind + kEpiAmax
  kEpiAmax = 6
};
__host__ __device__ constexpr bool epi_amax(int k) { return k >= kEpiAmax; }
__host__ __device__ constexpr int epi_base(int k) {
  return k < kEpiAmax ? k : (k == kEpiAmax ? kEpiPlain : k - kEpiAmax);
}
__host__ __device__ constexpr bool epi_staged(int k) {
  return epi_base(k) == kEpiPlain || epi_base(k) >= kEpiStagedBias;
}

// ------------------------------------------------------------- epilogue --

// Output of one wave's (32 FM) x 128 block: the wave's rows start at
// wave_row0, its columns at wave_col0.  acc(i, j, r) gives the float32 sum
// in register r of MFMA tile (i, j) as an MFMA issued W x A^T leaves it
// (acc_in: the accumulator array, or a callable giving that sum):
// lane (h, c) = (lane / 32, lane % 32) of tile (i, j) owns row 32 i + c
// and, for q = 0..3, the 4 consecutive columns 32 j + 8 q + 4 h .. +3
// (registers 4 q .. 4 q + 3); it is called where the value is consumed, so
// that values derived from the accumulators need not all be live.  Every output
// is acc * rs[i] (the row's scale), then + bias, then GELU, then rounded to
// the output type; rows and columns past the output read the last valid
// bias entry and are never stored.  stg: this wave's 8 KB (per pass of 32
// rows) of idle LDS for the staged bf16 kinds.
template <int kEpi, int FM, class Acc>
__device__ __forceinline__ void store_tile(const Acc& acc_in, const float (&rs)[FM],
                                           int64_t wave_row0, int64_t wave_col0, uint8_t* stg,
                                           const EpiArgs& e, int lane) {
  // Acc: the f32x16 [FM][4] accumulators themselves (read here: passing
  // them through a caller's lambda measured a few spilled registers in the
  // fp16 kernel) or a callable (i, j, r) -> float
  auto acc = [&](int i, int j, int r) -> float {
    if constexpr (std::is_array<Acc>::value)
      return acc_in[i][j][r];
    else
      return acc_in(i, j, r);
  };
  const int c = lane & 31, lh = lane >> 5;
  if constexpr (epi_staged(kEpi)) {
    // bf16 staged per 32-row slice through this wave's own 8 KB of the idle
    // ring -- rows of 256 bytes, 16-byte chunk k of row r at slot k ^ (r &
    // 15) -- and stored as 4 rows x 256 contiguous bytes per instruction
    constexpr int kB = epi_base(kEpi);
    constexpr bool kBias = kB == kEpiStagedBias || kB == kEpiStagedBiasGelu;
    constexpr bool kGelu = kB == kEpiStagedGelu || kB == kEpiStagedBiasGelu;
    uint32_t amx = 0;        // |max| of this lane's stored values (bf16 patterns)
    // bias of the lane's 64 columns (columns past N read column N-1)
    float bv[kBias ? 4 : 1][4][4];
    if constexpr (kBias)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            bv[j][q][t] = __uint_as_float(
                (uint32_t)e.bias[min<int64_t>(wave_col0 + 32 * j + 8 * q + 4 * lh + t, e.N - 1)] << 16);
#pragma unroll
    for (int pi = 0; pi < FM; pi += kPassTiles) {
#pragma unroll
      for (int ii = 0; ii < kPassTiles; ++ii) {
        const int i = pi + ii;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float v[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              v[t] = acc(i, j, 4 * q + t) * rs[i];
              if constexpr (kBias) v[t] += bv[j][q][t];
              if constexpr (kGelu) v[t] = gelu_tanh(v[t]);
            }
            *reinterpret_cast<u32x2*>(stg + (32 * ii + c) * 256 + (((4 * j + q) ^ (c & 15)) << 4) +
                                      8 * lh) = u32x2{bf16_pack(v[0], v[1]), bf16_pack(v[2], v[3])};
          }
      }
      // a wave's LDS operations run in order, so the reads below see these
      // writes without a wait; the fence only keeps the compiler's order
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      asm volatile("" ::: "memory");
      // this pass's (32 kPassTiles) x 128 block: rows below e.M - prow0,
      // columns below e.N - wave_col0 exist
      const int64_t prow0 = wave_row0 + pi * 32;
      uint16_t* const ybase = static_cast<uint16_t*>(e.y) + prow0 * e.ldy + wave_col0;
      const int64_t rows_left = e.M - prow0, cols_left = e.N - wave_col0;
      const int k = lane & 15;
      u32x4 d[8 * kPassTiles];
#pragma unroll
      for (int it = 0; it < 8 * kPassTiles; ++it) {
        const int r = it * 4 + (lane >> 4);
        d[it] = *reinterpret_cast<const u32x4*>(stg + r * 256 + ((k ^ (r & 15)) << 4));
      }
      if (cols_left >= 128 && e.ldy < (1 << 24)) {
        // whole 256-byte row segments: buffer stores over this pass's rows
        // that exist; rows past the output fall outside the buffer's range
        // and are dropped (the whole offset is in the vector offset, which
        // the range check covers; the scalar offset stays 0)
        const uint32_t row_bytes = 2u * (uint32_t)e.ldy;
        const uint32_t nrows = (uint32_t)max<int64_t>(0, min<int64_t>(rows_left, 32 * kPassTiles));
        const __amdgpu_buffer_rsrc_t ry = buffer_rsrc(ybase, nrows * row_bytes);
        const uint32_t voff = (uint32_t)(lane >> 4) * row_bytes + (uint32_t)k * 16u;
#pragma unroll
        for (int it = 0; it < 8 * kPassTiles; ++it) {
          __builtin_amdgcn_raw_buffer_store_b128(d[it], ry, (int)(voff + (uint32_t)it * 4u * row_bytes),
                                                 0, 0);
          if constexpr (epi_amax(kEpi))
            if (it * 4 + (lane >> 4) < rows_left)
              amx = max(amx, fold_max(abs_max8_pk(d[it], u16x2{0, 0})));
        }
      } else {
#pragma unroll
      for (int it = 0; it < 8 * kPassTiles; ++it) {
        const int r = it * 4 + (lane >> 4);
        if (r < rows_left && k * 8 < cols_left) {
          uint16_t* yp = ybase + (int64_t)r * e.ldy + k * 8;
          if (k * 8 + 8 <= cols_left) {
            *reinterpret_cast<u32x4*>(yp) = d[it];
            if constexpr (epi_amax(kEpi)) amx = max(amx, fold_max(abs_max8_pk(d[it], u16x2{0, 0})));
          } else {
            for (int t = 0; k * 8 + t < cols_left; ++t) {
              const uint32_t b = (d[it][t >> 1] >> (16 * (t & 1))) & 0xFFFFu;
              yp[t] = (uint16_t)b;
              if constexpr (epi_amax(kEpi)) amx = max(amx, b & 0x7FFFu);
            }
          }
        }
      }
      }
      // the next pass overwrites the slice after these reads (in order)
      asm volatile("" ::: "memory");
    }
    if constexpr (epi_amax(kEpi)) {
      // |bf16| patterns of the stored values order as the values do: the
      // wave's integer maximum, then one atomic maximum per wave of its
      // float bits (pattern << 16), as the act_quant amax pass reads them
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) amx = max(amx, (uint32_t)__shfl_xor((int)amx, o, 64));
      if (lane == 0) atomicMax(e.amax + (blockIdx.x % kAmaxSlots), amx << 16);
    }
  } else if constexpr (kEpi == kEpiQuant) {
    // NVFP4 output with the given tensor scale s_T: every output is rounded
    // to bf16 and goes through the encoder's arithmetic (16-column groups
    // along the row, E4M3 scale from the group's |max|, E2M1 codes), so the
    // codes equal act_quant (given s_T) of the bf16 output.  In 32-column
    // block j, group p holds columns 16p .. 16p+15: lane (h, c) owns its
    // columns 4h .. 4h+3 (q = 2p) and 8+4h .. 8+4h+3 (q = 2p+1).  The two
    // lanes of a group (c and c+32) exchange their maxima and their code
    // halves; lane h stores code bytes 4h .. 4h+3 of the group's 8 and lane
    // 0 of the pair the scale byte.  (Staging these small stores through
    // LDS into whole row segments measured slower.)
    const float s_t = *e.y_ts;
    const float gsc = recip0(6.0f * s_t);
    const int64_t cpr = e.N / 2, spr = e.N / 16;       // code and scale bytes per row
    auto store = [&](auto has_bias, auto has_gelu) {
      constexpr bool kBias = decltype(has_bias)::value, kGelu = decltype(has_gelu)::value;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int64_t col0 = wave_col0 + j * 32 + p * 16;   // the group's first column
          float bv[8];
          if constexpr (kBias)
#pragma unroll
            for (int t = 0; t < 8; ++t)
              bv[t] = __uint_as_float(
                  (uint32_t)e.bias[min<int64_t>(col0 + 8 * (t >> 2) + 4 * lh + (t & 3), e.N - 1)] << 16);
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            float v[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              v[t] = acc(i, j, 4 * (2 * p + (t >> 2)) + (t & 3)) * rs[i];
              if constexpr (kBias) v[t] += bv[t];
              if constexpr (kGelu) v[t] = gelu_tanh(v[t]);
            }
            const u32x4 w = {bf16_pack(v[0], v[1]), bf16_pack(v[2], v[3]), bf16_pack(v[4], v[5]),
                             bf16_pack(v[6], v[7])};
            uint32_t mx = fold_max(abs_max8_pk(w, u16x2{0, 0}));
            mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32));
            const uint32_t enc = e4m3_encode(__uint_as_float(mx << 16) * gsc);
            const float inv = recip0(e4m3_decode(enc) * s_t);
            const uint32_t own = e2m1_pack8(w, inv);
            const uint32_t other = (uint32_t)__shfl_xor((int)own, 32);
            const uint32_t word = lh == 0 ? ((own & 0xFFFFu) | (other << 16))
                                          : ((other >> 16) | (own & 0xFFFF0000u));
            const int64_t row = wave_row0 + i * 32 + c;
            if (row < e.M && col0 < e.N) {
              *reinterpret_cast<uint32_t*>(e.yq + row * cpr + col0 / 2 + 4 * lh) = word;
              if (lh == 0) e.ys[row * spr + col0 / 16] = (uint8_t)enc;
            }
          }
        }
    };
    using T = std::true_type;
    using F = std::false_type;
    if (e.bias && e.gelu)
      store(T(), T());
    else if (e.bias)
      store(T(), F());
    else if (e.gelu)
      store(F(), T());
    else
      store(F(), F());
  } else {
    // general: from registers, 4 consecutive outputs per lane and (i, j, q)
    auto store = [&](auto has_bias, auto has_gelu) {
      constexpr bool kBias = decltype(has_bias)::value, kGelu = decltype(has_gelu)::value;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t col = wave_col0 + j * 32 + q * 8 + lh * 4;
          float bv[4];
          if constexpr (kBias)
#pragma unroll
            for (int t = 0; t < 4; ++t)
              bv[t] = __uint_as_float((uint32_t)e.bias[min<int64_t>(col + t, e.N - 1)] << 16);
          const bool full = col + 4 <= e.N && e.vec_ok;
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const int64_t row = wave_row0 + i * 32 + c;
            if (row >= e.M || col >= e.N) continue;
            float v[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              v[t] = acc(i, j, 4 * q + t) * rs[i];
              if constexpr (kBias) v[t] += bv[t];
              if constexpr (kGelu) v[t] = gelu_tanh(v[t]);
            }
            if (e.out_f32) {
              float* yp = static_cast<float*>(e.y) + row * e.ldy + col;
              if (full)
                *reinterpret_cast<f32x4*>(yp) = f32x4{v[0], v[1], v[2], v[3]};
              else
                for (int t = 0; t < 4 && col + t < e.N; ++t) yp[t] = v[t];
            } else {
              uint16_t* yp = static_cast<uint16_t*>(e.y) + row * e.ldy + col;
              const uint32_t p01 = bf16_pack(v[0], v[1]), p23 = bf16_pack(v[2], v[3]);
              if (full) {
                *reinterpret_cast<u32x2*>(yp) = u32x2{p01, p23};
              } else {
                const uint32_t pk[4] = {p01 & 0xFFFFu, p01 >> 16, p23 & 0xFFFFu, p23 >> 16};
                for (int t = 0; t < 4 && col + t < e.N; ++t) yp[t] = (uint16_t)pk[t];
              }
            }
          }
        }
    };
    using T = std::true_type;
    using F = std::false_type;
    if (e.bias && e.gelu)
      store(T(), T());
    else if (e.bias)
      store(T(), F());
    else if (e.gelu)
      store(F(), T());
    else
      store(F(), F());
  }
}

}  // namespace qact
