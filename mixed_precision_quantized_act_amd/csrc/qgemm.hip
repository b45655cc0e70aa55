// Quantized linear GEMMs on gfx950 MFMA:  Y = dequant(A) dequant(W)^T.
//
// 6Bit-Diffusion, abstract and Fig. 2 caption: every internal linear of a
// DiT block runs with NVFP4 (4-bit) weights and NVFP4 or INT8 activations.
//
// No gfx950 matrix instruction takes NVFP4's E4M3 scale per 16 elements
// (its block-scaled FP4 MFMA takes power-of-two scales per 32), and an E2M1
// value times an E4M3 scale needs up to 6 significant bits, more than any
// FP8/FP6/FP4 element holds.  Both paths therefore feed exact operands:
//
//  * NVFP4 x NVFP4: each operand is dequantized exactly to bf16 (E2M1 value
//    times E4M3 scale; the float32 tensor scales are applied in the
//    epilogue) and multiplied on v_mfma_f32_32x32x16_bf16.
//  * INT8 x NVFP4: each weight row is written as s_Tw 2^(Fr-11) I with an
//    integer I = c M 2^(F-Fr) (c = 2*E2M1, scale = M 2^(F-10)), split into
//    two int8 digit planes I = 128 hi + lo; both planes run against the
//    int8 activations on v_mfma_i32_32x32x32_i8 with exact int32 sums,
//    combined in float64 per output.  Rows whose scale exponents spread by
//    more than 6 (never for Gaussian weights) are computed by a separate
//    exact kernel.
//
// Tiling (both paths): 256 threads = 4 waves in a 2x2 grid, a 256 x 256
// output tile (INT8: 256 x 128 columns times 2 digit planes), K stages of
// 128 bytes per row (64 bf16 or 128 int8) double-buffered in LDS (2 x 64
// KB), rows stored with a 16-byte-chunk XOR swizzle so that the 16-byte
// fragment reads of 32 consecutive rows hit distinct banks.  Each wave owns
// a 128 x 128 block of accumulators (16 MFMA tiles of 32 x 32).  Workgroups
// are remapped so each XCD works a contiguous band of tiles (L2 reuse).
#include <type_traits>

#include "qact_device.h"
#include "qact_internal.h"

namespace qact {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(16))) int i32x16;

static constexpr int kThreads = 256;
static constexpr int kTileM = 256;
static constexpr int kTileRowsB = 256;        // B tile rows per stage (bf16: N; int8: 2 x 128)
static constexpr int kRowBytes = 128;         // bytes per tile row per K stage
static constexpr int kStageBytes = (kTileM + kTileRowsB) * kRowBytes;
static constexpr int kGroupM = 8;

static inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// ------------------------------------------------------------ operands --

// NVFP4 -> bf16 without the tensor scale (exact), into a zero-padded
// [rows_pad][kpad] matrix.  One 16-element group per thread.
__global__ void __launch_bounds__(256)
nvfp4_to_bf16_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s, int64_t rows,
                     int64_t K, int64_t rows_pad, int64_t kpad, uint16_t* __restrict__ dst) {
  const int64_t gpr = kpad / 16;
  const int64_t total = rows_pad * gpr;
  for (int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gi < total;
       gi += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = gi / gpr, g = gi - r * gpr;
    u32x4 o0 = {0, 0, 0, 0}, o1 = {0, 0, 0, 0};
    if (r < rows && g * 16 < K) {
      const u32x2 c = *reinterpret_cast<const u32x2*>(q + r * (K / 2) + g * 8);
      const float sc = e4m3_decode(s[r * (K / 16) + g]);
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t byte = (c[i >> 2] >> (8 * (i & 3))) & 0xFFu;
        const float v0 = (float)e2m1_twice(byte & 0xFu) * 0.5f * sc;
        const float v1 = (float)e2m1_twice(byte >> 4) * 0.5f * sc;
        w[i] = (__float_as_uint(v0) >> 16) | (__float_as_uint(v1) & 0xFFFF0000u);
      }
      o0 = u32x4{w[0], w[1], w[2], w[3]};
      o1 = u32x4{w[4], w[5], w[6], w[7]};
    }
    u32x4* d = reinterpret_cast<u32x4*>(dst + r * kpad + g * 16);
    d[0] = o0;
    d[1] = o1;
  }
}

// NVFP4 weight -> two int8 digit planes [2][n_pad][kpad], the per-column
// scale s_Tw 2^(Fr-11) and the irregular-row flags.  One wave per row.
__global__ void __launch_bounds__(256)
nvfp4_to_int8_digits_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
                            const float* __restrict__ w_ts /* null: 1 */, int64_t N, int64_t K,
                            int64_t n_pad, int64_t kpad, int8_t* __restrict__ planes,
                            float* __restrict__ colscale, uint8_t* __restrict__ irregular) {
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (n >= n_pad) return;
  const int64_t gpr = K / 16;
  int fmin = 99, fmax = 0;
  if (n < N) {
    for (int64_t g = lane; g < gpr; g += 64) {
      const uint32_t c = s[n * gpr + g];
      const uint32_t e = c >> 3, m = c & 7u;
      const uint32_t sig = e ? 8u + m : m;
      const int f = e ? (int)e : 1;
      if (sig) {
        fmin = min(fmin, f);
        fmax = max(fmax, f);
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    fmin = min(fmin, __shfl_xor(fmin, o, 64));
    fmax = max(fmax, __shfl_xor(fmax, o, 64));
  }
  const int fr = fmin == 99 ? 1 : fmin;
  const bool irr = (n < N) && fmin != 99 && (fmax - fr) > 6;
  int8_t* p_hi = planes + n * kpad;
  int8_t* p_lo = planes + n_pad * kpad + n * kpad;
  for (int64_t g = lane; g < kpad / 16; g += 64) {
    u32x4 hi4 = {0, 0, 0, 0}, lo4 = {0, 0, 0, 0};
    if (n < N && g < gpr && !irr) {
      const uint32_t c = s[n * gpr + g];
      const uint32_t e = c >> 3, m = c & 7u;
      const int sig = (int)(e ? 8u + m : m);
      const int f = e ? (int)e : 1;
      const int mult = sig ? (sig << (f - fr)) : 0;
      const u32x2 codes = *reinterpret_cast<const u32x2*>(q + n * (K / 2) + g * 8);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t code = (codes[i >> 3] >> (4 * (i & 7))) & 0xFu;
        const int I = e2m1_twice(code) * mult;
        const int lo = ((I + 64) & 127) - 64;
        const int hi = (I - lo) >> 7;
        hi4[i >> 2] |= ((uint32_t)hi & 0xFFu) << (8 * (i & 3));
        lo4[i >> 2] |= ((uint32_t)lo & 0xFFu) << (8 * (i & 3));
      }
    }
    *reinterpret_cast<u32x4*>(p_hi + g * 16) = hi4;
    *reinterpret_cast<u32x4*>(p_lo + g * 16) = lo4;
  }
  if (lane == 0) {
    colscale[n] = (n < N) ? ldexpf(w_ts ? *w_ts : 1.0f, fr - 11) : 0.0f;
    irregular[n] = irr ? 1 : 0;
  }
}

// ------------------------------------------------------------ epilogue --

__device__ __forceinline__ float gelu_tanh(float v) {
  return 0.5f * v * (1.0f + tanhf(0.7978845608028654f * (v + 0.044715f * v * v * v)));
}

struct EpiArgs {
  void* y;
  int64_t ldy;
  int out_f32;
  int gelu;
  const uint16_t* bias;
  int64_t M, N;
};

__device__ __forceinline__ void store_out(const EpiArgs& e, int64_t row, int64_t col, float v) {
  if (e.bias) v += __uint_as_float((uint32_t)e.bias[col] << 16);
  if (e.gelu) v = gelu_tanh(v);
  if (e.out_f32)
    static_cast<float*>(e.y)[row * e.ldy + col] = v;
  else
    static_cast<uint16_t*>(e.y)[row * e.ldy + col] = (uint16_t)f32_to_bf16(v);
}

// ---------------------------------------------------------------- GEMM --

struct GemmArgs {
  const uint8_t* A;      // rows of kRowBytes-aligned K bytes
  int64_t lda;           // bytes
  int64_t a_rows;        // rows that exist (loads clamp to a_rows - 1)
  int64_t a_kbytes;      // K bytes that exist (later chunks load as 0)
  const uint8_t* B;
  int64_t ldb;           // bytes
  int64_t b_plane;       // bytes between the two int8 digit planes
  int k_tiles;           // K stages of kRowBytes
  int mt, nt;            // tile counts
  // epilogue inputs
  const float* a_ts;     // NVFP4: activation tensor scale
  const float* w_ts;     // NVFP4: weight tensor scale
  const float* a_s;      // INT8: per-row activation scale
  const float* colscale; // INT8: per-column s_Tw 2^(Fr-11)
  int32_t* acc_hi;       // INT8 verification dump (or null)
  int32_t* acc_lo;
};

template <bool I8>
__device__ __forceinline__ int b_tile_row(int wn, int j, int lane) {
  if (I8) return (j >> 1) * 128 + wn * 64 + (j & 1) * 32 + (lane & 31);
  return wn * 128 + j * 32 + (lane & 31);
}

template <bool I8>
__global__ void __launch_bounds__(kThreads, 1)
qgemm_kernel(GemmArgs g, EpiArgs e) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes];

  // XCD-aware tile order: hardware deals workgroups to the 8 XCDs in turn;
  // give each XCD a contiguous range of logical tiles, grouped kGroupM
  // tile-rows at a time so that concurrent tiles share A rows and B columns.
  const int total = g.mt * g.nt;
  const int per_xcd = (total + 7) / 8;
  const int logical = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (logical >= total) return;
  const int group = logical / (kGroupM * g.nt);
  const int first_m = group * kGroupM;
  const int gsz = min(g.mt - first_m, kGroupM);
  const int in_group = logical - group * kGroupM * g.nt;
  const int tm = first_m + in_group % gsz;
  const int tn = in_group / gsz;
  const int64_t m0 = (int64_t)tm * kTileM;
  const int64_t nb0 = (int64_t)tn * (I8 ? 128 : 256);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // global -> register staging: per K stage each thread moves 8 chunks of
  // 16 bytes of A and 8 of B; chunk i covers tile row i*32 + tid/8, byte
  // column (tid%8)*16, so rows step by 32 and the LDS slot by 32 rows.
  const int r8 = tid >> 3, ch8 = tid & 7;
  const int lds_base = r8 * kRowBytes + ((ch8 ^ (r8 & 7)) << 4);
  const uint8_t* b_base = g.B + (nb0 + r8) * g.ldb + ch8 * 16;
  u32x4 ra[8], rb[8];
  auto load_stage = [&](int kt) {
    const int64_t kb = (int64_t)kt * kRowBytes;
    // only the INT8 activation operand is the caller's unpadded buffer:
    // its rows past M are clamped (the results are not stored) and its
    // K chunks past K load as zero
    const bool kin = !I8 || kb + ch8 * 16 < g.a_kbytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int64_t ar = m0 + i * 32 + r8;
      if (I8) ar = ar < g.a_rows ? ar : g.a_rows - 1;
      if (kin)
        ra[i] = *reinterpret_cast<const u32x4*>(g.A + ar * g.lda + kb + ch8 * 16);
      else
        ra[i] = u32x4{0, 0, 0, 0};
      const int64_t boff = I8 ? (int64_t)(i >> 2) * g.b_plane + (int64_t)((i & 3) * 32) * g.ldb
                              : (int64_t)(i * 32) * g.ldb;
      rb[i] = *reinterpret_cast<const u32x4*>(b_base + boff + kb);
    }
  };
  auto store_stage = [&](int buf) {
    uint8_t* sa = smem + buf * kStageBytes + lds_base;
    uint8_t* sb = sa + kTileM * kRowBytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<u32x4*>(sa + i * 32 * kRowBytes) = ra[i];
      *reinterpret_cast<u32x4*>(sb + i * 32 * kRowBytes) = rb[i];
    }
  };

  typedef typename std::conditional<I8, i32x16, f32x16>::type acc_t;
  acc_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  int a_frag_off[4], b_frag_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a_frag_off[i] = (wm * 128 + i * 32 + (lane & 31)) * kRowBytes;
    b_frag_off[i] = b_tile_row<I8>(wn, i, lane) * kRowBytes;
  }
  const int row_sw = lane & 7;           // (row & 7) of every fragment row of this lane

  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int kt = 0; kt < g.k_tiles; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < g.k_tiles;
    if (more) load_stage(kt + 1);
    const uint8_t* sa = smem + cur * kStageBytes;
    const uint8_t* sb = sa + kTileM * kRowBytes;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = 2 * s + (lane >> 5);
      const int coff = (ch ^ row_sw) << 4;
      u32x4 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = *reinterpret_cast<const u32x4*>(sa + a_frag_off[i] + coff);
        bf[i] = *reinterpret_cast<const u32x4*>(sb + b_frag_off[i] + coff);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (I8)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                __builtin_bit_cast(i32x4, af[i]), __builtin_bit_cast(i32x4, bf[j]), acc[i][j], 0,
                0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, af[i]), __builtin_bit_cast(bf16x8, bf[j]), acc[i][j],
                0, 0, 0);
        }
    }
    if (more) store_stage(cur ^ 1);
    __syncthreads();
  }

  // epilogue: accumulator r of a 32x32 tile holds row (r/4)*8 + (lane/32)*4
  // + r%4 and column lane%32
  const int64_t row_base = m0 + wm * 128 + (lane >> 5) * 4;
  if constexpr (I8) {
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
      const int64_t col = nb0 + wn * 64 + jn * 32 + (lane & 31);
      const bool col_ok = col < e.N;
      const float cs = col_ok ? g.colscale[col] : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = row_base + i * 32 + (r >> 2) * 8 + (r & 3);
          if (col_ok && row < e.M) {
            const int hi = acc[i][jn][r], lo = acc[i][jn + 2][r];
            if (g.acc_hi) {
              g.acc_hi[row * e.N + col] = hi;
              g.acc_lo[row * e.N + col] = lo;
            } else {
              const double t = 128.0 * (double)hi + (double)lo;
              store_out(e, row, col, (float)t * g.a_s[row] * cs);
            }
          }
        }
    }
  } else {
    const float alpha = (*g.a_ts) * (*g.w_ts);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = nb0 + wn * 128 + j * 32 + (lane & 31);
      const bool col_ok = col < e.N;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = row_base + i * 32 + (r >> 2) * 8 + (r & 3);
          if (col_ok && row < e.M) store_out(e, row, col, acc[i][j][r] * alpha);
        }
    }
  }
}

// Exact INT8 x NVFP4 columns for irregular weight rows: per 16-group integer
// sums scaled by the group's E4M3 value in float64.
__global__ void __launch_bounds__(256)
int8_irregular_kernel(const int8_t* __restrict__ a_q, const float* __restrict__ a_s,
                      const uint8_t* __restrict__ w_q, const uint8_t* __restrict__ w_s,
                      const float* __restrict__ w_ts, int64_t K,
                      const uint8_t* __restrict__ irregular, EpiArgs e) {
  const int64_t gpr = K / 16;
  for (int64_t n = blockIdx.x; n < e.N; n += gridDim.x) {
    if (!irregular[n]) continue;
    for (int64_t m = threadIdx.x; m < e.M; m += blockDim.x) {
      double acc = 0.0;
      for (int64_t gi = 0; gi < gpr; ++gi) {
        const u32x2 c = *reinterpret_cast<const u32x2*>(w_q + n * (K / 2) + gi * 8);
        const int8_t* qa = a_q + m * K + gi * 16;
        int p = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          p += (int)qa[i] * e2m1_twice((c[i >> 3] >> (4 * (i & 7))) & 0xFu);
        acc += (double)p * (double)e4m3_decode(w_s[n * gpr + gi]);
      }
      store_out(e, m, n, (float)(acc * 0.5 * (double)a_s[m] * (double)(*w_ts)));
    }
  }
}

// ---------------------------------------------------------------- host --

static int64_t kpad_bytes(int64_t k_bytes) { return round_up(k_bytes, kRowBytes); }

size_t nvfp4_gemm_ws_bytes(int64_t M, int64_t N, int64_t K) {
  const int64_t kp = kpad_bytes(2 * K) / 2;
  return (size_t)round_up(round_up(M, 256) * kp * 2, 256) + (size_t)round_up(N, 256) * kp * 2;
}

size_t int8_gemm_ws_bytes(int64_t, int64_t N, int64_t K) {
  const int64_t kp = kpad_bytes(K), np = round_up(N, 128);
  return (size_t)round_up(2 * np * kp, 256) + (size_t)round_up(np * 4, 256) + (size_t)np;
}

static hipEvent_t g_ev_before = nullptr, g_ev_after = nullptr;

void set_gemm_events(hipEvent_t before, hipEvent_t after) {
  g_ev_before = before;
  g_ev_after = after;
}

static hipError_t launch_gemm(bool i8, const GemmArgs& g, const EpiArgs& e, hipStream_t st) {
  const int total = g.mt * g.nt;
  const int grid = 8 * ((total + 7) / 8);
  if (g_ev_before) {
    hipError_t err = hipEventRecord(g_ev_before, st);
    if (err != hipSuccess) return err;
  }
  if (i8)
    hipLaunchKernelGGL(qgemm_kernel<true>, dim3(grid), dim3(kThreads), 0, st, g, e);
  else
    hipLaunchKernelGGL(qgemm_kernel<false>, dim3(grid), dim3(kThreads), 0, st, g, e);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess && g_ev_after) err = hipEventRecord(g_ev_after, st);
  return err;
}

hipError_t launch_nvfp4_gemm(const uint8_t* a_q, const uint8_t* a_s, const float* a_ts,
                             const uint8_t* w_q, const uint8_t* w_s, const float* w_ts,
                             int64_t M, int64_t N, int64_t K, const GemmOut& o, void* ws,
                             hipStream_t st) {
  const int64_t kp = kpad_bytes(2 * K) / 2;
  const int64_t mp = round_up(M, 256), np = round_up(N, 256);
  uint16_t* a_bf = static_cast<uint16_t*>(ws);
  uint16_t* w_bf = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + round_up(mp * kp * 2, 256));
  auto grid_for = [](int64_t groups) {
    int64_t b = (groups + 255) / 256;
    return (unsigned)(b > 16384 ? 16384 : (b < 1 ? 1 : b));
  };
  hipLaunchKernelGGL(nvfp4_to_bf16_kernel, dim3(grid_for(mp * kp / 16)), dim3(256), 0, st, a_q,
                     a_s, M, K, mp, kp, a_bf);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(nvfp4_to_bf16_kernel, dim3(grid_for(np * kp / 16)), dim3(256), 0, st, w_q,
                     w_s, N, K, np, kp, w_bf);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  GemmArgs g = {};
  g.A = reinterpret_cast<const uint8_t*>(a_bf);
  g.lda = kp * 2;
  g.a_rows = mp;
  g.a_kbytes = kp * 2;
  g.B = reinterpret_cast<const uint8_t*>(w_bf);
  g.ldb = kp * 2;
  g.k_tiles = (int)(kp * 2 / kRowBytes);
  g.mt = (int)(mp / 256);
  g.nt = (int)(np / 256);
  g.a_ts = a_ts;
  g.w_ts = w_ts;
  EpiArgs e = {o.y, o.ldy, o.out_f32, o.gelu, o.bias, M, N};
  return launch_gemm(false, g, e, st);
}

hipError_t launch_int8_gemm(const int8_t* a_q, const float* a_s, const uint8_t* w_q,
                            const uint8_t* w_s, const float* w_ts, int64_t M, int64_t N,
                            int64_t K, const GemmOut& o, int32_t* acc_hi, int32_t* acc_lo,
                            void* ws, hipStream_t st) {
  const int64_t kp = kpad_bytes(K), np = round_up(N, 128);
  int8_t* planes = static_cast<int8_t*>(ws);
  float* colscale = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + round_up(2 * np * kp, 256));
  uint8_t* irregular = reinterpret_cast<uint8_t*>(colscale) + round_up(np * 4, 256);
  hipLaunchKernelGGL(nvfp4_to_int8_digits_kernel, dim3((unsigned)((np + 3) / 4)), dim3(256), 0,
                     st, w_q, w_s, w_ts, N, K, np, kp, planes, colscale, irregular);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  GemmArgs g = {};
  g.A = reinterpret_cast<const uint8_t*>(a_q);
  g.lda = K;
  g.a_rows = M;
  g.a_kbytes = K;
  g.B = reinterpret_cast<const uint8_t*>(planes);
  g.ldb = kp;
  g.b_plane = np * kp;
  g.k_tiles = (int)(kp / kRowBytes);
  g.mt = (int)((M + 255) / 256);
  g.nt = (int)(np / 128);
  g.a_s = a_s;
  g.colscale = colscale;
  g.acc_hi = acc_hi;
  g.acc_lo = acc_lo;
  EpiArgs e = {o.y, o.ldy, o.out_f32, o.gelu, o.bias, M, N};
  err = launch_gemm(true, g, e, st);
  if (err != hipSuccess || acc_hi) return err;
  hipLaunchKernelGGL(int8_irregular_kernel, dim3(64), dim3(256), 0, st, a_q, a_s, w_q, w_s, w_ts,
                     K, irregular, e);
  return hipGetLastError();
}

}  // namespace qact
