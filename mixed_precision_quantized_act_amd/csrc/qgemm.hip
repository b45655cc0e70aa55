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
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(16))) int i32x16;

static constexpr int kTileM = 256;
static constexpr int kTileRowsB = 256;        // B tile rows per stage (bf16: N; int8: 2 x 128)
static constexpr int kRowBytes = 128;         // bytes per tile row per K stage
static constexpr int kStageBytes = (kTileM + kTileRowsB) * kRowBytes;
static constexpr int kGroupM = 8;
static constexpr int kEpiStride = 72;         // floats per staged output row
static constexpr int kSmemBytes = 4 * 128 * kEpiStride * 4;   // >= 2 operand stages

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
  int vec_ok;            // y 16-byte aligned and ldy % 4 == 0: vector stores
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

// Wave grid of a workgroup: WM x WN waves (WM = 2).  A wave owns a
// (256/WM) x (256/WN) block of the 256 x 256 output tile (INT8: (256/WM) x
// (128/WN) columns of each of the two digit planes), as FM x FN MFMA tiles
// of 32 x 32.
template <int WN>
struct Cfg {
  static constexpr int WM = 2;
  static constexpr int NW = WM * WN;              // waves
  static constexpr int NT = 64 * NW;              // threads
  static constexpr int FM = 256 / WM / 32;        // A fragments per wave
  static constexpr int FN = 256 / WN / 32;        // B fragments per wave
  static constexpr int RPP = NT / 8;              // tile rows per staging pass
  static constexpr int PASSES = 256 / RPP;        // staging passes per operand
  static constexpr int EP_FM = NW == 4 ? 4 : 2;   // A fragments per epilogue pass
};

template <bool I8, int WN>
__device__ __forceinline__ int b_frag_row(int wn, int j, int lane) {
  constexpr int FN = Cfg<WN>::FN;
  if (I8) {
    constexpr int half = FN / 2;                  // column fragments per digit plane
    return (j / half) * 128 + wn * (128 / WN) + (j % half) * 32 + (lane & 31);
  }
  return wn * (256 / WN) + j * 32 + (lane & 31);
}

// LDS swizzle: 16-byte chunk c of tile row r sits in chunk slot
// c ^ ((r >> 1) & 7) of its 128-byte row.  A 16-lane group of a 16-byte
// fragment read covers 16 consecutive rows at one chunk: even rows land in
// one half of the 64 banks and odd rows in the other, and (r >> 1) & 7
// spreads each half's 8 rows over the 8 slots, so the group hits 64
// distinct banks.  The staging writes (8 lanes per row) are conflict-free
// too.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  // raw buffer (stride 0): loads at offsets >= bytes return zero
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

template <bool I8, bool DUMP, int WN>
__global__ void __launch_bounds__(Cfg<WN>::NT, 1)
qgemm_kernel(GemmArgs g, EpiArgs e) {
  using C = Cfg<WN>;
  static_assert(kSmemBytes >= 2 * kStageBytes, "LDS holds two operand stages");
  static_assert(C::NW * C::EP_FM * 32 * kEpiStride * 4 <= kSmemBytes, "epilogue staging fits");
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];

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
  const int wm = wave / WN, wn = wave % WN;

  // Buffer resources based at this tile's first row: rows past the operand
  // (INT8 activations: rows >= M) fall outside the range and load zero.
  int64_t a_bytes = (g.a_rows - m0) * g.lda;
  if (a_bytes > 0x7FFFFFF0) a_bytes = 0x7FFFFFF0;
  const __amdgpu_buffer_rsrc_t ra_src = buffer_rsrc(g.A + m0 * g.lda, (uint32_t)a_bytes);
  const __amdgpu_buffer_rsrc_t rb_src = buffer_rsrc(g.B + nb0 * g.ldb, 0x7FFFFFF0u);

  // global -> register staging: per K stage each thread moves PASSES chunks
  // of 16 bytes of A and of B; chunk i covers tile row i*RPP + tid/8, byte
  // column (tid%8)*16 (RPP is a multiple of 16, so every chunk of a thread
  // has the same swizzle).
  const int r8 = tid >> 3, ch8 = tid & 7;
  const int lds_base = r8 * kRowBytes + ((ch8 ^ swz(r8)) << 4);
  const uint32_t a_off = (uint32_t)(r8 * g.lda + ch8 * 16);
  const uint32_t a_step = (uint32_t)(C::RPP * g.lda);
  const uint32_t b_off = (uint32_t)(r8 * g.ldb + ch8 * 16);
  u32x4 ra[C::PASSES], rb[C::PASSES];
  auto gload = [&](int kt) {
    const uint32_t kb = (uint32_t)kt * kRowBytes;
    // the INT8 activation rows are unpadded: a chunk past K loads zero
    const bool kin = !I8 || (int64_t)kb + ch8 * 16 < g.a_kbytes;
#pragma unroll
    for (int i = 0; i < C::PASSES; ++i) {
      ra[i] = buffer_load16(ra_src, kin ? a_off + i * a_step + kb : 0x7FFFFFF0u);
      const int trow = i * C::RPP;                // first tile row of this pass
      const uint32_t bo = I8 ? (uint32_t)(trow / 128) * (uint32_t)g.b_plane +
                                   (uint32_t)((trow % 128) * g.ldb)
                             : (uint32_t)(trow * g.ldb);
      rb[i] = buffer_load16(rb_src, b_off + bo + kb);
    }
  };
  auto lds_store = [&](int buf) {
    uint8_t* sa = smem + buf * kStageBytes + lds_base;
    uint8_t* sb = sa + kTileM * kRowBytes;
#pragma unroll
    for (int i = 0; i < C::PASSES; ++i) {
      *reinterpret_cast<u32x4*>(sa + i * C::RPP * kRowBytes) = ra[i];
      *reinterpret_cast<u32x4*>(sb + i * C::RPP * kRowBytes) = rb[i];
    }
  };

  typedef typename std::conditional<I8, i32x16, f32x16>::type acc_t;
  acc_t acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  // fragment rows of this lane are (multiple of 32) + lane % 32, so they
  // all share the swizzle of lane % 32
  const int a_frag = (wm * (256 / C::WM) + (lane & 31)) * kRowBytes;
  const int row_sw = swz(lane & 31);
  auto frags = [&](int buf, int s, u32x4 (&af)[C::FM], u32x4 (&bf)[C::FN]) {
    const uint8_t* sa = smem + buf * kStageBytes;
    const uint8_t* sb = sa + kTileM * kRowBytes;
    const int coff = ((2 * s + (lane >> 5)) ^ row_sw) << 4;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
      af[i] = *reinterpret_cast<const u32x4*>(sa + a_frag + i * 32 * kRowBytes + coff);
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      bf[j] = *reinterpret_cast<const u32x4*>(sb + b_frag_row<I8, WN>(wn, j, lane) * kRowBytes +
                                              coff);
  };
  auto mfmas = [&](const u32x4 (&af)[C::FM], const u32x4 (&bf)[C::FN]) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        if constexpr (I8)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, af[i]),
                                                            __builtin_bit_cast(i32x4, bf[j]),
                                                            acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[i]),
                                                              __builtin_bit_cast(bf16x8, bf[j]),
                                                              acc[i][j], 0, 0, 0);
      }
  };

  // Pipeline: LDS holds stage kt while registers carry stage kt+1 from
  // global memory; fragments of substep s+1 are read while the MFMAs of
  // substep s run.  At substep 3 the next stage goes to the other LDS
  // buffer (one barrier per stage) and the loads of stage kt+2 are issued.
  gload(0);
  lds_store(0);
  __syncthreads();
  if (g.k_tiles > 1) gload(1);
  u32x4 fa0[C::FM], fb0[C::FN], fa1[C::FM], fb1[C::FN];
  frags(0, 0, fa0, fb0);
  for (int kt = 0; kt < g.k_tiles; ++kt) {
    const int cur = kt & 1;
    frags(cur, 1, fa1, fb1);
    mfmas(fa0, fb0);
    frags(cur, 2, fa0, fb0);
    mfmas(fa1, fb1);
    frags(cur, 3, fa1, fb1);
    mfmas(fa0, fb0);
    if (kt + 1 < g.k_tiles) {
      lds_store(cur ^ 1);
      __syncthreads();
      frags(cur ^ 1, 0, fa0, fb0);
      if (kt + 2 < g.k_tiles) gload(kt + 2);
    }
    mfmas(fa1, fb1);
  }

  // ---- epilogue.  Accumulator r of a 32x32 MFMA tile holds row
  // (r/4)*8 + (lane/32)*4 + r%4 and column lane%32.  In passes of EP_FM row
  // fragments x 64 columns, each wave stages its values as float32 in LDS
  // (row stride kEpiStride floats: the two half-waves write disjoint
  // banks), then reads them back row-contiguous and stores 4 consecutive
  // outputs per lane.
  __syncthreads();                       // every wave is done with the operand tiles
  const int lrow = (lane >> 5) * 4, lcol = lane & 31;
  constexpr int OUT_FRAGS = I8 ? C::FN / 2 : C::FN;     // 32-column output blocks per wave
  const int64_t wave_row0 = m0 + wm * (256 / C::WM);
  const int64_t wave_col0 = nb0 + wn * (OUT_FRAGS * 32);
  if constexpr (I8 && DUMP) {          // verification dump of the exact sums
#pragma unroll
    for (int jn = 0; jn < OUT_FRAGS; ++jn)
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = wave_row0 + i * 32 + (r >> 2) * 8 + lrow + (r & 3);
          const int64_t col = wave_col0 + jn * 32 + lcol;
          if (row < e.M && col < e.N) {
            g.acc_hi[row * e.N + col] = acc[i][jn][r];
            g.acc_lo[row * e.N + col] = acc[i][jn + OUT_FRAGS][r];
          }
        }
    return;
  }
  float* ep = reinterpret_cast<float*>(smem) + wave * (C::EP_FM * 32 * kEpiStride);
  const float alpha = I8 ? 1.0f : (*g.a_ts) * (*g.w_ts);
#pragma unroll
  for (int ip = 0; ip < C::FM; ip += C::EP_FM)
#pragma unroll
    for (int jp = 0; jp < OUT_FRAGS; jp += 2) {
#pragma unroll
      for (int i = 0; i < C::EP_FM; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float v;
            if constexpr (I8)
              v = fmaf(128.0f, (float)acc[ip + i][jp + jj][r],
                       (float)acc[ip + i][jp + jj + OUT_FRAGS][r]);
            else
              v = acc[ip + i][jp + jj][r] * alpha;
            ep[(i * 32 + (r >> 2) * 8 + lrow + (r & 3)) * kEpiStride + jj * 32 + lcol] = v;
          }
      __syncthreads();
      for (int it = 0; it < C::EP_FM * 8; ++it) {
        const int idx = it * 64 + lane;
        const int rl = idx >> 4, c4 = (idx & 15) * 4;
        const int64_t row = wave_row0 + ip * 32 + rl;
        const int64_t col = wave_col0 + jp * 32 + c4;
        if (row >= e.M || col >= e.N) continue;
        const f32x4 v4 = *reinterpret_cast<const f32x4*>(ep + rl * kEpiStride + c4);
        float v[4] = {v4[0], v4[1], v4[2], v4[3]};
        const float rs = I8 ? g.a_s[row] : 1.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (I8 && col + q < e.N) v[q] = v[q] * rs * g.colscale[col + q];
          if (e.bias && col + q < e.N) v[q] += __uint_as_float((uint32_t)e.bias[col + q] << 16);
          if (e.gelu) v[q] = gelu_tanh(v[q]);
        }
        const bool full = col + 4 <= e.N && e.vec_ok;
        if (e.out_f32) {
          float* yp = static_cast<float*>(e.y) + row * e.ldy + col;
          if (full)
            *reinterpret_cast<f32x4*>(yp) = f32x4{v[0], v[1], v[2], v[3]};
          else
            for (int q = 0; q < 4 && col + q < e.N; ++q) yp[q] = v[q];
        } else {
          uint16_t* yp = static_cast<uint16_t*>(e.y) + row * e.ldy + col;
          if (full) {
            u32x2 o = {f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16),
                       f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16)};
            *reinterpret_cast<u32x2*>(yp) = o;
          } else {
            for (int q = 0; q < 4 && col + q < e.N; ++q) yp[q] = (uint16_t)f32_to_bf16(v[q]);
          }
        }
      }
      __syncthreads();
    }
}

// Exact INT8 x NVFP4 columns for irregular weight rows: per 16-group integer
// sums scaled by the group's E4M3 value in float64.  Each workgroup scans
// 256 row flags at once (one per thread) and then walks the flagged rows
// in index order; with no irregular rows it only reads the flags.
__global__ void __launch_bounds__(256)
int8_irregular_kernel(const int8_t* __restrict__ a_q, const float* __restrict__ a_s,
                      const uint8_t* __restrict__ w_q, const uint8_t* __restrict__ w_s,
                      const float* __restrict__ w_ts, int64_t K,
                      const uint8_t* __restrict__ irregular, EpiArgs e) {
  __shared__ uint64_t masks[4];
  const int64_t gpr = K / 16;
  const int wave = threadIdx.x >> 6;
  for (int64_t nb = (int64_t)blockIdx.x * 256; nb < e.N; nb += (int64_t)gridDim.x * 256) {
    const int64_t mine = nb + threadIdx.x;
    const bool flag = mine < e.N && irregular[mine] != 0;
    const uint64_t bal = __ballot(flag);
    if ((threadIdx.x & 63) == 0) masks[wave] = bal;
    __syncthreads();
    for (int w = 0; w < 4; ++w) {
      uint64_t bits = masks[w];
      while (bits) {
        const int bit = __ffsll((unsigned long long)bits) - 1;
        bits &= bits - 1;
        const int64_t n = nb + w * 64 + bit;
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
    __syncthreads();
  }
}

// ---------------------------------------------------------------- host --

static int vec_ok(const GemmOut& o) {
  return (reinterpret_cast<uintptr_t>(o.y) % 16 == 0) && (o.ldy % 4 == 0);
}

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

#ifndef QACT_BF16_WN
#define QACT_BF16_WN 2
#endif

static hipError_t launch_gemm(bool i8, const GemmArgs& g, const EpiArgs& e, hipStream_t st) {
  const int total = g.mt * g.nt;
  const int grid = 8 * ((total + 7) / 8);
  if (g_ev_before) {
    hipError_t err = hipEventRecord(g_ev_before, st);
    if (err != hipSuccess) return err;
  }
  constexpr int kWnBf16 = QACT_BF16_WN;
  if (i8 && g.acc_hi)
    hipLaunchKernelGGL((qgemm_kernel<true, true, 2>), dim3(grid), dim3(Cfg<2>::NT), 0, st, g, e);
  else if (i8)
    hipLaunchKernelGGL((qgemm_kernel<true, false, 2>), dim3(grid), dim3(Cfg<2>::NT), 0, st, g, e);
  else
    hipLaunchKernelGGL((qgemm_kernel<false, false, kWnBf16>), dim3(grid), dim3(Cfg<kWnBf16>::NT),
                       0, st, g, e);
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
  EpiArgs e = {o.y, o.ldy, o.out_f32, o.gelu, o.bias, M, N, vec_ok(o)};
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
  EpiArgs e = {o.y, o.ldy, o.out_f32, o.gelu, o.bias, M, N, vec_ok(o)};
  err = launch_gemm(true, g, e, st);
  if (err != hipSuccess || acc_hi) return err;
  const int64_t fb = (N + 255) / 256;
  hipLaunchKernelGGL(int8_irregular_kernel, dim3((unsigned)(fb < 1024 ? fb : 1024)), dim3(256), 0,
                     st, a_q, a_s, w_q, w_s, w_ts, K, irregular, e);
  return hipGetLastError();
}

}  // namespace qact
