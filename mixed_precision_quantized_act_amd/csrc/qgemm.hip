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
//    combined per output.  Rows whose scale exponents spread by more than 6
//    (never for Gaussian weights) are computed by a separate exact kernel.
//
// Tiling (both paths): a workgroup of 4 waves (2 x 2) computes a 256 x 128
// tile of B rows (NVFP4: 128 output columns; INT8: 64 output columns in
// each of the two digit planes); each wave owns 128 x 64 as 4 x 2 MFMA
// tiles of 32 x 32.  K advances in stages of 64 bytes per row (32 bf16 or
// 64 int8), loaded straight from global memory into a 3-deep LDS ring
// (24 KB per stage) by buffer loads whose out-of-range lanes return zero
// (ragged M and K of the unpadded INT8 activations).  With 72 KB of LDS
// and at most 256 registers per lane, two workgroups share a CU, so one
// workgroup's barriers, prologue and epilogue run under the other's
// MFMAs.  Workgroups are remapped so each XCD works a contiguous band of
// tiles (L2 reuse).
#include <type_traits>

#include "qact_device.h"
#include "qact_internal.h"

namespace qact {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(16))) int i32x16;

static constexpr int kThreads = 256;          // 4 waves, 2 x 2
static constexpr int kTileM = 256;            // A rows per tile
static constexpr int kTileB = 128;            // B rows per tile (INT8: 2 planes x 64)
static constexpr int kRowBytes = 64;          // bytes per tile row per K stage
static constexpr int kStageBytes = (kTileM + kTileB) * kRowBytes;   // 24 KB
static constexpr int kStages = 3;             // LDS ring depth: 2 stages in flight
static constexpr int kGroupM = 8;
static constexpr int kFM = 4, kFN = 2;        // MFMA tiles per wave (rows, B columns)
static constexpr int kEpiStride = 72;         // floats per staged output row
static constexpr int kEpiBytes = 4 * 32 * kEpiStride * 4;          // 32 rows per wave per pass
static constexpr int kScaleFloats = 128 + 32;                      // INT8: row + column scales
static constexpr int kRingBytes = kStages * kStageBytes;
static constexpr int kSmemBytes = kRingBytes + 4 * kScaleFloats * 4;

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
  int64_t a_rows;        // rows that exist (the buffer range ends there)
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

// LDS swizzle: 16-byte chunk c of a 64-byte tile row r sits in slot
// c ^ ((r >> 2) & 3).  A 16-lane group of a 16-byte fragment read covers 16
// consecutive rows at one chunk; 4 rows fill the 64 banks and (r >> 2) & 3
// moves each row quartet to different slots, so the group hits 64 distinct
// banks.  The direct-to-LDS loads write each wave's 1 KB lane-linearly.
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  // raw buffer (stride 0): loads at offsets >= bytes return zero
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// lds + 16 * l (the LDS address is wave-uniform and goes through M0).
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void* lds,
                                                  uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds, 16, (int)off, 0, 0, 0);
}

// Wait until at most n vector-memory operations of this wave are in flight.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// B-tile row of MFMA fragment j of wave column wn (lane's row inside it is
// lane % 32).  INT8: fragment 0 is the hi plane, 1 the lo plane, same columns.
template <bool I8>
__device__ __forceinline__ int b_frag_row(int wn, int j) {
  if (I8) return j * 64 + wn * 32;
  return wn * 64 + j * 32;
}

template <bool I8, bool DUMP>
__global__ void __launch_bounds__(kThreads, 2)
qgemm_kernel(GemmArgs g, EpiArgs e) {
  static_assert(kEpiBytes <= kRingBytes, "epilogue staging reuses the ring");
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
  const int64_t nb0 = (int64_t)tn * (I8 ? kTileB / 2 : kTileB);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Buffer resources based at this tile's first row: rows past the operand
  // (INT8 activations: rows >= M) fall outside the range and load zero.
  int64_t a_bytes = (g.a_rows - m0) * g.lda;
  if (a_bytes > 0x7FFFFFF0) a_bytes = 0x7FFFFFF0;
  const __amdgpu_buffer_rsrc_t ra_src = buffer_rsrc(g.A + m0 * g.lda, (uint32_t)a_bytes);
  const __amdgpu_buffer_rsrc_t rb_src = buffer_rsrc(g.B + nb0 * g.ldb, 0x7FFFFFF0u);

  // Direct-to-LDS staging.  A stage holds 256 A rows then 128 B rows of 64
  // bytes; one wave instruction fills 16 rows (1 KB): lane l takes row l/4
  // of its 16 and the chunk that belongs in slot l%4 of that row.  The 16 A
  // groups and 8 B groups of a stage are spread over the 4 waves.
  constexpr int kAGroups = kTileM / 16 / 4, kBGroups = kTileB / 16 / 4;   // per wave
  const int ld_chunk = (lane & 3) ^ ((lane >> 4) & 3);
  const uint32_t lane_a = (uint32_t)((lane >> 2) * g.lda + ld_chunk * 16);
  const uint32_t lane_b = (uint32_t)((lane >> 2) * g.ldb + ld_chunk * 16);
  auto issue = [&](int kt, int buf) {
    uint8_t* sbase = smem + buf * kStageBytes;
    const uint32_t kb = (uint32_t)kt * kRowBytes;
    // the INT8 activation rows are unpadded: a chunk past K loads zero
    const bool kin = !I8 || (int64_t)kb + ld_chunk * 16 < g.a_kbytes;
#pragma unroll
    for (int i = 0; i < kAGroups; ++i) {
      const int grp = i * 4 + wave;                // 16-row group of A, 0..15
      const uint32_t ao = (uint32_t)(grp * 16) * (uint32_t)g.lda + lane_a + kb;
      buffer_load_lds16(ra_src, sbase + grp * 1024, kin ? ao : 0x7FFFFFF0u);
    }
#pragma unroll
    for (int i = 0; i < kBGroups; ++i) {
      const int grp = i * 4 + wave;                // 16-row group of B, 0..7
      const int trow = grp * 16;
      const uint32_t bo = I8 ? (uint32_t)(trow / 64) * (uint32_t)g.b_plane +
                                   (uint32_t)(trow % 64) * (uint32_t)g.ldb
                             : (uint32_t)trow * (uint32_t)g.ldb;
      buffer_load_lds16(rb_src, sbase + kTileM * kRowBytes + grp * 1024, bo + lane_b + kb);
    }
  };

  typedef typename std::conditional<I8, i32x16, f32x16>::type acc_t;
  acc_t acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  // fragment rows of this lane are (multiple of 32) + lane % 32, so they
  // all share the swizzle of lane % 32
  const int a_frag = (wm * 128 + (lane & 31)) * kRowBytes;
  const int b_frag = (lane & 31) * kRowBytes;
  const int row_sw = swz(lane & 31);
  auto frags = [&](int buf, int s, u32x4 (&af)[kFM], u32x4 (&bf)[kFN]) {
    const uint8_t* sa = smem + buf * kStageBytes;
    const uint8_t* sb = sa + kTileM * kRowBytes;
    const int coff = ((2 * s + (lane >> 5)) ^ row_sw) << 4;
#pragma unroll
    for (int i = 0; i < kFM; ++i)
      af[i] = *reinterpret_cast<const u32x4*>(sa + a_frag + i * 32 * kRowBytes + coff);
#pragma unroll
    for (int j = 0; j < kFN; ++j)
      bf[j] = *reinterpret_cast<const u32x4*>(sb + b_frag + b_frag_row<I8>(wn, j) * kRowBytes +
                                              coff);
  };
  auto mfmas = [&](const u32x4 (&af)[kFM], const u32x4 (&bf)[kFN]) {
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j) {
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

  // Pipeline over the LDS ring: stages kt+1 and kt+2 are in flight while
  // stage kt is multiplied.  Before stage kt is read, each wave waits for
  // its own loads of stage kt (the loads of the younger stage may stay
  // outstanding) and a barrier makes every wave's loads visible; the same
  // barrier guarantees that stage kt-1's buffer, which the loads of stage
  // kt+2 overwrite, is no longer read.
  constexpr int kLoadsPerStage = kAGroups + kBGroups;
  const int nk = g.k_tiles;
  for (int p = 0; p < kStages - 1 && p < nk; ++p) issue(p, p);
  u32x4 fa0[kFM], fb0[kFN], fa1[kFM], fb1[kFN];
  int buf = 0, nbuf = kStages - 1;
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk)
      wait_vm<kLoadsPerStage>();
    else
      wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    if (kt + kStages - 1 < nk) issue(kt + kStages - 1, nbuf);
    frags(buf, 0, fa0, fb0);
    frags(buf, 1, fa1, fb1);
    mfmas(fa0, fb0);
    mfmas(fa1, fb1);
    buf = buf + 1 == kStages ? 0 : buf + 1;
    nbuf = nbuf + 1 == kStages ? 0 : nbuf + 1;
  }

  // ---- epilogue.  Accumulator r of a 32x32 MFMA tile holds row
  // (r/4)*8 + (lane/32)*4 + r%4 and column lane%32.  In passes of 32 rows,
  // each wave stages its values as float32 in LDS (row stride kEpiStride
  // floats: the two half-waves write disjoint banks), then reads them back
  // row-contiguous and stores 4 consecutive outputs per lane.
  __syncthreads();                       // every wave is done with the operand ring
  const int lrow = (lane >> 5) * 4, lcol = lane & 31;
  constexpr int kOutCols = I8 ? 32 : 64;           // output columns per wave
  const int64_t wave_row0 = m0 + wm * 128;
  const int64_t wave_col0 = nb0 + wn * kOutCols;
  if constexpr (I8 && DUMP) {          // verification dump of the exact sums
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = wave_row0 + i * 32 + (r >> 2) * 8 + lrow + (r & 3);
        const int64_t col = wave_col0 + lcol;
        if (row < e.M && col < e.N) {
          g.acc_hi[row * e.N + col] = acc[i][0][r];
          g.acc_lo[row * e.N + col] = acc[i][1][r];
        }
      }
    return;
  }
  float* ep = reinterpret_cast<float*>(smem) + wave * (32 * kEpiStride);
  const float alpha = I8 ? 1.0f : (*g.a_ts) * (*g.w_ts);
  // INT8: the wave's row scales (s_a) and column scales (s_Tw 2^(Fr-11))
  // go to LDS once, so the store loop reads no scale from global memory
  float* sc_row = reinterpret_cast<float*>(smem + kRingBytes) + wave * kScaleFloats;
  float* sc_col = sc_row + 128;
  if constexpr (I8) {
    for (int i = lane; i < 128; i += 64) {
      const int64_t row = wave_row0 + i;
      sc_row[i] = row < e.M ? g.a_s[row] : 0.0f;
    }
    if (lane < 32) {
      const int64_t col = wave_col0 + lane;
      sc_col[lane] = col < e.N ? g.colscale[col] : 0.0f;
    }
  }
  constexpr int kLanesPerRow = kOutCols / 4;       // 4 outputs per lane
  constexpr int kRowsPerIter = 64 / kLanesPerRow;
#pragma unroll
  for (int ip = 0; ip < kFM; ++ip) {
#pragma unroll
    for (int jj = 0; jj < kOutCols / 32; ++jj)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v;
        if constexpr (I8)
          v = fmaf(128.0f, (float)acc[ip][0][r], (float)acc[ip][1][r]);
        else
          v = acc[ip][jj][r] * alpha;
        ep[((r >> 2) * 8 + lrow + (r & 3)) * kEpiStride + jj * 32 + lcol] = v;
      }
    __syncthreads();
    for (int it = 0; it < 32 / kRowsPerIter; ++it) {
      const int rl = it * kRowsPerIter + lane / kLanesPerRow;
      const int c4 = (lane % kLanesPerRow) * 4;
      const int64_t row = wave_row0 + ip * 32 + rl;
      const int64_t col = wave_col0 + c4;
      if (row >= e.M || col >= e.N) continue;
      const f32x4 v4 = *reinterpret_cast<const f32x4*>(ep + rl * kEpiStride + c4);
      float v[4] = {v4[0], v4[1], v4[2], v4[3]};
      const float rs = I8 ? sc_row[ip * 32 + rl] : 1.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (I8) v[q] = v[q] * rs * sc_col[c4 + q];
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
  return (size_t)round_up(round_up(M, kTileM) * kp * 2, 256) +
         (size_t)round_up(N, kTileB) * kp * 2;
}

size_t int8_gemm_ws_bytes(int64_t, int64_t N, int64_t K) {
  const int64_t kp = kpad_bytes(K), np = round_up(N, kTileB / 2);
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
  if (i8 && g.acc_hi)
    hipLaunchKernelGGL((qgemm_kernel<true, true>), dim3(grid), dim3(kThreads), 0, st, g, e);
  else if (i8)
    hipLaunchKernelGGL((qgemm_kernel<true, false>), dim3(grid), dim3(kThreads), 0, st, g, e);
  else
    hipLaunchKernelGGL((qgemm_kernel<false, false>), dim3(grid), dim3(kThreads), 0, st, g, e);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess && g_ev_after) err = hipEventRecord(g_ev_after, st);
  return err;
}

hipError_t launch_nvfp4_gemm(const uint8_t* a_q, const uint8_t* a_s, const float* a_ts,
                             const uint8_t* w_q, const uint8_t* w_s, const float* w_ts,
                             int64_t M, int64_t N, int64_t K, const GemmOut& o, void* ws,
                             hipStream_t st) {
  const int64_t kp = kpad_bytes(2 * K) / 2;
  const int64_t mp = round_up(M, kTileM), np = round_up(N, kTileB);
  uint16_t* a_bf = static_cast<uint16_t*>(ws);
  uint16_t* w_bf =
      reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + round_up(mp * kp * 2, 256));
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
  g.mt = (int)(mp / kTileM);
  g.nt = (int)(np / kTileB);
  g.a_ts = a_ts;
  g.w_ts = w_ts;
  EpiArgs e = {o.y, o.ldy, o.out_f32, o.gelu, o.bias, M, N, vec_ok(o)};
  return launch_gemm(false, g, e, st);
}

hipError_t launch_int8_gemm(const int8_t* a_q, const float* a_s, const uint8_t* w_q,
                            const uint8_t* w_s, const float* w_ts, int64_t M, int64_t N,
                            int64_t K, const GemmOut& o, int32_t* acc_hi, int32_t* acc_lo,
                            void* ws, hipStream_t st) {
  const int64_t kp = kpad_bytes(K), np = round_up(N, kTileB / 2);
  int8_t* planes = static_cast<int8_t*>(ws);
  float* colscale =
      reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + round_up(2 * np * kp, 256));
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
  g.mt = (int)((M + kTileM - 1) / kTileM);
  g.nt = (int)(np / (kTileB / 2));
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
