// Quantized linear GEMMs on gfx950 MFMA:  Y = dequant(A) dequant(W)^T.
//
// 6Bit-Diffusion, abstract and Fig. 2 caption: every internal linear of a
// DiT block runs with NVFP4 (4-bit) weights and NVFP4 or INT8 activations.
//
// No gfx950 matrix instruction takes NVFP4's E4M3 scale per 16 elements
// (its block-scaled FP4 MFMA takes power-of-two scales per 32).  Every
// NVFP4 value -- an E2M1 value times an E4M3 scale, at most 6 significant
// bits between 2^-10 and 2688 -- and every int8 is exact in fp16, and their
// products are exact in the fp32 accumulator of v_mfma_f32_32x32x16_f16.
// The kernel therefore reads the quantized operands as they are stored and
// expands them to fp16 inside the workgroup ("dequant on load"): the bytes
// that cross L2 are the 4-bit codes (plus one scale byte per 16) or the
// int8 activations, not a 2-byte copy of each operand.  The float32 tensor
// scales (and the INT8 per-row scales) are applied in the epilogue.
//
// Workgroup: 8 waves, a 256 x 256 output tile; wave (wm, wn) owns rows
// 128 wm .. +128 and columns 64 wn .. +64 as 4 x 2 MFMA tiles of 32 x 32.
// K runs in fp16 stages of 32 (a 64-byte row slice per operand row).
//
// Data path per stage, all of it overlapped with the MFMAs:
//   global --(DMA, buffer_load ... lds)--> raw ring in LDS, 4 units of two
//   stages (NVFP4 rows: 32 bytes of codes; INT8 rows: 64 bytes; one 4-byte
//   word of E4M3 scales per row from a per-tile copy of the scales);
//   A: raw ring --(ds_read, expand to fp16, ds_write)--> fp16 ring (3
//   stages) --(ds_read)--> MFMA fragments;
//   W: raw ring --(ds_read, expand to fp16)--> MFMA fragments directly.
// LDS writes are the scarce resource on gfx950 (about a third of the read
// bandwidth), so only A -- which 4 waves share -- is written back as fp16;
// each W fragment is used by 2 waves, which both expand it.  Within a stage
// the K order is permuted so that a lane's W words are contiguous: MFMA
// k-step s, lane half h takes K elements 8 (2h + s) .. +7 of the stage
// (the same for A and W, so the products pair up as before).
//
// Schedule: the wave rows form two groups, X (wm 0) and Y (wm 1); each SIMD
// holds one wave of each.  A wave alternates a memory phase (issue DMA,
// convert the next stage, read this stage's fragments) and a compute phase
// (16 MFMAs), with a workgroup barrier after each.  Y runs one barrier
// behind X, so on every SIMD one wave multiplies while the other moves and
// converts data.  Workgroups are remapped so each XCD works a contiguous,
// grouped band of tiles (L2 reuse).
#include "qact_device.h"
#include "qact_internal.h"

namespace qact {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

static constexpr int kThreads = 512;
static constexpr int kTileM = 256, kTileN = 256;
static constexpr int kStageK = 32;              // K per fp16 stage
static constexpr int kUnitK = 64;               // K per raw unit (two stages)
static constexpr int kRowBytes = 64;            // fp16 bytes per tile row per stage
static constexpr int kF16Stage = kTileM * kRowBytes;   // A only: 16 KB
static constexpr int kF16Bufs = 3;
static constexpr int kRawSlots = 4;
#ifndef QACT_GROUP_M
#define QACT_GROUP_M 8
#endif
#ifndef QACT_VALU_PER_MFMA
#define QACT_VALU_PER_MFMA 3
#endif
#ifndef QACT_COMPUTE_PRIO
#define QACT_COMPUTE_PRIO 0
#endif
static constexpr int kGroupM = QACT_GROUP_M;
static constexpr int kFM = 4, kFN = 2;          // MFMA tiles per wave (rows, columns)

// One raw unit in LDS: A codes, B codes, A scale words, B scale words.
// B starts half a bank row (128 bytes) after the end of A, so that the A
// and B words a lane reads sit in different banks.
template <bool I8>
struct Raw {
  static constexpr int kA = 0;
  static constexpr int kB = kTileM * (I8 ? 64 : 32) + 128;
  static constexpr int kAS = kB + kTileN * 32;
  static constexpr int kBS = kAS + kTileM * 4 + 128;
  static constexpr int kSlot = kBS + kTileN * 4 + 128;
  static constexpr int kSmem = kF16Bufs * kF16Stage + kRawSlots * kSlot;
  static constexpr int kLoads = I8 ? 4 : 3;     // DMA instructions per wave per unit
};
static_assert(Raw<true>::kSmem <= 160 * 1024, "LDS");

static inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
static inline int64_t units_of(int64_t K) { return (K + kUnitK - 1) / kUnitK; }

// ------------------------------------------------------- scale re-layout --

// E4M3 scales [rows][K/16] -> per 256-row tile and K unit of 64, the 4
// scale bytes of each row as one word: dst[(tile * units + u) * 256 + r].
// Rows past `rows` and groups past K/16 read as 0 (a zero scale makes the
// corresponding fp16 values zero, whatever codes the raw unit holds there).
// One workgroup per (tile, unit), one thread per row.
__global__ void __launch_bounds__(256)
scale_tiles_kernel(const uint8_t* __restrict__ s, int64_t rows, int64_t K, int units,
                   uint32_t* __restrict__ dst) {
  const int tu = (int)blockIdx.x;
  const int u = tu % units, t = tu / units;
  const int64_t row = (int64_t)t * 256 + threadIdx.x;
  const int64_t gpr = K / 16;
  uint32_t v = 0;
  if (row < rows) {
    const uint8_t* p = s + row * gpr + 4 * u;
    if ((gpr & 3) == 0 && (reinterpret_cast<uintptr_t>(s) & 3) == 0 && 4 * (int64_t)u + 4 <= gpr) {
      v = *reinterpret_cast<const uint32_t*>(p);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * (int64_t)u + j < gpr) v |= (uint32_t)p[j] << (8 * j);
    }
  }
  dst[(int64_t)tu * 256 + threadIdx.x] = v;
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

// ---------------------------------------------------------------- GEMM --

struct GemmArgs {
  const uint8_t* a;      // NVFP4 codes [M][K/2] or int8 [M][K]
  const uint32_t* a_st;  // NVFP4: per-tile scale words of A
  const uint8_t* b;      // NVFP4 codes [N][K/2]
  const uint32_t* b_st;  // per-tile scale words of W
  int64_t K;
  int units, nk;         // raw units of 64 and fp16 stages of 32 along K
  int mt, nt;            // tile counts
  const float* a_ts;     // NVFP4: activation tensor scale
  const float* w_ts;     // weight tensor scale
  const float* a_rs;     // INT8: per-row activation scale
};

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

// fp16 tile rows: 16-byte chunk c (K elements 8c .. 8c+7 of the stage) of
// row r sits in slot c ^ ((r >> 2) & 3), so that 16 consecutive rows at one
// chunk (an MFMA fragment read, a conversion write) hit 64 distinct banks.
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

// 8 E2M1 codes (one word, element 2i in the low nibble of byte i) times the
// fp16 scale pair sc -> 8 fp16 values.  The conversion with a unit scale
// and the fp16 product are both exact.
__device__ __forceinline__ u32x4 nvfp4_chunk(uint32_t w, f16x2 sc) {
  u32x4 o;
  o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sc);
  o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sc);
  o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sc);
  o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sc);
  return o;
}

// 4 int8 -> 4 fp16: byte b + 128 placed under the fp16 exponent of 1024
// gives 1024 + b + 128 exactly; subtracting 1152 leaves b.
__device__ __forceinline__ u32x2 int8_quad(uint32_t w) {
  const uint32_t x = w ^ 0x80808080u;
  const f16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  const f16x2 lo =
      __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u)) - bias;
  const f16x2 hi =
      __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u)) - bias;
  return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// E4M3 scale byte `idx` (0..3) of a scale word -> the fp16 pair {s, s}
// (every E4M3 value is exact in fp16).
__device__ __forceinline__ f16x2 scale_pair(uint32_t word, int idx) {
  const f16x2 two = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(idx >= 2 ? word >> 16 : word, 1.0f, false);
  const _Float16 s = (idx & 1) ? two[1] : two[0];
  return f16x2{s, s};
}

template <bool I8>
__global__ void __launch_bounds__(kThreads, 1)
qgemm_kernel(GemmArgs g, EpiArgs e) {
  using R = Raw<I8>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[R::kSmem];
  uint8_t* const raw_base = smem + kF16Bufs * kF16Stage;

  // XCD-aware tile order: hardware deals workgroups to the 8 XCDs in turn;
  // give each XCD a contiguous range of logical tiles, grouped kGroupM
  // tile-rows at a time so that concurrent tiles share A rows and B rows.
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
  const int64_t m0 = (int64_t)tm * kTileM, n0 = (int64_t)tn * kTileN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);     // uniform per wave
  const int wm = wave >> 2, wn = wave & 3;
  const int64_t K = g.K;

  // Buffer resources based at this tile's first row; rows past the operand
  // fall outside the range and load zero.
  const int64_t a_row = I8 ? K : K / 2, b_row = K / 2;
  const int64_t a_rows = min<int64_t>(e.M - m0, kTileM), b_rows = min<int64_t>(e.N - n0, kTileN);
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(g.a + m0 * a_row, (uint32_t)(a_rows * a_row));
  const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(g.b + n0 * b_row, (uint32_t)(b_rows * b_row));
  const uint32_t st_bytes = (uint32_t)g.units * 1024u;
  const __amdgpu_buffer_rsrc_t ras =
      buffer_rsrc(I8 ? g.b_st : g.a_st + (size_t)tm * g.units * 256, I8 ? 0u : st_bytes);
  const __amdgpu_buffer_rsrc_t rbs = buffer_rsrc(g.b_st + (size_t)tn * g.units * 256, st_bytes);
  constexpr uint32_t kOOB = 0x7FFFFFF0u;

  // ---- DMA of raw unit u into slot u % 3.  Each wave moves rows 32w ..
  // 32w+31 of the codes of A and of B, and one scale block of 64 rows.
  // NVFP4 rows (32 bytes per unit): lane l takes row l/2 and the half that
  // the conversion reads without bank conflicts from slot l%2 (global half
  // slot ^ ((row >> 3) & 1)).  INT8 rows (64 bytes): two instructions of
  // 16 rows; lane l takes row l/4 and for slot l%4 the global chunk
  // slot ^ (((row >> 2) & 1) * 2).  Chunks past the end of a row load zero.
  const uint32_t nv_row = (uint32_t)(32 * wave + (lane >> 1));
  const uint32_t nv_half = (uint32_t)((lane & 1) ^ ((nv_row >> 3) & 1));
  auto issue_unit = [&](int u) {
    uint8_t* s = raw_base + (u % kRawSlots) * R::kSlot;
    const uint32_t kb_nv = (uint32_t)u * 32u + nv_half * 16u;      // byte in an NVFP4 row
    if constexpr (I8) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t row = (uint32_t)(32 * wave + 16 * i + (lane >> 2));
        const uint32_t c = (uint32_t)((lane & 3) ^ (((row >> 2) & 1) * 2));
        const uint32_t kb = (uint32_t)u * 64u + c * 16u;
        dma16(ra, s + R::kA + (32 * wave + 16 * i) * 64,
                kb < (uint32_t)K ? row * (uint32_t)a_row + kb : kOOB);
      }
    } else {
      dma16(ra, s + R::kA + 32 * wave * 32,
              kb_nv < (uint32_t)b_row ? nv_row * (uint32_t)a_row + kb_nv : kOOB);
    }
    dma16(rb, s + R::kB + 32 * wave * 32,
            kb_nv < (uint32_t)b_row ? nv_row * (uint32_t)b_row + kb_nv : kOOB);
    // scale words: NVFP4 waves 0-3 take A, 4-7 take B; INT8 waves 0-3 take
    // B and waves 4-7 issue a load that reads zero into the unused A area
    const int sw = wave & 3;
    const uint32_t so = (uint32_t)u * 1024u + (uint32_t)(64 * sw + lane) * 4u;
    if (I8 ? wave >= 4 : wave < 4)
      dma4(ras, s + R::kAS + 64 * sw * 4, I8 ? kOOB : so);
    else
      dma4(rbs, s + R::kBS + 64 * sw * 4, so);
  };
  // wait for this wave's DMA of unit `need`; units up to `last` issued
  auto wait_unit = [&](int need, int last) {
    const int younger = min(g.units - 1, last) - need;
    if (younger >= 3)
      wait_vm<3 * R::kLoads>();
    else if (younger == 2)
      wait_vm<2 * R::kLoads>();
    else if (younger == 1)
      wait_vm<R::kLoads>();
    else
      wait_vm<0>();
  };

  // ---- A: expansion of fp16 stage st into fp16 buffer st % 3.  The
  // thread handles row (128 wm + t/2), K elements 16h .. 16h+15 of the
  // stage (one E4M3 scale group, fp16 chunks 2h and 2h+1), h = t % 2.
  const int ct = tid & 255;
  const int crow = wm * 128 + (ct >> 1), chf = ct & 1;
  const int crow_sw = swz(crow);
  struct RawA {
    u32x4 a;             // NVFP4: a[0..1] codes; INT8: 16 int8
    uint32_t as;         // NVFP4: scale word
  };
  auto read_a = [&](int st) {
    const uint8_t* s = raw_base + ((st >> 1) % kRawSlots) * R::kSlot;
    const int sh = st & 1;                       // stage within the unit
    RawA r;
    if constexpr (I8) {
      r.as = 0;
      r.a = *reinterpret_cast<const u32x4*>(
          s + R::kA + crow * 64 + 16 * ((2 * sh + chf) ^ (((crow >> 2) & 1) * 2)));
    } else {
      r.as = *reinterpret_cast<const uint32_t*>(s + R::kAS + crow * 4);
      const u32x2 a2 = *reinterpret_cast<const u32x2*>(
          s + R::kA + crow * 32 + 16 * (sh ^ ((crow >> 3) & 1)) + 8 * chf);
      r.a = u32x4{a2[0], a2[1], 0u, 0u};
    }
    return r;
  };
  auto store_a = [&](int st, const RawA& r) {
    uint8_t* fa = smem + (st % kF16Bufs) * kF16Stage + crow * kRowBytes;
    const int c0 = 2 * chf, c1 = 2 * chf + 1;
    if constexpr (I8) {
      const u32x2 q0 = int8_quad(r.a[0]), q1 = int8_quad(r.a[1]);
      const u32x2 q2 = int8_quad(r.a[2]), q3 = int8_quad(r.a[3]);
      *reinterpret_cast<u32x4*>(fa + ((c0 ^ crow_sw) << 4)) = u32x4{q0[0], q0[1], q1[0], q1[1]};
      *reinterpret_cast<u32x4*>(fa + ((c1 ^ crow_sw) << 4)) = u32x4{q2[0], q2[1], q3[0], q3[1]};
    } else {
      const f16x2 asc = scale_pair(r.as, 2 * (st & 1) + chf);
      *reinterpret_cast<u32x4*>(fa + ((c0 ^ crow_sw) << 4)) = nvfp4_chunk(r.a[0], asc);
      *reinterpret_cast<u32x4*>(fa + ((c1 ^ crow_sw) << 4)) = nvfp4_chunk(r.a[1], asc);
    }
  };
  auto expand_a = [&](int st) { store_a(st, read_a(st)); };

  f32x16 acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // A fragment rows of this lane are (multiple of 32) + lane % 32, so they
  // all share the swizzle of lane % 32; k-step s reads fp16 chunk 2h + s.
  const int a_frag = (wm * 128 + (lane & 31)) * kRowBytes;
  const int row_sw = swz(lane & 31);
  const int lh = lane >> 5;
  auto frags_a = [&](int st, int s, u32x4 (&af)[kFM]) {
    const uint8_t* sb = smem + (st % kF16Bufs) * kF16Stage;
    const int coff = ((2 * lh + s) ^ row_sw) << 4;
#pragma unroll
    for (int i = 0; i < kFM; ++i)
      af[i] = *reinterpret_cast<const u32x4*>(sb + a_frag + i * 32 * kRowBytes + coff);
  };
  // W fragments of stage st straight from the raw unit: lane (h, n) reads
  // the 8 code bytes 8h .. 8h+7 of row n's stage (words 2h, 2h+1: one scale
  // group) and expands word 2h+s into the fragment of k-step s.
  struct RawB {
    u32x2 w[kFN];
    uint32_t sw[kFN];
  };
  auto read_b = [&](int st) {
    const uint8_t* s = raw_base + ((st >> 1) % kRawSlots) * R::kSlot;
    const int sh = st & 1;
    RawB r;
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      const int n = wn * 64 + j * 32 + (lane & 31);
      r.w[j] = *reinterpret_cast<const u32x2*>(s + R::kB + n * 32 + 16 * (sh ^ ((n >> 3) & 1)) +
                                               8 * lh);
      r.sw[j] = *reinterpret_cast<const uint32_t*>(s + R::kBS + n * 4);
    }
    return r;
  };
  auto conv_b = [&](int st, const RawB& r, u32x4 (&b0)[kFN], u32x4 (&b1)[kFN]) {
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      const f16x2 sc = scale_pair(r.sw[j], 2 * (st & 1) + lh);
      b0[j] = nvfp4_chunk(r.w[j][0], sc);
      b1[j] = nvfp4_chunk(r.w[j][1], sc);
    }
  };
  auto frags_b = [&](int st, u32x4 (&b0)[kFN], u32x4 (&b1)[kFN]) { conv_b(st, read_b(st), b0, b1); };
  // The MFMA is issued as W x A^T: accumulator r of tile (i, j) then holds
  // output row 32i + lane % 32 of the wave's rows and output column
  // 32j + (r/4)*8 + (lane/32)*4 + r%4 of its columns, so that each lane
  // owns runs of 4 consecutive outputs of one row (stored directly).
  auto mfmas = [&](const u32x4 (&af)[kFM], const u32x4 (&bf)[kFN]) {
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, bf[j]),
                                                           __builtin_bit_cast(f16x8, af[i]),
                                                           acc[i][j], 0, 0, 0);
  };
  // a workgroup barrier that the compiler moves no instruction across
  auto barrier = [] {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto wait_lds = [] { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); };
  // an opaque identity at this point of the program: arithmetic that uses
  // the value cannot be hoisted above it (nor above the barrier before it)
  auto pin = [](auto& v) { asm volatile("" : "+v"(v)); };

  // ---- pipeline.  Memory phase k of a wave: (even k >= 2) issue raw unit
  // k/2 + 3, read the A fragments of stage k, wait for its own DMA of the
  // unit of stage k+3; it also reads the raw words of W stage k+1 and A
  // stage k+2 into registers.  Compute phase k: the MFMAs of stage k and,
  // under them, the expansion of those words into the W fragments of stage
  // k+1 and the A rows of stage k+2 (fp16 buffer (k+2) % 3).  X runs
  // memory phase k at phase 2k and compute phase k at 2k+1; Y runs each
  // one phase later; every phase ends with lgkmcnt(0) and a workgroup
  // barrier.
  //  * fp16 stage k+2 is written by X and Y in their compute phases k
  //    (phases 2k+1, 2k+2) and read in their memory phases k+2 (2k+4,
  //    2k+5); its buffer held stage k-1, last read in phase 2k-1;
  //  * raw unit v is first read in memory phase 2v-2 (X: phase 4v-4);
  //    every wave waited for its own DMA of it in memory phase 2v-3 (Y:
  //    phase 4v-5) or, for v <= 1, before the loop;
  //  * raw unit v+4, issued in memory phase 2v+2 (phase 4v+4 at the
  //    earliest), overwrites unit v, whose last reads (W words of stage
  //    2v+1 in memory phase 2v, phase 4v+1 at the latest) have completed.
  const int nk = g.nk;
  for (int u = 0; u < kRawSlots && u < g.units; ++u) issue_unit(u);
  if (g.units > 1)
    wait_unit(1, kRawSlots - 1);
  else
    wait_unit(0, kRawSlots - 1);
  barrier();
  expand_a(0);
  if (nk > 1) expand_a(1);
  u32x4 fbA0[kFN], fbA1[kFN], fbB0[kFN], fbB1[kFN];
  frags_b(0, fbA0, fbA1);
#pragma unroll
  for (int j = 0; j < kFN; ++j) {
    pin(fbA0[j]);
    pin(fbA1[j]);
  }
  wait_lds();
  barrier();
  if (wm == 1) barrier();
  u32x4 fa0[kFM], fa1[kFM];
  // one stage; (b0, b1) hold its W fragments, (n0, n1) receive stage kt+1's
  auto step = [&](int kt, u32x4 (&b0)[kFN], u32x4 (&b1)[kFN], u32x4 (&n0)[kFN],
                  u32x4 (&n1)[kFN]) {
    // memory phase
    if (kt >= 2 && !(kt & 1)) {
      const int u = (kt >> 1) + 3;
      if (u < g.units) issue_unit(u);
    }
    frags_a(kt, 0, fa0);
    frags_a(kt, 1, fa1);
    // raw words of the next expansions (their units are already visible:
    // the unit of stage kt+2 was waited for by every wave in its memory
    // phase kt-1).  Past the last stage these are stale words whose
    // expansions land in registers and an fp16 buffer no longer read.
    const RawB rb = read_b(kt + 1);
    const RawA ra = read_a(kt + 2);
    if (kt + 3 < nk) wait_unit((kt + 3) >> 1, (kt >> 1) + 3);
    wait_lds();
    barrier();
    // compute phase, free of branches so that the expansions interleave
    // with the MFMAs: one MFMA and three VALU instructions at a time, then
    // the fp16 stores of A stage kt+2 into buffer (kt+2) % 3 (which holds
    // no stage that is still to be read).
    RawB rbp = rb;
    RawA rap = ra;
    pin(rbp.w[0]); pin(rbp.w[1]); pin(rbp.sw[0]); pin(rbp.sw[1]);
    pin(rap.a); pin(rap.as);
    if (QACT_COMPUTE_PRIO) __builtin_amdgcn_s_setprio(QACT_COMPUTE_PRIO);
    mfmas(fa0, b0);
    mfmas(fa1, b1);
    conv_b(kt + 1, rbp, n0, n1);
    store_a(kt + 2, rap);
#pragma unroll
    for (int i = 0; i < 2 * kFM * kFN; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, QACT_VALU_PER_MFMA, 0);   // VALU
    }
    __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);     // DS writes
    // the W fragments of stage kt+1 are complete here (not sunk into the
    // next memory phase)
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      pin(n0[j]);
      pin(n1[j]);
    }
    if (QACT_COMPUTE_PRIO) __builtin_amdgcn_s_setprio(0);
    wait_lds();
    barrier();
  };
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, fbA0, fbA1, fbB0, fbB1);
    if (kt + 1 < nk) step(kt + 1, fbB0, fbB1, fbA0, fbA1);
  }
  if (wm == 0) barrier();

  // ---- epilogue.  Lane (h, c) of accumulator tile (i, j) owns row 32i + c
  // and, for q = 0..3, the 4 consecutive columns 32j + 8q + 4h .. +3
  // (h = lane/32, c = lane%32).  Scale, bias, GELU and the rounding are
  // applied in registers.  bf16 output (the usual case) is staged per
  // 32-row slice through this wave's own 4 KB of the (now idle) fp16 area
  // -- rows of 128 bytes, 16-byte chunk k of row r at slot k ^ (r & 7) --
  // and leaves as 8 rows x 128 contiguous bytes per store instruction;
  // f32 or unaligned output is stored straight from the registers.
  wait_vm<0>();          // no DMA into LDS outlives the workgroup
  __syncthreads();       // every wave is past its last read of the rings
  const int64_t wave_row0 = m0 + wm * 128;
  const int64_t wave_col0 = n0 + wn * 64;
  const float alpha = I8 ? *g.w_ts : (*g.a_ts) * (*g.w_ts);
  auto epi_vals = [&](int i, int j, int q, float rs, float (&v)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) v[t] = acc[i][j][4 * q + t] * rs;
    if (e.bias) {
      const int64_t col = wave_col0 + j * 32 + q * 8 + lh * 4;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (col + t < e.N) v[t] += __uint_as_float((uint32_t)e.bias[col + t] << 16);
    }
    if (e.gelu)
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = gelu_tanh(v[t]);
  };
  if (!e.out_f32 && e.vec_ok) {
    uint8_t* const stg = smem + wave * 4096;
    const int c = lane & 31;
#pragma unroll
    for (int i = 0; i < kFM; ++i) {
      const int64_t arow = wave_row0 + i * 32 + c;
      const float rs = I8 ? (arow < e.M ? g.a_rs[arow] : 0.0f) * alpha : alpha;
#pragma unroll
      for (int j = 0; j < kFN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v[4];
          epi_vals(i, j, q, rs, v);
          *reinterpret_cast<u32x2*>(stg + c * 128 + (((4 * j + q) ^ (c & 7)) << 4) + 8 * lh) =
              u32x2{bf16_pack(v[0], v[1]), bf16_pack(v[2], v[3])};
        }
      wait_lds();
      // this pass's 32 x 64 block: rows below e.M - prow0, columns below
      // e.N - wave_col0 exist
      const int64_t prow0 = wave_row0 + i * 32;
      uint16_t* const ybase = static_cast<uint16_t*>(e.y) + prow0 * e.ldy + wave_col0;
      const int64_t rows_left = e.M - prow0, cols_left = e.N - wave_col0;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int r = it * 8 + (lane >> 3), k = lane & 7;
        const u32x4 d = *reinterpret_cast<const u32x4*>(stg + r * 128 + ((k ^ (r & 7)) << 4));
        if (r < rows_left && k * 8 < cols_left) {
          uint16_t* yp = ybase + (int64_t)r * e.ldy + k * 8;
          if (k * 8 + 8 <= cols_left)
            *reinterpret_cast<u32x4*>(yp) = d;
          else
            for (int t = 0; k * 8 + t < cols_left; ++t)
              yp[t] = (uint16_t)(d[t >> 1] >> (16 * (t & 1)));
        }
      }
      wait_lds();
    }
  } else {
#pragma unroll
    for (int i = 0; i < kFM; ++i) {
      const int64_t row = wave_row0 + i * 32 + (lane & 31);
      if (row >= e.M) continue;
      const float rs = I8 ? g.a_rs[row] * alpha : alpha;
#pragma unroll
      for (int j = 0; j < kFN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t col = wave_col0 + j * 32 + q * 8 + lh * 4;
          if (col >= e.N) continue;
          float v[4];
          epi_vals(i, j, q, rs, v);
          if (e.out_f32) {
            float* yp = static_cast<float*>(e.y) + row * e.ldy + col;
            if (col + 4 <= e.N && e.vec_ok)
              *reinterpret_cast<f32x4*>(yp) = f32x4{v[0], v[1], v[2], v[3]};
            else
              for (int t = 0; t < 4 && col + t < e.N; ++t) yp[t] = v[t];
          } else {
            uint16_t* yp = static_cast<uint16_t*>(e.y) + row * e.ldy + col;
            const uint32_t p01 = bf16_pack(v[0], v[1]), p23 = bf16_pack(v[2], v[3]);
            const uint32_t pk[4] = {p01 & 0xFFFFu, p01 >> 16, p23 & 0xFFFFu, p23 >> 16};
            for (int t = 0; t < 4 && col + t < e.N; ++t) yp[t] = (uint16_t)pk[t];
          }
        }
    }
  }
}

// ---------------------------------------------------------------- host --

static int vec_ok(const GemmOut& o) {
  return (reinterpret_cast<uintptr_t>(o.y) % 16 == 0) && (o.ldy % 4 == 0);
}

static size_t scale_tiles_bytes(int64_t rows, int64_t K) {
  return (size_t)((rows + kTileM - 1) / kTileM) * (size_t)units_of(K) * 1024u;
}

size_t nvfp4_gemm_ws_bytes(int64_t M, int64_t N, int64_t K) {
  return (size_t)round_up((int64_t)scale_tiles_bytes(M, K), 256) + scale_tiles_bytes(N, K);
}

size_t int8_gemm_ws_bytes(int64_t, int64_t N, int64_t K) { return scale_tiles_bytes(N, K); }

static hipEvent_t g_ev_before = nullptr, g_ev_after = nullptr;

void set_gemm_events(hipEvent_t before, hipEvent_t after) {
  g_ev_before = before;
  g_ev_after = after;
}

static hipError_t launch_scale_tiles(const uint8_t* s, int64_t rows, int64_t K, uint32_t* dst,
                                     hipStream_t st) {
  const int64_t tiles = (rows + kTileM - 1) / kTileM, units = units_of(K);
  hipLaunchKernelGGL(scale_tiles_kernel, dim3((unsigned)(tiles * units)), dim3(256), 0, st, s, rows,
                     K, (int)units, dst);
  return hipGetLastError();
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

static GemmArgs base_args(int64_t M, int64_t N, int64_t K) {
  GemmArgs g = {};
  g.K = K;
  g.units = (int)units_of(K);
  g.nk = (int)((K + kStageK - 1) / kStageK);
  g.mt = (int)((M + kTileM - 1) / kTileM);
  g.nt = (int)((N + kTileN - 1) / kTileN);
  return g;
}

hipError_t launch_nvfp4_gemm(const uint8_t* a_q, const uint8_t* a_s, const float* a_ts,
                             const uint8_t* w_q, const uint8_t* w_s, const float* w_ts,
                             int64_t M, int64_t N, int64_t K, const GemmOut& o, void* ws,
                             hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  uint32_t* a_st = static_cast<uint32_t*>(ws);
  uint32_t* b_st = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) +
                                               round_up((int64_t)scale_tiles_bytes(M, K), 256));
  hipError_t err = launch_scale_tiles(a_s, M, K, a_st, st);
  if (err == hipSuccess) err = launch_scale_tiles(w_s, N, K, b_st, st);
  if (err != hipSuccess) return err;
  GemmArgs g = base_args(M, N, K);
  g.a = a_q;
  g.a_st = a_st;
  g.b = w_q;
  g.b_st = b_st;
  g.a_ts = a_ts;
  g.w_ts = w_ts;
  EpiArgs e = {o.y, o.ldy, o.out_f32, o.gelu, o.bias, M, N, vec_ok(o)};
  return launch_gemm(false, g, e, st);
}

hipError_t launch_int8_gemm(const int8_t* a_q, const float* a_s, const uint8_t* w_q,
                            const uint8_t* w_s, const float* w_ts, int64_t M, int64_t N,
                            int64_t K, const GemmOut& o, void* ws, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  uint32_t* b_st = static_cast<uint32_t*>(ws);
  hipError_t err = launch_scale_tiles(w_s, N, K, b_st, st);
  if (err != hipSuccess) return err;
  GemmArgs g = base_args(M, N, K);
  g.a = reinterpret_cast<const uint8_t*>(a_q);
  g.b = w_q;
  g.b_st = b_st;
  g.w_ts = w_ts;
  g.a_rs = a_s;
  EpiArgs e = {o.y, o.ldy, o.out_f32, o.gelu, o.bias, M, N, vec_ok(o)};
  return launch_gemm(true, g, e, st);
}

}  // namespace qact
