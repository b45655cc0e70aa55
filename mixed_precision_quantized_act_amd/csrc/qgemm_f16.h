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
// expands them to fp16 in registers ("dequant on load"): the bytes that
// cross L2 and LDS are the 4-bit codes (plus one scale byte per 16) or the
// int8 activations, not a 2-byte copy of each operand.  The float32 tensor
// scales (and the INT8 per-row scales) are applied in the epilogue.
//
// Workgroup: 4 waves (one per SIMD), a 256 x 256 output tile; wave (wm, wn)
// owns rows 128 wm .. +128 and columns 128 wn .. +128 as 4 x 4 MFMA tiles
// of 32 x 32 (256 accumulators per lane).  K runs in stages of 32.
//
// Data path:
//   global --(DMA, buffer_load ... lds)--> raw ring in LDS, kRawSlots (4) units of two
//   stages (NVFP4 rows: 32 bytes of codes; INT8 rows: 64 bytes; one 4-byte
//   word of E4M3 scales per row from a per-tile copy of the scales);
//   raw ring --(ds_read, expand to fp16 in registers)--> MFMA fragments,
//   for A and for W alike.
// LDS traffic is therefore the DMA writes plus one read of each raw byte per
// wave that uses it (about 20 KB per stage), and the waves meet at one
// barrier per unit (two stages), which hands a ring slot back to the DMA.
// Each A row is expanded by the 2 waves that use it, each W row likewise.
// Within a stage the K order is permuted so that a lane's words are
// contiguous: MFMA k-step s, lane half h takes K elements 8 (2h + s) .. +7
// of the stage (the same for A and W, so the products pair up as before).
//
// Schedule per stage t: the raw words of stage t+2 are read, the words of
// stage t+1 (read one stage earlier) are expanded under the 32 MFMAs of
// stage t (about five VALU instructions per MFMA).  Workgroups are
// remapped so each XCD works a contiguous, grouped band of tiles (L2 reuse).
//
// This header holds the kernel's device code (in namespace qact::f16k, so
// that the INT8 integer kernel's translation unit can include it beside its
// own for the routed linear); qgemm.hip holds its launches.
#pragma once

#include <type_traits>

#include "qgemm_common.h"

namespace qact {

// Arguments of the fp16-MFMA kernel (at namespace qact, so that its
// kernels keep the names qact::qgemm_kernel<...>(qact::GemmArgs, ...)).
struct GemmArgs {
  const uint8_t* a;      // NVFP4 codes [M][K/2] or int8 [M][K]
  const uint32_t* a_st;  // NVFP4: per-tile scale words of A (or the E4M3 array, a_direct)
  const uint8_t* b;      // NVFP4 codes [N][K/2]
  const uint32_t* b_st;  // per-tile scale words of W (or the E4M3 array, b_direct)
  int64_t K;
  int units, nk;         // raw units of 64 and fp16 stages of 32 along K
  int mt, nt;            // tile counts
  const float* a_ts;     // NVFP4: activation tensor scale
  const float* w_ts;     // weight tensor scale
  const float* a_rs;     // INT8: per-row activation scale
  int a_direct;          // NVFP4: A's scale words read from the [M][K/16] array itself
  int b_direct;          // W's scale words read from the [N][K/16] array itself
  // K split of the last, partly filled round of tiles (see split_plan)
  int main_tiles;        // tiles computed whole, by workgroups 0 .. grid_main-1
  int grid_main;         // a multiple of 8
  int splits;            // K slices per tail tile (1: no split)
  int split_units;       // raw units per slice (the last slice may have fewer)
  float* part;           // slice partial sums, kPartTile floats per (tail tile, slice)
  Gate gate;             // the call's device-side gate
};

namespace f16k {

static constexpr int kThreads = 256;
static constexpr int kTileM = 256, kTileN = 256;
static constexpr int kStageK = 32;              // K per stage
static constexpr int kUnitK = 64;               // K per raw unit (two stages)
#ifndef QACT_RAW_SLOTS
#define QACT_RAW_SLOTS 4
#endif
// DMA runs kRawSlots - 1 units ahead; 5 slots measured no faster than 4
static constexpr int kRawSlots = QACT_RAW_SLOTS;
static_assert(kRawSlots >= 2, "the ring needs a slot being read and one being filled");
#ifndef QACT_GROUP_M
#define QACT_GROUP_M 8
#endif
#ifndef QACT_VALU_PER_MFMA
#define QACT_VALU_PER_MFMA 5
#endif
#ifndef QACT_DS_READS
#define QACT_DS_READS 0
#endif
static constexpr int kGroupM = QACT_GROUP_M;
static constexpr int kFM = 4, kFN = 4;          // MFMA tiles per wave (rows, columns)

// One raw unit in LDS: A codes, B codes, A scale words (NVFP4), B scale
// words.  Pads of 128 bytes keep the regions off each other's banks.
template <bool I8>
struct Raw {
  static constexpr int kA = 0;
  static constexpr int kB = kTileM * (I8 ? 64 : 32) + 128;
  static constexpr int kAS = kB + kTileN * 32;
  static constexpr int kBS = kAS + (I8 ? 0 : kTileM * 4 + 128);
  static constexpr int kSlot = kBS + kTileN * 4 + 128;
  static constexpr int kSmem = kRawSlots * kSlot;
  static constexpr int kLoads = I8 ? 7 : 6;     // DMA instructions per wave per unit
};
// the epilogue stages (32 kPassTiles) rows x 128 bf16 per wave through the idle ring
static_assert(Raw<false>::kSmem >= 4 * 8192 * kPassTiles, "epilogue staging");
static_assert(Raw<true>::kSmem <= 160 * 1024, "LDS");

static inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
static inline int64_t units_of(int64_t K) { return (K + kUnitK - 1) / kUnitK; }

// ---------------------------------------------------------------- GEMM --


// fp32 partial sums of one tile: 4 waves x 256 accumulators x 64 lanes
static constexpr int kPartTile = 4 * 256 * 64;
// K split of the last round of tiles (see split_plan): CUs of the device
// (one workgroup each) and slices per tile, at most
static constexpr int kCUs = 256;
static constexpr int kMaxSplits = 4;
static constexpr int kSplitMinSaved = 24;   // raw units a split must take off the last round

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
struct RawWords {
  typedef u32x2 A;       // NVFP4: the lane's 8 code bytes of a row's stage
};
template <>
struct RawWords<true> {
  typedef u32x4 A;       // INT8: the lane's 16 bytes of a row's stage
};

// Launch modes: kWhole -- whole tiles (all of them, or all but the tail
// tiles of a K-split call); kSlice -- one K slice of a tail tile per
// workgroup, storing its fp32 partial sums; kFixup -- four workgroups per
// tail tile, one per quadrant (the slices' partial sums of one wave of the
// slice workgroups), each of whose waves adds one row of MFMA tiles' sums
// (in slice order) and runs the epilogue on those 32 x 128 outputs.  Each is its own kernel so that the whole-tile kernel carries
// none of the slice bookkeeping (modes kWhole, kSlice, kFixup).

// The kernel body: workgroup `bid` of a launch in mode kMode, with the
// launch's LDS (Raw<I8>::kSmem bytes, 16-byte aligned) at smem.
template <bool I8, int kEpi, int kMode>
__device__ __forceinline__ void qgemm_body(const GemmArgs& g, const EpiArgs& e, uint8_t* smem,
                                           int bid) {
  using R = Raw<I8>;
  using AW = typename RawWords<I8>::A;
  if (gated_off(g.gate)) return;

  // XCD-aware tile order: hardware deals workgroups to the 8 XCDs in turn;
  // give each XCD a contiguous range of logical tiles, grouped kGroupM
  // tile-rows at a time so that concurrent tiles share A rows and B rows.
  // A kSlice workgroup computes slice `slice` of tail tile main_tiles +
  // bid / splits: raw units u_begin .. u_begin + u_count - 1.
  // a fixup launch has four workgroups per tail tile, one per quadrant
  // (the partial sums of the slices' wave fq), each wave adding one row
  // of 32 x 128 outputs
  const int fq = bid & 3;
  TileWork tw;
  if (!tile_work(kMode, kMode == kFixup ? (bid >> 2) : bid, g.main_tiles, g.splits,
                 g.split_units, g.units, tw))
    return;
  const int logical = tw.logical, slice = tw.slice, u_begin = tw.u_begin, u_count = tw.u_count;
  int tm, tn;
  tile_coords(logical, g.mt, g.nt, kGroupM, tm, tn);
  const int64_t m0 = (int64_t)tm * kTileM, n0 = (int64_t)tn * kTileN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);     // uniform per wave
  const int wm = kMode == kFixup ? (fq >> 1) : (wave >> 1);
  const int wn = kMode == kFixup ? (fq & 1) : (wave & 1);
  const int64_t K = g.K;

  // Buffer resources based at this tile's first row; rows past the operand
  // fall outside the range and load zero.
  // A K slice starts its buffers u_begin units in (a_lim, b_lim: the row
  // bytes left from there).
  const int64_t a_row = I8 ? K : K / 2, b_row = K / 2;
  const int64_t a_rows = min<int64_t>(e.M - m0, kTileM), b_rows = min<int64_t>(e.N - n0, kTileN);
  const uint32_t a_skip = (uint32_t)u_begin * (I8 ? 64u : 32u), b_skip = (uint32_t)u_begin * 32u;
  const uint32_t a_lim = (uint32_t)a_row - a_skip, b_lim = (uint32_t)b_row - b_skip;
  const __amdgpu_buffer_rsrc_t ra =
      buffer_rsrc(g.a + m0 * a_row + a_skip, (uint32_t)(a_rows * a_row) - a_skip);
  const __amdgpu_buffer_rsrc_t rb =
      buffer_rsrc(g.b + n0 * b_row + b_skip, (uint32_t)(b_rows * b_row) - b_skip);
  // Scale words: word u * 256 + r of the tile's re-laid-out copy holds the
  // 4 scales of row r and unit u; with a_direct / b_direct (K a multiple
  // of 64, rows are whole words) the word is bytes 4u .. 4u+3 of row r of
  // the operand's own array (rows past the operand's end fall outside the
  // buffer range and read as 0).
  const uint32_t gpr = (uint32_t)(K / 16);
  const bool ad = !I8 && g.a_direct != 0;
  const bool bd = g.b_direct != 0;
  const uint32_t s_skip = (uint32_t)u_begin * 1024u;
  const uint32_t st_bytes = (uint32_t)g.units * 1024u - s_skip;
  const uint8_t* const bs_base =
      bd ? reinterpret_cast<const uint8_t*>(g.b_st) + n0 * gpr + 4 * u_begin
         : reinterpret_cast<const uint8_t*>(g.b_st + (size_t)tn * g.units * 256) + s_skip;
  const __amdgpu_buffer_rsrc_t ras = buffer_rsrc(
      I8   ? static_cast<const void*>(g.b_st)
      : ad ? reinterpret_cast<const uint8_t*>(g.a_st) + m0 * gpr + 4 * u_begin
           : reinterpret_cast<const uint8_t*>(g.a_st + (size_t)tm * g.units * 256) + s_skip,
      I8 ? 0u : ad ? (uint32_t)(a_rows * gpr) - 4u * (uint32_t)u_begin : st_bytes);
  const __amdgpu_buffer_rsrc_t rbs =
      buffer_rsrc(bs_base, bd ? (uint32_t)(b_rows * gpr) - 4u * (uint32_t)u_begin : st_bytes);
  constexpr uint32_t kOOB = 0x7FFFFFF0u;

  // ---- DMA of raw unit u into slot u % kRawSlots.  The destination of one
  // instruction is 64 consecutive lanes' bytes: 32 NVFP4 rows (lane l: row
  // l/2, LDS half l%2 = global half (l%2) ^ ((row >> 3) & 1)), 16 INT8 rows
  // (lane l: row l/4, LDS chunk l%4 = global chunk (l%4) ^ (((row >> 2) & 1)
  // * 2)) or 64 scale words.  Wave w moves the row blocks w, w+4, ... of
  // each operand and scale words 64w .. 64w+63.  Chunks past the end of a
  // row load zero; NVFP4 bytes that a 16-byte load takes from the next row
  // meet a zero scale word.
  auto issue_unit = [&](int u) {
    uint8_t* s = smem + (u % kRawSlots) * R::kSlot;
    const bool real = u < u_count;                  // past the last unit: zeros into a free slot
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int blk = wave + 4 * i;
      const uint32_t row = (uint32_t)(32 * blk + (lane >> 1));
      const uint32_t half = (uint32_t)((lane & 1) ^ ((row >> 3) & 1));
      const uint32_t kb = (uint32_t)u * 32u + half * 16u;     // byte in an NVFP4 row
      if constexpr (!I8)
        dma16(ra, s + R::kA + blk * 1024, real && kb < b_lim ? row * (uint32_t)a_row + kb : kOOB);
      dma16(rb, s + R::kB + blk * 1024, real && kb < b_lim ? row * (uint32_t)b_row + kb : kOOB);
    }
    if constexpr (I8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int blk = wave + 4 * i;
        const uint32_t row = (uint32_t)(16 * blk + (lane >> 2));
        const uint32_t c = (uint32_t)((lane & 3) ^ (((row >> 2) & 1) * 2));
        const uint32_t kb = (uint32_t)u * 64u + c * 16u;
        dma16(ra, s + R::kA + blk * 1024, real && kb < a_lim ? row * (uint32_t)a_row + kb : kOOB);
      }
    }
    const uint32_t srow = (uint32_t)(64 * wave + lane);
    const uint32_t so_a = ad ? srow * gpr + 4u * (uint32_t)u : (uint32_t)u * 1024u + srow * 4u;
    const uint32_t so_b = bd ? srow * gpr + 4u * (uint32_t)u : (uint32_t)u * 1024u + srow * 4u;
    if constexpr (!I8) dma4(ras, s + R::kAS + 256 * wave, real ? so_a : kOOB);
    dma4(rbs, s + R::kBS + 256 * wave, real ? so_b : kOOB);
  };
  // ---- raw words of a stage.  Lane (h, r) = (lane / 32, lane % 32) of
  // tile i takes row 32 i + r of the wave's rows: for NVFP4 the 8 code
  // bytes 8h .. 8h+7 of the row's stage (words 2h, 2h+1: one scale group,
  // k-steps 0 and 1) and the row's scale word; for INT8 the 16 bytes
  // 16h .. 16h+15 of the row's stage.  The same for the W rows of tile j.
  const int lr = lane & 31, lh = lane >> 5;
  const int nv_off = 16 * ((lr >> 3) & 1) + 8 * lh;   // half swizzle of rows lr (mod 32)
  const int i8_sw = ((lr >> 2) & 1) * 2;               // chunk swizzle of INT8 rows lr (mod 32)
  const int a_base = (wm * 128 + lr), b_base = (wn * 128 + lr);
  struct RawS {
    AW a[kFM];
    uint32_t as[kFM];
    u32x2 b[kFN];
    uint32_t bs[kFN];
  };
  // each stage's reads address from one lane base per region (A codes, A
  // scale words, W codes, W scale words): the tiles' offsets are constants
  // that the LDS reads take as immediates
  const uint32_t la = (uint32_t)a_base * (I8 ? 64u : 32u), lb = (uint32_t)b_base * 32u;
  const uint32_t las = (uint32_t)a_base * 4u, lbs = (uint32_t)b_base * 4u;
  auto read_raw = [&](int t, RawS& r) {
    const uint8_t* s = smem + ((t >> 1) % kRawSlots) * R::kSlot;
    const int sh = t & 1;
    const uint8_t* const pa =
        s + la + (I8 ? 16u * (uint32_t)((2 * sh + lh) ^ i8_sw) : (uint32_t)((16 * sh) ^ nv_off));
    const uint8_t* const pb = s + lb + (uint32_t)((16 * sh) ^ nv_off);
    const uint8_t* const pas = s + las;
    const uint8_t* const pbs = s + lbs;
#pragma unroll
    for (int i = 0; i < kFM; ++i) {
      if constexpr (I8) {
        r.a[i] = *reinterpret_cast<const AW*>(pa + R::kA + 32 * 64 * i);
        r.as[i] = 0u;
      } else {
        r.a[i] = *reinterpret_cast<const AW*>(pa + R::kA + 32 * 32 * i);
        r.as[i] = *reinterpret_cast<const uint32_t*>(pas + R::kAS + 32 * 4 * i);
      }
    }
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      r.b[j] = *reinterpret_cast<const u32x2*>(pb + R::kB + 32 * 32 * j);
      r.bs[j] = *reinterpret_cast<const uint32_t*>(pbs + R::kBS + 32 * 4 * j);
    }
  };
  // fp16 fragments of a stage: (a0, b0) for k-step 0, (a1, b1) for k-step 1
  struct Ops {
    u32x4 a0[kFM], a1[kFM], b0[kFN], b1[kFN];
  };
  auto expand = [&](int t, const RawS& r, Ops& o) {
    const int grp = 2 * (t & 1) + lh;                  // scale group of the lane's K elements
#pragma unroll
    for (int i = 0; i < kFM; ++i) {
      if constexpr (I8) {
        const u32x2 q0 = int8_quad(r.a[i][0]), q1 = int8_quad(r.a[i][1]);
        const u32x2 q2 = int8_quad(r.a[i][2]), q3 = int8_quad(r.a[i][3]);
        o.a0[i] = u32x4{q0[0], q0[1], q1[0], q1[1]};
        o.a1[i] = u32x4{q2[0], q2[1], q3[0], q3[1]};
      } else {
        const f16x2 sc = scale_pair(r.as[i], grp);
        o.a0[i] = nvfp4_chunk(r.a[i][0], sc);
        o.a1[i] = nvfp4_chunk(r.a[i][1], sc);
      }
    }
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      const f16x2 sc = scale_pair(r.bs[j], grp);
      o.b0[j] = nvfp4_chunk(r.b[j][0], sc);
      o.b1[j] = nvfp4_chunk(r.b[j][1], sc);
    }
  };

  f32x16 acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // The MFMA is issued as W x A^T: accumulator r of tile (i, j) then holds
  // output row 32i + lane % 32 of the wave's rows and output column
  // 32j + (r/4)*8 + (lane/32)*4 + r%4 of its columns, so that each lane
  // owns runs of 4 consecutive outputs of one row.
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
  // the value cannot be hoisted above it
  auto pin = [](auto& v) { asm volatile("" : "+v"(v)); };
  auto pin_raw = [&](RawS& r) {
#pragma unroll
    for (int i = 0; i < kFM; ++i) {
      pin(r.a[i]);
      if constexpr (!I8) pin(r.as[i]);
    }
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      pin(r.b[j]);
      pin(r.bs[j]);
    }
  };
  auto pin_ops = [&](Ops& o) {
#pragma unroll
    for (int i = 0; i < kFM; ++i) {
      pin(o.a0[i]);
      pin(o.a1[i]);
    }
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      pin(o.b0[j]);
      pin(o.b1[j]);
    }
  };

  // epilogue scales, read now so that their latency hides under the loop:
  // the tensor scales and (INT8, plain epilogue) the row scales of the
  // lane's rows (rows past M read row M-1; they are never stored)
  const float alpha = I8 ? *g.w_ts : (*g.a_ts) * (*g.w_ts);
  float row_scale[kFM];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
    row_scale[i] = I8 && epi_staged(kEpi) ? g.a_rs[min<int64_t>(m0 + wm * 128 + 32 * i + (lane & 31), e.M - 1)]
                                : 1.0f;

  // ---- pipeline.  Units are issued in order, one per two stages, with
  // units past the last one issued as zero loads, so that a wave always has
  // the same number of DMA instructions in flight and every stage past K
  // (the second stage of a last unit that K ends inside, the reads ahead
  // of the last stage) sees zero words, which expand to zero fragments.
  // Unit v (stages 2v, 2v+1): before the pair, wait for this wave's DMA of
  // unit v+1 (the kRawSlots - 2 units after it may still be in flight), then a
  // workgroup barrier, after which that unit is visible to all and the slot
  // of unit v -- whose last words (stage 2v+1) every wave read and waited
  // for in stage 2v-1 -- takes unit v+kRawSlots.  Stage t reads the raw words of
  // stage t+2 and runs its 32 MFMAs with the expansion of stage t+1's words
  // under them.  The loop body has no branch, so that the accumulators
  // stay in the accumulation registers across it.
  const int nk = 2 * u_count;
  // the raw-word reads of stage t+2 (NVFP4: 16, INT8: 12) go one per MFMA
  // from the start of the stage: the scheduling template offers a read
  // slot after every MFMA (measured 12 % faster for NVFP4 and 4 % for INT8
  // than offering 8 slots)
  constexpr int kDsReads = QACT_DS_READS > 0 ? QACT_DS_READS : 2 * kFM * kFN;
  if constexpr (kMode != kFixup) {
#pragma unroll
  for (int u = 0; u < kRawSlots; ++u) issue_unit(u);
  wait_vm<(kRawSlots - 1) * R::kLoads>();
  barrier();
  Ops opA, opB;
  RawS rwA, rwB;
  read_raw(0, rwA);
  read_raw(1, rwB);
  expand(0, rwA, opA);
  auto compute = [&](int t, Ops& cur, Ops& nxt, RawS& rn, RawS& rf) {
    // rn: words of stage t+1 (read in stage t-1); rf receives stage t+2's
    pin_raw(rn);
    read_raw(t + 2, rf);
    mfmas(cur.a0, cur.b0);
    mfmas(cur.a1, cur.b1);
    expand(t + 1, rn, nxt);
#pragma unroll
    for (int i = 0; i < 2 * kFM * kFN; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                     // MFMA
      if (i < kDsReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // DS read
      __builtin_amdgcn_sched_group_barrier(0x002, QACT_VALU_PER_MFMA, 0);   // VALU
    }
    pin_ops(nxt);
  };
  auto sync_unit = [&](int t) {
    wait_vm<(kRawSlots - 2) * R::kLoads>();
    wait_lds();
    barrier();
    issue_unit((t >> 1) + kRawSlots);
  };
  for (int t = 0; t < nk; t += 2) {
    sync_unit(t);
    compute(t, opA, opB, rwB, rwA);
    compute(t + 1, opB, opA, rwA, rwB);
  }

  wait_vm<0>();          // no DMA into LDS outlives the workgroup
  __syncthreads();       // every wave is past its last read of the ring

  // ---- K slice of a tail tile: store the partial sums for the fixup
  // launch and stop.  Partial chunk (i, j, r4) -- accumulators 4 r4 .. 4 r4
  // + 3 of MFMA tile (i, j) -- of lane l of wave w sits at f32x4 index
  // (w * 64 + chunk) * 64 + l of the slice's kPartTile floats.
  if constexpr (kMode == kSlice) {
    f32x4* const mine = reinterpret_cast<f32x4*>(g.part) +
                        ((size_t)(logical - g.main_tiles) * g.splits + slice) * (kPartTile / 4) +
                        wave * 4096 + lane;
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          mine[((i * kFN + j) * 4 + r4) * 64] =
              f32x4{acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]};
    return;
  }
  } else {
    // the tile's sum over its K slices, added in slice order
    const f32x4* const base = reinterpret_cast<const f32x4*>(g.part) +
                              (size_t)(logical - g.main_tiles) * g.splits * (kPartTile / 4) +
                              fq * 4096 + lane;
    const int ns = g.splits;
    constexpr int kPair = 2;              // MFMA tiles whose chunks load together
    {
      const int i = wave;                 // this wave's row of MFMA tiles
#pragma unroll
      for (int j0 = 0; j0 < kFN; j0 += kPair) {
        // the 4 chunks of MFMA tiles (i, j0 .. j0 + kPair - 1) from every
        // slice, loads issued together
        f32x4 v[kPair][4][kMaxSplits];
#pragma unroll
        for (int jj = 0; jj < kPair; ++jj)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
            for (int sl = 0; sl < kMaxSplits; ++sl)
              v[jj][r4][sl] =
                  sl < ns ? base[(size_t)sl * (kPartTile / 4) + ((i * kFN + j0 + jj) * 4 + r4) * 64]
                          : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int jj = 0; jj < kPair; ++jj) {
          f32x16 tot;
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            f32x4 sum = v[jj][r4][0];
#pragma unroll
            for (int sl = 1; sl < kMaxSplits; ++sl)
              if (sl < ns) sum += v[jj][r4][sl];
#pragma unroll
            for (int t = 0; t < 4; ++t) tot[4 * r4 + t] = sum[t];
          }
          // into the accumulation registers through an MFMA with zero
          // operands (it adds +0, which changes no sum: none is -0), so
          // that the 256 sums do not crowd the ordinary registers
          const f16x8 z = {};
          acc[0][j0 + jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(z, z, tot, 0, 0, 0);
        }
        // bound the loads in flight to kPair MFMA tiles' chunks
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if constexpr (kMode != kSlice) {

  // ---- epilogue (store_tile): the tensor scales, and for INT8 the row
  // scales of the lane's rows (rows past M read row M-1; never stored)
  const int c = lane & 31;
  if constexpr (kMode == kFixup) {
    const int64_t wave_row0 = m0 + wm * 128 + 32 * wave;
    const int64_t wave_col0 = n0 + wn * 128;
    float rs[1];
    rs[0] = I8 ? g.a_rs[min<int64_t>(wave_row0 + c, e.M - 1)] * alpha : alpha;
    store_tile<kEpi, 1>(acc, rs, wave_row0, wave_col0, smem + wave * 8192 * kPassTiles, e, lane);
  } else {
  const int64_t wave_row0 = m0 + wm * 128;
  const int64_t wave_col0 = n0 + wn * 128;
  float rs[kFM];
#pragma unroll
  for (int i = 0; i < kFM; ++i) {
    if constexpr (I8 && !epi_staged(kEpi))   // (the other kernels read them here)
      row_scale[i] = g.a_rs[min<int64_t>(wave_row0 + 32 * i + c, e.M - 1)];
    rs[i] = I8 ? row_scale[i] * alpha : alpha;
  }
  store_tile<kEpi, kFM>(acc, rs, wave_row0, wave_col0, smem + wave * 8192 * kPassTiles, e, lane);
  }
  }
}

}  // namespace f16k

// The NVFP4 linear set up for a caller that may launch its whole tiles
// itself (the routed linear): the scale re-layout, when the scales are not
// read in place, enqueued under `gate`; the kernel arguments (with gate
// `gate`) in g and e (qgemm.hip).
hipError_t nvfp4_gemm_prepare(const uint8_t* a_q, const uint8_t* a_s, const float* a_ts,
                              const uint8_t* w_q, const uint8_t* w_s, const float* w_ts,
                              int64_t M, int64_t N, int64_t K, const GemmOut& o, void* ws,
                              size_t ws_bytes, Gate gate, hipStream_t st, GemmArgs& g,
                              EpiArgs& e);
// the launches of a linear so prepared, under g.gate: the whole tiles and,
// when its last round is split, the K slices and fixup (tails_only: just
// the latter)
hipError_t nvfp4_gemm_launch(const GemmArgs& g, const EpiArgs& e, hipStream_t st,
                             bool tails_only);

}  // namespace qact
