// INT8-activation linear on gfx950 integer MFMA with exact int32 sums.
//
// 6Bit-Diffusion, abstract: volatile layers keep INT8 activations; Table 2
// ("W4A6"): the weights stay 4-bit NVFP4.  The layer is
//   Y[m][n] = s_a[m] s_Tw sum_k q[m][k] E4M3(sw[n][k/16]) E2M1(w[n][k]).
//
// Integer form of an NVFP4 weight row.  An E4M3 scale is c 2^x with an
// integer significand c (normal codes: 8 + mantissa, x = exponent - 10;
// subnormal codes: mantissa, x = -9) and an E2M1 value is v / 2 with
// v in {0, 1, 2, 3, 4, 6, 8, 12} (with sign).  With X[n] the smallest x over
// the row's non-zero scales,
//   W[n][k] = s_Tw 2^(X[n] - 1) I[n][k],   I = v c 2^(x - X[n]),
// an integer with |I| <= 180 2^spread (spread = largest minus smallest x of
// the row).  For spread <= 7, |I| <= 23040 splits into two int8 digits,
// I = 256 hi + lo with lo in [-128, 127] and |hi| <= 90, so that
//   Y[m][n] = s_a[m] s_Tw 2^(X[n] - 1) (256 H[m][n] + L[m][n]),
//   H = sum_k q hi,  L = sum_k q lo,
// two exact int32 sums (|H|, |L| <= K 127 128 < 2^31 for K < 2^17) from
// v_mfma_i32_32x32x32_i8.  The digit planes are made once per weight at
// set-up (int8_planes_kernel) in the layout the GEMM loads: no conversion
// of either operand in the GEMM's loop.  Rows with a wider spread are
// reported at set-up; their linears take the exact-operand fp16 kernel.
//
// Workgroup: 4 waves (one per SIMD), 256 activation rows x 128 weight rows,
// i.e. a 256 x 256 integer tile against the two planes.  Wave w owns
// activation rows 64 w .. +64 and all 256 plane rows (2 x 8 MFMA tiles of
// 32 x 32; tiles j < 4 take the lo plane, j >= 4 the hi plane of the same
// 128 columns).  K runs in units of 64 (two MFMA k-steps of 32): per unit
// the tile's 16 KB of activations and 16 KB of plane rows are DMA'd
// (buffer_load ... lds) into a 4-slot LDS ring, three units ahead; each wave
// reads its fragments straight from the ring, one unit ahead.  Both kinds of
// memory instruction are spread over the unit's 32 MFMAs.  Two kernels:
// qgemm_i8_kernel takes one tile per workgroup (and the K slices of a split
// last round, and their fixup); qgemm_i8_persist, for short K loops over
// more than one round of tiles, walks several tiles per workgroup through
// one continuous stream of units.
#include <hip/hip_ext.h>

#include "qgemm_common.h"
#include "qgemm_f16.h"

namespace qact {

namespace {

constexpr int kThreads = 256;
constexpr int kTileM = 256;                     // activation rows per tile
constexpr int kTileN = 128;                     // weight rows (output columns) per tile
constexpr int kUnitK = 64;                      // K per unit (two k-steps of 32)
constexpr int kSlots = 4;                       // LDS ring slots (units)
constexpr int kUnitBytes = 256 * kUnitK;        // one operand's unit in LDS
constexpr int kWOff = kUnitBytes + 128;         // plane rows after the activations
constexpr int kSlot = 2 * kWOff;
constexpr int kColF = kSlots * kSlot;           // the tile's 128 column factors (float)
constexpr int kRowS = kColF + kTileN * 4;       // and its 256 row scales s_a s_Tw (float)
constexpr int kSmem = kRowS + kTileM * 4;
constexpr int kLoads = 8;                       // DMA instructions per wave per unit
constexpr int kFM = 2, kFN = 8;                 // MFMA tiles per wave (rows, plane rows)
constexpr int kSpreadMax = 7;                   // largest exponent spread of a row
static_assert(kSmem <= 160 * 1024, "LDS");
static_assert(kSmem >= 4 * 8192 * kPassTiles, "epilogue staging");

// K split of the last round of tiles (as in the fp16 kernel): one
// workgroup per CU, at most 4 slices, each at least 2 units, taken when it
// takes at least kSplitMinSaved units off the last round (the fixup
// launch reads 256 KB per slice and tile: it costs about as much as the
// fp16 kernel's 15-20 units, i.e. 30-40 of these half-length units).
constexpr int kCUs = 256;
constexpr int kMaxSplits = 4;
constexpr int kSplitMinSaved = 40;
constexpr int kPartTile = 4 * 256 * 64;         // int32 partial sums of one tile

inline int64_t units_of(int64_t K) { return (K + kUnitK - 1) / kUnitK; }
inline int64_t ntiles_of(int64_t N) { return (N + kTileN - 1) / kTileN; }
inline size_t r256(size_t v) { return (v + 255) / 256 * 256; }

// LDS / packed-plane position of 16-byte chunk c (K bytes 16c .. 16c+15
// of a unit) of row r: chunks are XOR-swizzled by bit 2 of the row so that
// the 32 rows of a fragment read spread over the banks.
__host__ __device__ constexpr int chunk_slot(int r, int c) { return c ^ (((r >> 2) & 1) * 2); }

// E4M3 code -> (c, x) with value c 2^x.
__device__ __forceinline__ void e4m3_sig_exp(uint32_t s, int& c, int& x) {
  const int e = (int)((s >> 3) & 15u), m = (int)(s & 7u);
  c = e ? 8 + m : m;
  x = e ? e - 10 : -9;
}

}  // namespace

// --------------------------------------------------------- weight planes --

// Packed planes of an NVFP4 weight [N][K]: for weight-row tile t (128
// rows) and unit u, 16 KB at ((t * units + u) * 16384): plane row
// pr = plane * 128 + r (plane 0 = lo, 1 = hi) holds its 64 digits at
// pr * 64, chunk c at slot chunk_slot(pr, c).  Rows past N and K past the
// weight are zero.  Then float rowf[tiles * 128] = 2^(X[n] - 1) (0 for
// all-zero, irregular and padding rows) and the int32 count of irregular
// rows.  One wave per row; lane l takes element 64 u + l of each unit.
__global__ void __launch_bounds__(256)
int8_planes_kernel(const uint8_t* __restrict__ w_q, const uint8_t* __restrict__ w_s, int64_t N,
                   int64_t K, int units, int8_t* __restrict__ planes, float* __restrict__ rowf,
                   int* __restrict__ irregular) {
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // < tiles * 128
  const int lane = threadIdx.x & 63;
  const int64_t gpr = K / 16;
  int xmin = 64, xmax = -64;
  if (n < N)
    for (int64_t gi = lane; gi < gpr; gi += 64) {
      int c, x;
      e4m3_sig_exp(w_s[n * gpr + gi], c, x);
      if (c) {
        xmin = min(xmin, x);
        xmax = max(xmax, x);
      }
    }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    xmin = min(xmin, __shfl_xor(xmin, o, 64));
    xmax = max(xmax, __shfl_xor(xmax, o, 64));
  }
  const bool live = xmin <= xmax;                 // a non-zero scale exists
  const bool regular = !live || xmax - xmin <= kSpreadMax;
  if (lane == 0) {
    rowf[n] = live && regular ? ldexpf(1.0f, xmin - 1) : 0.0f;
    if (!regular) atomicAdd(irregular, 1);
  }
  const int r = (int)(n % kTileN);
  int8_t* const tile = planes + (n / kTileN) * (int64_t)units * kUnitBytes;
  for (int u = 0; u < units; ++u) {
    const int64_t k = (int64_t)u * kUnitK + lane;
    int I = 0;
    if (live && regular && k < K) {
      const uint32_t code = (w_q[n * (K / 2) + k / 2] >> (4 * (k & 1))) & 15u;
      int c, x;
      e4m3_sig_exp(w_s[n * gpr + k / 16], c, x);
      I = c ? e2m1_twice(code) * c * (1 << (x - xmin)) : 0;
    }
    const int lo = ((I + 128) & 255) - 128;
    const int hi = (I - lo) / 256;
    int8_t* const unit = tile + (int64_t)u * kUnitBytes;
    const int c = lane >> 4, b = lane & 15;
    unit[r * 64 + 16 * chunk_slot(r, c) + b] = (int8_t)lo;
    unit[(kTileN + r) * 64 + 16 * chunk_slot(kTileN + r, c) + b] = (int8_t)hi;
  }
}

size_t int8_planes_bytes(int64_t N, int64_t K) {
  const int64_t t = ntiles_of(N);
  return r256((size_t)(t * units_of(K)) * kUnitBytes) + r256((size_t)t * kTileN * 4) + 256;
}

hipError_t launch_int8_planes(const uint8_t* w_q, const uint8_t* w_s, int64_t N, int64_t K,
                              void* w8, int* irregular_dev, hipStream_t st) {
  const int64_t t = ntiles_of(N);
  int8_t* planes = static_cast<int8_t*>(w8);
  float* rowf = reinterpret_cast<float*>(static_cast<uint8_t*>(w8) +
                                         r256((size_t)(t * units_of(K)) * kUnitBytes));
  hipLaunchKernelGGL(int8_planes_kernel, dim3((unsigned)(t * kTileN / 4)), dim3(256), 0, st, w_q,
                     w_s, N, K, (int)units_of(K), planes, rowf, irregular_dev);
  return hipGetLastError();
}

int* int8_planes_counter(void* w8, int64_t N, int64_t K) {
  const int64_t t = ntiles_of(N);
  return reinterpret_cast<int*>(static_cast<uint8_t*>(w8) +
                                r256((size_t)(t * units_of(K)) * kUnitBytes) +
                                r256((size_t)t * kTileN * 4));
}

// ------------------------------------------------------------------ GEMM --

struct I8Args {
  const uint8_t* a;          // int8 activations [M][K]
  const int8_t* planes;      // packed weight planes
  const float* rowf;         // 2^(X[n] - 1) per weight row
  const float* a_rs;         // activation row scales s_a
  const float* w_ts;         // weight tensor scale s_Tw
  int64_t K;
  int units;
  int mt, nt;                // tile counts
  int main_tiles, grid_main; // whole tiles and their grid (a multiple of 8)
  int splits, split_units;   // K split of the tail tiles
  int32_t* part;             // slice partial sums, kPartTile per (tail tile, slice)
  int32_t* acc_hi;           // kEpiAcc: the sums H and L, int32 [M][N]
  int32_t* acc_lo;
  Gate gate;
};

// the test-only epilogue: store H and L themselves
constexpr int kEpiAcc = 100;

// ---- pieces of the pipeline shared by the two GEMM kernels
namespace {

constexpr uint32_t kOOB = 0x7FFFFFF0u;          // an offset past every buffer range

// MFMA operands of one unit for a wave: for k-step s, lane (lh, lr) holds
// the 16 bytes of K 32 s + 16 lh .. +15 of row 32 i + lr of the wave's
// activation rows (tile i) and of plane row 32 j + lr (tile j).
struct Frag {
  i32x4 a[2][kFM];
  i32x4 w[2][kFN];
};
constexpr int kReads = 2 * (kFM + kFN);          // fragment reads per unit

// DMA instruction idx (0..7) of unit u into the ring slot at s.  One
// instruction fills 1 KB of LDS: 16 activation rows (lane l: row l/4, LDS
// chunk l%4 = chunk chunk_slot(row, l%4)), or 1 KB of the packed planes as
// they lie.  Wave w moves the 1 KB blocks w, w+4, w+8, w+12 of the
// activations (idx 0..3), then of the planes (4..7).  ra: the tile's
// activation rows from the unit base (a_lim bytes of K left in a row);
// rw: its planes from the same unit.  real = false: zero loads.
__device__ __forceinline__ void dma_one(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rw,
                                        uint8_t* s, uint32_t u, int idx, int wave, int ln,
                                        uint32_t K, uint32_t a_lim, bool real) {
  const int blk = wave + 4 * (idx & 3);
  if (idx < 4) {
    const uint32_t row = (uint32_t)(16 * blk + (ln >> 2));
    const uint32_t kb = u * kUnitK + 16u * (uint32_t)chunk_slot((int)row, ln & 3);
    dma16(ra, s + blk * 1024, real && kb < a_lim ? row * K + kb : kOOB);
  } else {
    dma16(rw, s + kWOff + blk * 1024,
          real ? u * kUnitBytes + (uint32_t)(blk * 1024 + ln * 16) : kOOB);
  }
}

// Fragment read idx (0..19: k-step idx / 10; activation tiles 0, 1, then
// plane tiles 0..7) of the unit in the ring slot at s.  Bit 2 of the rows
// read is bit 2 of lr, so one swizzle serves all.
__device__ __forceinline__ void read_one(const uint8_t* s, int idx, Frag& f, int wave, int ln) {
  const int ks = idx / (kFM + kFN), r = idx % (kFM + kFN);
  const int lr = ln & 31;
  const int off = 16 * chunk_slot(lr, 2 * ks + (ln >> 5));
  if (r < kFM)
    f.a[ks][r] = *reinterpret_cast<const i32x4*>(s + (64 * wave + 32 * r + lr) * 64 + off);
  else
    f.w[ks][r - kFM] =
        *reinterpret_cast<const i32x4*>(s + kWOff + (32 * (r - kFM) + lr) * 64 + off);
}

// fragments are in their registers at this point of the program
__device__ __forceinline__ void pin_frag(Frag& f) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int i = 0; i < kFM; ++i) asm volatile("" : "+v"(f.a[ks][i]));
#pragma unroll
    for (int j = 0; j < kFN; ++j) asm volatile("" : "+v"(f.w[ks][j]));
  }
}

// a workgroup barrier that the compiler moves no instruction across
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// the lane index as an opaque value: offsets formed from it are formed
// where it is taken rather than hoisted and kept live
__device__ __forceinline__ int opaque_lane(int lane) {
  asm volatile("" : "+v"(lane));
  return lane;
}

// The 32 MFMAs of a unit on cur, issued as W x A^T (accumulator r of tile
// (i, j): output row 32 i + lr of the wave's rows, plane row 32 j + 8 (r/4)
// + 4 lh + r%4), in 8 segments of 4.  With kMem, segment g also issues DMA
// instruction g (dma(g)) and the fragment reads kFirstRead[g] ..
// kFirstRead[g+1]-1 (read(idx)), so that the memory instructions trickle
// out under the MFMAs (a burst of 8 LDS-DMA instructions after the barrier
// holds the wave's issue long enough to idle its MFMA unit: measured 7-9 %
// slower at the CogVideoX linear shapes).  kFirst: the first k-step starts
// the sums from zero.
template <bool kFirst, bool kMem, class Dma, class Read>
__device__ __forceinline__ void unit_mfmas(i32x16 (&acc)[kFM][kFN], Frag& cur, const Dma& dma,
                                           const Read& read) {
  constexpr int kSegs = 8;
  static_assert(kLoads == kSegs && 2 * kFM * kFN == 4 * kSegs, "segment layout");
  constexpr int kFirstRead[kSegs + 1] = {0, 3, 6, 9, 12, 14, 16, 18, kReads};
  const i32x16 zero = {};
  pin_frag(cur);
#pragma unroll
  for (int seg = 0; seg < kSegs; ++seg) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int x = seg * 4 + m, ks = x / (kFM * kFN), i = (x / kFN) % kFM, j = x % kFN;
      acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur.w[ks][j], cur.a[ks][i],
                                                        kFirst && ks == 0 ? zero : acc[i][j],
                                                        0, 0, 0);
    }
    if constexpr (kMem) {
      dma(seg);
#pragma unroll
      for (int r = 0; r < 3; ++r)
        if (kFirstRead[seg] + r < kFirstRead[seg + 1]) read(kFirstRead[seg] + r);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Epilogue of a wave's 64 rows x 128 columns: 256 H + L in float32 (one
// rounding: fmaf of two exact conversions while |H|, |L| < 2^24), times
// 2^(X[n] - 1) of the column (colf, LDS), times the row scale rows[r] *
// rs_mul (LDS), then store_tile with its staging at stg.  ln: the lane;
// lr, lh: ln % 32 and ln / 32.
template <int kEpi>
__device__ __forceinline__ void i8_epilogue(const i32x16 (&acc)[kFM][kFN], const float* colf,
                                            const float* rows, float rs_mul, int64_t wave_row0,
                                            int64_t n0, uint8_t* stg, const EpiArgs& e, int wave,
                                            int ln, int lr, int lh) {
  float rs[kFM];
#pragma unroll
  for (int i = 0; i < kFM; ++i) rs[i] = rows[64 * wave + 32 * i + lr] * rs_mul;
  f32x4 cf[kFN / 2][4];
#pragma unroll
  for (int j = 0; j < kFN / 2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      cf[j][q] = *reinterpret_cast<const f32x4*>(colf + 32 * j + 8 * q + 4 * lh);
  // formed where the epilogue consumes it, so that only the values of the
  // pass being stored are live in ordinary registers
  auto val = [&](int i, int j, int r) {
    return __builtin_fmaf((float)acc[i][j + kFN / 2][r], 256.0f, (float)acc[i][j][r]) *
           cf[j][r >> 2][r & 3];
  };
  store_tile<kEpi, kFM>(val, rs, wave_row0, n0, stg, e, ln);
}

}  // namespace


// The per-tile kernel's body: workgroup `bid` of a launch in mode kMode,
// with the launch's LDS (kSmem bytes, 16-byte aligned) at smem.
template <int kEpi, int kMode>
__device__ __forceinline__ void i8_tile_body(const I8Args& g, const EpiArgs& e, uint8_t* smem,
                                             int bid) {
  if (gated_off(g.gate)) return;

  // tile of this workgroup: XCD-aware order as in the fp16 kernel (each
  // XCD a contiguous range of logical tiles, grouped 8 tile-rows at a time)
  // a fixup launch has two workgroups per tail tile (half fh of its rows)
  const int fh = bid & 1;
  TileWork tw;
  if (!tile_work(kMode, kMode == kFixup ? (bid >> 1) : bid, g.main_tiles, g.splits,
                 g.split_units, g.units, tw))
    return;
  const int logical = tw.logical, slice = tw.slice, u_begin = tw.u_begin, u_count = tw.u_count;
  int tm, tn;
  tile_coords(logical, g.mt, g.nt, 8, tm, tn);
  const int64_t m0 = (int64_t)tm * kTileM, n0 = (int64_t)tn * kTileN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t K = g.K;
  const int lr = lane & 31, lh = lane >> 5;

  i32x16 acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  // epilogue factors, read now so that their latency hides under the loop
  // and kept in LDS (written once the loop has started; a loop barrier
  // makes them visible): the tile's 128 column factors 2^(X[n] - 1) (the
  // array is padded to whole tiles) and its 256 row scales s_a s_Tw (rows
  // past M read row M-1; they are never stored)
  constexpr bool kFactors = kEpi != kEpiAcc && kMode != kSlice;
  const int64_t wave_row0 = m0 + 64 * wave;
  float cfv = 0.0f, rsv = 0.0f;
  float* const colf = reinterpret_cast<float*>(smem + kColF);
  float* const rows = reinterpret_cast<float*>(smem + kRowS);
  auto put_factors = [&] {
    if (tid < kTileN) colf[tid] = cfv;
    rows[tid] = rsv;
  };
  if constexpr (kFactors) {
    rsv = g.a_rs[min<int64_t>(m0 + tid, e.M - 1)] * *g.w_ts;
    if (tid < kTileN) cfv = g.rowf[n0 + tid];
    if constexpr (kMode == kFixup) {
      put_factors();
      __syncthreads();
    }
  }

  if constexpr (kMode != kFixup) {
    // Activations: rows m0 .. (at most 256), K bytes from the slice start;
    // rows past M fall outside the buffer and load zero, as do chunks past
    // K (passed the out-of-range offset).  Planes: the tile's units from the
    // slice start, always in range (padded at set-up).
    const int64_t a_rows = min<int64_t>(e.M - m0, kTileM);
    const uint32_t a_skip = (uint32_t)u_begin * kUnitK;
    const uint32_t a_lim = (uint32_t)K - a_skip;
    const __amdgpu_buffer_rsrc_t ra =
        buffer_rsrc(g.a + m0 * K + a_skip, (uint32_t)(a_rows * K) - a_skip);
    const __amdgpu_buffer_rsrc_t rw =
        buffer_rsrc(g.planes + ((int64_t)tn * g.units + u_begin) * kUnitBytes,
                    (uint32_t)u_count * (uint32_t)kUnitBytes);
    // DMA of unit u into slot u % kSlots; units past the last are issued
    // as zero loads into their free slot
    auto issue_one = [&](int u, int idx) {
      dma_one(ra, rw, smem + (u % kSlots) * kSlot, (uint32_t)u, idx, wave, lane, (uint32_t)K,
              a_lim, u < u_count);
    };
    auto issue_unit = [&](int u) {
#pragma unroll
      for (int idx = 0; idx < kLoads; ++idx) issue_one(u, idx);
    };
    auto read_unit = [&](int u, Frag& f) {
#pragma unroll
      for (int idx = 0; idx < kReads; ++idx) read_one(smem + (u % kSlots) * kSlot, idx, f, wave, lane);
    };
    // unit u on cur, with the DMA of unit u_dma and the reads of unit u_next
    auto compute = [&](Frag& cur, int u_next, Frag& nxt, int u_dma) {
      unit_mfmas<false, true>(
          acc, cur, [&](int idx) { issue_one(u_dma, idx); },
          [&](int idx) { read_one(smem + (u_next % kSlots) * kSlot, idx, nxt, wave, lane); });
      pin_frag(nxt);
    };
    // Unit u: wait for this wave's DMA of unit u+1 (units u+2, u+3 may still
    // be in flight) and for its reads of unit u (done one unit earlier);
    // after the barrier unit u+1 is visible to every wave and no wave reads
    // the slot of unit u any more, so that compute(u) may DMA unit u +
    // kSlots into it.
    auto sync_unit = [&] {
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<(kSlots - 2) * kLoads>();
      wait_lds();
      ring_barrier();
    };
#pragma unroll
    for (int u = 0; u < kSlots; ++u) issue_unit(u);
    wait_vm<(kSlots - 1) * kLoads>();
    ring_barrier();
    Frag f0, f1;
    read_unit(0, f0);
    if constexpr (kFactors) put_factors();
    for (int u = 0; u < u_count; u += 2) {
      sync_unit();
      compute(f0, u + 1, f1, u + kSlots);
      sync_unit();
      compute(f1, u + 2, f0, u + 1 + kSlots);
    }
    wait_vm<0>();       // no DMA into LDS outlives the workgroup
    wait_lds();
    __syncthreads();    // every wave is past its last read of the ring

    if constexpr (kMode == kSlice) {
      // partial sums of this slice: chunk (i, j, r4) of lane l of wave w at
      // i32x4 index (w * 64 + chunk) * 64 + l of the slice's kPartTile ints
      i32x4* const mine = reinterpret_cast<i32x4*>(g.part) +
                          ((size_t)(logical - g.main_tiles) * g.splits + slice) * (kPartTile / 4) +
                          wave * 4096 + lane;
#pragma unroll
      for (int i = 0; i < kFM; ++i)
#pragma unroll
        for (int j = 0; j < kFN; ++j)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
            mine[((i * kFN + j) * 4 + r4) * 64] =
                i32x4{acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2],
                      acc[i][j][4 * r4 + 3]};
      return;
    }
  } else {
    // the tile's sums over its K slices (integer sums: exact in any order).
    // Workgroup half fh takes the slice waves fq = 2 fh, 2 fh + 1; its wave
    // w adds row tile w & 1 of slice wave 2 fh + (w >> 1): all 8 plane
    // tiles of one 32-row block, into acc[0][*]
    const int fq = 2 * fh + (wave >> 1), i = wave & 1;
    const i32x4* const base = reinterpret_cast<const i32x4*>(g.part) +
                              (size_t)(logical - g.main_tiles) * g.splits * (kPartTile / 4) +
                              fq * 4096 + lane;
    const int ns = g.splits;
    constexpr int kPair = 2;              // plane tiles whose chunks load together
#pragma unroll
    for (int j0 = 0; j0 < kFN; j0 += kPair) {
      i32x4 v[kPair][4][kMaxSplits];
#pragma unroll
      for (int jj = 0; jj < kPair; ++jj)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
          for (int sl = 0; sl < kMaxSplits; ++sl)
            v[jj][r4][sl] =
                sl < ns ? base[(size_t)sl * (kPartTile / 4) + ((i * kFN + j0 + jj) * 4 + r4) * 64]
                        : i32x4{0, 0, 0, 0};
#pragma unroll
      for (int jj = 0; jj < kPair; ++jj) {
        i32x16 tot;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          i32x4 sum = v[jj][r4][0];
#pragma unroll
          for (int sl = 1; sl < kMaxSplits; ++sl) sum += v[jj][r4][sl];
#pragma unroll
          for (int t = 0; t < 4; ++t) tot[4 * r4 + t] = sum[t];
        }
        // into the accumulation registers through an MFMA with zero operands
        const i32x4 z = {0, 0, 0, 0};
        acc[0][j0 + jj] = __builtin_amdgcn_mfma_i32_32x32x32_i8(z, z, tot, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  if constexpr (kMode != kSlice) {
    // a fixup wave owns one 32-row block of the tile, b0 (row tile 0 of
    // acc); the others their 64 rows
    constexpr int FM = kMode == kFixup ? 1 : kFM;
    const int b0 = kMode == kFixup ? 2 * (2 * fh + (wave >> 1)) + (wave & 1) : 0;
    const int64_t row0 = kMode == kFixup ? m0 + 32 * b0 : wave_row0;
    if constexpr (kEpi == kEpiAcc) {
      // H (hi plane, tiles j >= 4) and L (lo plane) as they are
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int64_t row = row0 + 32 * i + lr;
#pragma unroll
        for (int j = 0; j < kFN / 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t col = n0 + 32 * j + 8 * (r >> 2) + 4 * lh + (r & 3);
            if (row < e.M && col < e.N) {
              g.acc_lo[row * e.N + col] = acc[i][j][r];
              g.acc_hi[row * e.N + col] = acc[i][j + kFN / 2][r];
            }
          }
      }
    } else {
      // rows holds s_a s_Tw (multiplied once per row as it was staged)
      // i8_epilogue's arithmetic, written out: called here, the register
      // allocation of this kernel spills 12-37 registers
      float rs[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        rs[i] = rows[(kMode == kFixup ? 32 * b0 : 64 * wave) + 32 * i + lr];
      f32x4 cf[kFN / 2][4];
#pragma unroll
      for (int j = 0; j < kFN / 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          cf[j][q] = *reinterpret_cast<const f32x4*>(colf + 32 * j + 8 * q + 4 * lh);
      auto val = [&](int i, int j, int r) {
        return __builtin_fmaf((float)acc[i][j + kFN / 2][r], 256.0f, (float)acc[i][j][r]) *
               cf[j][r >> 2][r & 3];
      };
      store_tile<kEpi, FM>(val, rs, row0, n0, smem + wave * 8192 * kPassTiles, e, lane);
    }
  }
}

template <int kEpi, int kMode>
__global__ void __launch_bounds__(kThreads, 1)
qgemm_i8_kernel(I8Args g, EpiArgs e) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmem];
  i8_tile_body<kEpi, kMode>(g, e, smem, (int)blockIdx.x);
}

// Persistent whole-tile kernel for short K loops: a grid of one workgroup
// per CU, each taking the tiles blockIdx.x, blockIdx.x + gridDim.x, ... of
// the whole-tile order (gridDim.x a multiple of 8, so that a workgroup
// stays in its XCD's range).  The units of a workgroup's tiles form one
// stream through the LDS ring: the DMA of the next tile's first three units
// runs under the current tile's last units, so that a tile starts without
// a fresh workgroup's launch and first-load latency.  At a tile's end:
//   - the last unit issues no DMA and no reads, so that its slot is free
//     for the epilogue's staging;
//   - before the epilogue, every DMA issued so far has landed (the next
//     tile's units 0 .. 2): the epilogue's stores are then the only
//     memory operations in flight older than later DMAs, and no
//     count-based wait assumes an order between loads and stores (a
//     tile's first two syncs wait for no DMA);
//   - after it, wave 0 DMAs the next tile's factors, every wave the next
//     tile's unit 3 (into the staging slot), then reads unit 0.
// Requires an even number of units, at least 6.
template <int kEpi>
__global__ void __launch_bounds__(kThreads, 1)
qgemm_i8_persist(I8Args g, EpiArgs e) {
  // the ring, then the tile's 128 column factors and 256 activation row
  // scales s_a, both moved in by DMA (1 KB each)
  constexpr int kPColF = kSlots * kSlot, kPRowS = kPColF + 1024;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kPRowS + 1024];
  static_assert(kPRowS + 1024 <= 160 * 1024, "LDS");
  static_assert(kSlot >= 4 * 8192 * kPassTiles, "epilogue staging in one ring slot");
  static_assert((kSlots & (kSlots - 1)) == 0, "ring of a power of two");
  if (gated_off(g.gate)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int units = g.units;
  const uint32_t K = (uint32_t)g.K;

  // tile k of this workgroup: origin and operand ranges (rows past M fall
  // outside the activation range and load zero); past the last tile ok =
  // false and the ranges are empty, so that its loads are all zero
  struct Tile {
    int64_t m0, n0;
    const uint8_t* a;
    const int8_t* w;
    uint32_t a_bytes, w_bytes;
    bool ok;
  };
  auto tile_k = [&](int k, Tile& t) {
    const int bid = (int)blockIdx.x + k * (int)gridDim.x;
    TileWork tw;
    t.ok = bid < g.grid_main &&
           tile_work(kWhole, bid, g.main_tiles, g.splits, g.split_units, units, tw);
    int tm = 0, tn = 0;
    if (t.ok) tile_coords(tw.logical, g.mt, g.nt, 8, tm, tn);
    t.m0 = (int64_t)tm * kTileM;
    t.n0 = (int64_t)tn * kTileN;
    t.a = g.a + t.m0 * g.K;
    t.w = g.planes + (int64_t)tn * units * kUnitBytes;
    t.a_bytes = t.ok ? (uint32_t)(min<int64_t>(e.M - t.m0, kTileM) * g.K) : 0u;
    t.w_bytes = t.ok ? (uint32_t)units * (uint32_t)kUnitBytes : 0u;
  };
  Tile cur, nxt;
  tile_k(0, cur);
  if (!cur.ok) return;

  // ring slot of unit u of the current tile (u >= units: the next tile's
  // unit u - units), stream position sbase + u
  int sbase = 0;
  auto slot = [&](int u) { return smem + ((sbase + u) & (kSlots - 1)) * kSlot; };
  // the DMA of unit u of the stream, instruction idx
  auto issue_one = [&](int u, int idx, int ln) {
    const bool in_next = u >= units;
    const Tile& t = in_next ? nxt : cur;
    dma_one(buffer_rsrc(t.a, t.a_bytes), buffer_rsrc(t.w, t.w_bytes), slot(u),
            (uint32_t)(in_next ? u - units : u), idx, wave, ln, K, K, true);
  };
  // the factors of tile t by wave 0, 4 bytes per lane: 2^(X[n] - 1) of its
  // 128 columns (the array is padded to whole tiles) and s_a of its 256
  // rows (rows past M fall outside the range and read 0; never stored)
  const float* const colf = reinterpret_cast<const float*>(smem + kPColF);
  const float* const rows = reinterpret_cast<const float*>(smem + kPRowS);
  auto dma_factors = [&](const Tile& t) {
    if (wave != 0) return;
    const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(g.rowf + t.n0, kTileN * 4);
    const __amdgpu_buffer_rsrc_t rr = buffer_rsrc(
        g.a_rs + t.m0, (uint32_t)(min<int64_t>(e.M - t.m0, kTileM) * 4));
#pragma unroll
    for (int i = 0; i < kTileN / 64; ++i) dma4(rc, smem + kPColF + 256 * i, 256u * i + 4u * lane);
#pragma unroll
    for (int i = 0; i < kTileM / 64; ++i) dma4(rr, smem + kPRowS + 256 * i, 256u * i + 4u * lane);
  };
  // before unit u (u >= 2): this wave's DMA of unit u+1 has landed (units
  // u+2, u+3 may be in flight); before units 0 and 1 nothing is in flight
  // that they need.  Then this wave's reads are done, then the barrier.
  auto sync_unit = [&](auto vm) {
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (decltype(vm)::value) wait_vm<(kSlots - 2) * kLoads>();
    wait_lds();
    ring_barrier();
  };
  using T = std::true_type;
  using F = std::false_type;
  i32x16 acc[kFM][kFN];
  // unit u on cur: with the DMA of unit u + kSlots and the reads of unit
  // u + 1 into nf (kMem), the first unit starting the sums (first)
  auto compute = [&](auto first, auto mem, Frag& cf_, int u, Frag& nf, int ln) {
    unit_mfmas<decltype(first)::value, decltype(mem)::value>(
        acc, cf_, [&](int idx) { issue_one(u + kSlots, idx, ln); },
        [&](int idx) { read_one(slot(u + 1), idx, nf, wave, ln); });
    if constexpr (decltype(mem)::value) pin_frag(nf);
  };

  // first tile: its factors, then units 0 .. kSlots - 1, all landed
  dma_factors(cur);
  tile_k(1, nxt);
#pragma unroll
  for (int u = 0; u < kSlots; ++u)
#pragma unroll
    for (int idx = 0; idx < kLoads; ++idx) issue_one(u, idx, lane);
  wait_vm<0>();
  ring_barrier();
  Frag f0, f1;
#pragma unroll
  for (int idx = 0; idx < kReads; ++idx) read_one(slot(0), idx, f0, wave, lane);

  for (int k = 0;; ++k) {
    // per-lane offsets formed once per tile (live through its unit loop,
    // not through the epilogue)
    const int ln = opaque_lane(lane);
    sync_unit(F());
    compute(T(), T(), f0, 0, f1, ln);
    sync_unit(F());
    compute(F(), T(), f1, 1, f0, ln);
    for (int u = 2; u < units - 2; u += 2) {
      sync_unit(T());
      compute(F(), T(), f0, u, f1, ln);
      sync_unit(T());
      compute(F(), T(), f1, u + 1, f0, ln);
    }
    sync_unit(T());
    compute(F(), T(), f0, units - 2, f1, ln);
    sync_unit(T());
    compute(F(), F(), f1, units - 1, f0, ln);
    wait_vm<0>();
    const int lne = opaque_lane(lane);
    i8_epilogue<kEpi>(acc, colf, rows, *g.w_ts, cur.m0 + 64 * wave, cur.n0,
                      slot(units - 1) + wave * 8192 * kPassTiles, e, wave, lne, lne & 31, lne >> 5);
    // every wave is past its reads of the staging slot and of the factors
    wait_lds();
    ring_barrier();
    if (!nxt.ok) break;
    dma_factors(nxt);
    const int ln2 = opaque_lane(lane);
#pragma unroll
    for (int idx = 0; idx < kLoads; ++idx) issue_one(units + kSlots - 1, idx, ln2);
#pragma unroll
    for (int idx = 0; idx < kReads; ++idx) read_one(slot(units), idx, f0, wave, ln2);
    cur = nxt;
    sbase = (sbase + units) & (kSlots - 1);
    tile_k(k + 2, nxt);
  }
  wait_vm<0>();   // no DMA into LDS outlives the workgroup
}

// Routed linear: the whole tiles of either format in one launch, the
// format read from the device byte *route (kRouteNvfp4: the fp16-MFMA
// NVFP4 kernel's body; otherwise kRouteInt8: the per-tile integer kernel's
// body; neither: nothing), for a step enqueued or captured before its
// decisions are known.  The grid covers the larger of the two whole-tile
// grids; each body takes only the workgroups of its own.  The LDS holds
// either body's.
template <int kEpi>
__global__ void __launch_bounds__(kThreads, 1)
qgemm_routed_kernel(GemmArgs gf, I8Args gi, EpiArgs e, const uint8_t* route) {
  constexpr int kF16 = f16k::Raw<false>::kSmem;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kF16 > kSmem ? kF16 : kSmem];
  const uint32_t r = *route;
  const int bid = (int)blockIdx.x;
  if (r & kRouteNvfp4) {
    if (bid < gf.grid_main) f16k::qgemm_body<false, kEpi, kWhole>(gf, e, smem, bid);
  } else if (r & kRouteInt8) {
    if (bid < gi.grid_main) i8_tile_body<kEpi, kWhole>(gi, e, smem, bid);
  }
}

// ------------------------------------------------------------------ host --

namespace {

SplitPlan split_plan(int64_t M, int64_t N, int64_t K) {
  const int total = (int)(((M + kTileM - 1) / kTileM) * ntiles_of(N));
  return plan_split(total, (int)units_of(K), kCUs, kMaxSplits, kSplitMinSaved);
}

hipEvent_t g_ev_before = nullptr, g_ev_after = nullptr;

template <int kEpi, int kMode>
void launch_mode(int grid, hipEvent_t before, hipEvent_t after, const I8Args& g, const EpiArgs& e,
                 hipStream_t st) {
  if (before || after)
    hipExtLaunchKernelGGL((qgemm_i8_kernel<kEpi, kMode>), dim3(grid), dim3(kThreads), 0, st,
                          before, after, 0u, g, e);
  else
    hipLaunchKernelGGL((qgemm_i8_kernel<kEpi, kMode>), dim3(grid), dim3(kThreads), 0, st, g, e);
}

// the persistent kernel where a tile's start and end weigh most: short K
// loops (even, 6 .. kPersistMaxUnits units) over more than one round of
// tiles (measured 5-6 % faster at K = 1920, 1.6 % at 3072, 1 % slower at
// 7680, where the static assignment of tiles to workgroups costs more)
constexpr int kPersistMaxUnits = 64;
bool persist_fits(const I8Args& g) {
  return g.main_tiles && g.units % 2 == 0 && g.units >= 6 && g.units <= kPersistMaxUnits &&
         g.grid_main > kCUs;
}

template <int kEpi>
void launch_one(const I8Args& g, const EpiArgs& e, hipStream_t st) {
  const int tail = g.mt * g.nt - g.main_tiles;
  bool persist = false;
  if constexpr (kEpi != kEpiAcc) persist = persist_fits(g);
  if (persist) {
    if constexpr (kEpi != kEpiAcc) {
      hipEvent_t after = tail ? nullptr : g_ev_after;
      if (g_ev_before || after)
        hipExtLaunchKernelGGL((qgemm_i8_persist<kEpi>), dim3(kCUs), dim3(kThreads), 0, st,
                              g_ev_before, after, 0u, g, e);
      else
        hipLaunchKernelGGL((qgemm_i8_persist<kEpi>), dim3(kCUs), dim3(kThreads), 0, st, g, e);
    }
  } else if (g.main_tiles) {
    launch_mode<kEpi, kWhole>(g.grid_main, g_ev_before, tail ? nullptr : g_ev_after, g, e, st);
  }
  if (!tail) return;
  launch_mode<kEpiPlain, kSlice>(tail * g.splits, g.main_tiles ? nullptr : g_ev_before, nullptr,
                                 g, e, st);
  launch_mode<kEpi, kFixup>(2 * tail, nullptr, g_ev_after, g, e, st);
}

}  // namespace

void set_i8_gemm_events(hipEvent_t before, hipEvent_t after) {
  g_ev_before = before;
  g_ev_after = after;
}

size_t int8_i8_gemm_ws_bytes(int64_t M, int64_t N, int64_t K) {
  const SplitPlan p = split_plan(M, N, K);
  return (size_t)p.tail * p.splits * kPartTile * 4;
}

// the integer kernel's arguments (split: the K split of a partly filled
// last round, when the workspace holds it)
static I8Args i8_args(const int8_t* a_q, const float* a_s, const void* w8, const float* w_ts,
                      int64_t M, int64_t N, int64_t K, void* ws, bool split) {
  I8Args g = {};
  g.gate = current_gate();
  g.a = reinterpret_cast<const uint8_t*>(a_q);
  g.planes = static_cast<const int8_t*>(w8);
  const int64_t nt = ntiles_of(N);
  g.rowf = reinterpret_cast<const float*>(static_cast<const uint8_t*>(w8) +
                                          r256((size_t)(nt * units_of(K)) * kUnitBytes));
  g.a_rs = a_s;
  g.w_ts = w_ts;
  g.K = K;
  g.units = (int)units_of(K);
  g.mt = (int)((M + kTileM - 1) / kTileM);
  g.nt = (int)nt;
  const SplitPlan p = split ? split_plan(M, N, K) : SplitPlan{g.mt * g.nt, 0, 1, g.units};
  g.main_tiles = p.main_tiles;
  g.grid_main = 8 * ((p.main_tiles + 7) / 8);
  g.splits = p.splits;
  g.split_units = p.split_units;
  if (p.tail) g.part = static_cast<int32_t*>(ws);
  return g;
}

hipError_t launch_int8_i8_gemm(const int8_t* a_q, const float* a_s, const void* w8,
                               const float* w_ts, int64_t M, int64_t N, int64_t K,
                               const GemmOut& o, void* ws, size_t ws_bytes, int32_t* acc_hi,
                               int32_t* acc_lo, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  const bool split = acc_hi == nullptr && ws_bytes >= int8_i8_gemm_ws_bytes(M, N, K) &&
                     int8_i8_gemm_ws_bytes(M, N, K) > 0;
  I8Args g = i8_args(a_q, a_s, w8, w_ts, M, N, K, ws, split);
  g.acc_hi = acc_hi;
  g.acc_lo = acc_lo;
  const int vec = (reinterpret_cast<uintptr_t>(o.y) % 16 == 0) && (o.ldy % 4 == 0);
  EpiArgs e = {o.y, o.ldy, o.out_f32, o.gelu, o.bias, M, N, vec, o.yq, o.ys, o.y_ts, o.y_amax};
  if (acc_hi) {
    launch_one<kEpiAcc>(g, e, st);
    return hipGetLastError();
  }
  int kind = kEpiGeneral;
  if (o.yq)
    kind = kEpiQuant;
  else if (!o.out_f32 && vec)
    kind = (o.bias ? (o.gelu ? kEpiStagedBiasGelu : kEpiStagedBias)
                   : (o.gelu ? kEpiStagedGelu : kEpiPlain)) +
           (o.y_amax ? kEpiAmax : 0);
  switch (kind) {
    case kEpiPlain: launch_one<kEpiPlain>(g, e, st); break;
    case kEpiStagedBias: launch_one<kEpiStagedBias>(g, e, st); break;
    case kEpiStagedGelu: launch_one<kEpiStagedGelu>(g, e, st); break;
    case kEpiStagedBiasGelu: launch_one<kEpiStagedBiasGelu>(g, e, st); break;
    case kEpiAmax + kEpiPlain: launch_one<kEpiAmax + kEpiPlain>(g, e, st); break;
    case kEpiAmax + kEpiStagedBias: launch_one<kEpiAmax + kEpiStagedBias>(g, e, st); break;
    case kEpiAmax + kEpiStagedGelu: launch_one<kEpiAmax + kEpiStagedGelu>(g, e, st); break;
    case kEpiAmax + kEpiStagedBiasGelu: launch_one<kEpiAmax + kEpiStagedBiasGelu>(g, e, st); break;
    case kEpiQuant: launch_one<kEpiQuant>(g, e, st); break;
    default: launch_one<kEpiGeneral>(g, e, st); break;
  }
  return hipGetLastError();
}

// The routed linear: the NVFP4 scale re-layout (run only for kRouteNvfp4;
// none when the scales are read in place), one routed launch of the whole
// tiles, then the K slices and fixups of either format when its last round
// is split (each run only for its format).  Where the INT8 whole tiles
// take the persistent kernel (more than one round of short-K tiles), the
// per-tile body of a routed launch is the slower one and one launch more
// costs little beside the GEMM: there each format's own launches run, each
// under its part of the route.  Bf16 staged outputs only (the caller
// checks).
hipError_t launch_routed_gemm(const uint8_t* route, const uint8_t* a_q4, const uint8_t* a_s4,
                              const float* a_ts4, const int8_t* a_q8, const float* a_s8,
                              const uint8_t* w_q, const uint8_t* w_s, const float* w_ts,
                              const void* w8, int64_t M, int64_t N, int64_t K, const GemmOut& o,
                              void* ws, size_t ws_bytes, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  // every launch also honours the thread's gate (qa_set_gate), as a second
  // byte beside the route
  const Gate cur = current_gate();
  GemmArgs gf;
  EpiArgs e;
  hipError_t err = nvfp4_gemm_prepare(a_q4, a_s4, a_ts4, w_q, w_s, w_ts, M, N, K, o, ws, ws_bytes,
                                      Gate{route, kRouteNvfp4, 0u, cur.flags, cur.bits}, st,
                                      gf, e);
  if (err != hipSuccess) return err;
  const bool split = ws_bytes >= int8_i8_gemm_ws_bytes(M, N, K) &&
                     int8_i8_gemm_ws_bytes(M, N, K) > 0;
  I8Args gi = i8_args(a_q8, a_s8, w8, w_ts, M, N, K, ws, split);
  // a byte with both bits: NVFP4 only
  gi.gate = Gate{route, kRouteInt8, kRouteNvfp4, cur.flags, cur.bits};
  // the whole tiles: the kernel reads the route itself, its bodies check
  // the thread's gate
  GemmArgs gfm = gf;
  I8Args gim = gi;
  gfm.gate = cur;
  gim.gate = cur;
  if (!gfm.main_tiles) gfm.grid_main = 0;
  if (!gim.main_tiles) gim.grid_main = 0;
  const int grid = gfm.grid_main > gim.grid_main ? gfm.grid_main : gim.grid_main;
  const int kind = (o.bias ? (o.gelu ? kEpiStagedBiasGelu : kEpiStagedBias)
                           : (o.gelu ? kEpiStagedGelu : kEpiPlain)) +
                   (o.y_amax ? kEpiAmax : 0);
  const bool separate = persist_fits(gi);
  auto go = [&](auto kc) {
    constexpr int kEpi = decltype(kc)::value;
    if (separate) {
      launch_one<kEpi>(gi, e, st);
      return;
    }
    if (grid)
      hipLaunchKernelGGL((qgemm_routed_kernel<kEpi>), dim3(grid), dim3(kThreads), 0, st, gfm,
                         gim, e, route);
    const int tail = gi.mt * gi.nt - gi.main_tiles;
    if (tail) {
      launch_mode<kEpiPlain, kSlice>(tail * gi.splits, nullptr, nullptr, gi, e, st);
      launch_mode<kEpi, kFixup>(2 * tail, nullptr, nullptr, gi, e, st);
    }
  };
  switch (kind) {
    case kEpiPlain: go(std::integral_constant<int, kEpiPlain>()); break;
    case kEpiStagedBias: go(std::integral_constant<int, kEpiStagedBias>()); break;
    case kEpiStagedGelu: go(std::integral_constant<int, kEpiStagedGelu>()); break;
    case kEpiStagedBiasGelu: go(std::integral_constant<int, kEpiStagedBiasGelu>()); break;
    case kEpiAmax + kEpiPlain: go(std::integral_constant<int, kEpiAmax + kEpiPlain>()); break;
    case kEpiAmax + kEpiStagedBias: go(std::integral_constant<int, kEpiAmax + kEpiStagedBias>()); break;
    case kEpiAmax + kEpiStagedGelu: go(std::integral_constant<int, kEpiAmax + kEpiStagedGelu>()); break;
    default: go(std::integral_constant<int, kEpiAmax + kEpiStagedBiasGelu>()); break;
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  return nvfp4_gemm_launch(gf, e, st, !separate);
}

}  // namespace qact
