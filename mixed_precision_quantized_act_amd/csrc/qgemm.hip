// Quantized linear GEMMs on gfx950 MFMA (the fp16-MFMA kernel): its
// launches, the scale re-layout and the host code.  The kernel's design and
// device code are in qgemm_f16.h.
#include <hip/hip_ext.h>

#include <type_traits>

#include "qgemm_f16.h"

namespace qact {

using namespace f16k;

// ------------------------------------------------------- scale re-layout --

// E4M3 scales [rows][K/16] -> per 256-row tile and K unit of 64, the 4
// scale bytes of each row as one word: dst[(tile * units + u) * 256 + r].
// Rows past `rows` and groups past K/16 read as 0 (a zero scale makes the
// corresponding fp16 values zero, whatever codes the raw unit holds there).
// One workgroup per (tile, unit), one thread per row; the workgroups past
// tiles0 * units re-lay the second array (s1, rows1, dst1).
__global__ void __launch_bounds__(256)
scale_tiles_kernel(const uint8_t* __restrict__ s0, int64_t rows0, uint32_t* __restrict__ dst0,
                   int tiles0, const uint8_t* __restrict__ s1, int64_t rows1,
                   uint32_t* __restrict__ dst1, int64_t K, int units, Gate gate) {
  if (gated_off(gate)) return;
  int tu = (int)blockIdx.x;
  const bool second = tu >= tiles0 * units;
  if (second) tu -= tiles0 * units;
  const uint8_t* const s = second ? s1 : s0;
  const int64_t rows = second ? rows1 : rows0;
  uint32_t* const dst = second ? dst1 : dst0;
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

// the kernel: one workgroup's share of a launch in mode kMode
template <bool I8, int kEpi, int kMode>
__global__ void __launch_bounds__(kThreads, 1)
qgemm_kernel(GemmArgs g, EpiArgs e) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[Raw<I8>::kSmem];
  qgemm_body<I8, kEpi, kMode>(g, e, smem, (int)blockIdx.x);
}

// ---------------------------------------------------------------- host --

static int vec_ok(const GemmOut& o) {
  return (reinterpret_cast<uintptr_t>(o.y) % 16 == 0) && (o.ldy % 4 == 0);
}

bool gemm_out_staged(const GemmOut& o) { return !o.yq && !o.out_f32 && vec_ok(o); }

static size_t scale_tiles_bytes(int64_t rows, int64_t K) {
  return (size_t)((rows + kTileM - 1) / kTileM) * (size_t)units_of(K) * 1024u;
}
static size_t r256(size_t v) { return (v + 255) / 256 * 256; }

// K split of the last round.  With one workgroup per CU the tiles run in
// rounds of kCUs; when the last round is at most half full, each of its
// `tail` tiles is split along K into `splits` slices (at most kMaxSplits,
// at least 2 raw units each) so that the round holds tail * splits
// workgroups of 1/splits the length.  A pure function of the shape, so
// that workspace sizes are too; on a device with another CU count the plan
// is only less well fitted.  Every slice stores its fp32 partial sums in the workspace;
// a second launch adds them per tail tile and runs the epilogue (no
// workgroup waits for another inside a launch), four workgroups per tail
// tile so that the fixup's loads spread over more CUs and fewer sequential
// batches (74 tail tiles of the QKV shape: 22.7 us with one workgroup per
// tile).  (The split is worth it only if the round gets shorter by more
// than the slice and fixup launches cost: at 8 units the QKV and FFN-up
// shapes, 30 units in 3-4 slices, measured no faster, the 1920-wide O
// projection 2 % faster; the 7680-wide down projection, 120 units in 4,
// is 10 % faster.)
static SplitPlan split_plan(int64_t M, int64_t N, int64_t K) {
  const int total = (int)(((M + kTileM - 1) / kTileM) * ((N + kTileN - 1) / kTileN));
  return plan_split(total, (int)units_of(K), kCUs, kMaxSplits, kSplitMinSaved);
}
// the slices' partial sums
static size_t split_ws_bytes(const SplitPlan& p) {
  return (size_t)p.tail * p.splits * kPartTile * 4;
}

size_t nvfp4_gemm_ws_bytes(int64_t M, int64_t N, int64_t K) {
  return r256(scale_tiles_bytes(M, K)) + r256(scale_tiles_bytes(N, K)) +
         split_ws_bytes(split_plan(M, N, K));
}

size_t int8_gemm_ws_bytes(int64_t M, int64_t N, int64_t K) {
  return r256(scale_tiles_bytes(N, K)) + split_ws_bytes(split_plan(M, N, K));
}

// INT8: the weight scales are read in place when K is a multiple of 64 and
// the array is 4-byte aligned (no re-layout launch).  The NVFP4 kernel,
// whose raw loads already touch more rows per unit, measured about 5 %
// slower reading either scale array in place than after one re-layout
// launch of both, so it always takes the per-tile copies.
#ifndef QACT_INT8_W_DIRECT
#define QACT_INT8_W_DIRECT 1
#endif
static bool w_scales_direct(int64_t K, const void* w_s) {
  return QACT_INT8_W_DIRECT && K % kUnitK == 0 && (reinterpret_cast<uintptr_t>(w_s) & 3) == 0;
}

// NVFP4: both scale arrays are read in place (no re-layout launch) when K
// is a multiple of 64, both arrays are 4-byte aligned and the GEMM has at
// most kNvfp4DirectTiles tiles.  Measured per call (graph replays): up to
// one round of tiles the launch saved (about 2 us) outweighs the slower
// scale loads (256x768x256 13.5 -> 11.6 us, 8192x1920x1920 62.6 -> 61.4);
// past it the loads cost more (17776x5760x1920 363 -> 375 us).
#ifndef QACT_NVFP4_DIRECT_TILES
#define QACT_NVFP4_DIRECT_TILES 256
#endif
static constexpr int kNvfp4DirectTiles = QACT_NVFP4_DIRECT_TILES;
static bool nvfp4_scales_direct(int64_t M, int64_t N, int64_t K, const void* a_s,
                                const void* w_s) {
  const int64_t tiles = ((M + kTileM - 1) / kTileM) * ((N + kTileN - 1) / kTileN);
  return tiles <= kNvfp4DirectTiles && K % kUnitK == 0 &&
         ((reinterpret_cast<uintptr_t>(a_s) | reinterpret_cast<uintptr_t>(w_s)) & 3) == 0;
}

// the least workspace a call accepts: without the K split (which is used
// only when the workspace holds nvfp4/int8_gemm_ws_bytes)
size_t nvfp4_gemm_ws_need(int64_t M, int64_t N, int64_t K, const void*) {
  return r256(scale_tiles_bytes(M, K)) + scale_tiles_bytes(N, K);
}

size_t int8_gemm_ws_need(int64_t, int64_t N, int64_t K, const void* w_s) {
  return w_scales_direct(K, w_s) ? 0 : scale_tiles_bytes(N, K);
}

static hipEvent_t g_ev_before = nullptr, g_ev_after = nullptr;

void set_gemm_events(hipEvent_t before, hipEvent_t after) {
  g_ev_before = before;
  g_ev_after = after;
}

// one launch re-lays out (s0, rows0) and, when s1 is not null, (s1, rows1)
static hipError_t launch_scale_tiles(const uint8_t* s0, int64_t rows0, uint32_t* dst0,
                                     const uint8_t* s1, int64_t rows1, uint32_t* dst1, int64_t K,
                                     hipStream_t st, Gate gate = current_gate()) {
  const int64_t units = units_of(K);
  const int64_t t0 = (rows0 + kTileM - 1) / kTileM, t1 = s1 ? (rows1 + kTileM - 1) / kTileM : 0;
  hipLaunchKernelGGL(scale_tiles_kernel, dim3((unsigned)((t0 + t1) * units)), dim3(256), 0, st, s0,
                     rows0, dst0, (int)t0, s1, rows1, dst1, K, (int)units, gate);
  return hipGetLastError();
}

// The GEMM: the whole tiles, then with a K split the slices of the tail
// tiles and their fixup.  The events take the dispatches' own start and
// end timestamps (the start of the first, the end of the last): no marker
// packets are added to the stream around the kernels.
template <bool I8, int kEpi, int kMode>
static void launch_mode(int grid, hipEvent_t before, hipEvent_t after, const GemmArgs& g,
                        const EpiArgs& e, hipStream_t st) {
  if (before || after)
    hipExtLaunchKernelGGL((qgemm_kernel<I8, kEpi, kMode>), dim3(grid), dim3(kThreads), 0, st,
                          before, after, 0u, g, e);
  else
    hipLaunchKernelGGL((qgemm_kernel<I8, kEpi, kMode>), dim3(grid), dim3(kThreads), 0, st, g, e);
}

// parts: kPartsWhole, kPartsTails or both (the tails alone take no events)
enum { kPartsWhole = 1, kPartsTails = 2 };
template <bool I8, int kEpi>
static void launch_one(int parts, const GemmArgs& g, const EpiArgs& e, hipStream_t st) {
  const int tail = g.mt * g.nt - g.main_tiles;
  const bool ev = parts & kPartsWhole;
  if (g.main_tiles && (parts & kPartsWhole))
    launch_mode<I8, kEpi, kWhole>(g.grid_main, g_ev_before, tail ? nullptr : g_ev_after, g, e, st);
  if (!tail || !(parts & kPartsTails)) return;
  launch_mode<I8, kEpiPlain, kSlice>(tail * g.splits, ev && !g.main_tiles ? g_ev_before : nullptr,
                                     nullptr, g, e, st);
  launch_mode<I8, kEpi, kFixup>(4 * tail, nullptr, ev ? g_ev_after : nullptr, g, e, st);
}

static hipError_t launch_gemm(bool i8, const GemmArgs& g, const EpiArgs& e, hipStream_t st,
                              int parts = kPartsWhole | kPartsTails) {
  int kind = kEpiGeneral;
  if (e.yq)
    kind = kEpiQuant;
  else if (!e.out_f32 && e.vec_ok)
    kind = (e.bias ? (e.gelu ? kEpiStagedBiasGelu : kEpiStagedBias)
                   : (e.gelu ? kEpiStagedGelu : kEpiPlain)) +
           (e.amax ? kEpiAmax : 0);
  auto go = [&](auto i8c) {
    constexpr bool I8 = decltype(i8c)::value;
    switch (kind) {
      case kEpiPlain: launch_one<I8, kEpiPlain>(parts, g, e, st); break;
      case kEpiStagedBias: launch_one<I8, kEpiStagedBias>(parts, g, e, st); break;
      case kEpiStagedGelu: launch_one<I8, kEpiStagedGelu>(parts, g, e, st); break;
      case kEpiStagedBiasGelu: launch_one<I8, kEpiStagedBiasGelu>(parts, g, e, st); break;
      case kEpiAmax + kEpiPlain: launch_one<I8, kEpiAmax + kEpiPlain>(parts, g, e, st); break;
      case kEpiAmax + kEpiStagedBias: launch_one<I8, kEpiAmax + kEpiStagedBias>(parts, g, e, st); break;
      case kEpiAmax + kEpiStagedGelu: launch_one<I8, kEpiAmax + kEpiStagedGelu>(parts, g, e, st); break;
      case kEpiAmax + kEpiStagedBiasGelu:
        launch_one<I8, kEpiAmax + kEpiStagedBiasGelu>(parts, g, e, st);
        break;
      case kEpiQuant: launch_one<I8, kEpiQuant>(parts, g, e, st); break;
      default: launch_one<I8, kEpiGeneral>(parts, g, e, st); break;
    }
  };
  if (i8)
    go(std::true_type());
  else
    go(std::false_type());
  return hipGetLastError();
}

// split: the workspace region of the K split (null: no split)
static GemmArgs base_args(int64_t M, int64_t N, int64_t K, uint8_t* split) {
  GemmArgs g = {};
  g.gate = current_gate();
  g.K = K;
  g.units = (int)units_of(K);
  g.nk = (int)((K + kStageK - 1) / kStageK);
  g.mt = (int)((M + kTileM - 1) / kTileM);
  g.nt = (int)((N + kTileN - 1) / kTileN);
  const SplitPlan p = split ? split_plan(M, N, K) : SplitPlan{g.mt * g.nt, 0, 1, g.units};
  g.main_tiles = p.main_tiles;
  g.grid_main = 8 * ((p.main_tiles + 7) / 8);
  g.splits = p.splits;
  g.split_units = p.split_units;
  if (p.tail) g.part = reinterpret_cast<float*>(split);
  return g;
}

hipError_t nvfp4_gemm_prepare(const uint8_t* a_q, const uint8_t* a_s, const float* a_ts,
                              const uint8_t* w_q, const uint8_t* w_s, const float* w_ts,
                              int64_t M, int64_t N, int64_t K, const GemmOut& o, void* ws,
                              size_t ws_bytes, Gate gate, hipStream_t st, GemmArgs& g,
                              EpiArgs& e) {
  uint8_t* const w8 = static_cast<uint8_t*>(ws);
  const size_t tiles = r256(scale_tiles_bytes(M, K)) + r256(scale_tiles_bytes(N, K));
  g = base_args(M, N, K, ws_bytes >= nvfp4_gemm_ws_bytes(M, N, K) ? w8 + tiles : nullptr);
  g.gate = gate;
  if (nvfp4_scales_direct(M, N, K, a_s, w_s)) {
    g.a_direct = g.b_direct = 1;
    g.a_st = reinterpret_cast<const uint32_t*>(a_s);
    g.b_st = reinterpret_cast<const uint32_t*>(w_s);
  } else {
    uint32_t* a_st = static_cast<uint32_t*>(ws);
    uint32_t* b_st = reinterpret_cast<uint32_t*>(w8 + r256(scale_tiles_bytes(M, K)));
    hipError_t err = launch_scale_tiles(a_s, M, a_st, w_s, N, b_st, K, st, gate);
    if (err != hipSuccess) return err;
    g.a_direct = g.b_direct = 0;
    g.a_st = a_st;
    g.b_st = b_st;
  }
  g.a = a_q;
  g.b = w_q;
  g.a_ts = a_ts;
  g.w_ts = w_ts;
  e = EpiArgs{o.y, o.ldy, o.out_f32, o.gelu, o.bias, M, N, vec_ok(o), o.yq, o.ys, o.y_ts,
              o.y_amax};
  return hipSuccess;
}

hipError_t nvfp4_gemm_launch(const GemmArgs& g, const EpiArgs& e, hipStream_t st,
                             bool tails_only) {
  return launch_gemm(false, g, e, st, tails_only ? kPartsTails : kPartsWhole | kPartsTails);
}

hipError_t launch_nvfp4_gemm(const uint8_t* a_q, const uint8_t* a_s, const float* a_ts,
                             const uint8_t* w_q, const uint8_t* w_s, const float* w_ts,
                             int64_t M, int64_t N, int64_t K, const GemmOut& o, void* ws,
                             size_t ws_bytes, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  GemmArgs g;
  EpiArgs e;
  hipError_t err = nvfp4_gemm_prepare(a_q, a_s, a_ts, w_q, w_s, w_ts, M, N, K, o, ws, ws_bytes,
                                      current_gate(), st, g, e);
  if (err != hipSuccess) return err;
  return launch_gemm(false, g, e, st);
}

hipError_t launch_int8_gemm(const int8_t* a_q, const float* a_s, const uint8_t* w_q,
                            const uint8_t* w_s, const float* w_ts, int64_t M, int64_t N,
                            int64_t K, const GemmOut& o, void* ws, size_t ws_bytes,
                            hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  uint8_t* const w8 = static_cast<uint8_t*>(ws);
  GemmArgs g = base_args(M, N, K,
                         ws_bytes >= int8_gemm_ws_bytes(M, N, K) ? w8 + r256(scale_tiles_bytes(N, K))
                                                                 : nullptr);
  g.b_direct = w_scales_direct(K, w_s);
  if (g.b_direct) {
    g.b_st = reinterpret_cast<const uint32_t*>(w_s);
  } else {
    uint32_t* b_st = static_cast<uint32_t*>(ws);
    hipError_t err = launch_scale_tiles(w_s, N, b_st, nullptr, 0, nullptr, K, st);
    if (err != hipSuccess) return err;
    g.b_st = b_st;
  }
  g.a = reinterpret_cast<const uint8_t*>(a_q);
  g.b = w_q;
  g.w_ts = w_ts;
  g.a_rs = a_s;
  EpiArgs e = {o.y, o.ldy, o.out_f32, o.gelu, o.bias, M, N, vec_ok(o), o.yq, o.ys, o.y_ts,
               o.y_amax};
  return launch_gemm(true, g, e, st);
}

}  // namespace qact
