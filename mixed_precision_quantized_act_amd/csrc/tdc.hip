// Gamma, Temporal Delta Cache and relative-error kernels for gfx950
// (HBM-bound streams).
//
// 6Bit-Diffusion: Gamma is the relative L1 distance between a block's input
// and output (Fig. 2 and Fig. 3 captions); TDC caches the block residual
// Delta = out - in and reuses it for invariant blocks (abstract), comparing
// successive Deltas by relative L2 (Fig. 4 caption); E_rel, the layer-wise
// relative quantization error that the DMPQ predictor is fitted to (Fig. 3
// caption), is taken as the relative L2 error of the layer output; the
// cosine similarity of successive Deltas (Fig. 4 caption) is the other
// agreement measure the pages show.
//
// tdc_apply may run in place (dst == in): every element is read and then
// written by the same thread, so `in` and `dst` carry no restrict.
//
// One streaming pass: 16-byte vector loads of 8 bf16, per-thread float64
// partial sums of exact terms, a wave/workgroup reduction into one row of
// scratch per workgroup, then a one-workgroup pass that adds the rows in a
// fixed order.  No atomics, so sums are bit-reproducible.
#include "qact_device.h"
#include "qact_internal.h"

namespace qact {

#ifndef QACT_TDC_UNROLL
#define QACT_TDC_UNROLL 4
#endif
#ifndef QACT_TDC_BLOCKS
#define QACT_TDC_BLOCKS 2048
#endif
static constexpr int kRedBlocks = QACT_TDC_BLOCKS;
static constexpr int kThreads = 256;
static constexpr int kUnroll = QACT_TDC_UNROLL;
static_assert(kRedBlocks % kThreads == 0, "finalize loads kRedBlocks / kThreads rows per thread");

// MODE_APPLY_AMAX: tdc_apply that also max-combines the |max| of its
// bf16 outputs into a device word (the consumer's NVFP4 tensor amax)
enum { MODE_GAMMA = 0, MODE_UPDATE = 1, MODE_APPLY = 2, MODE_RELERR = 3, MODE_COS = 4,
       MODE_APPLY_AMAX = 5 };

struct Acc4 {
  double s[4];
};

template <int MODE, bool PREV>
__device__ __forceinline__ uint32_t tdc_pair(uint32_t xi, uint32_t bi, uint32_t pi, Acc4& a) {
  // xi, bi, pi: bf16 bit patterns (low 16 bits); returns the bf16 written
  const float x = __uint_as_float(xi << 16);
  const float b = __uint_as_float(bi << 16);
  if (MODE == MODE_COS) {
    // x = Delta_t, b = Delta_{t-1}: x b, x^2, b^2, each exact in float64
    const double xd = (double)x, bd = (double)b;
    a.s[0] = __fma_rn(xd, bd, a.s[0]);
    a.s[1] = __fma_rn(xd, xd, a.s[1]);
    a.s[2] = __fma_rn(bd, bd, a.s[2]);
    return 0;
  }
  if (MODE == MODE_RELERR) {
    // x = quantized output, b = reference: (x - b)^2 and b^2, each exact in
    // float64 (a bf16 difference has at most 17 significant bits)
    const double d = (double)x - (double)b;
    a.s[0] = __fma_rn(d, d, a.s[0]);
    a.s[1] = __fma_rn((double)b, (double)b, a.s[1]);
    return 0;
  }
  if (MODE == MODE_APPLY || MODE == MODE_APPLY_AMAX) {
    const uint32_t o = f32_to_bf16(x + b);
    const double od = (double)__uint_as_float(o << 16);
    a.s[0] += fabs(od - (double)x);
    a.s[1] += fabs((double)x);
    return o;
  }
  a.s[0] += fabs((double)b - (double)x);
  a.s[1] += fabs((double)x);
  if (MODE == MODE_GAMMA) return 0;
  const uint32_t dn = f32_to_bf16(b - x);
  if (PREV) {
    // fused multiply-add: each square joins the sum with one rounding (the
    // square of a short bf16 difference is exact in float64 anyway)
    const double p = (double)__uint_as_float(pi << 16);
    const double diff = (double)__uint_as_float(dn << 16) - p;
    a.s[2] = __fma_rn(diff, diff, a.s[2]);
    a.s[3] = __fma_rn(p, p, a.s[3]);
  }
  return dn;
}

// The operand set a kernel takes from a device byte (ring slot of the
// Delta cache): the primary pointers when (*sel & bits_a), the alternates
// when (*sel & bits_b), nothing otherwise; sel == nullptr: the primary ones.
__device__ __forceinline__ bool pick_route(const RingRoute& rt, const uint16_t*& b,
                                           const uint16_t*& prev, uint16_t*& dst) {
  if (!rt.sel) return true;
  const uint32_t v = *rt.sel;
  if (v & rt.bits_a) return true;
  if (v & rt.bits_b) {
    b = rt.b_alt;
    prev = rt.prev_alt;
    dst = rt.dst_alt;
    return true;
  }
  return false;
}

template <int MODE, bool PREV>
__global__ void __launch_bounds__(kThreads)
tdc_kernel(const uint16_t* in, const uint16_t* b, const uint16_t* prev, uint16_t* dst, int64_t n,
           double* __restrict__ partial, int want_sums, uint32_t* __restrict__ amax_out,
           RingRoute rt, Gate gate) {
  if (gated_off(gate)) return;
  if (!pick_route(rt, b, prev, dst)) return;
  constexpr bool kAmax = MODE == MODE_APPLY_AMAX;
  constexpr bool kWrites = MODE == MODE_UPDATE || MODE == MODE_APPLY || kAmax;
  uint32_t amx = 0;            // |max| of this thread's outputs (bf16 patterns)
  Acc4 a = {{0.0, 0.0, 0.0, 0.0}};
  const int64_t nvec = n / 8;
  // kUnroll vectors per thread and sweep: all loads issued before any use
  const int64_t sweep = (int64_t)gridDim.x * kThreads * kUnroll;
  for (int64_t v0 = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; v0 < nvec;
       v0 += sweep) {
    u32x4 xv[kUnroll], bv[kUnroll], pv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t v = v0 + u * kThreads;
      if (v < nvec) {
        xv[u] = reinterpret_cast<const u32x4*>(in)[v];
        bv[u] = reinterpret_cast<const u32x4*>(b)[v];
        pv[u] = PREV ? reinterpret_cast<const u32x4*>(prev)[v] : u32x4{0, 0, 0, 0};
      } else {
        xv[u] = bv[u] = pv[u] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t v = v0 + u * kThreads;
      u32x4 ov;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = tdc_pair<MODE, PREV>(xv[u][i] & 0xFFFFu, bv[u][i] & 0xFFFFu,
                                                 pv[u][i] & 0xFFFFu, a);
        const uint32_t hi = tdc_pair<MODE, PREV>(xv[u][i] >> 16, bv[u][i] >> 16, pv[u][i] >> 16, a);
        ov[i] = lo | (hi << 16);
      }
      if (kWrites && v < nvec) {
        // plain stores: nontemporal ones measured 5-8 % slower here
        reinterpret_cast<u32x4*>(dst)[v] = ov;
        if constexpr (kAmax) amx = max(amx, fold_max(abs_max8_pk(ov, u16x2{0, 0})));
      }
    }
  }
  // ragged tail (n % 8 elements), done by workgroup 0
  if (blockIdx.x == 0) {
    const int64_t e = nvec * 8 + threadIdx.x;
    if (e < n) {
      const uint32_t o = tdc_pair<MODE, PREV>(in[e], b[e], PREV ? prev[e] : 0u, a);
      if (kWrites) dst[e] = (uint16_t)o;
      if constexpr (kAmax) amx = max(amx, o & 0x7FFFu);
    }
  }
  if constexpr (kAmax) {
    // the wave's integer maximum, one atomic maximum per wave (float bits)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amx = max(amx, (uint32_t)__shfl_xor((int)amx, o, 64));
    if ((threadIdx.x & 63) == 0) atomicMax(amax_out + (blockIdx.x % kAmaxSlots), amx << 16);
  }
  if (!want_sums) return;
  __shared__ double red[4][kThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const double s = wave_sum(a.s[j]);
    if (lane == 0) red[j][wave] = s;
  }
  __syncthreads();
  if (threadIdx.x < 4) {
    double s = 0.0;
    for (int w = 0; w < kThreads / 64; ++w) s += red[threadIdx.x][w];
    partial[(int64_t)blockIdx.x * 4 + threadIdx.x] = s;
  }
}

// Fixed-order sum of the per-workgroup rows: thread t adds rows t, t+256,
// ... (all four columns, loads issued together), then the waves combine in
// order.
__global__ void __launch_bounds__(kThreads)
tdc_finalize_kernel(const double* __restrict__ partial, int rows, int ncols,
                    double* __restrict__ sums, RingRoute rt, Gate gate) {
  if (gated_off(gate)) return;
  if (rt.sel && (*rt.sel & (rt.bits_a | rt.bits_b)) == 0u) return;
  __shared__ double red[4][kThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double s[4] = {0.0, 0.0, 0.0, 0.0};
  // rows <= kRedBlocks: every load issued before the first add
  constexpr int kPer = kRedBlocks / kThreads;
  double4 p[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int r = threadIdx.x + kThreads * j;
    p[j] = r < rows ? reinterpret_cast<const double4*>(partial)[r] : double4{0.0, 0.0, 0.0, 0.0};
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    s[0] += p[j].x;
    s[1] += p[j].y;
    s[2] += p[j].z;
    s[3] += p[j].w;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const double t = wave_sum(s[j]);
    if (lane == 0) red[j][wave] = t;
  }
  __syncthreads();
  if (threadIdx.x < ncols) {
    double t = 0.0;
    for (int w = 0; w < kThreads / 64; ++w) t += red[threadIdx.x][w];
    sums[threadIdx.x] = t;
  }
}

// One timestep's decisions on the device, from the sums the previous
// step's calls left: for each block l (one thread each), first the state
// update the host loop makes after a step -- Gamma_{t-1} = S1/S2 of the
// block (tdc_update's or, for a skipped block, tdc_apply's), and for a
// block computed at t-1 its Delta going to the other ring slot and d =
// sqrt(S3)/sqrt(S4) once two Deltas are stored -- then the decisions of the
// DMPQ rule (p = alpha Gamma + beta > tau: INT8, ties NVFP4, all INT8 at t
// = 0; 6Bit-Diffusion, Fig. 3 caption) and of the TDC rule (skip when t >=
// 2, the block ran at t-1 and d < delta; abstract and Fig. 4 caption), and
// the gate bytes of the step's calls.  The step counter is advanced by
// thread 0 after every block's update.
__device__ __forceinline__ double ratio0_dev(double num, double den) {
  if (den == 0.0) return num == 0.0 ? 0.0 : __longlong_as_double(0x7FF0000000000000ll);
  return num / den;
}

__global__ void __launch_bounds__(kThreads)
decide_kernel(const double* __restrict__ sums, const float* __restrict__ alpha,
              const float* __restrict__ beta, double tau, double delta, int L, int J,
              int* __restrict__ t_ctr, uint8_t* __restrict__ bstate, double* __restrict__ d_prev,
              uint8_t* __restrict__ blk_flags, uint8_t* __restrict__ lin_flags,
              uint8_t* __restrict__ mask_out, uint8_t* __restrict__ skip_out) {
  const int t = *t_ctr;
  for (int l = threadIdx.x; l < L; l += blockDim.x) {
    uint32_t computed = bstate[4 * l], nst = bstate[4 * l + 1], last = bstate[4 * l + 2];
    double gamma = 0.0;
    if (t >= 1) {
      const double* sl = sums + 4 * (int64_t)l;
      gamma = ratio0_dev(sl[0], sl[1]);
      if (computed) {
        last ^= 1u;
        nst = nst < 2u ? nst + 1u : 2u;
        d_prev[l] = nst >= 2u ? ratio0_dev(sqrt(sl[2]), sqrt(sl[3]))
                              : __longlong_as_double(0x7FF0000000000000ll);
      }
    }
    const bool skip = t >= 2 && computed && d_prev[l] < delta;
    for (int j = 0; j < J; ++j) {
      const int i = l * J + j;
      const double p = (double)alpha[i] * gamma + (double)beta[i];
      const uint32_t m = (t == 0 || p > tau) ? 1u : 0u;   // 1: INT8
      lin_flags[i] = (uint8_t)(skip ? 0u : (m ? kRouteInt8 : kRouteNvfp4));
      if (mask_out) mask_out[i] = (uint8_t)m;
    }
    blk_flags[l] = (uint8_t)(skip ? (last ? kBlkSkip1 : kBlkSkip0) : (last ? kBlkRun1 : kBlkRun0));
    if (skip_out) skip_out[l] = skip ? 1 : 0;
    bstate[4 * l] = skip ? 0 : 1;
    bstate[4 * l + 1] = (uint8_t)nst;
    bstate[4 * l + 2] = (uint8_t)last;
  }
  __syncthreads();
  if (threadIdx.x == 0) *t_ctr = t + 1;
}

hipError_t launch_decide(const double* sums, const float* alpha, const float* beta, double tau,
                         double delta, int L, int J, int* t_ctr, uint8_t* bstate, double* d_prev,
                         uint8_t* blk_flags, uint8_t* lin_flags, uint8_t* mask_out,
                         uint8_t* skip_out, hipStream_t stream) {
  hipLaunchKernelGGL(decide_kernel, dim3(1), dim3(kThreads), 0, stream, sums, alpha, beta, tau,
                     delta, L, J, t_ctr, bstate, d_prev, blk_flags, lin_flags, mask_out, skip_out);
  return hipGetLastError();
}

size_t reduce_ws_bytes(int64_t) { return (size_t)kRedBlocks * 4 * sizeof(double); }

hipError_t launch_tdc(int mode, const uint16_t* in, const uint16_t* b, const uint16_t* prev,
                      uint16_t* dst, int64_t n, double* sums, void* ws, hipStream_t stream,
                      uint32_t* amax_out, const RingRoute* route) {
  const Gate gt = current_gate();
  const RingRoute rt = route ? *route : RingRoute{nullptr, 0u, 0u, nullptr, nullptr, nullptr};
  const int64_t nvec = n / 8;
  int64_t nb = (nvec + kThreads * kUnroll - 1) / (kThreads * kUnroll);
  // with sums, at most kRedBlocks partial rows; without, one sweep (measured
  // faster for tdc_apply: 37.0 -> 35.4 us at 17776 x 1920)
  if (nb > (sums ? kRedBlocks : 65535)) nb = sums ? kRedBlocks : 65535;
  if (nb < 1) nb = 1;
  double* partial = static_cast<double*>(ws);
  const int want = sums != nullptr;
  const dim3 g((unsigned)nb), t(kThreads);
  if (mode == MODE_GAMMA)
    hipLaunchKernelGGL((tdc_kernel<MODE_GAMMA, false>), g, t, 0, stream, in, b, prev, dst, n,
                       partial, want, amax_out, rt, gt);
  else if (mode == MODE_UPDATE && prev)
    hipLaunchKernelGGL((tdc_kernel<MODE_UPDATE, true>), g, t, 0, stream, in, b, prev, dst, n,
                       partial, want, amax_out, rt, gt);
  else if (mode == MODE_UPDATE)
    hipLaunchKernelGGL((tdc_kernel<MODE_UPDATE, false>), g, t, 0, stream, in, b, prev, dst, n,
                       partial, want, amax_out, rt, gt);
  else if (mode == MODE_APPLY)
    hipLaunchKernelGGL((tdc_kernel<MODE_APPLY, false>), g, t, 0, stream, in, b, prev, dst, n,
                       partial, want, amax_out, rt, gt);
  else if (mode == MODE_RELERR)
    hipLaunchKernelGGL((tdc_kernel<MODE_RELERR, false>), g, t, 0, stream, in, b, prev, dst, n,
                       partial, want, amax_out, rt, gt);
  else if (mode == MODE_COS)
    hipLaunchKernelGGL((tdc_kernel<MODE_COS, false>), g, t, 0, stream, in, b, prev, dst, n,
                       partial, want, amax_out, rt, gt);
  else
    hipLaunchKernelGGL((tdc_kernel<MODE_APPLY_AMAX, false>), g, t, 0, stream, in, b, prev, dst,
                       n, partial, want, amax_out, rt, gt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !want) return e;
  const int ncols = mode == MODE_UPDATE ? 4 : mode == MODE_COS ? 3 : 2;
  hipLaunchKernelGGL(tdc_finalize_kernel, dim3(1), t, 0, stream, partial, (int)nb, ncols, sums, rt,
                     gt);
  return hipGetLastError();
}

}  // namespace qact
