// C ABI of libqact: argument checks, scratch layout and the host-side
// decisions of 6Bit-Diffusion (the DMPQ precision rule of the Fig. 3
// caption and the Temporal Delta Cache skip rule of the Fig. 2 caption).
// Every device entry point validates everything before it enqueues work.
#include <hip/hip_runtime.h>

#include <cmath>
#include <new>
#include <math.h>
#include <stdint.h>

#include "qact.h"
#include "qact_internal.h"

using namespace qact;

static_assert(kRouteNvfp4 == QA_ROUTE_NVFP4 && kRouteInt8 == QA_ROUTE_INT8, "gate bytes");
static_assert(kBlkRun0 == QA_BLK_RUN0 && kBlkRun1 == QA_BLK_RUN1 && kBlkSkip0 == QA_BLK_SKIP0 &&
                  kBlkSkip1 == QA_BLK_SKIP1,
              "gate bytes");

namespace {

// Size limits.  The GEMM kernels address a tile's operand rows (at most 256
// rows of at most K bytes) with 32-bit buffer offsets and mark a load to be
// skipped with an offset just below 2^31, so 256 K must stay below 2^31;
// one workgroup of 256 threads per tile or per 4 activation rows keeps every
// grid below 2^32 threads.
constexpr int64_t kMaxRows = (int64_t)1 << 26;  // M, N
constexpr int64_t kMaxK = (int64_t)1 << 23;
constexpr int64_t kMaxTiles = (int64_t)1 << 24; // 256 x 128 output tiles of one linear

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round256(size_t v) { return (v + 255) / 256 * 256; }

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return an && bn && x < y + bn && y < x + an;
}

int hip_status(hipError_t e) { return e == hipSuccess ? QA_OK : QA_EHIP; }

int check_mk(int64_t M, int64_t K) {
  if (M < 0 || K <= 0 || M >= kMaxRows || K >= kMaxK) return QA_ESHAPE;
  if (K % 16) return QA_ESHAPE;
  return QA_OK;
}

// a linear's N and its tile count; the NVFP4 call's per-tile scale copy
// is one workgroup per (256-row tile, K unit of 64) of both operands
int check_nk(int64_t M, int64_t N, int64_t K) {
  if (N < 0 || N >= kMaxRows) return QA_ESHAPE;
  if (((M + 255) / 256) * ((N + 127) / 128) > kMaxTiles) return QA_ESHAPE;
  if (((M + 255) / 256 + (N + 255) / 256) * ((K + 63) / 64) > kMaxTiles) return QA_ESHAPE;
  return QA_OK;
}

int check_out(qa_out out, qa_epi epi) {
  if (out != QA_OUT_BF16 && out != QA_OUT_F32) return QA_EINVAL;
  if (epi != QA_EPI_NONE && epi != QA_EPI_GELU_TANH) return QA_EINVAL;
  return QA_OK;
}

// the calling thread's gate (qa_set_gate), applied to every launch it makes
thread_local Gate g_gate = {nullptr, 0u};
// set only for the duration of a qlinear_*_amax call: the output |max| target
thread_local uint32_t* g_out_amax = nullptr;

}  // namespace

namespace qact {
Gate current_gate() { return g_gate; }
}  // namespace qact

extern "C" {

const char* qa_strerror(int status) {
  switch (status) {
    case QA_OK: return "ok";
    case QA_EINVAL: return "invalid argument (null pointer, bad enum or negative size)";
    case QA_ESHAPE: return "bad shape (K must be a positive multiple of 16 below 2^23; ld >= K; rows below 2^26)";
    case QA_EALIGN: return "misaligned buffer (16-byte alignment required)";
    case QA_EUNSUPPORTED: return "unsupported combination";
    case QA_EWORKSPACE: return "workspace too small";
    case QA_EHIP: return "HIP launch failed";
    case QA_EALIAS: return "an output overlaps an input";
    case QA_ESCRATCH: return "the call needs more than the library's static scratch (64 MiB)";
    default: return "unknown status";
  }
}

const char* qa_build_info(void) { return "libqact 0.1 gfx950"; }

// ------------------------------------------------------------ act_quant --

size_t act_quant_workspace(qa_fmt fmt, int64_t M, int64_t K) {
  if (fmt == QA_NVFP4) return nvfp4_quant_ws_bytes(M, K);
  return 0;
}

int act_quant(qa_fmt fmt, const uint16_t* x, int64_t M, int64_t K, int64_t ldx, void* q,
              void* scales, float* tscale, uint32_t flags, void* ws, size_t ws_bytes,
              hipStream_t stream) {
  if (fmt != QA_NVFP4 && fmt != QA_INT8) return QA_EINVAL;
  if (!x || !q || !scales) return QA_EINVAL;
  if (int s = check_mk(M, K)) return s;
  if (ldx < K || ldx % 8) return QA_ESHAPE;
  if (!aligned16(x) || !aligned16(q)) return QA_EALIGN;
  if (flags & ~(QA_TSCALE_GIVEN | QA_AMAX_GIVEN)) return QA_EINVAL;
  if ((flags & QA_TSCALE_GIVEN) && (flags & QA_AMAX_GIVEN)) return QA_EINVAL;
  const size_t xbytes = M ? (size_t)((M - 1) * ldx + K) * 2 : 0;
  if (fmt == QA_INT8) {
    if (tscale || flags) return QA_EINVAL;
    if (reinterpret_cast<uintptr_t>(scales) & 3u) return QA_EALIGN;
    if (overlap(x, xbytes, q, (size_t)(M * K)) || overlap(x, xbytes, scales, (size_t)M * 4))
      return QA_EALIAS;
    if (M == 0) return QA_OK;
    return hip_status(launch_int8_quant(x, M, K, ldx, static_cast<int8_t*>(q),
                                        static_cast<float*>(scales), stream));
  }
  if (!tscale) return QA_EINVAL;
  if (reinterpret_cast<uintptr_t>(tscale) & 3u) return QA_EALIGN;
  const bool given = (flags & QA_TSCALE_GIVEN) != 0;
  const bool amax_given = (flags & QA_AMAX_GIVEN) != 0;
  if (!given && ws_bytes < nvfp4_quant_ws_bytes(M, K)) return QA_EWORKSPACE;
  if (!given && !ws) return QA_EINVAL;
  if (amax_given && (reinterpret_cast<uintptr_t>(ws) & 3u)) return QA_EALIGN;
  if (overlap(x, xbytes, q, (size_t)(M * K / 2)) || overlap(x, xbytes, scales, (size_t)(M * K / 16)))
    return QA_EALIAS;
  if (M == 0) return QA_OK;
  return hip_status(launch_nvfp4_quant(x, M, K, ldx, static_cast<uint8_t*>(q),
                                       static_cast<uint8_t*>(scales), tscale, given, amax_given,
                                       ws, stream));
}

int act_quant_routed(const uint8_t* route, const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                     uint8_t* q4, uint8_t* s4, float* ts4, uint32_t flags4, void* ws4,
                     size_t ws4_bytes, int8_t* q8, float* s8, hipStream_t stream) {
  if (!route || !x || !q4 || !s4 || !ts4 || !q8 || !s8) return QA_EINVAL;
  if (int s = check_mk(M, K)) return s;
  if (ldx < K || ldx % 8) return QA_ESHAPE;
  if (!aligned16(x) || !aligned16(q4) || !aligned16(q8)) return QA_EALIGN;
  if ((reinterpret_cast<uintptr_t>(ts4) & 3u) || (reinterpret_cast<uintptr_t>(s8) & 3u))
    return QA_EALIGN;
  if (flags4 & ~(QA_TSCALE_GIVEN | QA_AMAX_GIVEN)) return QA_EINVAL;
  if ((flags4 & QA_TSCALE_GIVEN) && (flags4 & QA_AMAX_GIVEN)) return QA_EINVAL;
  const bool given = (flags4 & QA_TSCALE_GIVEN) != 0;
  const bool amax_given = (flags4 & QA_AMAX_GIVEN) != 0;
  if (!given && (!ws4 || ws4_bytes < nvfp4_quant_ws_bytes(M, K))) return QA_EWORKSPACE;
  if (!given && (reinterpret_cast<uintptr_t>(ws4) & 3u)) return QA_EALIGN;
  const size_t xbytes = M ? (size_t)((M - 1) * ldx + K) * 2 : 0;
  const void* outs[4] = {q4, s4, q8, s8};
  const size_t ob[4] = {(size_t)(M * K / 2), (size_t)(M * K / 16), (size_t)(M * K), (size_t)M * 4};
  for (int i = 0; i < 4; ++i) {
    if (overlap(x, xbytes, outs[i], ob[i])) return QA_EALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], ob[i], outs[j], ob[j])) return QA_EALIAS;
  }
  if (M == 0) return QA_OK;
  return hip_status(launch_act_quant_routed(route, x, M, K, ldx, q4, s4, ts4, given, amax_given,
                                            ws4, q8, s8, stream));
}

// -------------------------------------------------------------- qlinear --

// the INT8 linear takes the integer-MFMA kernel when given w8 and the fp16
// kernel otherwise: its workspace covers either
static size_t int8_ws_bytes(int64_t M, int64_t N, int64_t K) {
  const size_t a = int8_gemm_ws_bytes(M, N, K), b = int8_i8_gemm_ws_bytes(M, N, K);
  return a > b ? a : b;
}

size_t qlinear_workspace(qa_fmt fmt, int64_t M, int64_t N, int64_t K) {
  if (check_mk(M, K) || check_nk(M, N, K)) return 0;
  return fmt == QA_NVFP4 ? nvfp4_gemm_ws_bytes(M, N, K) : int8_ws_bytes(M, N, K);
}

static int check_linear(int64_t M, int64_t N, int64_t K, const void* y, int64_t ldy,
                        qa_out out, qa_epi epi) {
  if (int s = check_mk(M, K)) return s;
  if (int s = check_nk(M, N, K)) return s;
  if (int s = check_out(out, epi)) return s;
  if (!y) return QA_EINVAL;
  if (ldy < N) return QA_ESHAPE;
  if (reinterpret_cast<uintptr_t>(y) & (out == QA_OUT_F32 ? 3u : 1u)) return QA_EALIGN;
  return QA_OK;
}

int qlinear_nvfp4(const uint8_t* a_q, const uint8_t* a_s, const float* a_ts,
                  const uint8_t* w_q, const uint8_t* w_s, const float* w_ts, int64_t M,
                  int64_t N, int64_t K, const uint16_t* bias, void* y, int64_t ldy, qa_out out,
                  qa_epi epi, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!a_q || !a_s || !a_ts || !w_q || !w_s || !w_ts) return QA_EINVAL;
  if (int s = check_linear(M, N, K, y, ldy, out, epi)) return s;
  if (!aligned16(a_q) || !aligned16(w_q)) return QA_EALIGN;
  {
    const size_t need = nvfp4_gemm_ws_need(M, N, K, w_s);
    if (ws_bytes < need || (need && !ws)) return QA_EWORKSPACE;
  }
  if (!aligned16(ws)) return QA_EALIGN;
  const size_t ybytes = M && N ? (size_t)((M - 1) * ldy + N) * (out == QA_OUT_F32 ? 4 : 2) : 0;
  if (overlap(y, ybytes, a_q, (size_t)(M * K / 2)) || overlap(y, ybytes, w_q, (size_t)(N * K / 2)) ||
      overlap(y, ybytes, ws, ws_bytes))
    return QA_EALIAS;
  if (M == 0 || N == 0) return QA_OK;
  GemmOut o = {y, ldy, out == QA_OUT_F32, epi == QA_EPI_GELU_TANH, bias};
  o.y_amax = g_out_amax;
  return hip_status(launch_nvfp4_gemm(a_q, a_s, a_ts, w_q, w_s, w_ts, M, N, K, o, ws, ws_bytes, stream));
}

// the INT8 linear's weight operands: the digit planes w8 (integer MFMA;
// w_q and w_s unused) or the NVFP4 weight itself (fp16 MFMA)
static int check_int8_weight(const uint8_t* w_q, const uint8_t* w_s, const void* w8) {
  if (w8) return (reinterpret_cast<uintptr_t>(w8) & 255u) ? QA_EALIGN : QA_OK;
  if (!w_q || !w_s) return QA_EINVAL;
  return aligned16(w_q) ? QA_OK : QA_EALIGN;
}
static size_t int8_ws_need(int64_t M, int64_t N, int64_t K, const uint8_t* w_s, const void* w8) {
  return w8 ? 0 : int8_gemm_ws_need(M, N, K, w_s);
}
static size_t int8_weight_bytes(int64_t N, int64_t K, const void* w8) {
  return w8 ? int8_planes_bytes(N, K) : (size_t)(N * K / 2);
}
static hipError_t launch_int8(const int8_t* a_q, const float* a_s, const uint8_t* w_q,
                              const uint8_t* w_s, const float* w_ts, const void* w8, int64_t M,
                              int64_t N, int64_t K, const GemmOut& o, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  if (w8)
    return launch_int8_i8_gemm(a_q, a_s, w8, w_ts, M, N, K, o, ws, ws_bytes, nullptr, nullptr,
                               stream);
  return launch_int8_gemm(a_q, a_s, w_q, w_s, w_ts, M, N, K, o, ws, ws_bytes, stream);
}

extern "C++" {
namespace qact {
// the checks of qlinear_int8 that do not involve the workspace
int int8_linear_status(const int8_t* a_q, const float* a_s, const uint8_t* w_q,
                       const uint8_t* w_s, const float* w_ts, const void* w8, int64_t M,
                       int64_t N, int64_t K, const void* y, int64_t ldy, qa_out out, qa_epi epi) {
  if (!a_q || !a_s || !w_ts) return QA_EINVAL;
  if (int s = check_int8_weight(w_q, w_s, w8)) return s;
  if (int s = check_linear(M, N, K, y, ldy, out, epi)) return s;
  if (!aligned16(a_q)) return QA_EALIGN;
  return QA_OK;
}
}  // namespace qact
}  // extern "C++"

int qlinear_int8(const int8_t* a_q, const float* a_s, const uint8_t* w_q, const uint8_t* w_s,
                 const float* w_ts, const void* w8, int64_t M, int64_t N, int64_t K,
                 const uint16_t* bias, void* y, int64_t ldy, qa_out out, qa_epi epi, void* ws,
                 size_t ws_bytes, hipStream_t stream) {
  if (int s = int8_linear_status(a_q, a_s, w_q, w_s, w_ts, w8, M, N, K, y, ldy, out, epi))
    return s;
  {
    const size_t need = int8_ws_need(M, N, K, w_s, w8);
    if (ws_bytes < need || (need && !ws)) return QA_EWORKSPACE;
  }
  if (!aligned16(ws)) return QA_EALIGN;
  const size_t ybytes = M && N ? (size_t)((M - 1) * ldy + N) * (out == QA_OUT_F32 ? 4 : 2) : 0;
  if (overlap(y, ybytes, a_q, (size_t)(M * K)) ||
      overlap(y, ybytes, w8 ? w8 : w_q, int8_weight_bytes(N, K, w8)) ||
      overlap(y, ybytes, ws, ws_bytes))
    return QA_EALIAS;
  if (M == 0 || N == 0) return QA_OK;
  GemmOut o = {y, ldy, out == QA_OUT_F32, epi == QA_EPI_GELU_TANH, bias};
  o.y_amax = g_out_amax;
  return hip_status(launch_int8(a_q, a_s, w_q, w_s, w_ts, w8, M, N, K, o, ws, ws_bytes, stream));
}

size_t int8_weight_planes_bytes(int64_t N, int64_t K) {
  if (N < 0 || K <= 0 || K % 16) return 0;
  return int8_planes_bytes(N, K);
}

int int8_weight_planes(const uint8_t* w_q, const uint8_t* w_s, int64_t N, int64_t K, void* w8,
                       size_t w8_bytes, int64_t* irregular_rows, hipStream_t stream) {
  if (!w_q || !w_s || !w8) return QA_EINVAL;
  if (int s = check_mk(N, K)) return s;
  if (reinterpret_cast<uintptr_t>(w8) & 255u) return QA_EALIGN;
  if (w8_bytes < int8_planes_bytes(N, K)) return QA_EWORKSPACE;
  if (overlap(w8, w8_bytes, w_q, (size_t)(N * K / 2)) || overlap(w8, w8_bytes, w_s, (size_t)(N * K / 16)))
    return QA_EALIAS;
  if (irregular_rows) *irregular_rows = 0;
  if (N == 0) return QA_OK;
  int* cnt = int8_planes_counter(w8, N, K);
  if (hipMemsetAsync(cnt, 0, sizeof(int), stream) != hipSuccess) return QA_EHIP;
  if (launch_int8_planes(w_q, w_s, N, K, w8, cnt, stream) != hipSuccess) return QA_EHIP;
  int host = 0;
  if (hipMemcpyAsync(&host, cnt, sizeof(int), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return QA_EHIP;
  if (irregular_rows) *irregular_rows = host;
  return host ? QA_EUNSUPPORTED : QA_OK;
}

int qlinear_int8_acc(const int8_t* a_q, const void* w8, int64_t M, int64_t N, int64_t K,
                     int32_t* acc_hi, int32_t* acc_lo, hipStream_t stream) {
  if (!a_q || !w8 || !acc_hi || !acc_lo) return QA_EINVAL;
  if (int s = check_mk(M, K)) return s;
  if (int s = check_nk(M, N, K)) return s;
  if (K >= ((int64_t)1 << 17)) return QA_ESHAPE;
  if (!aligned16(a_q)) return QA_EALIGN;
  if ((reinterpret_cast<uintptr_t>(w8) & 255u) || (reinterpret_cast<uintptr_t>(acc_hi) & 3u) ||
      (reinterpret_cast<uintptr_t>(acc_lo) & 3u))
    return QA_EALIGN;
  const size_t ab = (size_t)(M * N) * 4;
  if (overlap(acc_hi, ab, acc_lo, ab) || overlap(acc_hi, ab, a_q, (size_t)(M * K)) ||
      overlap(acc_lo, ab, a_q, (size_t)(M * K)) ||
      overlap(acc_hi, ab, w8, int8_planes_bytes(N, K)) ||
      overlap(acc_lo, ab, w8, int8_planes_bytes(N, K)))
    return QA_EALIAS;
  if (M == 0 || N == 0) return QA_OK;
  GemmOut o = {nullptr, N, 0, 0, nullptr};
  return hip_status(launch_int8_i8_gemm(a_q, nullptr, w8, nullptr, M, N, K, o, nullptr, 0, acc_hi,
                                        acc_lo, stream));
}

// bf16 output and its |max| (the tensor amax of a following NVFP4
// act_quant, which then skips its amax pass: QA_AMAX_GIVEN)
static int check_amax_out(const GemmOut& o, const uint32_t* y_amax, const void* y, size_t ybytes,
                          const void* ws, size_t ws_bytes) {
  if (!y_amax) return QA_EINVAL;
  if (reinterpret_cast<uintptr_t>(y_amax) & 3u) return QA_EALIGN;
  if (!gemm_out_staged(o)) return QA_EUNSUPPORTED;
  if (overlap(y, ybytes, y_amax, kAmaxSlots * 4) || overlap(ws, ws_bytes, y_amax, kAmaxSlots * 4))
    return QA_EALIAS;
  return QA_OK;
}

int qlinear_nvfp4_amax(const uint8_t* a_q, const uint8_t* a_s, const float* a_ts,
                       const uint8_t* w_q, const uint8_t* w_s, const float* w_ts, int64_t M,
                       int64_t N, int64_t K, const uint16_t* bias, void* y, int64_t ldy,
                       qa_epi epi, uint32_t* y_amax, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  GemmOut o = {y, ldy, 0, epi == QA_EPI_GELU_TANH, bias};
  o.y_amax = y_amax;
  if (y && ldy >= N && M > 0 && N > 0)
    if (int s = check_amax_out(o, y_amax, y, (size_t)((M - 1) * ldy + N) * 2, ws, ws_bytes))
      return s;
  if (!y_amax) return QA_EINVAL;
  g_out_amax = y_amax;
  const int s = qlinear_nvfp4(a_q, a_s, a_ts, w_q, w_s, w_ts, M, N, K, bias, y, ldy, QA_OUT_BF16,
                              epi, ws, ws_bytes, stream);
  g_out_amax = nullptr;
  return s;
}

int qlinear_int8_amax(const int8_t* a_q, const float* a_s, const uint8_t* w_q,
                      const uint8_t* w_s, const float* w_ts, const void* w8, int64_t M,
                      int64_t N, int64_t K, const uint16_t* bias, void* y, int64_t ldy,
                      qa_epi epi, uint32_t* y_amax, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  GemmOut o = {y, ldy, 0, epi == QA_EPI_GELU_TANH, bias};
  o.y_amax = y_amax;
  if (y && ldy >= N && M > 0 && N > 0)
    if (int s = check_amax_out(o, y_amax, y, (size_t)((M - 1) * ldy + N) * 2, ws, ws_bytes))
      return s;
  if (!y_amax) return QA_EINVAL;
  g_out_amax = y_amax;
  const int s = qlinear_int8(a_q, a_s, w_q, w_s, w_ts, w8, M, N, K, bias, y, ldy, QA_OUT_BF16,
                             epi, ws, ws_bytes, stream);
  g_out_amax = nullptr;
  return s;
}

// ------------------------------------------------------- routed linear --

size_t qlinear_routed_workspace(int64_t M, int64_t N, int64_t K) {
  if (check_mk(M, K) || check_nk(M, N, K) || K % 16) return 0;
  const size_t a = nvfp4_gemm_ws_bytes(M, N, K), b = int8_i8_gemm_ws_bytes(M, N, K);
  return a > b ? a : b;
}

int qlinear_routed(const uint8_t* route, const uint8_t* a_q4, const uint8_t* a_s4,
                   const float* a_ts4, const int8_t* a_q8, const float* a_s8, const uint8_t* w_q,
                   const uint8_t* w_s, const float* w_ts, const void* w8, int64_t M, int64_t N,
                   int64_t K, const uint16_t* bias, uint16_t* y, int64_t ldy, qa_epi epi,
                   uint32_t* y_amax, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!route || !a_q4 || !a_s4 || !a_ts4 || !a_q8 || !a_s8 || !w_q || !w_s || !w_ts || !w8)
    return QA_EINVAL;
  if (int s = check_linear(M, N, K, y, ldy, QA_OUT_BF16, epi)) return s;
  if (K % 16) return QA_ESHAPE;
  if (!aligned16(a_q4) || !aligned16(a_q8) || !aligned16(w_q)) return QA_EALIGN;
  if (reinterpret_cast<uintptr_t>(w8) & 255u) return QA_EALIGN;
  GemmOut o = {y, ldy, 0, epi == QA_EPI_GELU_TANH, bias};
  o.y_amax = y_amax;
  if (!gemm_out_staged(o)) return QA_EUNSUPPORTED;
  {
    const size_t need = nvfp4_gemm_ws_need(M, N, K, w_s);
    if (ws_bytes < need || (need && !ws)) return QA_EWORKSPACE;
  }
  if (!aligned16(ws)) return QA_EALIGN;
  const size_t ybytes = M && N ? (size_t)((M - 1) * ldy + N) * 2 : 0;
  if (y_amax && M > 0 && N > 0)
    if (int s = check_amax_out(o, y_amax, y, ybytes, ws, ws_bytes)) return s;
  if (overlap(y, ybytes, a_q4, (size_t)(M * K / 2)) || overlap(y, ybytes, a_q8, (size_t)(M * K)) ||
      overlap(y, ybytes, w_q, (size_t)(N * K / 2)) ||
      overlap(y, ybytes, w8, int8_planes_bytes(N, K)) || overlap(y, ybytes, ws, ws_bytes) ||
      overlap(y, ybytes, route, 1))
    return QA_EALIAS;
  if (M == 0 || N == 0) return QA_OK;
  return hip_status(launch_routed_gemm(route, a_q4, a_s4, a_ts4, a_q8, a_s8, w_q, w_s, w_ts, w8,
                                       M, N, K, o, ws, ws_bytes, stream));
}

// NVFP4 output of the linear (activation quantization of its consumer,
// fused into the producing GEMM's epilogue)
static int check_qout(int64_t M, int64_t N, int64_t K, qa_epi epi, const float* y_ts,
                      const uint8_t* y_q, const uint8_t* y_s) {
  if (int s = check_mk(M, K)) return s;
  if (int s = check_nk(M, N, K)) return s;
  if (N % 16) return QA_ESHAPE;
  if (int s = check_out(QA_OUT_BF16, epi)) return s;
  if (!y_ts || !y_q || !y_s) return QA_EINVAL;
  if (!aligned16(y_q)) return QA_EALIGN;
  return QA_OK;
}

static bool qout_aliases(const uint8_t* y_q, const uint8_t* y_s, int64_t M, int64_t N,
                         const void* a, size_t an, const void* w, size_t wn, const void* ws,
                         size_t ws_bytes) {
  const size_t qb = (size_t)(M * N / 2), sb = (size_t)(M * N / 16);
  return overlap(y_q, qb, y_s, sb) || overlap(y_q, qb, a, an) || overlap(y_s, sb, a, an) ||
         overlap(y_q, qb, w, wn) || overlap(y_s, sb, w, wn) || overlap(y_q, qb, ws, ws_bytes) ||
         overlap(y_s, sb, ws, ws_bytes);
}

int qlinear_nvfp4_q(const uint8_t* a_q, const uint8_t* a_s, const float* a_ts,
                    const uint8_t* w_q, const uint8_t* w_s, const float* w_ts, int64_t M,
                    int64_t N, int64_t K, const uint16_t* bias, qa_epi epi, const float* y_ts,
                    uint8_t* y_q, uint8_t* y_s, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!a_q || !a_s || !a_ts || !w_q || !w_s || !w_ts) return QA_EINVAL;
  if (int s = check_qout(M, N, K, epi, y_ts, y_q, y_s)) return s;
  if (!aligned16(a_q) || !aligned16(w_q)) return QA_EALIGN;
  {
    const size_t need = nvfp4_gemm_ws_need(M, N, K, w_s);
    if (ws_bytes < need || (need && !ws)) return QA_EWORKSPACE;
  }
  if (!aligned16(ws)) return QA_EALIGN;
  if (qout_aliases(y_q, y_s, M, N, a_q, (size_t)(M * K / 2), w_q, (size_t)(N * K / 2), ws,
                   ws_bytes))
    return QA_EALIAS;
  if (M == 0 || N == 0) return QA_OK;
  GemmOut o = {nullptr, N, 0, epi == QA_EPI_GELU_TANH, bias, y_q, y_s, y_ts};
  return hip_status(launch_nvfp4_gemm(a_q, a_s, a_ts, w_q, w_s, w_ts, M, N, K, o, ws, ws_bytes, stream));
}

int qlinear_int8_q(const int8_t* a_q, const float* a_s, const uint8_t* w_q, const uint8_t* w_s,
                   const float* w_ts, const void* w8, int64_t M, int64_t N, int64_t K,
                   const uint16_t* bias, qa_epi epi, const float* y_ts, uint8_t* y_q,
                   uint8_t* y_s, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!a_q || !a_s || !w_ts) return QA_EINVAL;
  if (int s = check_int8_weight(w_q, w_s, w8)) return s;
  if (int s = check_qout(M, N, K, epi, y_ts, y_q, y_s)) return s;
  if (!aligned16(a_q)) return QA_EALIGN;
  {
    const size_t need = int8_ws_need(M, N, K, w_s, w8);
    if (ws_bytes < need || (need && !ws)) return QA_EWORKSPACE;
  }
  if (!aligned16(ws)) return QA_EALIGN;
  if (qout_aliases(y_q, y_s, M, N, a_q, (size_t)(M * K), w8 ? w8 : w_q,
                   int8_weight_bytes(N, K, w8), ws, ws_bytes))
    return QA_EALIAS;
  if (M == 0 || N == 0) return QA_OK;
  GemmOut o = {nullptr, N, 0, epi == QA_EPI_GELU_TANH, bias, y_q, y_s, y_ts};
  return hip_status(launch_int8(a_q, a_s, w_q, w_s, w_ts, w8, M, N, K, o, ws, ws_bytes, stream));
}

size_t qlinear_layer_workspace(qa_fmt fmt, int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K <= 0) return 0;
  if (fmt == QA_NVFP4)
    return round256((size_t)(M * K / 2)) + round256((size_t)(M * K / 16)) +
           round256(nvfp4_quant_ws_bytes(M, K)) + nvfp4_gemm_ws_bytes(M, N, K);
  return round256((size_t)(M * K)) + round256((size_t)M * 4) + int8_ws_bytes(M, N, K);
}

int qlinear(qa_fmt fmt, const uint16_t* x, int64_t ldx, float* x_ts, uint32_t flags,
            const uint8_t* w_q, const uint8_t* w_s, const float* w_ts, const void* w8, int64_t M,
            int64_t N, int64_t K, const uint16_t* bias, void* y, int64_t ldy, qa_out out,
            qa_epi epi, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (fmt != QA_NVFP4 && fmt != QA_INT8) return QA_EINVAL;
  if (fmt == QA_NVFP4 && w8) return QA_EINVAL;
  if (int s = fmt == QA_INT8 ? check_int8_weight(w_q, w_s, w8) : QA_OK) return s;
  if (!x || !ws) return QA_EINVAL;
  if (int s = check_linear(M, N, K, y, ldy, out, epi)) return s;
  if (ws_bytes < qlinear_layer_workspace(fmt, M, N, K)) return QA_EWORKSPACE;
  if (!aligned16(ws)) return QA_EALIGN;
  uint8_t* p = static_cast<uint8_t*>(ws);
  if (fmt == QA_NVFP4) {
    if (!x_ts || (flags & QA_AMAX_GIVEN)) return QA_EINVAL;   // its act_quant workspace is internal
    uint8_t* aq = p;
    p += round256((size_t)(M * K / 2));
    uint8_t* as = p;
    p += round256((size_t)(M * K / 16));
    void* qws = p;
    p += round256(nvfp4_quant_ws_bytes(M, K));
    const size_t gws = nvfp4_gemm_ws_bytes(M, N, K);
    int s = act_quant(QA_NVFP4, x, M, K, ldx, aq, as, x_ts, flags, qws,
                      nvfp4_quant_ws_bytes(M, K), stream);
    if (s) return s;
    return qlinear_nvfp4(aq, as, x_ts, w_q, w_s, w_ts, M, N, K, bias, y, ldy, out, epi, p, gws,
                         stream);
  }
  if (flags) return QA_EINVAL;
  int8_t* aq = reinterpret_cast<int8_t*>(p);
  p += round256((size_t)(M * K));
  float* as = reinterpret_cast<float*>(p);
  p += round256((size_t)M * 4);
  int s = act_quant(QA_INT8, x, M, K, ldx, aq, as, nullptr, 0, nullptr, 0, stream);
  if (s) return s;
  return qlinear_int8(aq, as, w_q, w_s, w_ts, w8, M, N, K, bias, y, ldy, out, epi, p,
                      int8_ws_bytes(M, N, K), stream);
}

// ---------------------------------------------------------------- Gamma --

size_t reduce_workspace(int64_t n) { return reduce_ws_bytes(n); }

static int check_stream(const void* a, const void* b, int64_t n, void* ws, size_t ws_bytes,
                        bool need_ws) {
  if (!a || !b) return QA_EINVAL;
  if (n < 0) return QA_EINVAL;
  if (!aligned16(a) || !aligned16(b)) return QA_EALIGN;
  if (need_ws && (!ws || ws_bytes < reduce_ws_bytes(n))) return QA_EWORKSPACE;
  if (need_ws && (reinterpret_cast<uintptr_t>(ws) & 7u)) return QA_EALIGN;
  return QA_OK;
}

int block_gamma(const uint16_t* in, const uint16_t* out, int64_t n, double* sums2, void* ws,
                size_t ws_bytes, hipStream_t stream) {
  if (!sums2) return QA_EINVAL;
  if (int s = check_stream(in, out, n, ws, ws_bytes, true)) return s;
  return hip_status(launch_tdc(0, in, out, nullptr, nullptr, n, sums2, ws, stream));
}

int tdc_update(const uint16_t* in, const uint16_t* out, const uint16_t* delta_prev,
               uint16_t* delta_new, int64_t n, double* sums4, void* ws, size_t ws_bytes,
               hipStream_t stream) {
  if (!sums4 || !delta_new) return QA_EINVAL;
  if (int s = check_stream(in, out, n, ws, ws_bytes, true)) return s;
  if (!aligned16(delta_new) || (delta_prev && !aligned16(delta_prev))) return QA_EALIGN;
  const size_t b = (size_t)n * 2;
  if (overlap(delta_new, b, in, b) || overlap(delta_new, b, out, b) ||
      (delta_prev && overlap(delta_new, b, delta_prev, b)) || overlap(delta_new, b, ws, ws_bytes))
    return QA_EALIAS;
  return hip_status(launch_tdc(1, in, out, delta_prev, delta_new, n, sums4, ws, stream));
}

int tdc_apply(const uint16_t* in, const uint16_t* delta, uint16_t* out, int64_t n,
              double* sums2, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!out) return QA_EINVAL;
  if (int s = check_stream(in, delta, n, ws, ws_bytes, sums2 != nullptr)) return s;
  if (!aligned16(out)) return QA_EALIGN;
  const size_t b = (size_t)n * 2;
  if (overlap(out, b, delta, b)) return QA_EALIAS;
  if (out != in && overlap(out, b, in, b)) return QA_EALIAS;
  return hip_status(launch_tdc(2, in, delta, nullptr, out, n, sums2, ws, stream));
}

int tdc_apply_amax(const uint16_t* in, const uint16_t* delta, uint16_t* out, int64_t n,
                   double* sums2, uint32_t* out_amax, void* ws, size_t ws_bytes,
                   hipStream_t stream) {
  if (!out || !out_amax) return QA_EINVAL;
  if (int s = check_stream(in, delta, n, ws, ws_bytes, sums2 != nullptr)) return s;
  if (!aligned16(out)) return QA_EALIGN;
  if (reinterpret_cast<uintptr_t>(out_amax) & 3u) return QA_EALIGN;
  const size_t b = (size_t)n * 2;
  if (overlap(out, b, delta, b)) return QA_EALIAS;
  if (out != in && overlap(out, b, in, b)) return QA_EALIAS;
  const size_t ab = kAmaxSlots * 4;
  if (overlap(out_amax, ab, out, b) || overlap(out_amax, ab, in, b) ||
      overlap(out_amax, ab, delta, b) || overlap(out_amax, ab, ws, ws_bytes) ||
      (sums2 && overlap(out_amax, ab, sums2, 16)))
    return QA_EALIAS;
  return hip_status(launch_tdc(5, in, delta, nullptr, out, n, sums2, ws, stream, out_amax));
}

// the Delta ring of one block: two bf16 [n] slots, each 16-byte aligned,
// overlapping neither each other nor the other buffers of the call
static int check_ring(const uint8_t* blk, const uint16_t* ring0, const uint16_t* ring1,
                      const void* in, const void* other, int64_t n, const void* ws,
                      size_t ws_bytes) {
  if (!blk || !ring0 || !ring1) return QA_EINVAL;
  if (!aligned16(ring0) || !aligned16(ring1)) return QA_EALIGN;
  const size_t b = (size_t)n * 2;
  if (overlap(ring0, b, ring1, b)) return QA_EALIAS;
  for (const void* r : {static_cast<const void*>(ring0), static_cast<const void*>(ring1)})
    if (overlap(r, b, in, b) || overlap(r, b, other, b) || overlap(r, b, ws, ws_bytes))
      return QA_EALIAS;
  return QA_OK;
}

int tdc_update_ring(const uint8_t* blk, const uint16_t* in, const uint16_t* out, uint16_t* ring0,
                    uint16_t* ring1, int64_t n, double* sums4, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  if (!sums4) return QA_EINVAL;
  if (int s = check_stream(in, out, n, ws, ws_bytes, true)) return s;
  if (int s = check_ring(blk, ring0, ring1, in, out, n, ws, ws_bytes)) return s;
  const RingRoute rt = {blk, kBlkRun0, kBlkRun1, out, ring1, ring0};
  return hip_status(launch_tdc(1, in, out, ring0, ring1, n, sums4, ws, stream, nullptr, &rt));
}

int tdc_apply_ring(const uint8_t* blk, const uint16_t* in, const uint16_t* ring0,
                   const uint16_t* ring1, uint16_t* out, int64_t n, double* sums2,
                   uint32_t* out_amax, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!out) return QA_EINVAL;
  if (int s = check_stream(in, ring0, n, ws, ws_bytes, sums2 != nullptr)) return s;
  if (!aligned16(out)) return QA_EALIGN;
  const size_t b = (size_t)n * 2;
  if (out != in && overlap(out, b, in, b)) return QA_EALIAS;
  if (int s = check_ring(blk, ring0, ring1, in, out, n, ws, ws_bytes)) return s;
  if (out_amax) {
    if (reinterpret_cast<uintptr_t>(out_amax) & 3u) return QA_EALIGN;
    const size_t ab = kAmaxSlots * 4;
    if (overlap(out_amax, ab, out, b) || overlap(out_amax, ab, in, b) ||
        overlap(out_amax, ab, ring0, b) || overlap(out_amax, ab, ring1, b) ||
        overlap(out_amax, ab, ws, ws_bytes) || (sums2 && overlap(out_amax, ab, sums2, 16)))
      return QA_EALIAS;
  }
  const RingRoute rt = {blk, kBlkSkip0, kBlkSkip1, ring1, nullptr, out};
  return hip_status(launch_tdc(out_amax ? 5 : 2, in, ring0, nullptr, out, n, sums2, ws, stream,
                               out_amax, &rt));
}

int rel_err(const uint16_t* y_q, const uint16_t* y_ref, int64_t n, double* sums2, void* ws,
            size_t ws_bytes, hipStream_t stream) {
  if (!sums2) return QA_EINVAL;
  if (int s = check_stream(y_q, y_ref, n, ws, ws_bytes, true)) return s;
  if (overlap(sums2, 16, ws, ws_bytes)) return QA_EALIAS;
  return hip_status(launch_tdc(3, y_q, y_ref, nullptr, nullptr, n, sums2, ws, stream));
}

int delta_cosine(const uint16_t* d_new, const uint16_t* d_prev, int64_t n, double* sums3,
                 void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!sums3) return QA_EINVAL;
  if (int s = check_stream(d_new, d_prev, n, ws, ws_bytes, true)) return s;
  if (overlap(sums3, 24, ws, ws_bytes)) return QA_EALIAS;
  return hip_status(launch_tdc(4, d_new, d_prev, nullptr, nullptr, n, sums3, ws, stream));
}

int qa_test_convert(int op, uint32_t first, int64_t count, void* out, hipStream_t stream) {
  if (op < 0 || op > 2 || count < 0 || !out) return QA_EINVAL;
  if ((uint64_t)first + (uint64_t)count > ((uint64_t)1 << 32)) return QA_EINVAL;
  if (op == 2 && (reinterpret_cast<uintptr_t>(out) & 1u)) return QA_EALIGN;
  // the E4M3 scale encoder is defined on non-negative finite floats
  if (op == 1 && count && (uint64_t)first + (uint64_t)count - 1 > 0x7F7FFFFFu) return QA_EINVAL;
  if (count == 0) return QA_OK;
  return hip_status(launch_convert(op, first, count, out, stream));
}

int qa_test_stage_ab(int design, int iters, int blocks, const uint32_t* in, float* out,
                     hipStream_t stream) {
  if (design < 0 || design > 2 || iters < 0 || blocks < 1 || blocks > 65535 || !in || !out)
    return QA_EINVAL;
  if ((reinterpret_cast<uintptr_t>(in) & 3u) || (reinterpret_cast<uintptr_t>(out) & 3u))
    return QA_EALIGN;
  return hip_status(launch_stage_ab(design, iters, blocks, in, out, stream));
}

int qa_set_gemm_events(hipEvent_t before, hipEvent_t after) {
  if ((before == nullptr) != (after == nullptr)) return QA_EINVAL;
  set_gemm_events(before, after);
  set_i8_gemm_events(before, after);
  return QA_OK;
}

// ------------------------------------------------------ host decisions --

static double ratio0(double num, double den) {
  if (den == 0.0) return num == 0.0 ? 0.0 : INFINITY;
  return num / den;
}

// ------------------------------------------------ device-side step control --

int qa_set_gate(const uint8_t* flags, uint32_t bits) {
  if (flags && bits == 0) return QA_EINVAL;
  g_gate = Gate{flags, flags ? bits : 0u};
  return QA_OK;
}

int qa_decide_step(const double* sums, const float* alpha, const float* beta, double tau,
                   double delta, int L, int J, int* t_ctr, uint8_t* bstate, double* d_prev,
                   uint8_t* blk_flags, uint8_t* lin_flags, uint8_t* mask_out, uint8_t* skip_out,
                   hipStream_t stream) {
  if (L <= 0 || J <= 0 || L * J > (1 << 24)) return QA_ESHAPE;
  if (!sums || !alpha || !beta || !t_ctr || !bstate || !d_prev || !blk_flags || !lin_flags)
    return QA_EINVAL;
  if ((reinterpret_cast<uintptr_t>(sums) & 7u) || (reinterpret_cast<uintptr_t>(d_prev) & 7u) ||
      (reinterpret_cast<uintptr_t>(alpha) & 3u) || (reinterpret_cast<uintptr_t>(beta) & 3u) ||
      (reinterpret_cast<uintptr_t>(t_ctr) & 3u) || (reinterpret_cast<uintptr_t>(bstate) & 3u))
    return QA_EALIGN;
  return hip_status(launch_decide(sums, alpha, beta, tau, delta, L, J, t_ctr, bstate, d_prev,
                                  blk_flags, lin_flags, mask_out, skip_out, stream));
}

double qa_gamma_from_sums(const double* sums2) {
  return sums2 ? ratio0(sums2[0], sums2[1]) : NAN;
}

double qa_rel_l2_from_sums(const double* sums4) {
  return sums4 ? ratio0(sqrt(sums4[2]), sqrt(sums4[3])) : NAN;
}

double qa_cosine_from_sums(const double* sums3) {
  if (!sums3) return NAN;
  const double den = sqrt(sums3[1]) * sqrt(sums3[2]);
  return den == 0.0 ? 0.0 : sums3[0] / den;
}

int tdc_decide_cos(int t, const double* cos_prev, const uint8_t* computed_prev, int L,
                   double threshold, uint8_t* skip) {
  if (L < 0 || !skip || (L && t >= 2 && (!cos_prev || !computed_prev))) return QA_EINVAL;
  for (int l = 0; l < L; ++l)
    skip[l] = (uint8_t)(t >= 2 && computed_prev[l] && cos_prev[l] > threshold);
  return QA_OK;
}

double qa_rel_err_from_sums(const double* sums2) {
  return sums2 ? ratio0(sqrt(sums2[0]), sqrt(sums2[1])) : NAN;
}

// Least-squares line y = alpha x + beta through n points (two passes:
// means, then centred sums, in long double).  Fewer than two distinct x:
// alpha = 0 and beta = mean of y (0 without points).
static void fit_line(const long double* x, const long double* y, int n, float* alpha,
                     float* beta) {
  if (n == 0) {
    *alpha = 0.0f;
    *beta = 0.0f;
    return;
  }
  long double mx = 0, my = 0;
  for (int i = 0; i < n; ++i) {
    mx += x[i];
    my += y[i];
  }
  mx /= n;
  my /= n;
  long double sxx = 0, sxy = 0;
  for (int i = 0; i < n; ++i) {
    sxx += (x[i] - mx) * (x[i] - mx);
    sxy += (x[i] - mx) * (y[i] - my);
  }
  const long double a = sxx > 0 ? sxy / sxx : 0.0L;
  *alpha = (float)a;
  *beta = (float)(my - a * mx);
}

int dmpq_fit(const double* gamma, const double* erel, int T, int L, int J, float* alpha,
             float* beta) {
  if (T < 0 || L < 0 || J <= 0 || !alpha || !beta) return QA_EINVAL;
  if ((T > 0 && L > 0) && (!gamma || !erel)) return QA_EINVAL;
  const int np = T > 1 ? T - 1 : 0;
  long double* x = np ? new (std::nothrow) long double[2 * (size_t)np] : nullptr;
  if (np && !x) return QA_EINVAL;
  long double* y = x ? x + np : nullptr;
  for (int l = 0; l < L; ++l)
    for (int j = 0; j < J; ++j) {
      int n = 0;
      for (int t = 1; t < T; ++t) {
        const double g = gamma[(size_t)(t - 1) * L + l];
        const double e = erel[(size_t)t * L * J + (size_t)l * J + j];
        if (!std::isfinite(g) || !std::isfinite(e)) continue;
        x[n] = g;
        y[n] = e;
        ++n;
      }
      fit_line(x, y, n, &alpha[(size_t)l * J + j], &beta[(size_t)l * J + j]);
    }
  delete[] x;
  return QA_OK;
}

int dmpq_mask(const double* gamma_prev, int L, int J, const float* alpha, const float* beta,
              double tau, uint8_t* mask) {
  if (L < 0 || J <= 0 || !mask) return QA_EINVAL;
  if (gamma_prev && (!alpha || !beta)) return QA_EINVAL;
  for (int l = 0; l < L; ++l)
    for (int j = 0; j < J; ++j) {
      const int i = l * J + j;
      if (!gamma_prev) {
        mask[i] = 1;
        continue;
      }
      const double p = (double)alpha[i] * gamma_prev[l] + (double)beta[i];
      mask[i] = p > tau ? 1 : 0;
    }
  return QA_OK;
}

int tdc_decide(int t, const double* d_prev, const uint8_t* computed_prev, int L, double delta,
               uint8_t* skip) {
  if (L < 0 || !skip || (L && t >= 2 && (!d_prev || !computed_prev))) return QA_EINVAL;
  for (int l = 0; l < L; ++l)
    skip[l] = (t >= 2 && computed_prev[l] && d_prev[l] < delta) ? 1 : 0;
  return QA_OK;
}

}  // extern "C"
