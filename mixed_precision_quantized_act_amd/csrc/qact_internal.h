// Internal launch entry points of libqact (host side).  Each returns the
// HIP error of its launches; argument checking is done by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qact.h"

namespace qact {

// Device-side gate of a call: every kernel of the call reads the byte
// *flags on the device and does nothing unless (*flags & bits) != 0 and
// (*flags & veto) == 0, and, when flags2 is set, (*flags2 & bits2) != 0.
// flags == nullptr: no gate.  Set per host thread through qa_set_gate
// (veto 0, no flags2); a routed call builds its own per format, with the
// thread's gate as the second byte.
struct Gate {
  const uint8_t* flags;
  uint32_t bits;
  uint32_t veto = 0u;
  const uint8_t* flags2 = nullptr;
  uint32_t bits2 = 0u;
};
Gate current_gate();

// A producer-computed tensor amax (qlinear_*_amax, tdc_apply_amax) is kept
// as kAmaxSlots partial maxima (float bits, non-negative: they order as
// integers), workgroup b max-combining into slot b % kAmaxSlots so that the
// atomics spread over many addresses; act_quant's workspace holds exactly
// these slots, and QA_AMAX_GIVEN folds them as it folds its own amax pass.
constexpr int kAmaxSlots = 1024;

// Gate bits written by the device-side decisions (launch_decide): per
// linear, which activation format runs (none when its block is skipped);
// per block, the compute path with ring slot `last` = 0 or 1 (the Delta
// cache reads slot last and writes slot last ^ 1) or the skip path reading
// slot last.
enum : uint32_t {
  kRouteNvfp4 = 1u, kRouteInt8 = 2u,
  kBlkRun0 = 1u, kBlkRun1 = 2u, kBlkSkip0 = 4u, kBlkSkip1 = 8u
};
hipError_t launch_decide(const double* sums, const float* alpha, const float* beta, double tau,
                         double delta, int L, int J, int* t_ctr, uint8_t* bstate, double* d_prev,
                         uint8_t* blk_flags, uint8_t* lin_flags, uint8_t* mask_out,
                         uint8_t* skip_out, hipStream_t stream);

// ---- activation quantization (act_quant.hip)
size_t nvfp4_quant_ws_bytes(int64_t M, int64_t K);
// amax_given: the tensor |max| is the float at ws[0] (no amax pass)
hipError_t launch_nvfp4_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                              uint8_t* q, uint8_t* scales, float* tscale, bool given,
                              bool amax_given, void* ws, hipStream_t stream);
hipError_t launch_int8_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                             float* scale, hipStream_t stream);
// both formats in one launch, the format read from the device byte *route
// (kRouteNvfp4 / kRouteInt8; the tensor-max pass, when needed, is a second
// launch that runs only for kRouteNvfp4)
hipError_t launch_act_quant_routed(const uint8_t* route, const uint16_t* x, int64_t M, int64_t K,
                                   int64_t ldx, uint8_t* q4, uint8_t* s4, float* ts4, bool given,
                                   bool amax_given, void* ws, int8_t* q8, float* s8,
                                   hipStream_t stream);

// ---- test-only element conversions (convert_check.hip)
hipError_t launch_convert(int op, uint32_t first, int64_t count, void* out, hipStream_t stream);

// ---- test/benchmark-only compute stages of three NVFP4 GEMM designs (stage_ab.hip)
hipError_t launch_stage_ab(int design, int iters, int blocks, const uint32_t* in, float* out,
                           hipStream_t stream);

// ---- profiling hook: events recorded around each main GEMM kernel
void set_gemm_events(hipEvent_t before, hipEvent_t after);

// ---- quantized GEMMs (qgemm.hip)
struct GemmOut {
  void* y;
  int64_t ldy;
  int out_f32;            // 0: bf16, 1: f32
  int gelu;               // 0: none, 1: GELU-tanh
  const uint16_t* bias;   // bf16 [N] or null
  uint8_t* yq = nullptr;  // non-null: NVFP4 output (codes [M][N/2], scales [M][N/16])
  uint8_t* ys = nullptr;  //   quantized with the given tensor scale *y_ts instead of y
  const float* y_ts = nullptr;
  uint32_t* y_amax = nullptr;  // bf16 staged output: atomic max of its |values| (float bits)
};
// true when the output takes the bf16 staged epilogue (the one that can
// also produce the output's |max|)
bool gemm_out_staged(const GemmOut& o);
size_t nvfp4_gemm_ws_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_nvfp4_gemm(const uint8_t* a_q, const uint8_t* a_s, const float* a_ts,
                             const uint8_t* w_q, const uint8_t* w_s, const float* w_ts,
                             int64_t M, int64_t N, int64_t K, const GemmOut& o, void* ws,
                             size_t ws_bytes, hipStream_t stream);
size_t int8_gemm_ws_bytes(int64_t M, int64_t N, int64_t K);
// the least workspace a call accepts (INT8 reads the weight scales in
// place when K is a multiple of 64 and w_s is 4-byte aligned); with the
// full *_gemm_ws_bytes the last round of tiles is split along K
size_t nvfp4_gemm_ws_need(int64_t M, int64_t N, int64_t K, const void* w_s);
size_t int8_gemm_ws_need(int64_t M, int64_t N, int64_t K, const void* w_s);
hipError_t launch_int8_gemm(const int8_t* a_q, const float* a_s, const uint8_t* w_q,
                            const uint8_t* w_s, const float* w_ts, int64_t M, int64_t N,
                            int64_t K, const GemmOut& o, void* ws, size_t ws_bytes,
                            hipStream_t stream);

// ---- INT8 path on integer MFMA (qgemm_i8.hip): the NVFP4 weight as two
// int8 digit planes made once at set-up, and the GEMM with exact int32 sums
size_t int8_planes_bytes(int64_t N, int64_t K);
// device int32 counter of the irregular rows inside the planes buffer
int* int8_planes_counter(void* w8, int64_t N, int64_t K);
hipError_t launch_int8_planes(const uint8_t* w_q, const uint8_t* w_s, int64_t N, int64_t K,
                              void* w8, int* irregular_dev, hipStream_t stream);
size_t int8_i8_gemm_ws_bytes(int64_t M, int64_t N, int64_t K);
// acc_hi/acc_lo non-null: store the int32 sums H and L [M][N] instead of y
hipError_t launch_int8_i8_gemm(const int8_t* a_q, const float* a_s, const void* w8,
                               const float* w_ts, int64_t M, int64_t N, int64_t K,
                               const GemmOut& o, void* ws, size_t ws_bytes, int32_t* acc_hi,
                               int32_t* acc_lo, hipStream_t stream);
void set_i8_gemm_events(hipEvent_t before, hipEvent_t after);
// the linear in the format the device byte *route selects (kRouteNvfp4:
// the NVFP4 operands; kRouteInt8: the INT8 operands with w8), whole tiles
// in one launch; bf16 staged outputs only (the ABI checks)
hipError_t launch_routed_gemm(const uint8_t* route, const uint8_t* a_q4, const uint8_t* a_s4,
                              const float* a_ts4, const int8_t* a_q8, const float* a_s8,
                              const uint8_t* w_q, const uint8_t* w_s, const float* w_ts,
                              const void* w8, int64_t M, int64_t N, int64_t K, const GemmOut& o,
                              void* ws, size_t ws_bytes, hipStream_t stream);

// ---- Gamma / Temporal Delta Cache (tdc.hip)
// qlinear_int8's argument checks other than those of its workspace
int int8_linear_status(const int8_t* a_q, const float* a_s, const uint8_t* w_q,
                       const uint8_t* w_s, const float* w_ts, const void* w8, int64_t M,
                       int64_t N, int64_t K, const void* y, int64_t ldy, qa_out out, qa_epi epi);

size_t reduce_ws_bytes(int64_t n);
// Operands chosen on the device from the byte *sel: the call's own (b,
// delta_prev, dst) when (*sel & bits_a), these when (*sel & bits_b), no work
// otherwise (the Delta ring slot of a block, from qa_decide_step).
struct RingRoute {
  const uint8_t* sel;
  uint32_t bits_a, bits_b;
  const uint16_t* b_alt;
  const uint16_t* prev_alt;
  uint16_t* dst_alt;
};
// mode 0: block_gamma, 1: tdc_update, 2: tdc_apply, 3: rel_err, 4: delta_cosine,
// 5: tdc_apply that also max-combines |out| into *amax_out
hipError_t launch_tdc(int mode, const uint16_t* in, const uint16_t* b, const uint16_t* delta_prev,
                      uint16_t* dst, int64_t n, double* sums, void* ws, hipStream_t stream,
                      uint32_t* amax_out = nullptr, const RingRoute* route = nullptr);

}  // namespace qact
