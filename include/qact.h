/*
 * qact.h - C ABI of the MI355X (gfx950) quantized-linear library libqact.so.
 *
 * The operations are those of 6Bit-Diffusion (arXiv 2603.18742): each
 * internal linear layer of a video-DiT block quantizes its activations at
 * inference time to NVFP4 or INT8, chosen per layer (abstract; Fig. 2
 * caption), and multiplies them with 4-bit NVFP4 weights (Table 2, "W4");
 * the choice comes from a linear predictor on the block's input/output
 * relative L1 distance Gamma at the preceding timestep (Fig. 3 caption);
 * the Temporal Delta Cache stores a block's residual Delta = out - in and
 * reuses it when the two preceding Deltas agree (abstract; Fig. 2 and
 * Fig. 4 captions).
 *
 * Formats (the pages name NVFP4 and INT8 and print no rounding rules; the
 * readings below hold throughout):
 *   NVFP4  codes  u8 [rows][K/2]: E2M1 element 2j in the low nibble, 2j+1
 *                 in the high nibble; bit 3 of a nibble is the sign.
 *          scales u8 [rows][K/16]: one OCP E4M3FN scale per 16 elements.
 *          tscale f32 scalar: the tensor scale s_T.
 *          Encode (float32, in order; recip(y) = y == 0 ? 0 : 1/y):
 *            s_T = amax/2688; g = recip(6 s_T); enc = E4M3(amax_group * g);
 *            inv = recip(E4M3value(enc) * s_T); code = E2M1(x * inv).
 *          E2M1 and E4M3 round to nearest, ties to the even code, and
 *          saturate (6 and 448); a negative x that rounds to 0 keeps its
 *          sign bit.  K must be a multiple of 16.
 *   INT8   q i8 [rows][K], scale f32 [rows], per token (row), symmetric:
 *          s = amax_row/127, inv = recip(s), q = clamp(rint(x*inv), +-127).
 *   bf16   uint16 bit patterns; tensors are row-major.
 *
 * Conventions for every device entry point:
 *   - tensor pointers are DEVICE pointers owned by the caller; the library
 *     allocates nothing; ``ws``/``ws_bytes`` is caller-owned device scratch
 *     of at least the size the matching *_workspace() call returns;
 *   - arguments are validated on the host first; when a call returns an
 *     error, nothing was enqueued;
 *   - work is enqueued on ``stream`` and the call returns without waiting;
 *     device faults surface at the caller's next synchronisation;
 *   - vector buffers must be 16-byte aligned; row strides are in elements;
 *   - results are deterministic: no floating-point atomics anywhere (the
 *     producer-side tensor amax uses integer atomic maxima, whose result
 *     does not depend on their order);
 *   - calls on different streams must not share output or scratch buffers;
 *   - a gate set with qa_set_gate applies to every later call of the same
 *     host thread until cleared.
 */
#ifndef QACT_H
#define QACT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QA_OK = 0,
  QA_EINVAL = -1,        /* null pointer, bad enum, negative size         */
  QA_ESHAPE = -2,        /* K % 16 != 0, ld < K, sizes beyond the limits  */
  QA_EALIGN = -3,        /* a vector buffer is not 16-byte aligned        */
  QA_EUNSUPPORTED = -4,  /* a valid but unimplemented combination         */
  QA_EWORKSPACE = -5,    /* ws_bytes below the required size              */
  QA_EHIP = -6,          /* a HIP launch failed                           */
  QA_EALIAS = -7,        /* an output overlaps an input it must not alias */
  QA_ESCRATCH = -8       /* the call needs more than the library's static
                            scratch (QA_NOALLOC_SCRATCH_BYTES)            */
} qa_status;

typedef enum { QA_NVFP4 = 0, QA_INT8 = 1 } qa_fmt;
typedef enum { QA_OUT_BF16 = 0, QA_OUT_F32 = 1 } qa_out;
typedef enum { QA_EPI_NONE = 0, QA_EPI_GELU_TANH = 1 } qa_epi;

/* NVFP4 only: *tscale is an input (a calibrated or producer-computed s_T)
 * and the tensor amax pass is skipped. */
#define QA_TSCALE_GIVEN 1u
/* NVFP4 only: the tensor |max| amax_T is already in ws, as the 1024
 * partial maxima (float bits) that qlinear_nvfp4_amax, qlinear_int8_amax
 * or tdc_apply_amax leave there (the whole act_quant workspace, 4 KB); the
 * amax pass is skipped, amax_T is their maximum and s_T = amax_T / 2688 is
 * written to *tscale -- the same s_T, bit for bit, as without the flag. */
#define QA_AMAX_GIVEN 2u

/* Human-readable name of a status code (static storage). */
const char* qa_strerror(int status);

/* Library version and the GPU architecture the kernels were built for. */
const char* qa_build_info(void);

/* ------------------------------------------------------------------------
 * Activation (and weight) quantization.  Abstract: activations are
 * quantized on the fly to NVFP4 or INT8; Fig. 2 caption: the bits are per
 * linear layer.  Weights use the same NVFP4 call once at set-up.
 *
 * x      bf16 [M][ldx] (first K columns used), 16-byte aligned, ldx % 8 == 0
 * q      NVFP4: u8 [M][K/2];  INT8: i8 [M][K]
 * scales NVFP4: u8 [M][K/16];  INT8: f32 [M]
 * tscale NVFP4: f32 device scalar, output (or input with QA_TSCALE_GIVEN);
 *        QA_AMAX_GIVEN takes amax_T from ws (see above), needs ws 4-aligned;
 *        INT8: must be NULL
 * 0 <= M < 2^26 (M == 0 enqueues nothing), 0 < K < 2^23, K % 16 == 0 for
 * NVFP4 (QA_ESHAPE otherwise).
 * ------------------------------------------------------------------------ */
size_t act_quant_workspace(qa_fmt fmt, int64_t M, int64_t K);
int act_quant(qa_fmt fmt, const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
              void* q, void* scales, float* tscale, uint32_t flags,
              void* ws, size_t ws_bytes, hipStream_t stream);

/* act_quant_routed: act_quant in the format that the device byte *route
 * selects, in one launch, for a timestep enqueued (or captured in a graph)
 * before its decisions are known (6Bit-Diffusion, Fig. 2 caption: each
 * linear's activation format is chosen per timestep).  *route is a linear
 * gate byte of qa_decide_step: (*route & 1) NVFP4 into (q4, s4, *ts4) with
 * flags4 and ws4 as for act_quant (QA_TSCALE_GIVEN or QA_AMAX_GIVEN: the
 * encoder alone; neither: a tensor-max launch first, which also runs only
 * for NVFP4); otherwise (*route & 2) INT8 into (q8, s8); 0: nothing.  The outputs of
 * the format not chosen are left as they were.  Arguments as for act_quant
 * (both formats' buffers required); the outputs overlap neither each other
 * nor x. */
int act_quant_routed(const uint8_t* route, const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                     uint8_t* q4, uint8_t* s4, float* ts4, uint32_t flags4, void* ws4,
                     size_t ws4_bytes, int8_t* q8, float* s8, hipStream_t stream);

/* ------------------------------------------------------------------------
 * qlinear_nvfp4_q / qlinear_int8_q: the same linears with the output
 * quantized to NVFP4 in the GEMM epilogue, for a consumer linear that
 * takes NVFP4 activations (6Bit-Diffusion, Fig. 2 caption: the activations
 * of each internal linear are quantized; fusing that quantization into the
 * producer removes the bf16 round trip of the intermediate).  Every output
 * value (scale, bias, GELU as for qlinear_*) is rounded to bf16 and then
 * encoded exactly as act_quant NVFP4 with QA_TSCALE_GIVEN and tensor scale
 * *y_ts (device float32, read by the kernel): y_q u8 [M][N/2] codes (low
 * nibble first), y_s u8 [M][N/16] E4M3 scales.  The tensor scale is an
 * input because the whole output's |max| is not known while the output
 * tiles are produced.  Requires N % 16 == 0; y_q 16-byte aligned; y_q and
 * y_s must not overlap each other, the inputs or the workspace.
 * Workspace: as for qlinear_nvfp4 / qlinear_int8.
 * ------------------------------------------------------------------------ */
int qlinear_nvfp4_q(const uint8_t* a_q, const uint8_t* a_s, const float* a_ts,
                    const uint8_t* w_q, const uint8_t* w_s, const float* w_ts,
                    int64_t M, int64_t N, int64_t K, const uint16_t* bias, qa_epi epi,
                    const float* y_ts, uint8_t* y_q, uint8_t* y_s, void* ws, size_t ws_bytes,
                    hipStream_t stream);
int qlinear_int8_q(const int8_t* a_q, const float* a_s, const uint8_t* w_q,
                   const uint8_t* w_s, const float* w_ts, const void* w8, int64_t M, int64_t N,
                   int64_t K, const uint16_t* bias, qa_epi epi, const float* y_ts, uint8_t* y_q,
                   uint8_t* y_s, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Quantized linear  Y[M][N] = dequant(A) dequant(W)^T (+ bias) (-> GELU).
 * Abstract and Fig. 2: each internal linear runs on NVFP4 or INT8
 * activations against 4-bit (NVFP4) weights.
 *
 * A NVFP4 (a_q, a_s, a_ts) or INT8 (a_q, a_s) as produced by act_quant;
 * W NVFP4 [N][K] (w_q, w_s, w_ts).  bias: bf16 [N] or NULL.
 * y: bf16 or f32 [M][ldy], ldy >= N.  epi: QA_EPI_GELU_TANH applies
 * 0.5 v (1 + tanh(sqrt(2/pi)(v + 0.044715 v^3))) after the bias.
 * INT8 activations with w8 (the weight's digit planes from
 * int8_weight_planes, below): integer MFMA, exact int32 sums H and L per
 * output (see qlinear_int8_acc), Y = s_a[m] s_Tw 2^(X[n]-1) (256 H + L)
 * formed in float32 (three roundings); w_q and w_s are then not read and
 * may be NULL.  Without w8 (NULL), and always for NVFP4 activations, both
 * operands are expanded exactly to fp16 (each NVFP4 value E2M1 x E4M3 and
 * each int8 is exact in fp16) and multiplied on fp16 MFMA with float32
 * accumulation, the tensor scales and the INT8 row scales applied to the
 * sums: an output then differs from the exact (float64) product by the
 * float32 accumulation over K -- about K 2^-24 times sum_k |a_k w_k| at
 * worst -- plus the final rounding to the output type.  Either way the
 * relative Frobenius error is far below 1e-3.
 * Workspace: qlinear_workspace() bytes, device memory that the call may
 * overwrite: a per-tile copy of the E4M3 scales of the operands (about
 * (M + N) K / 16 bytes) and, for shapes whose last round of 256 x 256
 * tiles (one per CU, 256 CUs) is at most half full and deep enough in K,
 * fp32 partial sums of that round's tiles split along K into up to 4
 * slices (256 KB per slice).  A call given less than qlinear_workspace()
 * but at least the scale copies computes the same outputs without the
 * split (summed in another order: equal within the accuracy above).  When
 * K is a multiple of 64 and w_s is 4-byte aligned the INT8 call reads the
 * weight scales in place and needs no more workspace than the split's (it
 * may then be NULL, and runs unsplit).  With w8 the INT8 call needs no
 * scale copies; its K split keeps int32 partial sums (256 KB per slice).
 * y must not overlap any input.  Requires 0 < K < 2^23, K % 16 == 0,
 * 0 <= M, N < 2^26 (QA_ESHAPE otherwise: the kernels address a tile's
 * 256 operand rows with 32-bit offsets below 2^31).
 * ------------------------------------------------------------------------ */
size_t qlinear_workspace(qa_fmt fmt, int64_t M, int64_t N, int64_t K);  /* 0 if rejected */
int qlinear_nvfp4(const uint8_t* a_q, const uint8_t* a_s, const float* a_ts,
                  const uint8_t* w_q, const uint8_t* w_s, const float* w_ts,
                  int64_t M, int64_t N, int64_t K, const uint16_t* bias,
                  void* y, int64_t ldy, qa_out out, qa_epi epi,
                  void* ws, size_t ws_bytes, hipStream_t stream);
int qlinear_int8(const int8_t* a_q, const float* a_s,
                 const uint8_t* w_q, const uint8_t* w_s, const float* w_ts, const void* w8,
                 int64_t M, int64_t N, int64_t K, const uint16_t* bias,
                 void* y, int64_t ldy, qa_out out, qa_epi epi,
                 void* ws, size_t ws_bytes, hipStream_t stream);

/* qlinear_int8_noalloc: for callers that cannot allocate device memory
 * (code under stream capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The same call as qlinear_int8 -- same arguments without
 * ws/ws_bytes, same kernels, same outputs bit for bit -- with its
 * workspace in a device array of the library's own, QA_NOALLOC_SCRATCH_BYTES
 * (64 MiB) per GPU, held from the first call on that GPU until the process
 * ends.  It allocates nothing: the first call on a device looks up the
 * array's address there (a symbol query; QA_EHIP if it fails), later calls
 * reuse it.  A shape whose qlinear_workspace(QA_INT8, M, N, K) exceeds the
 * array returns QA_ESCRATCH with nothing enqueued (the linears of the
 * CogVideoX-2B and -5B blocks at 17776 tokens need at most 57 MiB).  A
 * call that qlinear_int8 would reject returns its status first.  `stream` (NULL: the null
 * stream) must belong to the current device
 * (QA_EINVAL otherwise).  Every call on one GPU shares that GPU's array:
 * calls that may overlap in time there (other streams, other host threads)
 * race on it and must be serialised by the caller.  No word of the array
 * needs to start at zero, and it keeps whatever the last call left. */
#define QA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int qlinear_int8_noalloc(const int8_t* a_q, const float* a_s, const uint8_t* w_q,
                         const uint8_t* w_s, const float* w_ts, const void* w8, int64_t M,
                         int64_t N, int64_t K, const uint16_t* bias, void* y, int64_t ldy,
                         qa_out out, qa_epi epi, hipStream_t stream);

/* ------------------------------------------------------------------------
 * INT8 path on integer MFMA.  6Bit-Diffusion, abstract: volatile layers
 * keep INT8 activations; Table 2 ("W4A6"): the weights stay 4-bit NVFP4.
 *
 * int8_weight_planes (set-up, once per weight; SYNCHRONISES `stream`):
 * writes into w8 (device, int8_weight_planes_bytes(N, K) bytes, 256-byte
 * aligned, owned by the caller and passed to the INT8 linears) the NVFP4
 * weight (w_q, w_s) [N][K] in integer form.  An E4M3 scale is c 2^x (normal
 * codes: c = 8 + mantissa, x = exponent field - 10; subnormal: c =
 * mantissa, x = -9) and an E2M1 value v/2 (v in 0, 1, 2, 3, 4, 6, 8, 12,
 * signed); with X[n] the smallest x over row n's non-zero scales,
 * W[n][k] = s_Tw 2^(X[n]-1) I[n][k], I = v c 2^(x - X[n]), and
 * I = 256 hi + lo with int8 digits lo in [-128, 127], |hi| <= 90.  This
 * holds for rows whose x spread (largest minus smallest) is at most 7;
 * other rows are "irregular": their count goes to *irregular_rows (host,
 * nullable) and the call returns QA_EUNSUPPORTED (the buffer must then
 * not be used; the linear runs without w8).  The tensor scale is not
 * part of w8 (w_ts is passed to each linear).
 *
 * qlinear_int8_acc (verification): the exact int32 sums of the linear,
 * acc_hi[m][n] = H = sum_k q[m][k] hi[n][k] and acc_lo = L = sum_k
 * q[m][k] lo[n][k] (int32 device arrays [M][N]) from the same integer
 * MFMA kernel.  Requires K < 2^17 (|H|, |L| < 2^31).  acc_hi and acc_lo
 * must not overlap each other or the inputs.
 * ------------------------------------------------------------------------ */
size_t int8_weight_planes_bytes(int64_t N, int64_t K);
int int8_weight_planes(const uint8_t* w_q, const uint8_t* w_s, int64_t N, int64_t K,
                       void* w8, size_t w8_bytes, int64_t* irregular_rows,
                       hipStream_t stream);
int qlinear_int8_acc(const int8_t* a_q, const void* w8, int64_t M, int64_t N, int64_t K,
                     int32_t* acc_hi, int32_t* acc_lo, hipStream_t stream);

/* qlinear_nvfp4_amax / qlinear_int8_amax: qlinear_nvfp4 / qlinear_int8
 * with a bf16 output (16-byte aligned, ldy % 4 == 0; otherwise
 * QA_EUNSUPPORTED) whose |max| over the stored values is also taken in the
 * GEMM epilogue and atomically max-combined into the 1024 device words
 * y_amax[0..1023] (float bits; workgroup b into word b % 1024, so that the
 * atomics spread; the caller zero-fills the 4 KB before the call).  Point
 * y_amax at the workspace of the act_quant NVFP4 call that quantizes y for
 * the next linear and pass QA_AMAX_GIVEN there: that call then skips its read of the
 * whole tensor for amax_T (6Bit-Diffusion, Fig. 2 caption: the consumer's
 * activations are quantized per linear; the producer already holds every
 * value).  y_amax[0..1023] must not overlap y, the inputs or ws. */
int qlinear_nvfp4_amax(const uint8_t* a_q, const uint8_t* a_s, const float* a_ts,
                       const uint8_t* w_q, const uint8_t* w_s, const float* w_ts, int64_t M,
                       int64_t N, int64_t K, const uint16_t* bias, void* y, int64_t ldy,
                       qa_epi epi, uint32_t* y_amax, void* ws, size_t ws_bytes,
                       hipStream_t stream);
int qlinear_int8_amax(const int8_t* a_q, const float* a_s, const uint8_t* w_q,
                      const uint8_t* w_s, const float* w_ts, const void* w8, int64_t M,
                      int64_t N, int64_t K, const uint16_t* bias, void* y, int64_t ldy,
                      qa_epi epi, uint32_t* y_amax, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/* qlinear_routed: the linear in the activation format that the device byte
 * *route selects, with one GEMM launch for both formats, for a timestep
 * enqueued (or captured in a graph) before its decisions are known
 * (6Bit-Diffusion, Fig. 2 caption: each linear's activation format is
 * chosen per timestep).  *route is a linear gate byte of qa_decide_step:
 * (*route & 1) qlinear_nvfp4 on (a_q4, a_s4, a_ts4); otherwise (*route & 2)
 * qlinear_int8 on (a_q8, a_s8) with w8 (the integer kernel); 0: nothing,
 * y and y_amax left as they were.  The outputs are those of the call the
 * byte selects, bit for bit.  Both formats' operands are required (w_q,
 * w_s for NVFP4, w8 for INT8, w_ts for both); y bf16 [M][ldy], 16-byte
 * aligned, ldy % 4 == 0 (QA_EUNSUPPORTED otherwise); y_amax: NULL or as
 * for qlinear_*_amax.  K % 16 == 0.  ws: qlinear_routed_workspace(M, N, K)
 * bytes (0 if the shape is rejected) split the last round of tiles along K
 * as the plain calls do; at least qlinear_workspace(QA_NVFP4, ...) without
 * the split.  Launches: the NVFP4 scale re-layout (runs only for NVFP4;
 * none at most 256 tiles of 256x256 with K % 64 == 0, where the scales
 * are read in place), the whole tiles of either format, and, when the last
 * round is split, each format's K slices and fixup (each runs only for its
 * format).  Where the INT8 whole tiles take the persistent kernel (more
 * than 256 tiles of 256x128, K / 64 even and 6..64), each format's whole
 * tiles launch on their own instead (each runs only for its format).  A
 * gate set with qa_set_gate applies to every one of these launches as
 * well. */
size_t qlinear_routed_workspace(int64_t M, int64_t N, int64_t K);
int qlinear_routed(const uint8_t* route, const uint8_t* a_q4, const uint8_t* a_s4,
                   const float* a_ts4, const int8_t* a_q8, const float* a_s8, const uint8_t* w_q,
                   const uint8_t* w_s, const float* w_ts, const void* w8, int64_t M, int64_t N,
                   int64_t K, const uint16_t* bias, uint16_t* y, int64_t ldy, qa_epi epi,
                   uint32_t* y_amax, void* ws, size_t ws_bytes, hipStream_t stream);

/* act_quant of x followed by the matching qlinear_* (one layer).  For
 * NVFP4 the tensor scale is computed from x (flags may hold
 * QA_TSCALE_GIVEN with *x_ts an input); for INT8 x_ts is unused and w8
 * (nullable) selects the integer-MFMA kernel; for NVFP4 w8 must be NULL. */
size_t qlinear_layer_workspace(qa_fmt fmt, int64_t M, int64_t N, int64_t K);
int qlinear(qa_fmt fmt, const uint16_t* x, int64_t ldx, float* x_ts, uint32_t flags,
            const uint8_t* w_q, const uint8_t* w_s, const float* w_ts, const void* w8,
            int64_t M, int64_t N, int64_t K, const uint16_t* bias,
            void* y, int64_t ldy, qa_out out, qa_epi epi,
            void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Gamma and the Temporal Delta Cache.  All tensors are bf16 [n] (a whole
 * block hidden state, flattened); sums are float64 device arrays.  Sums
 * are deterministic (fixed-order reduction, no atomics) and equal the
 * exact sums to about 1e-15 relative.
 *
 * block_gamma (Fig. 2 and Fig. 3 captions: the block's input/output
 * relative L1 distance):  sums2 = { sum|out-in|, sum|in| }.
 *
 * tdc_update (abstract: the residual between block input and output is
 * cached; Fig. 4 caption: successive updates compared by relative L2):
 *   delta_new = bf16(out - in), rounded once, and
 *   sums4 = { sum|out-in|, sum|in|, sum (delta_new-delta_prev)^2,
 *             sum delta_prev^2 }  (the last two 0 when delta_prev is NULL).
 *   delta_new must not overlap in, out or delta_prev.
 *
 * tdc_apply (abstract: skip the invariant block):  out = bf16(in + delta),
 *   rounded once; out may equal in (in place) but must not overlap delta;
 *   sums2 (nullable) = { sum|out-in|, sum|in| } of the applied pair.
 * ------------------------------------------------------------------------ */
size_t reduce_workspace(int64_t n);
int block_gamma(const uint16_t* in, const uint16_t* out, int64_t n, double* sums2,
                void* ws, size_t ws_bytes, hipStream_t stream);
int tdc_update(const uint16_t* in, const uint16_t* out, const uint16_t* delta_prev,
               uint16_t* delta_new, int64_t n, double* sums4,
               void* ws, size_t ws_bytes, hipStream_t stream);
int tdc_apply(const uint16_t* in, const uint16_t* delta, uint16_t* out, int64_t n,
              double* sums2, void* ws, size_t ws_bytes, hipStream_t stream);
/* tdc_apply that also takes the |max| of its bf16 outputs (each wave's
 * integer maximum of the |bf16| patterns, one atomic maximum per wave of
 * the float bits) into the 1024 device words out_amax[0..1023] (workgroup
 * b into word b % 1024), which the caller zero-fills before the call: the
 * tensor amax of the next linear's NVFP4 act_quant with QA_AMAX_GIVEN when
 * out_amax is that call's workspace (the block input or the
 * residual-added hidden state feeds the next linear).  out_amax: 4-byte
 * aligned, its 4 KB overlapping no other buffer. */
int tdc_apply_amax(const uint16_t* in, const uint16_t* delta, uint16_t* out, int64_t n,
                   double* sums2, uint32_t* out_amax, void* ws, size_t ws_bytes,
                   hipStream_t stream);

/* tdc_update_ring / tdc_apply_ring: tdc_update / tdc_apply on a block's
 * Delta ring (two bf16 [n] slots), the slot chosen on the device from the
 * block's gate byte *blk of qa_decide_step (abstract and Fig. 2 caption:
 * the cached residual of a block is refreshed when it runs and reused when
 * it is skipped):
 *   tdc_update_ring: QA_BLK_RUN0 (1) reads Delta_prev from ring0 and writes
 *     Delta_new to ring1; QA_BLK_RUN1 (2) reads ring1, writes ring0;
 *   tdc_apply_ring: QA_BLK_SKIP0 (4) applies ring0, QA_BLK_SKIP1 (8) ring1,
 *     with the |max| of the outputs into out_amax (nullable) as
 *     tdc_apply_amax;
 * any other byte: nothing, outputs and sums left as they were.  One launch
 * (plus the sums' finalize) instead of one per slot.  The slots must not
 * overlap each other or the call's other buffers. */
int tdc_update_ring(const uint8_t* blk, const uint16_t* in, const uint16_t* out, uint16_t* ring0,
                    uint16_t* ring1, int64_t n, double* sums4, void* ws, size_t ws_bytes,
                    hipStream_t stream);
int tdc_apply_ring(const uint8_t* blk, const uint16_t* in, const uint16_t* ring0,
                   const uint16_t* ring1, uint16_t* out, int64_t n, double* sums2,
                   uint32_t* out_amax, void* ws, size_t ws_bytes, hipStream_t stream);

/* rel_err (Fig. 3 caption: E_rel, the layer-wise relative quantization
 * error at a timestep, to which the DMPQ predictor is fitted; read here as
 * the relative L2 error of the layer output against its bf16 computation):
 *   sums2 = { sum (y_q - y_ref)^2, sum y_ref^2 } over bf16 [n] arrays
 *   (device, 16-byte aligned), float64 device output; E_rel =
 *   sqrt(sums2[0]) / sqrt(sums2[1]) (qa_rel_err_from_sums; 0/0 = 0,
 *   x/0 = +inf).  Workspace: reduce_workspace(n) bytes, as for the Gamma
 *   and TDC sums; sums2 must not lie in it. */
int rel_err(const uint16_t* y_q, const uint16_t* y_ref, int64_t n, double* sums2,
            void* ws, size_t ws_bytes, hipStream_t stream);

/* delta_cosine (Fig. 4 caption: the agreement of a block's successive
 * residual updates Delta_t and Delta_{t-1}, shown as cosine similarity
 * beside the relative L2 difference):  sums3 = { sum d_new d_prev,
 * sum d_new^2, sum d_prev^2 } over bf16 [n] device arrays, float64 device
 * output (exact terms, fixed-order sums); the cosine is
 * sums3[0] / (sqrt(sums3[1]) sqrt(sums3[2])) (qa_cosine_from_sums; 0 when
 * either norm is 0).  Workspace: reduce_workspace(n) bytes; sums3 must not
 * lie in it. */
int delta_cosine(const uint16_t* d_new, const uint16_t* d_prev, int64_t n, double* sums3,
                 void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Host-side decisions (pure functions on HOST arrays; no GPU work).
 *
 * dmpq_mask (abstract: NVFP4 for temporally stable layers, INT8 for
 * volatile ones; Fig. 3 caption: E_rel ~ alpha Gamma_{t-1} + beta per
 * internal linear):  for block l and linear j (entry l*J + j),
 *   p = alpha[l*J+j] * gamma_prev[l] + beta[l*J+j]   (float64)
 *   mask = p > tau ? 1 (INT8) : 0 (NVFP4); a tie is NVFP4.
 *   gamma_prev == NULL (no preceding timestep): every mask entry is 1.
 *   Gamma values are ratios sum|out-in| / sum|in| (0/0 = 0, x/0 = +inf).
 *
 * tdc_decide (Fig. 2 caption: skip from the two preceding block updates):
 *   skip[l] = t >= 2 && computed_prev[l] && d_prev[l] < delta, where
 *   d_prev[l] = ||Delta_{t-1} - Delta_{t-2}|| / ||Delta_{t-2}|| from the
 *   sums of the block's last tdc_update (0/0 = 0, x/0 = +inf).
 * ------------------------------------------------------------------------ */
int dmpq_mask(const double* gamma_prev, int L, int J, const float* alpha,
              const float* beta, double tau, uint8_t* mask);
/* dmpq_fit (Fig. 3 caption: over a calibration run, the time-shifted pairs
 * of a block's Gamma at t-1 and each internal linear's E_rel at t give a
 * linear regression y = alpha x + beta per linear):  gamma [T][L] (block l
 * at timestep t), erel [T][L*J] (linear l*J+j at timestep t), host arrays.
 * For every linear the pairs (gamma[t-1][l], erel[t][l*J+j]), t = 1..T-1,
 * with both values finite, are fitted by ordinary least squares (centred
 * sums in long double); alpha/beta [L*J] float32 host outputs, rounded to
 * nearest.  Fewer than two distinct x: alpha = 0 and beta = the mean of y
 * (0 without pairs).  Errors: QA_EINVAL for negative sizes, J <= 0 or null
 * arrays that are needed. */
int dmpq_fit(const double* gamma, const double* erel, int T, int L, int J, float* alpha,
             float* beta);
int tdc_decide(int t, const double* d_prev, const uint8_t* computed_prev, int L,
               double delta, uint8_t* skip);
/* tdc_decide_cos: the same rule with the cosine of Fig. 4 as the agreement
 * measure (a page variant of the relative-L2 rule):
 *   skip[l] = t >= 2 && computed_prev[l] && cos_prev[l] > threshold,
 * cos_prev[l] the cosine of the block's last two Deltas (delta_cosine). */
int tdc_decide_cos(int t, const double* cos_prev, const uint8_t* computed_prev, int L,
                   double threshold, uint8_t* skip);
/* ---- Device-side step control (a timestep without host decisions) -------
 * The host loop of a diffusion step decides on the host: DMPQ masks from
 * Gamma_{t-1} (dmpq_mask) and TDC skips (tdc_decide), after copying the
 * sums of the previous step back.  These two calls let the whole step be
 * enqueued -- or captured once in a graph and replayed -- with the
 * decisions made on the device:
 *
 * qa_decide_step: one launch, at the start of step t, on `stream`.  Per
 * block l (L blocks of J linears), from sums [L][4] as the previous step's
 * calls left them (S1, S2 of tdc_update for a computed block, of tdc_apply
 * for a skipped one; S3, S4 of tdc_update), with device state that the
 * caller zero-fills once before step 0 and that the call carries on:
 *   t_ctr   int32: steps decided so far (t);
 *   bstate  u8 [L][4]: the block ran at t-1, Deltas stored (0..2), ring slot
 *           `last` holding the newest Delta, unused;
 *   d_prev  f64 [L]: relative L2 distance of the last two Deltas.
 * It first applies step t-1's outcome as the host loop does (Gamma =
 * S1/S2; a computed block's Delta went to slot last ^ 1, and d = sqrt(S3) /
 * sqrt(S4) once two are stored; x/0 = +inf, 0/0 = 0), then decides exactly
 * as dmpq_mask (alpha, beta: device f32 [L*J]; tau) and tdc_decide (delta)
 * would on those values, and writes the gate bytes of step t:
 *   lin_flags u8 [L*J]: 1 = NVFP4 path, 2 = INT8 path, 0 = block skipped;
 *   blk_flags u8 [L]:   1 / 2 = compute, Delta ring slot last = 0 / 1
 *                       (tdc_update reads slot last, writes last ^ 1);
 *                       4 / 8 = skip, tdc_apply with slot last = 0 / 1;
 *   mask_out [L*J], skip_out [L] (nullable): the decisions themselves.
 * The ring slots must hold zeros before step 0 (a first Delta is then
 * compared with zeros: d = +inf, as with no previous Delta).
 *
 * qa_set_gate: until cleared (flags NULL), every kernel of every library
 * call made from the calling thread reads the device byte *flags and does
 * nothing unless (*flags & bits) != 0 -- the call's outputs, sums
 * included, are then left as they were.  Host-side checks still run.  A
 * step thus enqueues every path (both formats of each linear, the compute
 * and skip paths of each block, the Delta update for either ring slot),
 * each under its gate byte and bits.  Per thread; bits != 0 when flags is
 * set. */
/* gate bytes written by qa_decide_step */
#define QA_ROUTE_NVFP4 1u   /* lin_flags: the linear runs on NVFP4 activations */
#define QA_ROUTE_INT8 2u    /* lin_flags: ... on INT8 activations */
#define QA_BLK_RUN0 1u      /* blk_flags: compute, Delta ring slot last = 0 */
#define QA_BLK_RUN1 2u      /* blk_flags: compute, last = 1 */
#define QA_BLK_SKIP0 4u     /* blk_flags: skip, apply slot 0 */
#define QA_BLK_SKIP1 8u     /* blk_flags: skip, apply slot 1 */
int qa_decide_step(const double* sums, const float* alpha, const float* beta, double tau,
                   double delta, int L, int J, int* t_ctr, uint8_t* bstate, double* d_prev,
                   uint8_t* blk_flags, uint8_t* lin_flags, uint8_t* mask_out, uint8_t* skip_out,
                   hipStream_t stream);
int qa_set_gate(const uint8_t* flags, uint32_t bits);

/* Test-only: the element conversions the quantizers and epilogues are built
 * on, applied to the float32 bit patterns first .. first + count - 1
 * (count >= 0, first + count <= 2^32), one output per pattern, so that a
 * test can check them on every input against the format rules (NVFP4:
 * 6Bit-Diffusion, abstract):
 *   op 0  E2M1 code (u8 out; low nibble, bit 3 the sign) as the NVFP4
 *         encoders convert x * inv: nearest, ties to the even code,
 *         saturating at 6;
 *   op 1  E4M3FN code (u8 out) of a group scale: inputs must be
 *         non-negative and finite (patterns <= 0x7F7FFFFF);
 *   op 2  bf16 bits (u16 out, 2-byte aligned) as the epilogues round
 *         float32 outputs: nearest, ties to even.
 * Outputs for NaN or infinite inputs (ops 0 and 2) are not specified. */
int qa_test_convert(int op, uint32_t first, int64_t count, void* out, hipStream_t stream);

/* Test and benchmark only: the compute stage of three designs of the NVFP4
 * linear (6Bit-Diffusion, abstract: NVFP4 activations and weights, one E4M3
 * scale per 16 elements) on register-resident operands, `iters` 16-element
 * scale groups per wave, `blocks` workgroups of 256 lanes:
 *   design 0  both operands expanded exactly to fp16 with their group
 *             scales, fp16 MFMA accumulating across groups (the library's);
 *   design 1  codes as fp8, one fp8 MFMA per group from zero, the partial
 *             product rescaled by s_a s_w per output into float32 sums;
 *   design 2  activations scaled into fp16, weight codes unscaled, fp16
 *             MFMA per group from zero, rescaled by s_w per output.
 * in: device u32 [1024][64] per-lane operands (layout in stage_ab.hip);
 * out: device f32 [1024][256], lane (g % 1024)'s accumulators.  Lanes g and
 * g + 1024 k read and write the same rows with the same values. */
int qa_test_stage_ab(int design, int iters, int blocks, const uint32_t* in, float* out,
                     hipStream_t stream);

/* Profiling hook: while set, each qlinear_nvfp4 / qlinear_int8 call (also
 * inside qlinear) launches its main GEMM kernel with hipExtLaunchKernel so
 * that `before` and `after` take that dispatch's start and end timestamps
 * (no extra packets on the stream); hipEventElapsedTime(before, after) is
 * then that kernel's duration.  The events are created and owned by the
 * caller; pass NULL, NULL to stop.  Process-wide setting, not thread-safe. */
int qa_set_gemm_events(hipEvent_t before, hipEvent_t after);

/* Helpers for the host: Gamma and d from the device sums once copied back. */
double qa_gamma_from_sums(const double* sums2);
double qa_rel_l2_from_sums(const double* sums4);
double qa_rel_err_from_sums(const double* sums2);
double qa_cosine_from_sums(const double* sums3);

#ifdef __cplusplus
}
#endif
#endif /* QACT_H */
