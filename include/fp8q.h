/*
 * fp8q.h - C ABI of libfp8q: FP8 E4M3 linear layers (per-tensor scales, or per-token
 * activation and per-channel weight scales) and the
 * NestedFP dual-precision GEMM on AMD MI355X (gfx950).
 *
 * Pages whose statement of the problem these calls follow:
 *   [RTX4060]  the page on a 7B model on an RTX 4060 with FP8
 *              (intelliparadigm.com/article/weixin_29051149/2151670)
 *   [C++FP8]   "C++与FP8量化：大模型推理部署的系统级优化实践" (tqpw.cn/news/201730)
 *   [NestedFP] "NestedFP双精度推理框架：LLM部署中的内存与计算优化"
 *              (intelliparadigm.com/article/weixin_42537919/2229392)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named x, q, qa, qw, y, w, hi, lo, a, scale, amax, sa, sw are
 *    DEVICE pointers on the current HIP device.  The caller owns every buffer;
 *    the library allocates no device memory on any call.
 *  - Matrices are dense, row-major, without strides: activations [M,K],
 *    weights and NestedFP planes [N,K] (K contiguous: the "tn" layout of the
 *    FP8 GEMM named in [C++FP8] §3.3), outputs [M,N].
 *  - 16-bit floating-point tensors (bf16, fp16) are passed as their uint16
 *    bit patterns; FP8 tensors as uint8 codes (OCP E4M3 "FN": bias 7, max 448,
 *    0x7F/0xFF NaN; E5M2: bias 15).
 *  - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL is the null stream) and never synchronizes the host.  Scales and
 *    amax stay on the device.
 *  - Arguments are validated on the host before any HIP call; on a validation
 *    error nothing is launched.  Base pointers must be 16-byte aligned.
 *  - No output buffer may share a byte with another buffer of the same call,
 *    input or output (FP8Q_ERR_OVERLAP): other workgroups still read and
 *    write those bytes.  Inputs may share memory with each other.  The one
 *    exception is the y of the linear calls (fp8_linear, fp8_linear_rowwise,
 *    fp8_linear_delayed, nested_linear_fp8, nested_linear_fp8_e4m3), which
 *    may lie over their activation input (in place).
 *    A failed launch returns FP8Q_ERR_LAUNCH; faults inside a kernel surface
 *    at the caller's next synchronization, as for any HIP work.
 *  - Calls on different streams are independent (no shared mutable state).
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8Q_ABI_VERSION 3

/* 32-bit words of the delayed-scaling state (see fp8_quantize_act_delayed). */
#define FP8Q_DELAYED_STATE_WORDS 288

typedef enum {
    FP8Q_OK = 0,
    FP8Q_ERR_NULL = 1,    /* a required pointer is NULL                        */
    FP8Q_ERR_SHAPE = 2,   /* a size is out of range (see each call)            */
    FP8Q_ERR_ALIGN = 3,   /* a base pointer is not 16-byte aligned             */
    FP8Q_ERR_DTYPE = 4,   /* unknown input dtype                               */
    FP8Q_ERR_LAUNCH = 5,  /* a HIP call or kernel launch failed                */
    FP8Q_ERR_DEVICE = 6,  /* the current device is not a gfx950 GPU            */
    FP8Q_ERR_OVERLAP = 7  /* an output overlaps another buffer of the call     */
} fp8q_status;

typedef enum { FP8Q_BF16 = 0, FP8Q_FP16 = 1 } fp8q_dtype;

typedef void* fp8q_stream; /* hipStream_t */

/* Symbols of the shared library; everything else in it is hidden. */
#if defined(FP8Q_BUILD)
#define FP8Q_API __attribute__((visibility("default")))
#else
#define FP8Q_API
#endif

/* Returns FP8Q_ABI_VERSION of the built library. */
FP8Q_API int fp8q_abi_version(void);

/* Static, never-NULL description of a status code. */
FP8Q_API const char* fp8q_status_str(int status);

/* Text of the last HIP error seen by this thread's calls ("" if none). */
FP8Q_API const char* fp8q_last_error(void);

/*
 * fp8_quantize_act - dynamic per-tensor E4M3 quantization.
 *   [RTX4060] §2.2: activations are quantized at run time from the layer's
 *   amax; §6.1: scaled values stay within 448 and the E4M3 exponent does not
 *   saturate.  The same call quantizes weights offline (static quantization,
 *   [RTX4060] §2.2) when given the fp16 weight tensor.
 *
 *   x[n]     in : bf16 (dtype FP8Q_BF16) or fp16 (FP8Q_FP16) bit patterns
 *   q[n]     out: E4M3 codes, q_i = E4M3_rne_sat(fl32(x_i / s))
 *   *scale   out: s = fl32(amax / 448), or 1.0 when amax == 0
 *   *amax    out: max_i |x_i| (also used as the reduction accumulator; its
 *                 previous contents are ignored)
 *   n >= 1.  E4M3 rounding: nearest, ties to even, subnormals kept,
 *   |v| > 448 (and +-inf) saturate to +-448.  NaN inputs are outside the
 *   contract.
 */
FP8Q_API fp8q_status fp8_quantize_act(const void* x, int dtype, int64_t n, uint8_t* q,
                             float* scale, float* amax, fp8q_stream stream);

/*
 * fp8_gemm - y = bf16( (qa . qw^T) * fl32(*sa * *sw) ), fp32 accumulation.
 *   The FP8 GEMM of [C++FP8] §3.3 (E4M3 operands, fp32 accumulate, bf16
 *   output, "tn" layout), on statically quantized weights ([RTX4060] §2.2).
 *
 *   qa[M,K]  in : E4M3 activation codes        *sa in: activation scale
 *   qw[N,K]  in : E4M3 weight codes            *sw in: weight scale
 *   y[M,N]   out: bf16 bit patterns, round to nearest even
 *   1 <= M, N <= 2^31-1;  16 <= K <= 2^22 and K % 16 == 0.
 *   M <= 16 runs the weight-streaming decode kernels, larger M the MFMA tile
 *   GEMM.
 */
FP8Q_API fp8q_status fp8_gemm(const uint8_t* qa, const float* sa, const uint8_t* qw,
                     const float* sw, uint16_t* y, int64_t M, int64_t N, int64_t K,
                     fp8q_stream stream);

/*
 * fp8_linear - one FP8 linear layer: fp8_quantize_act on the activation,
 *   then fp8_gemm on its codes ([RTX4060] §2.2: dynamic activation
 *   quantization against statically quantized weights; [C++FP8] §3.3: the
 *   FP8 GEMM).  Results are bit-identical to the two calls made in sequence:
 *
 *   x[M,K]   in : bf16/fp16 activation (dtype as for fp8_quantize_act)
 *   qw[N,K], *sw in: E4M3 weight codes and scale
 *   y[M,N]   out: bf16 bit patterns
 *   q[M,K], *scale, *amax out: the activation codes, scale and amax
 *   Size rules as fp8_gemm.  For M <= 16 with M*K <= 32768, and for
 *   3 <= M <= 16 with M*K <= 65536 and N > 16384, the whole layer is one
 *   kernel (each workgroup quantizes the activation in LDS);
 *   otherwise it launches the quantizer and then the GEMM, and while the
 *   quantizer runs y (not yet written) may hold its per-workgroup partial
 *   maxima.  y may lie over x (in place): then the layer always takes the
 *   two launches and the quantizer uses no scratch.  Every other overlap of
 *   an output returns FP8Q_ERR_OVERLAP.
 */
FP8Q_API fp8q_status fp8_linear(const void* x, int dtype, const uint8_t* qw, const float* sw,
                       uint16_t* y, uint8_t* q, float* scale, float* amax, int64_t M,
                       int64_t N, int64_t K, fp8q_stream stream);

/*
 * fp8_quantize_rows - one E4M3 scale per row of x[rows, cols]: per-token
 *   activation scales, or per-channel weight scales when x is a weight
 *   matrix [N, K] (the per-token / per-channel options of the TensorRT-LLM
 *   build in [C++FP8] §4.2).  Row r is quantized exactly as fp8_quantize_act
 *   quantizes it on its own:
 *
 *   x[rows,cols]  in : bf16/fp16 bit patterns (dtype as for fp8_quantize_act)
 *   q[rows,cols]  out: E4M3 codes of row r with scale[r]
 *   scale[rows]   out: fl32(amax[r] / 448), or 1.0 when amax[r] == 0
 *   amax[rows]    out: max over row r of |x|
 *   1 <= rows <= 2^31-1;  16 <= cols <= 2^22 and cols % 16 == 0.
 */
FP8Q_API fp8q_status fp8_quantize_rows(const void* x, int dtype, int64_t rows, int64_t cols,
                                       uint8_t* q, float* scale, float* amax,
                                       fp8q_stream stream);

/*
 * fp8_gemm_rowwise - fp8_gemm with a scale per activation row and per weight
 *   row: y[m,n] = bf16( (sum_k dec(qa[m,k]) dec(qw[n,k])) * fl32(sa[m] * sw[n]) ),
 *   fp32 accumulation, the epilogue applied once per element.
 *
 *   qa[M,K], sa[M] in: E4M3 activation codes and per-token scales
 *   qw[N,K], sw[N] in: E4M3 weight codes and per-channel scales
 *   y[M,N]         out: bf16 bit patterns
 *   Size rules and dispatch as fp8_gemm.
 */
FP8Q_API fp8q_status fp8_gemm_rowwise(const uint8_t* qa, const float* sa, const uint8_t* qw,
                                      const float* sw, uint16_t* y, int64_t M, int64_t N,
                                      int64_t K, fp8q_stream stream);

/*
 * fp8_linear_rowwise - fp8_quantize_rows on the activation, then
 *   fp8_gemm_rowwise on its codes; bit-identical to the two calls made in
 *   sequence.
 *
 *   x[M,K]    in : bf16/fp16 activation
 *   qw[N,K], sw[N] in: E4M3 weight codes and per-channel scales
 *   y[M,N]    out: bf16 bit patterns
 *   q[M,K], sa[M], amax[M] out: activation codes, per-token scales and amax
 *   Size rules as fp8_gemm.  For M <= 2 and M*K <= 32768 one kernel (each
 *   workgroup quantizes both rows in LDS) unless y lies over x; otherwise
 *   two launches.
 */
FP8Q_API fp8q_status fp8_linear_rowwise(const void* x, int dtype, const uint8_t* qw,
                                        const float* sw, uint16_t* y, uint8_t* q, float* sa,
                                        float* amax, int64_t M, int64_t N, int64_t K,
                                        fp8q_stream stream);

/*
 * fp8_quantize_kv - FP8 KV cache: E4M3 codes of a K or V block with one scale
 *   per head ([RTX4060] §1 stores the KV cache in FP8, [C++FP8] §4.2 builds
 *   with an FP8 KV-cache type; attention itself is not part of this library).
 *
 *   x[T,H,D]  in : bf16/fp16 bit patterns, tokens x heads x head dimension
 *   q[T,H,D]  out: E4M3 codes; head h quantized with scale[h]
 *   scale[H]  out: fl32(amax[h] / 448), or 1.0 when amax[h] == 0
 *   amax[H]   out: max over all tokens and the head dimension of |x[:,h,:]|
 *   Head h is quantized exactly as fp8_quantize_act would quantize the
 *   gathered x[:,h,:].  T, H >= 1 (H <= 2^20); 8 <= D <= 2^16, D % 8 == 0;
 *   T*H*D <= 2^40.  Heads of at most 32768 elements: one launch; larger:
 *   three (partial maxima, kept in q until the last pass; per-head amax and
 *   scale; quantization).
 */
FP8Q_API fp8q_status fp8_quantize_kv(const void* x, int dtype, int64_t tokens, int64_t heads,
                                     int64_t head_dim, uint8_t* q, float* scale, float* amax,
                                     fp8q_stream stream);

/*
 * Delayed scaling with an amax history ([RTX4060] §6.1: the history should be
 * at least 1024 long).  A call quantizes with the scale that the amax of the
 * earlier calls gives, then records its own amax, so the activation is read
 * once and no reduction precedes the quantization:
 *
 *   history[L]  in/out: the amax of the last L calls on this tensor (ring)
 *   state[FP8Q_DELAYED_STATE_WORDS]
 *               in/out: [0] float bits of the scale the next call uses
 *               (0 = no history yet, meaning 1), [2] ring position, [4] float
 *               bits of max(history); every other word is an accumulator of a
 *               call in progress (0 between calls: the workgroups of a call
 *               count their arrival in eight 128-byte lines, so that their
 *               atomics do not all queue on one address)
 *   Both are device memory owned by the caller, zero-filled once before the
 *   first call, and changed only by these calls (a saved pair is restored
 *   whole); state is 16-byte aligned.  Calls on one (history, state) must not
 *   overlap in time (issue them on one stream).  1 <= L <= 2^24.
 *
 *   Call t: s = scale from state[0] (1 if 0); q_i = E4M3_rne_sat(fl32(x_i / s)),
 *   so values beyond 448 s saturate to +-448; a = max_i |x_i|;
 *   history[pos] = a; pos = (pos + 1) mod L; state[0] = fl32(max(history) / 448)
 *   (1.0 when the history holds only zeros).
 */

/*
 * fp8_quantize_act_delayed - fp8_quantize_act with delayed scaling:
 *   x[n] in; q[n] out; *scale out: the scale s used; *amax out: max_i |x_i|.
 *   One launch (a grid-stride pass whose last workgroup updates the history).
 */
FP8Q_API fp8q_status fp8_quantize_act_delayed(const void* x, int dtype, int64_t n, uint8_t* q,
                                              float* scale, float* amax, float* history,
                                              int64_t history_len, uint32_t* state,
                                              fp8q_stream stream);

/*
 * fp8_linear_delayed - fp8_linear with delayed activation scaling: the
 *   activation is quantized as fp8_quantize_act_delayed does, then multiplied
 *   with fp8_gemm; bit-identical to the two calls in sequence.  For M <= 2
 *   and M*K <= 32768 one kernel, whose quantization needs no reduction over
 *   the activation first, unless y lies over x (then two launches).  history
 *   and state, like the outputs, may share no byte with another buffer of
 *   the call.  Size rules as fp8_gemm.
 */
FP8Q_API fp8q_status fp8_linear_delayed(const void* x, int dtype, const uint8_t* qw,
                                        const float* sw, uint16_t* y, uint8_t* q, float* scale,
                                        float* amax, float* history, int64_t history_len,
                                        uint32_t* state, int64_t M, int64_t N, int64_t K,
                                        fp8q_stream stream);

/*
 * nested_split - NestedFP byte split of fp16 weights ([NestedFP] §2.1):
 *   hi[i] = w[i] >> 8, lo[i] = w[i] & 0xFF.   n >= 1.
 */
FP8Q_API fp8q_status nested_split(const uint16_t* w, uint8_t* hi, uint8_t* lo, int64_t n,
                         fp8q_stream stream);

/*
 * nested_rebuild_fp16 - the FP16-mode rebuild of [NestedFP] §2.1 on its own:
 *   w[i] = (hi[i] << 8) | lo[i].   n >= 1.  Uses the same device routine as
 *   nested_gemm_fp16; exported so the rebuild can be checked exhaustively.
 */
FP8Q_API fp8q_status nested_rebuild_fp16(const uint8_t* hi, const uint8_t* lo, uint16_t* w,
                                int64_t n, fp8q_stream stream);

/*
 * nested_gemm_fp16 - NestedFP FP16 mode ([NestedFP] §2.1, §2.2): weights are
 *   rebuilt in-kernel as fp16 (hi<<8)|lo, bit-exactly, then
 *   y = fp16( a . w^T ), fp32 accumulation, round to nearest even.
 *
 *   a[M,K]   in : fp16 activations;  hi[N,K], lo[N,K] in: byte planes
 *   y[M,N]   out: fp16 bit patterns
 *   Same size rules as fp8_gemm.
 */
FP8Q_API fp8q_status nested_gemm_fp16(const uint16_t* a, const uint8_t* hi, const uint8_t* lo,
                             uint16_t* y, int64_t M, int64_t N, int64_t K,
                             fp8q_stream stream);

/*
 * nested_gemm_fp8 - NestedFP FP8 mode ([NestedFP] §2.1): only the hi plane is
 *   read, as an 8-bit float; the upper byte of an fp16 word is exactly an E5M2
 *   code, so its value is fp16(hi << 8).  Activations are E4M3 codes from
 *   fp8_quantize_act (on the fp16 activation) with scale *sa:
 *   y = fp16( (qa . E5M2(hi)^T) * *sa ), fp32 accumulation.
 *
 *   qa[M,K] in, *sa in, hi[N,K] in, y[M,N] out (fp16 bits).
 *   Same size rules as fp8_gemm.
 */
FP8Q_API fp8q_status nested_gemm_fp8(const uint8_t* qa, const float* sa, const uint8_t* hi,
                            uint16_t* y, int64_t M, int64_t N, int64_t K,
                            fp8q_stream stream);

/*
 * nested_linear_fp8 - one NestedFP FP8-mode linear layer ([NestedFP] §2.1):
 *   fp8_quantize_act on the fp16 activation, then nested_gemm_fp8 on its
 *   codes.  Results are bit-identical to the two calls made in sequence:
 *
 *   a[M,K]   in : fp16 activation bit patterns
 *   hi[N,K]  in : hi byte plane of the fp16 weights, read as E5M2
 *   y[M,N]   out: fp16 bit patterns
 *   q[M,K], *scale, *amax out: the activation codes, scale and amax
 *   Size rules as fp8_gemm.  One kernel for the same sizes as fp8_linear
 *   (M <= 16 with M*K <= 32768, or 3 <= M <= 16 with M*K <= 65536 and
 *   N > 16384); otherwise the
 *   quantizer runs first and may keep its per-workgroup partial maxima in y
 *   (not yet written); y lying over a (in place) takes the two launches
 *   without that scratch.
 */
FP8Q_API fp8q_status nested_linear_fp8(const uint16_t* a, const uint8_t* hi, uint16_t* y,
                              uint8_t* q, float* scale, float* amax, int64_t M, int64_t N,
                              int64_t K, fp8q_stream stream);

/*
 * NestedFP with an E4M3 upper byte ([NestedFP] §2.1 also names E4M3 as the
 * upper byte's format).  Reading: the fp16 word s|e4..e0|m9..m0 is split into
 *   hi = s | e3..e0 | m9..m7   (the E4M3 code of w * 2^8, truncated toward
 *                               zero, whenever e4 == 0; fp16 subnormals land
 *                               on E4M3 subnormals, so nothing underflows)
 *   lo = e4 | m6..m0
 * so the rebuild is exact for every fp16 word, and the FP8 mode (hi as E4M3,
 * scale 2^-8) holds for finite |w| < 1.875 (beyond, e4 == 1 or hi would read
 * as NaN).  One more mantissa bit than the plain split's E5M2 upper byte.
 *
 * nested_split_e4m3 - the split above.  *out_of_range (device, 8-byte
 *   aligned, zero-filled by the caller; may be NULL) gains the number of
 *   words outside |w| < 1.875 (NaN and inf included).   n >= 1.
 * nested_rebuild_e4m3 - w = (hi & 0x80) << 8 | (lo & 0x80) << 7 |
 *   (hi & 0x7F) << 7 | (lo & 0x7F), the FP16-mode rebuild on its own.
 * nested_gemm_fp16_e4m3 - nested_gemm_fp16 on planes of this split.
 * nested_gemm_fp8_e4m3 - y = fp16((qa . E4M3(hi)^T) * fl32(*sa * 2^-8)).
 * nested_linear_fp8_e4m3 - fp8_quantize_act on the fp16 activation, then
 *   nested_gemm_fp8_e4m3; bit-identical to the two calls in sequence.
 *   Size rules and dispatch as the plain-split calls.
 */
FP8Q_API fp8q_status nested_split_e4m3(const uint16_t* w, uint8_t* hi, uint8_t* lo, int64_t n,
                                       uint64_t* out_of_range, fp8q_stream stream);
FP8Q_API fp8q_status nested_rebuild_e4m3(const uint8_t* hi, const uint8_t* lo, uint16_t* w,
                                         int64_t n, fp8q_stream stream);
FP8Q_API fp8q_status nested_gemm_fp16_e4m3(const uint16_t* a, const uint8_t* hi,
                                           const uint8_t* lo, uint16_t* y, int64_t M, int64_t N,
                                           int64_t K, fp8q_stream stream);
FP8Q_API fp8q_status nested_gemm_fp8_e4m3(const uint8_t* qa, const float* sa, const uint8_t* hi,
                                          uint16_t* y, int64_t M, int64_t N, int64_t K,
                                          fp8q_stream stream);
FP8Q_API fp8q_status nested_linear_fp8_e4m3(const uint16_t* a, const uint8_t* hi, uint16_t* y,
                                            uint8_t* q, float* scale, float* amax, int64_t M,
                                            int64_t N, int64_t K, fp8q_stream stream);

/*
 * fp8q_e4m3_encode_f32 - the device E4M3 encoder used by fp8_quantize_act,
 *   applied to binary32 values directly: q[i] = E4M3_rne_sat(v[i]).  n >= 1.
 *   Exported so the encoder can be checked exhaustively; not on the hot path.
 */
FP8Q_API fp8q_status fp8q_e4m3_encode_f32(const float* v, uint8_t* q, int64_t n,
                                 fp8q_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
