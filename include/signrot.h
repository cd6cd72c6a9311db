/*
 * signrot.h -- C ABI of libsignrot, SignRot's online activation path on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (pages: the SignRot abstract, arXiv 2611.16502, and the explainer
 * "SignRot for 4-bit LLM quantization -- Sign-adjusted Hadamard rotation"):
 * at the input of an LLM down-projection every token x (a row of n bf16
 * values) is rotated by an orthonormal Hadamard matrix, y = x.H / sqrt(n)
 * (explainer, paragraph on rotation: every entry of H is +-1/sqrt(n), applied
 * with a fast Walsh-Hadamard transform, paragraph on the down-projection); the
 * columns of H are sign-flipped by a calibrated vector d so that the one
 * massive-outlier channel reaches every output with the same sign
 * (explainer, paragraph on the sign adjustment; abstract); and the result is
 * quantized per token to 16 evenly spaced levels between the token's minimum
 * and maximum, an asymmetric INT4 code with a zero-point (explainer,
 * paragraphs on the quantizer and on symmetric versus asymmetric quantizers).
 *
 * Hadamard order (n <= 32768).  n = 2^k (k >= 1) uses the Sylvester matrix in
 * natural order, H[i][j] = (-1)^popcount(i & j).  Any other n = o * 2^v (o
 * odd) uses H = H_m (x) H_{2^k} with index i = a * 2^k + b (a < m, b < 2^k),
 * where m = o * 2^j for the smallest j >= 2 for which Paley's construction I
 * (q = m - 1 a prime power = 3 mod 4: H_m = I + S, S the Jacobsthal matrix of
 * the quadratic character of GF(q) bordered by a row of +1 and a column of -1)
 * or, failing that, construction II (q = m/2 - 1 a prime power = 1 mod 4:
 * H_m = C (x) [[1,1],[1,-1]] + I (x) [[1,-1],[-1,-1]], C the symmetric
 * conference matrix) exists with m <= 512.  GF(p^e) is GF(p)[t] modulo the
 * first monic irreducible polynomial in lexicographic order of its
 * coefficients.  So 28 * 2^k uses H28 over GF(27) = GF(3)[t]/(t^3 + 2t + 1),
 * 13824 = 108 * 2^7 uses construction I over GF(107), and 11008 = 344 * 2^5
 * uses construction I over GF(7^3) (172 * 2^6 has no Paley factor).  The
 * pages only ask for some Hadamard matrix; these are the library's choices.
 * Orientation: y_j = sum_i x_i H[i][j] (x is a row vector; the outlier at
 * channel c reaches the outputs through row c of H).
 *
 * Conventions shared by every call:
 *   - All sizes are element counts.  Device pointers are plain HIP device
 *     addresses (e.g. from torch).  `stream` is a hipStream_t passed as
 *     void*; NULL means the default stream.  Every tensor is owned by the
 *     caller; the library keeps no pointer after a call returns.
 *   - Activations are bf16 bit patterns, row-major [tokens][ld], ld >= n,
 *     with the base pointer 16-byte aligned and ld a multiple of 8 (so each
 *     row starts 16-byte aligned).
 *   - Calls return a signrot_status.  Argument errors are detected on the
 *     host before any HIP call and leave every output untouched.  A HIP
 *     error returns SIGNROT_EHIP; outputs are then unspecified and
 *     signrot_last_error() holds the HIP message.  Nothing throws.
 *   - tokens == 0 is a successful no-op (null pointers are then allowed).
 *   - Non-finite inputs, or inputs so large that the rotated values overflow
 *     binary32, give unspecified outputs (no checks on the hot path).
 *   - Calls are reentrant; concurrent calls on different streams are allowed.
 *   - Device memory the library itself allocates: (1) per device, the sign
 *     table of an outer factor H_m with m != 28 (and the transposed table for
 *     the outer-order MFMA kernel), at most 32 KiB each, copied there by the
 *     first call that needs it (hipMalloc + hipMemcpy) and kept until the
 *     process ends; a first call made while `stream` is being captured into
 *     a graph returns SIGNROT_EHIP instead and leaves the capture intact.
 *     H28 (every width 28 * 2^k) and the Sylvester-only widths with their own
 *     kernel need no table: H28 travels by value in the kernel arguments.
 *     (2) Stream-ordered scratch (hipMallocAsync / hipFreeAsync on `stream`),
 *     named at each call that uses it.  Nothing else.
 */
#ifndef SIGNROT_H
#define SIGNROT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SIGNROT_OK = 0,
  SIGNROT_EINVAL = -1,          /* bad pointer, size, stride or alignment   */
  SIGNROT_EUNSUPPORTED_N = -2,  /* n has no factorisation of the rule above  */
  SIGNROT_EHIP = -3             /* a HIP runtime call or launch failed       */
} signrot_status;

/* 1 if n factors by the rule above (n <= 32768), else 0. */
int signrot_supported_n(int64_t n);

/* The outer order m of n by that rule (1 for n = 2^k), or 0 when n is
 * unsupported. */
int signrot_outer_order(int64_t n);

/*
 * Calibration (abstract: one calibration forward pass; explainer, paragraph
 * on the sign adjustment: the channel with the largest absolute activation,
 * and a flip of each column j of H by the sign of that row's entry).
 *
 *   x_bf16  device, [tokens][ld] bf16 calibration batch (tokens < 2^28).
 *   d_out   device, [n] int8: d_j = sign(M_c) * H[c][j], values +1/-1, where
 *           c is the channel of the largest |x| over the batch and M_c the
 *           signed value there.  Ties: smallest channel, then smallest token.
 *           sign(+0) = sign(-0) = +1.
 *   c_out   host, may be NULL: the channel c.
 *   t_out   host, may be NULL: the token t holding M_c.
 *   mc_out  host, may be NULL: M_c widened to float.
 *
 * Enqueues its kernels on `stream`, then synchronizes that stream (the host
 * outputs need the result).  Uses a 16-byte stream-ordered scratch buffer
 * (hipMallocAsync / hipFreeAsync).  Unlike the other calls, tokens == 0 ->
 * SIGNROT_EINVAL: an empty batch has no largest activation, so there is no
 * channel to find.  t_out is reported in addition to c and M_c so that a
 * caller can check the argmax against its own data.
 */
int signrot_calibrate(const void* x_bf16, int64_t tokens, int64_t n, int64_t ld,
                      int8_t* d_out, int32_t* c_out, int64_t* t_out, float* mc_out,
                      void* stream);

/*
 * signrot_calibrate without any allocation, for callers that cannot allocate
 * device memory (tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, outputs and argument errors as signrot_calibrate.  The 16-byte
 * argmax record lives in a static device array of the library (one per GPU,
 * kept until the process ends; its address is looked up once per device)
 * instead of a stream-ordered allocation; each call clears it first.  The
 * record's size does not depend on the input, so no input is too large for
 * it.  Only widths whose Hadamard factors need no device table are taken,
 * n = 2^k and n = 28 * 2^k; any other supported n -> SIGNROT_EUNSUPPORTED_N
 * (use signrot_calibrate).  Calls that overlap on one GPU (several streams or
 * threads) race on the shared record: serialize them.  Synchronizes `stream`
 * before returning, as signrot_calibrate does.
 */
int signrot_calibrate_noalloc(const void* x_bf16, int64_t tokens, int64_t n, int64_t ld,
                              int8_t* d_out, int32_t* c_out, int64_t* t_out, float* mc_out,
                              void* stream);

/*
 * The online path: y = (x . H / sqrt(n)) (.) d, then per-token asymmetric
 * INT4 (explainer, paragraphs on rotation, on the sign adjustment and on the
 * quantizer).  Per token, with mn = min_j y_j and mx = max_j y_j:
 *   scale = (mx - mn) / 15, or 1 when mx == mn;
 *   zero  = -mn / scale, in code units, neither rounded nor clamped;
 *   q_j   = clamp(round((y_j - mn) / scale), 0, 15), round to nearest.
 *
 *   x_bf16  device, [tokens][ld] bf16.
 *   d       device, [n] int8, 16-byte aligned, every entry +1 or -1 (any
 *           other value gives unspecified output).  When d = sigma * (row c of H) -- the form
 *           signrot_calibrate produces -- the library recognises it and
 *           evaluates the identical quantity as ((x - x_c e_c) . H) (.) d plus
 *           the constant sigma * x_c / sqrt(n), so the outlier is added once
 *           instead of being rounded through every butterfly stage.
 *   codes   device, [tokens][n/2] uint8, 16-byte aligned: code of channel 2m
 *           in the low nibble of byte m, channel 2m+1 in the high nibble.
 *   scale   device, [tokens] float.
 *   zero    device, [tokens] float.
 *   y_out   device, [tokens][n] float, 16-byte aligned, or NULL: the
 *           rotated, flipped values in binary32 (a debugging output; the
 *           codes do not depend on it).
 *
 * A misaligned x, d, codes or y_out, ld < n or ld not a multiple of 8, a null
 * pointer (tokens > 0) or tokens < 0 -> SIGNROT_EINVAL; an unsupported n ->
 * SIGNROT_EUNSUPPORTED_N.
 *
 * Asynchronous: returns once the kernel is enqueued on `stream`.  Arithmetic
 * is binary32 throughout.
 */
int signrot_rotate_quant_int4(const void* x_bf16, int64_t tokens, int64_t n, int64_t ld,
                              const int8_t* d, uint8_t* codes, float* scale, float* zero,
                              float* y_out, void* stream);

/*
 * The online path for the sign vector in its calibrated form, given by the
 * outlier channel c and sigma = sign(M_c) instead of as the vector d
 * (explainer, paragraph on the sign adjustment: each column j of H is
 * multiplied by the sign of the outlier row's entry, so d_j = sigma * H[c][j]
 * with H the library's unnormalised +-1 matrix).  Computes exactly what
 * signrot_rotate_quant_int4 computes for that d, without reading d or
 * deciding its form on the device: about 1.7 us less per decode-sized call at
 * n = 14336, and under 1 us on a batch of 8192 tokens.
 *
 *   c       the channel signrot_calibrate returns in c_out, 0 <= c < n.
 *   sigma   +1 or -1: the sign of M_c (mc_out), with sign(+-0) = +1.
 *   the other arguments as for signrot_rotate_quant_int4.
 *
 * c outside [0, n) or sigma not +-1 -> SIGNROT_EINVAL; the other errors as
 * for signrot_rotate_quant_int4.  For the widths without a fast kernel, d is
 * built in a stream-ordered n-byte scratch (hipMallocAsync / hipFreeAsync).
 * Asynchronous.
 */
int signrot_rotate_quant_int4_outlier(const void* x_bf16, int64_t tokens, int64_t n, int64_t ld, int64_t c,
                                      int sigma, uint8_t* codes, float* scale, float* zero, float* y_out,
                                      void* stream);

/*
 * A variant with an integer zero-point (the GyRot abstract, on the pages as a
 * related paper: asymmetric quantization reformulated with a rounded
 * zero-point so that dequantization is integer arithmetic times one scale).
 * With the same scale s = (mx - mn) / 15 (1 when mx == mn):
 *   zero = rint(-mn / s), an integer (stored exactly in the float output);
 *   q_j  = clamp(rint(y_j / s) + zero, 0, 15),
 * so y_hat = s * (q - zero) with (q - zero) an integer.  Rounding the
 * zero-point moves the window of 16 levels by at most half a step, so
 * y / s + zero stays in [-0.5, 15.5] and every value is still within s/2 of
 * its level.
 *
 * The sign vector is given as (c, sigma) as for
 * signrot_rotate_quant_int4_outlier; there is no y_out.  Same arguments,
 * alignment and errors as that call.  Asynchronous.
 */
int signrot_rotate_quant_int4_zint(const void* x_bf16, int64_t tokens, int64_t n, int64_t ld, int64_t c, int sigma,
                                   uint8_t* codes, float* scale, float* zero, void* stream);

/*
 * The online path with its producer fused in (explainer, paragraph on the
 * down-projection: the gated nonlinearity between the up/gate projections and
 * the down-projection is why the rotation has to run online).  The
 * down-projection input is computed from the producer's two operands,
 *   x = bf16(SiLU(gate) * up),  SiLU(z) = z / (1 + e^-z),
 * in binary32 and rounded once to bf16 (nearest, ties to even), and then goes
 * through exactly what signrot_rotate_quant_int4_outlier computes for that x;
 * x itself never reaches memory.  (SwiGLU as the gated unit is a reading: the
 * pages name the nonlinearity, not its formula.)  The binary32 SiLU is within
 * about 2e-6 relative of the exact value for |gate| <= 16, so x equals the
 * exactly rounded bf16 value except where that value lies that close to a
 * point halfway between two bf16 numbers.
 *
 *   gate_bf16, up_bf16  device, [tokens][ld] bf16 each, same ld, 16-byte
 *                       aligned; ld >= n, ld % 8 == 0.
 *   c, sigma            the calibrated sign vector, as for
 *                       signrot_rotate_quant_int4_outlier (calibrated on x).
 *   codes, scale, zero, y_out   as for signrot_rotate_quant_int4.
 *
 * Only the widths with a fast kernel: n = 3584, 7168, 14336, 28672, 4096,
 * 8192, 16384; any other supported n -> SIGNROT_EUNSUPPORTED_N.  Other errors
 * as for signrot_rotate_quant_int4_outlier (a null or misaligned up ->
 * SIGNROT_EINVAL).  No allocation.  Asynchronous.
 */
int signrot_swiglu_rotate_quant_int4(const void* gate_bf16, const void* up_bf16, int64_t tokens, int64_t n, int64_t ld,
                                     int64_t c, int sigma, uint8_t* codes, float* scale, float* zero, float* y_out,
                                     void* stream);

/*
 * Dequantization (explainer, paragraph on the 4-bit quantizer: a token's 16
 * levels are spread evenly from its smallest to its largest value, so code q
 * stands for the level mn + q * scale; paragraph on symmetric versus
 * asymmetric quantizers: the asymmetric form carries a zero-point):
 * y_hat[t][j] = scale[t] * (q_j - zero[t]).
 *
 *   codes   device, [tokens][n/2] uint8, as signrot_rotate_quant_int4 or
 *           signrot_rotate_quant_int4_zint writes them.
 *   scale   device, [tokens] float; zero device, [tokens] float.
 *   y_hat   device, [tokens][n] float, 8-byte aligned.
 *
 * n must be supported (SIGNROT_EUNSUPPORTED_N otherwise); a null pointer or a
 * misaligned y_hat (tokens > 0) or tokens < 0 -> SIGNROT_EINVAL.  No
 * allocation.  Asynchronous.
 */
int signrot_dequant(const uint8_t* codes, const float* scale, const float* zero,
                    int64_t tokens, int64_t n, float* y_hat, void* stream);

/*
 * Offline weight fold (explainer, paragraph on the sign adjustment: the same
 * flip is folded into the weights offline; paragraph on rotation: H / sqrt(n)
 * is orthogonal, so rotating both factors of a product leaves it unchanged).
 * For a down-projection out = x . W^T with W [rows][n] (one row per output
 * feature), W' = W . H . D / sqrt(n): every row w of W becomes
 * (w . H / sqrt(n)) (.) d, the very transform applied to the activations, so
 * that out = x' . W'^T with x' = (x . H / sqrt(n)) (.) d.
 *
 *   w_bf16  device, [rows][ld] bf16, 16-byte aligned, ld >= n, ld % 8 == 0.
 *   d       device, [n] int8, 16-byte aligned, entries +1/-1 (the vector
 *           signrot_calibrate produced for the activations).
 *   w_out   device, [rows][n] float, 16-byte aligned.
 *
 * Runs the rotation kernels of signrot_rotate_quant_int4, whose INT4 codes
 * go to a stream-ordered scratch of rows * (n/2 + 8) bytes (hipMallocAsync /
 * hipFreeAsync on `stream`) and are discarded.  Asynchronous.  rows == 0 is a
 * no-op; argument errors as for signrot_rotate_quant_int4.
 */
int signrot_fold_weights(const void* w_bf16, int64_t rows, int64_t n, int64_t ld, const int8_t* d, float* w_out,
                         void* stream);

/*
 * Row sums of a folded weight, rowsum[k] = sum_j w[k][j] (explainer,
 * paragraph on symmetric versus asymmetric quantizers: the zero-point's share
 * of the product is the zero-point times a precomputed sum of the weights).
 * Computed once per weight, offline.
 *
 *   w_bf16  device, [rows][ld] bf16 (W' = W . H . D / sqrt(n) rounded to
 *           bf16), ld >= n; no alignment requirement.
 *   rowsum  device, [rows] float: the exact sum of the bf16 values,
 *           accumulated in binary64 and rounded once.
 *
 * rows == 0 is a no-op; rows < 0, n < 0, ld < n or a null pointer ->
 * SIGNROT_EINVAL.  Any n (the sum does not depend on the Hadamard order).
 * Asynchronous.
 */
int signrot_weight_rowsum(const void* w_bf16, int64_t rows, int64_t n, int64_t ld, float* rowsum, void* stream);

/*
 * The consumer of the INT4 activations: the down-projection on the folded
 * weight, out = yhat . W'^T with yhat = scale * (q - zero), evaluated as
 * (explainer, paragraph on symmetric versus asymmetric quantizers)
 *
 *   out[t][k] = scale[t] * (sum_j q[t][j] * w[k][j] - zero[t] * rowsum[k]),
 *
 * so the product itself runs on the unsigned integer codes.
 *
 *   codes   device, [tokens][n/2] uint8, as signrot_rotate_quant_int4 writes
 *           them (channel 2m in the low nibble of byte m).
 *   scale   device, [tokens] float; zero device, [tokens] float.
 *   w_bf16  device, [rows][ldw] bf16: row k is output feature k of W'.
 *   rowsum  device, [rows] float, from signrot_weight_rowsum.
 *   out     device, [tokens][rows] float.
 *
 * n even and >= 2 (any Hadamard order), ldw >= n.  The MFMA kernel runs when
 * n % 64 == 0, ldw % 8 == 0, rows * ldw < 2^31 and codes and w are 16-byte
 * aligned; other shapes take a plain one-thread-per-output kernel.  The
 * integer-by-bf16 products are exact; they are summed in binary32 (in an
 * order that differs between the two kernels).  tokens == 0 or rows == 0 is a
 * no-op; negative sizes, odd n, ldw < n, tokens or rows >= 2^31 or a null
 * pointer -> SIGNROT_EINVAL.  Asynchronous.
 */
int signrot_int4_linear(const uint8_t* codes, const float* scale, const float* zero, int64_t tokens, int64_t n,
                        const void* w_bf16, int64_t ldw, const float* rowsum, int64_t rows, float* out,
                        void* stream);

/* Which kernel signrot_int4_linear would launch for these operands (a static
 * string), or NULL when the arguments are invalid. */
const char* signrot_int4_linear_kernel_name(const uint8_t* codes, int64_t tokens, int64_t n, const void* w_bf16,
                                            int64_t ldw, int64_t rows);

/*
 * Measurement aid, not part of the method: a kernel that moves the bytes the
 * online path moves per token -- reads the bf16 row (2n bytes), writes n/2
 * bytes to out [tokens][n/2] and one float each to s0 [tokens] and
 * s1 [tokens] -- with no arithmetic (each 16-byte input chunk becomes the XOR
 * of its four words).  Its time is the memory system's ceiling for that
 * read/write mix at the shape.  n a multiple of 8 in [8, 32768], ld >= n and
 * a multiple of 8, tokens * n / 8 < 2^32, x 16-byte and out 4-byte aligned.
 * Asynchronous.
 */
int signrot_stream_ceiling(const void* x_bf16, int64_t tokens, int64_t n, int64_t ld, uint8_t* out, float* s0,
                           float* s1, void* stream);

/* Static text for a status code. */
const char* signrot_strerror(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* signrot_last_error(void);

/*
 * The library's own H28, row-major, entries +1/-1, written to host memory
 * out[784].  Lets a test compare it with an independently built table.
 */
int signrot_debug_h28(int8_t* out);

/*
 * The library's outer factor H_m (m = 28 or any Paley order of the rule above,
 * m <= 512), row-major, entries +1/-1, written to host memory out[m * m].
 * Host-only (no GPU needed).  SIGNROT_EINVAL when m has no construction.
 */
int signrot_debug_outer(int m, int8_t* out);

/*
 * The outer factor the rotate kernel uses when it reads n = m * 2^k as
 * (m 2^fold) * 2^(k - fold): H_m (x) Syl_{2^fold}, entry
 * (a 2^fold + u, a' 2^fold + v) = H_m[a][a'] (-1)^popcount(u & v), with
 * m = 1 (the Sylvester matrix alone), 28, or a Paley order.  Written
 * row-major to host memory out[(m 2^fold)^2].  Host-only.  SIGNROT_EINVAL
 * when m 2^fold > 512 or m has no construction.
 */
int signrot_debug_outer_folded(int m, int fold, int8_t* out);

/* How many Sylvester index bits the rotate kernel for n moves into its outer
 * factor (0: none), or -1 when n is unsupported.  Host-only. */
int signrot_outer_fold(int64_t n);

/* Which kernel variant signrot_rotate_quant_int4 would launch for n (a
 * static string naming it), or NULL when n is unsupported:
 *   "rq_mfma32_w8"   n = 4096, 8192, 16384 (Sylvester);
 *   "rq_mfma28_w7"   n = 28 * 2^k, k = 7, 8, 9;
 *   "rq_mfma28x2_w7" n = 28672 (two halves of the 14336 transform);
 *   "rq_outer_mfma"  n = m * 2^k with 16 <= 2^k <= 256 and ceil(m / 32)
 *                    at most 12, 12, 8, 6, 4 for 2^k = 16, 32, 64, 128, 256
 *                    (11008, 13824, 18944, 8960, 27648, 5120, 5504, 896,
 *                    1792 among them), and widths that reach such a shape
 *                    with Sylvester bits moved into the outer factor (24576,
 *                    20480, 12288, 10240, 6144, 64 .. 2048, 32768; most
 *                    2^k = 256 widths, e.g. 5120 and 17408, run as
 *                    (2 m) * 128);
 *   "rq_generic"     every other supported n.
 * Host-only (no GPU needed). */
const char* signrot_kernel_name(int64_t n);

#ifdef __cplusplus
}
#endif

#endif /* SIGNROT_H */
