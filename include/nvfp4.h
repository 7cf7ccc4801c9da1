/*
 * nvfp4.h -- C ABI of libnvfp4: NVFP4 microscaled quantization of training
 * tensors on AMD Instinct MI355X (gfx950), its IF4 variant, dequantization,
 * and the block-scaled FP4 GEMM that consumes the packed operands.
 *
 * Sources (the pages the operations follow):
 *   [QII-abs]  Quartet II: Accurate LLM Pre-Training in NVFP4 by Improved
 *              Unbiased Gradient Estimation, abstract (OpenAlex W7127094184).
 *   [QII-sum]  Quartet II news summary (mind-verse.de), sections
 *              "Kerninnovationen", "Quantisierung im Rueckwaertsdurchlauf",
 *              "Quantisierung im Vorwaertsdurchlauf".
 *   [PAL]      "Comparing INT4 and NVFP4 Palettes on Real Gradient Tensors"
 *              (sethwheeler.dev), opening paragraph and section "The two
 *              corners, and what the palette does to them".
 *   [IF4]      Adaptive Block-Scaled Data Types / IF4 (arXiv 2603.28765),
 *              abstract, Figure 1, Table 1, Figure 3.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named x, codes, scales, tensor_scale, ws, out, a_*, b_*, c are
 *   DEVICE pointers (HIP device memory of the current device).  The
 *   rht_signs / inv_rht_signs arrays are HOST pointers (4 words, read during
 *   the call).  The caller owns every buffer; the library allocates no device
 *   memory and keeps no state between calls.
 * - `stream` is a hipStream_t (NULL = the default stream).  Every entry point
 *   only enqueues work on that stream and returns; it never synchronizes.
 *   Faults inside kernels surface at the caller's next synchronization.
 * - Return value: NVFP4_OK (0) or a negative nvfp4_status.  On error nothing
 *   has been enqueued (validation happens before any launch), except for
 *   NVFP4_HIP_ERROR, which reports a failed launch.  nvfp4_last_error()
 *   returns a thread-local detail string for the last failing call.  The
 *   library never aborts or throws across this interface.
 * - Non-finite inputs, and tensors so small in magnitude that a block scale
 *   times the tensor scale underflows to zero, give unspecified (but
 *   memory-safe) results.
 *
 * Packed layout (the pages fix the format, not the bytes; this layout is the
 * library's own):
 *   codes  [rows_out x K/2] bytes, row-major; element 2j in the low nibble of
 *          byte j, element 2j+1 in the high nibble.  Nibble = sign<<3 | mag.
 *          NVFP4 magnitudes 0..7 index the E2M1 grid {0,.5,1,1.5,2,3,4,6}
 *          [PAL opening paragraph]; IF4 groups flagged INT hold integers 0..7
 *          (sign-magnitude, each value keeps its own sign [IF4 Figure 1]).
 *   scales [rows_out x K/16] bytes, row-major, one E4M3 ("FN": bias 7, max
 *          448, subnormals to 2^-9 [IF4 Table 1]) per 16 consecutive
 *          elements of a row [QII-sum "Quantisierung im Vorwaertsdurchlauf"].
 *          In IF4 output bit 7 is the INT flag [IF4 Figure 1].
 *   tensor_scale  one fp32 on the device [QII-sum, same section].
 *   Dequantized value = sign * (mag_value * (E4M3(scale & 0x7F) * tensor_scale)).
 * Quantization axis: axis 0 groups run along the contiguous dimension of the
 * row-major input x[rows][ld] and rows_out = rows, K = cols; axis 1 groups
 * run along the strided dimension (the reduction dimension of a row-major
 * activation or gradient, for the backward re-quantization of [QII-sum]) and
 * the output is the transpose: rows_out = cols, K = rows.
 * Element index (for the random streams) = row_out * K + k in the output
 * layout; block index = element index / 16.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 5

typedef enum nvfp4_status {
  NVFP4_OK = 0,
  NVFP4_INVALID_ARG = -1,   /* null pointer, bad enum, negative size          */
  NVFP4_BAD_SHAPE = -2,     /* K % 16, K % 128 with rotation/MS-EDEN-128, ld  */
  NVFP4_MISALIGNED = -3,    /* pointer or row stride not aligned as required  */
  NVFP4_WS_TOO_SMALL = -4,  /* workspace smaller than nvfp4_workspace_size()  */
  NVFP4_HIP_ERROR = -5,     /* a kernel launch failed                         */
  NVFP4_UNSUPPORTED = -6    /* valid request this build does not implement    */
} nvfp4_status;

typedef enum nvfp4_dtype { NVFP4_F32 = 0, NVFP4_BF16 = 1 } nvfp4_dtype;

typedef enum nvfp4_rounding {
  NVFP4_RTN = 0,     /* round-to-nearest-even codes, RNE block scales        */
  NVFP4_SR = 1,      /* stochastic element rounding, block scales rounded up */
  NVFP4_MSEDEN = 2   /* MS-EDEN: RTN codes, corrected scales rounded by SR   */
} nvfp4_rounding;

typedef enum nvfp4_format { NVFP4_FORMAT_NVFP4 = 0, NVFP4_FORMAT_IF4 = 1 } nvfp4_format;

/* How an RTN block scale is chosen (nvfp4_quantize_nvfp4 only). */
typedef enum nvfp4_scale_rule {
  NVFP4_SCALE_MAX6 = 0,    /* block maximum mapped to 6: e = E4M3((a/6)/s_t)   */
  NVFP4_SCALE_4OVER6 = 1,  /* Four Over Six: the better of maximum -> 6 and
                              maximum -> 4, s_t = max|z| / (6 * 256)           */
  NVFP4_SCALE_SEARCH = 2   /* the best of the 19 E4M3 scales e0-9 .. e0+9 around
                              the MAX6 byte e0, s_t = max|z| / (6 * 448)       */
} nvfp4_scale_rule;

typedef struct nvfp4_opts {
  int32_t rounding;        /* nvfp4_rounding                                   */
  int32_t axis;            /* 0 or 1, see above                                */
  int32_t rht;             /* 1: 128-point randomized Hadamard rotation first  */
  uint32_t rht_signs[4];   /* bit k of the 128-bit vector = bit k%32 of word
                              k/32; set = negate coordinate k before the
                              transform                                        */
  uint64_t seed;           /* Philox-4x32-10 key                               */
  uint32_t stream;         /* Philox counter word 3 (e.g. a step or trial id)  */
  int32_t eden_group;      /* MS-EDEN correction group: 128 (default) or 16    */
  const float *tensor_scale_in; /* DEVICE pointer to a given fp32 tensor scale
                              (positive and finite, else the codes are
                              unspecified), or NULL to compute it from this
                              tensor                                           */
  int32_t scale_rule;      /* nvfp4_scale_rule; other than MAX6 needs RTN      */
  float *amax_out;         /* DEVICE fp32 or NULL.  MS-EDEN with a computed
                              tensor scale also writes max|x| of the input as
                              given (before any rotation) here.               */
  const float *amax_in;    /* DEVICE fp32 or NULL.  A call without rotation
                              and without tensor_scale_in, other than MS-EDEN,
                              takes max|x| from here instead of reading the
                              input an extra time: s_t = amax_in / (6 * 448),
                              or / (6 * 256) for Four Over Six, 1 if it is 0. */
} nvfp4_opts;

/* Fills *o with defaults: RTN, axis 0, no rotation, seed 0, stream 0,
 * eden_group 128, computed tensor scale, scale rule NVFP4_SCALE_MAX6, no
 * amax_out / amax_in. */
void nvfp4_opts_init(nvfp4_opts *o);

/* Bytes of device workspace the quantizers need for this shape and options
 * (a multiple of 256; the ws pointer must be 256-byte aligned).  Holds
 * per-workgroup partial maxima and, for MS-EDEN, one fp32 target scale per
 * 16 elements. */
size_t nvfp4_workspace_size(int64_t rows, int64_t cols, const nvfp4_opts *o);

/*
 * NVFP4 quantization [QII-sum "Quantisierung im Vorwaertsdurchlauf" (RTN,
 * E4M3 per 16, fp32 per tensor); QII-abs and QII-sum "Quantisierung im
 * Rueckwaertsdurchlauf" (stochastic rounding, randomized Hadamard rotation
 * and MS-EDEN)].  Steps, per tensor:
 *   1. optional rotation z = 2^-3.5 * H_128 * diag(signs) * x of every
 *      128-group along the quantization axis (Sylvester order, stages of
 *      stride 1, 2, ..., 64);
 *   2. RTN/SR: tensor scale s_t = max|z| / (6 * 448) (1 if the tensor is 0);
 *      per 16-block a = max|z|, scale e = E4M3((a/6)/s_t) rounded to nearest
 *      even (RTN) or up (SR); codes = round(min(|z| / (e*s_t), 6)) on the
 *      E2M1 grid, to nearest even (RTN) or stochastically (SR, Philox tag 0,
 *      one 16-bit uniform per element);
 *   3. MS-EDEN: codes by RTN under the exact scale a/6; per correction group
 *      c = sum z^2 / sum z*zhat; target t = (a/6)*c; s_t = max t / 448;
 *      scale e = SR of min(t/s_t, 448) onto the E4M3 grid (Philox tag 1,
 *      one uniform per block).
 *   4. RTN with scale_rule NVFP4_SCALE_4OVER6 (Four Over Six, the local
 *      scaling option of the forward pass [QII-sum "Quantisierung im
 *      Vorwaertsdurchlauf"; IF4 Table 1, row "NVFP4 (4/6)"]): s_t =
 *      max|z| / (6 * 256); every block is coded by RTN twice, with
 *      e = E4M3((a/6)/s_t) and with e = E4M3((a/4)/s_t), and keeps the one
 *      with the smaller pairwise sum of squared errors (ties keep a/6).
 *      Output is plain NVFP4 (dequantize with NVFP4_FORMAT_NVFP4).
 *   5. RTN with scale_rule NVFP4_SCALE_SEARCH (a searched block scale [PAL
 *      "The two corners, and what the palette does to them"; the ScaleSearch
 *      abstract among the IF4 page's related papers]): s_t as in 2; every
 *      block is coded by RTN at the scale bytes e0, e0-1, e0+1, ..., e0-9,
 *      e0+9 (e0 = E4M3((a/6)/s_t); bytes outside 1..126 skipped) and keeps
 *      the first with a strictly smaller pairwise sum of squared errors.
 *      Output is plain NVFP4.
 * x: device, in_dtype elements, row-major with leading dimension ld >= cols
 * (elements).  axis 0 needs a 16-byte aligned base and ld * sizeof(elem) a
 * multiple of 16; axis 1 needs only element alignment (16-byte aligned rows
 * are loaded with vector loads, others element by element) and a row stride
 * ld * sizeof(elem) of at most 16 MiB (else NVFP4_UNSUPPORTED).
 * codes / scales: device, 16-byte aligned, sizes as in the layout above.
 * tensor_scale: device fp32 written with s_t (copied from tensor_scale_in if
 * given).  ws: device workspace of at least nvfp4_workspace_size() bytes,
 * 256-byte aligned; its contents on entry are ignored.
 * Shape rules: K % 16 == 0; K % 128 == 0 with rotation or MS-EDEN group 128.
 * Tensor maximum handed between calls (the training step quantizes X and W
 * row-wise for the forward product and column-wise for the weight and input
 * gradients; the maximum the tensor scale of the row-wise RTN needs is a
 * by-product of the column-wise MS-EDEN pass over the same tensor):
 * o->amax_out (MS-EDEN, tensor scale computed) receives max|x|, ready when
 * the call's work on the stream is; o->amax_in (no rotation, no
 * tensor_scale_in, not MS-EDEN) replaces the pass that finds it -- the
 * results are those of the call without it when *amax_in is the input's
 * max|x|.  Other combinations: NVFP4_UNSUPPORTED; either pointer not 4-byte
 * aligned: NVFP4_MISALIGNED.  An empty tensor writes 0 to amax_out and takes
 * the tensor scale 1 whatever amax_in holds.
 */
int nvfp4_quantize_nvfp4(const void *x, int in_dtype, int64_t rows, int64_t cols, int64_t ld,
                         const nvfp4_opts *o, uint8_t *codes, uint8_t *scales,
                         float *tensor_scale, void *ws, size_t ws_bytes, void *stream);

/*
 * MS-EDEN of one tensor along both axes from a single read of it: the
 * backward pass re-quantizes the output gradient row-wise (for the input
 * gradient) and along its reduction dimension (for the weight gradient)
 * [QII-sum "Quantisierung im Rueckwaertsdurchlauf"].  The results are those
 * of two nvfp4_quantize_nvfp4 calls with these options and axis 0 (codes_r,
 * scales_r, ts_r: [rows x cols/2], [rows x cols/16]) and axis 1 (codes_c,
 * scales_c, ts_c: [cols x rows/2], [cols x rows/16]); o->axis is ignored,
 * o->rounding must be NVFP4_MSEDEN, and each output has its own tensor scale
 * (both equal *o->tensor_scale_in when it is given).  Both axes must meet the
 * shape rules (multiples of 16, of 128 with rotation or group 128), rows must
 * be a multiple of 128 in any case (NVFP4_BAD_SHAPE), and x must meet the
 * axis-0 alignment and the axis-1 stride limit.  ws: at least nvfp4_workspace_size_dual() bytes,
 * 256-byte aligned.
 */
int nvfp4_quantize_nvfp4_dual(const void *x, int in_dtype, int64_t rows, int64_t cols, int64_t ld,
                              const nvfp4_opts *o, uint8_t *codes_r, uint8_t *scales_r, float *ts_r,
                              uint8_t *codes_c, uint8_t *scales_c, float *ts_c, void *ws,
                              size_t ws_bytes, void *stream);

/*
 * nvfp4_quantize_nvfp4 without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The library's own scratch array of
 * NVFP4_NOALLOC_SCRATCH_BYTES per GPU (reserved when the library's device
 * code is loaded on that GPU, and held until the process ends) stands in for
 * the workspace; the call itself allocates nothing.  Results, arguments and
 * errors are those of nvfp4_quantize_nvfp4; a call whose
 * nvfp4_workspace_size() exceeds the scratch (MS-EDEN with a computed tensor
 * scale on more than 24 * 2^20 blocks, about 403 M elements) returns
 * NVFP4_UNSUPPORTED before anything is enqueued.  Every call on one GPU
 * shares that GPU's scratch: calls that overlap on one GPU (on different
 * streams, or from several host threads) race and give unspecified results;
 * calls ordered on one stream do not.
 */
#define NVFP4_NOALLOC_SCRATCH_BYTES ((size_t)16384 + ((size_t)96 << 20))
int nvfp4_quantize_nvfp4_noalloc(const void *x, int in_dtype, int64_t rows, int64_t cols, int64_t ld,
                                 const nvfp4_opts *o, uint8_t *codes, uint8_t *scales,
                                 float *tensor_scale, void *stream);

/* Workspace bytes of nvfp4_quantize_nvfp4_dual (both axes' workspaces). */
size_t nvfp4_workspace_size_dual(int64_t rows, int64_t cols, const nvfp4_opts *o);

/*
 * IF4 quantization [IF4 abstract, Figure 1, Figure 3]: every 16-group is
 * coded two ways, as NVFP4 (E2M1 levels) and as scaled INT4 (integers 0..7),
 * and keeps the better one; the INT choice sets bit 7 of the scale byte.
 * Same arguments, options and layout rules as nvfp4_quantize_nvfp4 (scale
 * rule MAX6 only); o->rounding selects how:
 *   RTN: E2M1 under the RNE scale of a/6, integers under the RNE scale of
 *     a/7 (both RNE), keep the smaller pairwise sum of squared errors (ties
 *     keep FP4); s_t = max|z| / (6 * 448).
 *   SR (gradients; IF4 Figure 4): both branches as NVFP4 SR, scales rounded
 *     up from a/6 and from a/7, elements rounded stochastically (Philox tag
 *     0, the element's uniform whichever branch is kept); the branch is
 *     chosen before rounding, by the smaller expected squared error
 *     (S*S) * sum (y - l)(u - y) [PAL opening paragraph], ties FP4;
 *     s_t = max|z| / (6 * 448).
 *   MSEDEN (gradients; IF4 Figure 4 with QII-abs): RTN codes in both branches
 *     under the exact scales a/6 and a/7, keep the smaller pairwise squared
 *     error (ties FP4); the correction c = sum z^2 / sum z*zhat over the
 *     correction group uses the kept reconstructions; target t = (kept
 *     exact scale) * c, s_t = max t / 448, scale = SR of t/s_t onto E4M3
 *     (Philox tag 1) with the flag in bit 7.  amax_out as for NVFP4 MS-EDEN.
 */
int nvfp4_quantize_if4(const void *x, int in_dtype, int64_t rows, int64_t cols, int64_t ld,
                       const nvfp4_opts *o, uint8_t *codes, uint8_t *scales,
                       float *tensor_scale, void *ws, size_t ws_bytes, void *stream);

/*
 * Dequantization [PAL opening paragraph (the sixteen E2M1 values and the
 * per-block scale they are multiplied by); IF4 Figure 1 (a block flagged INT
 * in the scale's sign bit holds integers instead of E2M1 values); QII-sum
 * "Quantisierung im Vorwaertsdurchlauf" (E4M3 block scale times the fp32
 * tensor scale)]: out[r][k] =
 * sign * (v * (E4M3(scale & 0x7F) * tensor_scale)), v the E2M1 value or, for
 * IF4 groups with bit 7 set, the integer magnitude; then, if inv_rht_signs is
 * not NULL, the inverse rotation signs * (2^-3.5 * H_128 * z) of every
 * 128-group.  codes/scales/tensor_scale: device, as produced above;
 * inv_rht_signs: HOST, 4 words, or NULL.  out: device, [rows_out x k],
 * out_dtype (fp32, or bf16 rounded to nearest even), 16-byte aligned.
 * k % 16 == 0 (k % 128 == 0 with inverse rotation).
 */
int nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales, const float *tensor_scale,
                     int64_t rows_out, int64_t k, int format, const uint32_t *inv_rht_signs,
                     int out_dtype, void *out, void *stream);

/*
 * Block-scaled FP4 GEMM [QII-sum "Kerninnovationen" (NVFP4 GEMMs for linear
 * layers); QII-abs]:  C[M x N] = (ts_a * ts_b) * sum_k A[m][k] * B[n][k], with
 * A[m][k] = E2M1(code) * E4M3(scale) taken exactly, both operands K-major
 * packed NVFP4 as produced by nvfp4_quantize_nvfp4 (A: rows_out = M, B:
 * rows_out = N, both with the same K).  Accumulation in fp32 on the matrix
 * cores; the dequantized operands are exact in fp16, so the only rounding is
 * the accumulation's.  c: device, [M x ldc] row-major, out_dtype fp32 or bf16,
 * ldc >= N.  a_ts, b_ts: device fp32 tensor scales.  K % 16 == 0 and
 * K <= 16777200 (else NVFP4_UNSUPPORTED); codes and scales 16-byte aligned.
 * Operands must be NVFP4: this entry point reads every scale byte as an E4M3
 * value, so IF4 output (bit 7 = INT flag) gives wrong results here; use
 * nvfp4_gemm_if4 for it.
 */
int nvfp4_gemm_nvfp4(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_ts,
                     const uint8_t *b_codes, const uint8_t *b_scales, const float *b_ts,
                     int64_t M, int64_t N, int64_t K, void *c, int out_dtype, int64_t ldc,
                     void *stream);

/*
 * The same GEMM on IF4 operands [IF4 abstract, Figure 1; the IF4 page also
 * describes an IF4 multiply-accumulate unit, Figure 6]: a block whose scale
 * byte has bit 7 set holds sign-magnitude integers 0..7 (value
 * +-q * E4M3(scale & 0x7F)), any other block E2M1 codes.  NVFP4 operands are
 * valid IF4 operands (no flags), so either operand may be either format, as
 * produced by nvfp4_quantize_if4 or nvfp4_quantize_nvfp4.  Arguments, layout,
 * accuracy and errors as nvfp4_gemm_nvfp4.
 */
int nvfp4_gemm_if4(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_ts,
                   const uint8_t *b_codes, const uint8_t *b_scales, const float *b_ts,
                   int64_t M, int64_t N, int64_t K, void *c, int out_dtype, int64_t ldc,
                   void *stream);

/*
 * The NVFP4 GEMM with its output coded as NVFP4 in the same kernel [QII-sum
 * "Quantisierung im Vorwaertsdurchlauf" (RTN, one E4M3 scale per 16
 * elements, one fp32 scale per tensor); QII-abs (every linear-layer operand
 * in NVFP4)]: C = (ts_a * ts_b) * A_hat @ B_hat^T as in nvfp4_gemm_nvfp4,
 * then each row of C coded along N exactly as nvfp4_quantize_nvfp4 codes an
 * fp32 input with rounding RTN, axis 0, no rotation and tensor_scale_in =
 * c_ts: scale byte e = E4M3_RNE((max|block| / 6) / s_t), codes of
 * c / (E4M3(e) * s_t) on the E2M1 grid, round to nearest even.  The result
 * is the next layer's NVFP4 input without writing or re-reading C.
 * c_ts: DEVICE fp32, the tensor scale to code with (max |C| is not known
 * before C is computed, so it comes from the caller, e.g. from c_amax of an
 * earlier step divided by 6 * 448); it must be positive and finite, else
 * the codes are unspecified (the value is on the device, so no error is
 * returned for it).  c_codes: DEVICE [M x N/2] bytes,
 * c_scales: DEVICE [M x N/16] bytes, both 16-byte aligned, as the
 * quantizer's output for rows_out = M, K = N.  c_amax: DEVICE fp32 or NULL;
 * receives max |C| over all entries (cleared by the call itself).
 * Operands: NVFP4 only (IF4 blocks are read as E4M3 scales).  N % 16 == 0
 * (else NVFP4_BAD_SHAPE); other shapes, limits and errors as
 * nvfp4_gemm_nvfp4.  Codes can differ from coding the fp64 product where an
 * fp32 entry lies within accumulation error of a rounding boundary.
 */
int nvfp4_gemm_nvfp4_rtn(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_ts,
                         const uint8_t *b_codes, const uint8_t *b_scales, const float *b_ts,
                         int64_t M, int64_t N, int64_t K, const float *c_ts, uint8_t *c_codes,
                         uint8_t *c_scales, float *c_amax, void *stream);

/*
 * The randomized Hadamard rotation alone [QII-sum "Quantisierung im
 * Rueckwaertsdurchlauf" (the backward operands are rotated along the
 * micro-scaling groups before MS-EDEN); PAL opening paragraph (a random
 * sign flip followed by a Hadamard transform)], for checking it:
 * out[rows_out x K] fp32 = the rotated values of step 1 of
 * nvfp4_quantize_nvfp4, in the output layout of `axis`: for bf16 input the
 * product with the +-1 matrix H diag(signs) on the matrix cores (exact
 * products, fp32 sums), for fp32 input (and bf16 columns whose rows are not
 * 16-byte aligned) the butterfly stages in Sylvester order; then times
 * fp32(1/sqrt(128)).  The two evaluations of the same sums agree to fp32
 * rounding of the partial sums.
 * Same x rules; K % 128 == 0; out device, 16-byte aligned.
 */
int nvfp4_rht(const void *x, int in_dtype, int64_t rows, int64_t cols, int64_t ld, int axis,
              const uint32_t *rht_signs, float *out, void *stream);

const char *nvfp4_status_string(int status);
const char *nvfp4_last_error(void);
int nvfp4_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_H */
