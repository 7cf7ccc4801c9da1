/*
 * oracle.h -- plain, slow CPU reference for NVFP4 / MS-EDEN / IF4 quantization
 * and the block-scaled FP4 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library may include, link,
 * load or call this code.  Its users are the test-suite, the smoke check and
 * the CPU-baseline leg of the benchmark.  It shares no header, table, constant
 * or helper with the GPU sources.
 *
 * Arithmetic: IEEE fp32, round-to-nearest-even, one rounding per written
 * operation, no FMA contraction (built with -ffp-contract=off), denormals kept.
 * The GEMM ground truth accumulates in fp64.
 *
 * Parity status of each entry point is stated at its definition in oracle.c.
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element formats */
enum { ORC_FMT_NVFP4 = 0, ORC_FMT_IF4 = 1, ORC_FMT_NVINT4 = 2,
       ORC_FMT_NVFP4_4OVER6 = 3, /* NVFP4 codes, block maximum mapped to 6 or 4   */
       ORC_FMT_NVFP4_SEARCH = 4  /* NVFP4 codes, block scale searched (19 E4M3)   */ };
/* rounding of the E2M1 codes (and, for MS-EDEN, of the block scale) */
enum { ORC_RTN = 0, ORC_SR = 1, ORC_MSEDEN = 2 };

/* status codes */
enum { ORC_OK = 0, ORC_BAD_ARG = -1, ORC_BAD_SHAPE = -2 };

float orc_e2m1_value(int nibble);          /* signed nibble -> value          */
float orc_e4m3_value(int byte);            /* byte -> value (NaN for 0x7F/FF) */
int orc_e4m3_rne_sat(float v);             /* v >= 0 -> byte in [0, 0x7E]     */
int orc_e4m3_ceil_sat(float v);            /* v >= 0 -> byte in [0, 0x7E]     */
int orc_e2m1_rne(float a);                 /* 0 <= a <= 6 -> magnitude 0..7   */
int orc_int4_rne(float a);                 /* 0 <= a <= 7 -> 0..7             */
int orc_sr_e2m1(float a, uint32_t u16);    /* 0 <= a <= 6 -> magnitude 0..7   */
int orc_sr_e4m3(float a, uint32_t u16);    /* 0 <= a <= 448 -> byte           */
float orc_sr_expected_sq(float a, int is_int); /* (a-l)(u-a) on E2M1 / 0..7 */

/* the rules above over consecutive fp32 bit patterns (exhaustive checks) */
void orc_e2m1_rne_run(uint32_t bits_lo, uint64_t count, uint8_t *codes);
void orc_e4m3_run(uint32_t bits_lo, uint64_t count, int ceil_mode, uint8_t *bytes);
void orc_sr_e4m3_pairs(const float *a, const uint16_t *u16, uint64_t n, uint8_t *bytes);

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
uint32_t orc_uniform16(uint64_t seed, uint32_t tag, uint32_t stream, uint64_t idx);

void orc_fwht128(float *v);
void orc_rht128(const float *x, const uint32_t signs[4], float *z);
void orc_irht128(const float *z, const uint32_t signs[4], float *x);
float orc_pairwise_sum(const float *v, int n);

int orc_quantize(const float *x, int64_t rows, int64_t cols, int64_t ld,
                 int format, int rounding, int axis, int rht,
                 const uint32_t signs[4], uint64_t seed, uint32_t stream,
                 int eden_group, const float *ts_in,
                 uint8_t *codes, uint8_t *scales, float *ts_out,
                 float *z_out, float *tb_out);

int orc_dequantize(const uint8_t *codes, const uint8_t *scales, float ts,
                   int64_t rows_out, int64_t k, int format,
                   const uint32_t *inv_signs, float *out);

int orc_gemm_entries(const uint8_t *a_codes, const uint8_t *a_scales, float a_ts,
                     const uint8_t *b_codes, const uint8_t *b_scales, float b_ts,
                     int64_t M, int64_t N, int64_t K, int format,
                     const int64_t *im, const int64_t *in, int64_t count,
                     double *out);

int orc_gemm_full(const uint8_t *a_codes, const uint8_t *a_scales, float a_ts,
                  const uint8_t *b_codes, const uint8_t *b_scales, float b_ts,
                  int64_t M, int64_t N, int64_t K, int format, double *out);

int orc_num_threads(void);
void orc_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
