/*
 * oracle.c -- plain, slow CPU reference for NVFP4 microscaled quantization
 * (randomized Hadamard rotation, RTN, stochastic rounding, MS-EDEN), the IF4
 * per-group FP4/INT4 selection, dequantization and the block-scaled FP4 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
 * CPU-baseline leg are its only users.  The product library never includes,
 * links or calls it, and it shares no code with the GPU sources.
 *
 * Sources (the pages this follows), cited below by these short names:
 *   [QII-abs]  Quartet II: Accurate LLM Pre-Training in NVFP4 by Improved
 *              Unbiased Gradient Estimation -- abstract (OpenAlex W7127094184).
 *   [QII-sum]  Quartet II news summary (mind-verse.de), sections
 *              "Kerninnovationen", "Quantisierung im Rueckwaertsdurchlauf",
 *              "Quantisierung im Vorwaertsdurchlauf".
 *   [PAL]      "Comparing INT4 and NVFP4 Palettes on Real Gradient Tensors"
 *              (sethwheeler.dev): opening paragraph; section "The two corners,
 *              and what the palette does to them".
 *   [IF4]      Adaptive Block-Scaled Data Types / IF4 (arXiv 2603.28765, page
 *              on thelatestinai.com): abstract, Figure 1, Table 1, Figure 3.
 *   [Philox]   Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
 *              as 1, 2, 3", SC'11 -- the Philox-4x32 bijection (published
 *              method; the pages do not fix a generator).
 *
 * Arithmetic: fp32 with one rounding per written operation (compiled with
 * -ffp-contract=off), denormals kept.  Where the pages leave a step open the
 * plainest reading is taken; each is marked READING.
 *
 * Parity pins (what each function is checked against, outside itself) are
 * listed at each function.  Every function here is pinned.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads the parallel loops below use from now on (the CPU baseline times
 * the oracle on one thread and on all of them). */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ======================================================================
 * Element and scale formats
 * ==================================================================== */

/* E2M1 magnitudes by 3-bit code: the sixteen values of the FP4 menu are
 * {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6} [PAL opening paragraph].
 * Code = sign<<3 | magnitude code.
 * Pinned by: the grid fixture from [PAL]; gap ratio 4 from [PAL]. */
static const float GRID_E2M1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

float orc_e2m1_value(int nibble) {
  float m = GRID_E2M1[nibble & 7];
  return (nibble & 8) ? -m : m;
}

/* E4M3 (OCP "FN" variant): sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, no infinities, 0x7F/0xFF are NaN.  Largest finite 448 and smallest
 * subnormal 2^-9 are what [IF4 Table 1] prints ("6 x 448", "0.5 x 2^-9").
 * Pinned by: max 448, min 2^-9, 126 positive finite values. */
float orc_e4m3_value(int byte) {
  int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
  float v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexpf((float)m, -9);               /* m/8 * 2^(1-7) */
  else
    v = ldexpf(1.0f + (float)m / 8.0f, e - 7);
  return s ? -v : v;
}

/* The 127 non-negative finite E4M3 values, ascending, indexed by byte. */
static float e4m3_pos(int byte) { return orc_e4m3_value(byte); }

/* Largest j in [0, n-1) with grid(j) <= v (grid ascending, grid(0) <= v). */
static int floor_index_e4m3(float v) {
  int lo = 0, hi = 126; /* invariant: value(lo) <= v < value(hi) or hi==126 */
  if (v >= e4m3_pos(126)) return 126;
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (e4m3_pos(mid) <= v) lo = mid; else hi = mid;
  }
  return lo;
}

/* READING (block-scale rounding for RTN and IF4): nearest E4M3 value, ties to
 * the even mantissa, saturating at 448 (no infinities in E4M3 "FN"). */
int orc_e4m3_rne_sat(float v) {
  if (!(v > 0.0f)) return 0;
  if (v >= 448.0f) return 0x7E;
  int j = floor_index_e4m3(v);
  float lo = e4m3_pos(j), hi = e4m3_pos(j + 1);
  float dl = v - lo, dh = hi - v;
  if (dl < dh) return j;
  if (dh < dl) return j + 1;
  return (j & 1) ? j + 1 : j;
}

/* READING (block-scale rounding for elementwise SR): round the scale UP, so
 * that no element of the block lands above the top grid point -- the SR
 * corner of [PAL] scales each block so that nothing clips.  Saturates at 448. */
int orc_e4m3_ceil_sat(float v) {
  if (!(v > 0.0f)) return 0;
  if (v >= 448.0f) return 0x7E;
  int j = floor_index_e4m3(v);
  return (e4m3_pos(j) == v) ? j : j + 1;
}

/* READING (E2M1 round-to-nearest): nearest grid value, ties to the code with
 * an even mantissa bit (0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4,
 * 5->4).  Input is a magnitude already clipped to [0, 6]. */
int orc_e2m1_rne(float a) {
  int j = 0;
  if (a >= 6.0f) return 7;
  while (j < 7 && GRID_E2M1[j + 1] <= a) j++;
  float dl = a - GRID_E2M1[j], dh = GRID_E2M1[j + 1] - a;
  if (dl < dh) return j;
  if (dh < dl) return j + 1;
  return (j & 1) ? j + 1 : j;
}

/* Scaled-INT4 magnitudes 0..7 [IF4 Table 1, NVINT4 row: max 7, min 1].
 * Round to nearest integer, ties to even; input clipped to [0, 7]. */
int orc_int4_rne(float a) {
  if (a >= 7.0f) return 7;
  float f = floorf(a);
  float frac = a - f;
  int q = (int)f;
  if (frac > 0.5f) q += 1;
  else if (frac == 0.5f && (q & 1)) q += 1;
  return q;
}

/* Stochastic rounding onto an ascending grid (elementwise SR of [QII-abs],
 * [QII-sum]; unbiased: it rounds up with probability (a-l)/(u-l) [PAL]).
 * READING (uniforms): a 16-bit uniform u; round up iff u < p * 65536, where
 * p = (a - l)/(u - l).  Every grid gap here is a power of two, so p is exact.
 * A value at the top of the grid keeps it.
 * Pinned by: exact enumeration of all 65536 uniforms against the closed form
 * E[(q - a)^2] = (a - l)(u - a) of [PAL]. */
static int sr_on_grid(const float *grid, int n, float a, uint32_t u16) {
  if (a >= grid[n - 1]) return n - 1;
  int j = 0;
  while (j < n - 1 && grid[j + 1] <= a) j++;
  float lo = grid[j], hi = grid[j + 1];
  float p = (a - lo) / (hi - lo);
  return ((float)u16 < p * 65536.0f) ? j + 1 : j;
}

int orc_sr_e2m1(float a, uint32_t u16) { return sr_on_grid(GRID_E2M1, 8, a, u16); }

int orc_sr_e4m3(float a, uint32_t u16) {
  if (!(a > 0.0f)) return 0;
  if (a >= 448.0f) return 0x7E;
  int j = floor_index_e4m3(a);
  float lo = e4m3_pos(j), hi = e4m3_pos(j + 1);
  float p = (a - lo) / (hi - lo);
  return ((float)u16 < p * 65536.0f) ? j + 1 : j;
}

/* Scaled-INT4 magnitudes as a grid, for stochastic rounding onto integers. */
static const float GRID_INT4[8] = {0.0f, 1.0f, 2.0f, 3.0f, 4.0f, 5.0f, 6.0f, 7.0f};

/* Expected squared error, in grid units, of stochastically rounding a onto
 * an ascending grid: (a - l)(u - a) with l <= a < u the bracketing points
 * [PAL opening paragraph: SR's error for a value between two levels]; 0 at
 * the top of the grid, which a value there keeps.
 * Pinned by: exact enumeration of all 65536 uniforms of sr_on_grid. */
static float sr_expected_sq(const float *grid, int n, float a) {
  if (a >= grid[n - 1]) return 0.0f;
  int j = 0;
  while (j < n - 1 && grid[j + 1] <= a) j++;
  return (a - grid[j]) * (grid[j + 1] - a);
}

float orc_sr_expected_sq(float a, int is_int) {
  return sr_expected_sq(is_int ? GRID_INT4 : GRID_E2M1, 8, a);
}

/* Array forms of the rules above, over a run of consecutive fp32 bit
 * patterns (bits_lo, bits_lo + 1, ...), for the exhaustive comparison with
 * the device's conversions: no arithmetic beyond the functions they loop.
 *   codes: the nibble of an RTN-coded value y as the block coding below
 *          forms it, sign<<3 | E2M1_RNE(min(|y|, 6)), two per byte (even
 *          pattern in the low nibble); count even.
 *   bytes: E4M3 byte of v by RNE (ceil_mode 0) or rounded up (1). */
void orc_e2m1_rne_run(uint32_t bits_lo, uint64_t count, uint8_t *codes) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)(count / 2); i++) {
    int nib[2];
    for (int j = 0; j < 2; j++) {
      uint32_t b = bits_lo + (uint32_t)(2 * i + j);
      float y;
      memcpy(&y, &b, sizeof(y));
      nib[j] = (signbit(y) ? 8 : 0) | orc_e2m1_rne(fminf(fabsf(y), 6.0f));
    }
    codes[i] = (uint8_t)(nib[0] | (nib[1] << 4));
  }
}

void orc_e4m3_run(uint32_t bits_lo, uint64_t count, int ceil_mode, uint8_t *bytes) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)count; i++) {
    uint32_t b = bits_lo + (uint32_t)i;
    float v;
    memcpy(&v, &b, sizeof(v));
    bytes[i] = (uint8_t)(ceil_mode ? orc_e4m3_ceil_sat(v) : orc_e4m3_rne_sat(v));
  }
}

/* The scale rounding of MS-EDEN's second half over given pairs:
 * bytes[i] = orc_sr_e4m3(a[i], u16[i]) (exhaustive and boundary checks of
 * the device's form; no arithmetic beyond the function it loops). */
void orc_sr_e4m3_pairs(const float *a, const uint16_t *u16, uint64_t n, uint8_t *bytes) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; i++) bytes[i] = (uint8_t)orc_sr_e4m3(a[i], u16[i]);
}

/* ======================================================================
 * Counter-based RNG: Philox-4x32 with 10 rounds [Philox].
 * Each round multiplies words 0 and 2 by the two round multipliers, swaps
 * in the high halves XORed with the other words and the round key; the key
 * advances by the two Weyl increments between rounds.
 * Pinned by: the published known-answer vectors.
 * ==================================================================== */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; round++) {
    if (round > 0) { k0 += W0; k1 += W1; }
    uint64_t p0 = (uint64_t)M0 * (uint64_t)x0;
    uint64_t p1 = (uint64_t)M1 * (uint64_t)x2;
    uint32_t y0 = (uint32_t)(p1 >> 32) ^ x1 ^ k0;
    uint32_t y1 = (uint32_t)p1;
    uint32_t y2 = (uint32_t)(p0 >> 32) ^ x3 ^ k1;
    uint32_t y3 = (uint32_t)p0;
    x0 = y0; x1 = y1; x2 = y2; x3 = y3;
  }
  out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* READING (RNG keying): key = seed (lo, hi words); counter = (idx>>3 lo,
 * idx>>3 hi, tag, stream).  One Philox call yields eight 16-bit uniforms;
 * uniform number (idx & 7) is half (idx & 1) of word (idx & 7) >> 1.
 * tag 0 draws element roundings, tag 1 draws MS-EDEN scale roundings;
 * idx is the element (tag 0) or block (tag 1) index in the output layout. */
uint32_t orc_uniform16(uint64_t seed, uint32_t tag, uint32_t stream, uint64_t idx) {
  uint64_t call = idx >> 3;
  uint32_t ctr[4] = {(uint32_t)call, (uint32_t)(call >> 32), tag, stream};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t w[4];
  orc_philox4x32_10(ctr, key, w);
  uint32_t word = w[(idx & 7) >> 1];
  return (word >> (16 * (idx & 1))) & 0xFFFFu;
}

/* ======================================================================
 * Randomized Hadamard rotation along the micro-scaling groups
 * [QII-sum "Quantisierung im Rueckwaertsdurchlauf"; PAL opening paragraph].
 * READING: 128-point Sylvester Hadamard in natural order, applied after a
 * per-coordinate sign flip, normalized by fp32(1/sqrt(128)).  The fast
 * transform runs stages of stride 1, 2, 4, ..., 64; each butterfly maps
 * (a, b) -> (a + b, a - b) with a the lower index.
 * Pinned by: H H^T = 128 I and H[i][j] = (-1)^popcount(i & j) (textbook
 * Sylvester form), norm preservation, round trip, inner products of pairs
 * rotated with the same signs.
 * ==================================================================== */
void orc_fwht128(float *v) {
  for (int h = 1; h < 128; h *= 2)
    for (int i = 0; i < 128; i += 2 * h)
      for (int j = i; j < i + h; j++) {
        float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
}

static float rht_norm(void) { return (float)(1.0 / sqrt(128.0)); }

static int sign_bit(const uint32_t signs[4], int k) { return (signs[k >> 5] >> (k & 31)) & 1; }

void orc_rht128(const float *x, const uint32_t signs[4], float *z) {
  float w[128];
  for (int k = 0; k < 128; k++) w[k] = sign_bit(signs, k) ? -x[k] : x[k];
  orc_fwht128(w);
  const float c = rht_norm();
  for (int k = 0; k < 128; k++) z[k] = w[k] * c;
}

void orc_irht128(const float *z, const uint32_t signs[4], float *x) {
  float w[128];
  for (int k = 0; k < 128; k++) w[k] = z[k];
  orc_fwht128(w);
  const float c = rht_norm();
  for (int k = 0; k < 128; k++) {
    float u = w[k] * c;
    x[k] = sign_bit(signs, k) ? -u : u;
  }
}

/* READING (reduction order): pairwise binary tree over the indices in their
 * natural order, sum(v[0..n)) = sum(first half) + sum(second half). */
float orc_pairwise_sum(const float *v, int n) {
  if (n == 1) return v[0];
  return orc_pairwise_sum(v, n / 2) + orc_pairwise_sum(v + n / 2, n - n / 2);
}

/* ======================================================================
 * Quantization
 * ==================================================================== */

static void put_nibble(uint8_t *codes_row, int64_t k, int nib) {
  if (k & 1) codes_row[k >> 1] = (uint8_t)((codes_row[k >> 1] & 0x0F) | (nib << 4));
  else codes_row[k >> 1] = (uint8_t)((codes_row[k >> 1] & 0xF0) | nib);
}

/* NVFP4 with round-to-nearest (forward pass [QII-sum "Quantisierung im
 * Vorwaertsdurchlauf"]: one E4M3 scale per 16 elements under an fp32 tensor
 * scale) or elementwise stochastic rounding.  One 16-block:
 *   a_b = max |z|;  v = (a_b / 6) / s_t;  e = E4M3(v) (RNE for RTN, ceil for SR)
 *   S = value(e) * s_t;  y = z * (1 / S);  magnitude = round(min(|y|, 6)).
 * Pinned by: Table 1 MSE of NVFP4 on N(0,1) data [IF4 Table 1]; SR closed
 * form [PAL]; brute-force per-element nearest search. */
static void nvfp4_block(const float *z, float s_t, int rounding, uint64_t seed,
                        uint32_t stream, uint64_t idx0, uint8_t *codes_row,
                        int64_t k0, uint8_t *scale_out) {
  float a = 0.0f;
  for (int i = 0; i < 16; i++) a = fmaxf(a, fabsf(z[i]));
  float v = (a / 6.0f) / s_t;
  int e = (rounding == ORC_SR) ? orc_e4m3_ceil_sat(v) : orc_e4m3_rne_sat(v);
  *scale_out = (uint8_t)e;
  float r = 0.0f;
  if (e != 0) r = 1.0f / (orc_e4m3_value(e) * s_t);
  for (int i = 0; i < 16; i++) {
    int mag = 0;
    if (e != 0) {
      float y = fminf(fabsf(z[i] * r), 6.0f);
      if (rounding == ORC_SR)
        mag = orc_sr_e2m1(y, orc_uniform16(seed, 0, stream, idx0 + (uint64_t)i));
      else
        mag = orc_e2m1_rne(y);
    }
    put_nibble(codes_row, k0 + i, (signbit(z[i]) ? 8 : 0) | mag);
  }
}

/* One candidate coding of a 16-block: returns the scale byte, writes nibbles
 * into nib[], and the pairwise sum of squared errors into *sse.  The block
 * maximum is mapped to `top`:
 *   fp branch of IF4 and NVFP4: E2M1 values, top 6;
 *   int branch of IF4: integers 0..7, top 7 (the NVINT4 row of [IF4 Table 1],
 *   maximum 7 x 448);
 *   second candidate of Four Over Six: E2M1 values, top 4.
 * Magnitudes are clamped to the largest code (6 or 7). */
static int block_candidate(const float *z, float s_t, int is_int, float top, int nib[16],
                           float *sse) {
  float a = 0.0f;
  for (int i = 0; i < 16; i++) a = fmaxf(a, fabsf(z[i]));
  float vmax = is_int ? 7.0f : 6.0f;
  int e = orc_e4m3_rne_sat((a / top) / s_t);
  float S = orc_e4m3_value(e) * s_t;
  float r = (e != 0) ? 1.0f / S : 0.0f;
  float sq[16];
  for (int i = 0; i < 16; i++) {
    int mag = 0;
    if (e != 0) {
      float y = fminf(fabsf(z[i] * r), vmax);
      mag = is_int ? orc_int4_rne(y) : orc_e2m1_rne(y);
    }
    float val = is_int ? (float)mag : GRID_E2M1[mag];
    if (signbit(z[i])) val = -val;
    float d = z[i] - val * S;
    sq[i] = d * d;
    nib[i] = (signbit(z[i]) ? 8 : 0) | mag;
  }
  *sse = orc_pairwise_sum(sq, 16);
  return e;
}

/* IF4: quantize the 16-group both ways and keep the one with the smaller
 * squared error; the choice is the otherwise unused sign bit of the E4M3
 * scale (set = scaled INT4) [IF4 abstract, Figure 1, Figure 3].
 * READING: the INT branch has its own E4M3 scale a/7 under the shared tensor
 * scale; ties keep FP4; INT nibbles are sign-magnitude (each value keeps its
 * own sign bit [IF4 Figure 1]).
 * Pinned by: Table 1 MSE of IF4 and NVINT4 on N(0,1) [IF4 Table 1];
 * brute-force minimum over both branches on small blocks. */
static void if4_block(const float *z, float s_t, int format, uint8_t *codes_row,
                      int64_t k0, uint8_t *scale_out) {
  int nf[16], ni[16];
  float sse_f = 0.0f, sse_i = 0.0f;
  int ei = block_candidate(z, s_t, 1, 7.0f, ni, &sse_i);
  if (format == ORC_FMT_NVINT4) {
    *scale_out = (uint8_t)ei;
    for (int i = 0; i < 16; i++) put_nibble(codes_row, k0 + i, ni[i]);
    return;
  }
  int ef = block_candidate(z, s_t, 0, 6.0f, nf, &sse_f);
  int use_int = sse_i < sse_f;
  *scale_out = (uint8_t)(use_int ? (ei | 0x80) : ef);
  for (int i = 0; i < 16; i++) put_nibble(codes_row, k0 + i, use_int ? ni[i] : nf[i]);
}

/* One stochastic-rounding candidate of a 16-block: the scale byte e =
 * E4M3 rounded up of (a/top)/s_t (so that nothing clips, as for NVFP4 SR),
 * S = value(e) * s_t, y_i = min(|z_i| / S, top), and the closed-form expected
 * squared error of the block, (S * S) * pairwise sum of (y - l)(u - y). */
static int sr_candidate(const float *z, float s_t, int is_int, float y[16], float *ese) {
  const float top = is_int ? 7.0f : 6.0f;
  const float *grid = is_int ? GRID_INT4 : GRID_E2M1;
  float a = 0.0f;
  for (int i = 0; i < 16; i++) a = fmaxf(a, fabsf(z[i]));
  int e = orc_e4m3_ceil_sat((a / top) / s_t);
  float S = orc_e4m3_value(e) * s_t;
  float r = (e != 0) ? 1.0f / S : 0.0f;
  float d[16];
  for (int i = 0; i < 16; i++) {
    y[i] = (e != 0) ? fminf(fabsf(z[i] * r), top) : 0.0f;
    d[i] = sr_expected_sq(grid, 8, y[i]);
  }
  *ese = (S * S) * orc_pairwise_sum(d, 16);
  return e;
}

/* IF4 with stochastic rounding, for gradients [IF4 page, Figure 4: IF4 also
 * pays in the backward pass, more so with MS-EDEN; IF4 abstract and Figure 1
 * for the per-16 FP4/INT4 choice in the scale's sign bit; PAL opening
 * paragraph for SR and its error (y - l)(u - y)].
 * READING: both branches are NVFP4-SR-like: E4M3 scale rounded up from a/6
 * (E2M1 grid) and from a/7 (integers 0..7) under the shared tensor scale,
 * elements rounded stochastically with the same uniform whichever branch is
 * kept; the branch is chosen BEFORE rounding, by the smaller closed-form
 * expected squared error (tie: FP4), so the choice does not depend on the
 * random draw and each element stays unbiased.
 * Pinned by: the exact expectation over all 65536 uniforms of the chosen
 * branch is the smaller one; Monte-Carlo unbiasedness; expected error never
 * above NVFP4 SR's (its FP4 branch is NVFP4 SR). */
static void if4_sr_block(const float *z, float s_t, uint64_t seed, uint32_t stream, uint64_t idx0,
                         uint8_t *codes_row, int64_t k0, uint8_t *scale_out) {
  float yf[16], yi[16], ese_f, ese_i;
  int ef = sr_candidate(z, s_t, 0, yf, &ese_f);
  int ei = sr_candidate(z, s_t, 1, yi, &ese_i);
  int use_int = ese_i < ese_f;
  *scale_out = (uint8_t)(use_int ? (ei | 0x80) : ef);
  for (int i = 0; i < 16; i++) {
    uint32_t u = orc_uniform16(seed, 0, stream, idx0 + (uint64_t)i);
    int mag = use_int ? (ei ? sr_on_grid(GRID_INT4, 8, yi[i], u) : 0)
                      : (ef ? orc_sr_e2m1(yf[i], u) : 0);
    put_nibble(codes_row, k0 + i, (signbit(z[i]) ? 8 : 0) | mag);
  }
}

/* Four Over Six, the local scaling option of the forward pass
 * [QII-sum "Quantisierung im Vorwaertsdurchlauf"; IF4 Table 1, row
 * "NVFP4 (4/6)": maximum 6 x 256, relative dynamic range 57.1 %].
 * READING: each 16-block is coded twice with RTN, its maximum mapped to 6
 * (the NVFP4 scale a/6) and to 4 (scale a/4, which moves the near-maximal
 * values off the coarse top of the grid); the block keeps the candidate with
 * the smaller pairwise squared error (tie: 6).  Codes and scale bytes are
 * plain NVFP4, so dequantization is unchanged.  The tensor scale maps the
 * absmax to 6 x 256, so that the candidate-4 scale (up to 384) still fits
 * E4M3.
 * Pinned by: Table 1 MSE of NVFP4 (4/6) on N(0,1) [IF4 Table 1]; per block
 * never worse than NVFP4 RTN at the same tensor scale; the choice is the
 * smaller of the two candidates' float64 squared errors. */
static void fos_block(const float *z, float s_t, uint8_t *codes_row, int64_t k0,
                      uint8_t *scale_out) {
  int n6[16], n4[16];
  float sse6 = 0.0f, sse4 = 0.0f;
  int e6 = block_candidate(z, s_t, 0, 6.0f, n6, &sse6);
  int e4 = block_candidate(z, s_t, 0, 4.0f, n4, &sse4);
  int use4 = sse4 < sse6;
  *scale_out = (uint8_t)(use4 ? e4 : e6);
  for (int i = 0; i < 16; i++) put_nibble(codes_row, k0 + i, use4 ? n4[i] : n6[i]);
}

/* Scale search, RTN with a searched block scale: the standard NVFP4 scale
 * (block maximum mapped to 6) is not the error-minimizing one; a search over
 * nearby scale values lowers the error [PAL section "The two corners, and
 * what the palette does to them": the low-error corner sweeps 19 candidate
 * scales per block, rounds to nearest and keeps the best, values above the
 * top level clipping; the ScaleSearch abstract among the IF4 page's related
 * papers: a fine-grained search over the scale's mantissa bits, 27 % lower
 * NVFP4 error].
 * READING: the candidates are the 19 E4M3 scale bytes e0-9 .. e0+9 around the
 * RNE byte e0 of (a/6)/s_t, visited nearest first (e0, e0-1, e0+1, ...) and
 * skipping bytes outside 1..126 (e0 itself is always tried); codes by RTN at
 * each candidate (magnitudes clamped to 6); the block keeps the first
 * candidate with a strictly smaller pairwise sum of squared errors.  The
 * tensor scale is NVFP4's amax / (6 x 448).  The study's least-squares
 * reconstruction scale is not applied: with E4M3 scales and codes re-rounded
 * at every candidate, the searched minimum already is the best E4M3 scale
 * for its codes within the window.
 * Pinned by: the 27 % error reduction against NVFP4 RTN on N(0,1) data; the
 * kept candidate is the float64 brute-force minimum over the window; never
 * worse than RTN per block. */
static void search_block(const float *z, float s_t, uint8_t *codes_row, int64_t k0,
                         uint8_t *scale_out) {
  float a = 0.0f;
  for (int i = 0; i < 16; i++) a = fmaxf(a, fabsf(z[i]));
  const int e0 = orc_e4m3_rne_sat((a / 6.0f) / s_t);
  int best_e = -1, best_nib[16];
  float best_sse = 0.0f;
  for (int t = 0; t < 19; t++) {
    const int d = (t + 1) / 2 * ((t & 1) ? -1 : 1);   /* 0, -1, +1, -2, +2, ... */
    const int e = e0 + d;
    if (t > 0 && (e < 1 || e > 126)) continue;
    const float S = orc_e4m3_value(e) * s_t;
    const float r = (e != 0) ? 1.0f / S : 0.0f;
    int nib[16];
    float sq[16];
    for (int i = 0; i < 16; i++) {
      int mag = (e != 0) ? orc_e2m1_rne(fminf(fabsf(z[i] * r), 6.0f)) : 0;
      float val = GRID_E2M1[mag];
      if (signbit(z[i])) val = -val;
      float dd = z[i] - val * S;
      sq[i] = dd * dd;
      nib[i] = (signbit(z[i]) ? 8 : 0) | mag;
    }
    const float sse = orc_pairwise_sum(sq, 16);
    if (best_e < 0 || sse < best_sse) {
      best_e = e;
      best_sse = sse;
      memcpy(best_nib, nib, sizeof(nib));
    }
  }
  *scale_out = (uint8_t)best_e;
  for (int i = 0; i < 16; i++) put_nibble(codes_row, k0 + i, best_nib[i]);
}

/* MS-EDEN, first half, for one correction group of G elements (G = 128, the
 * rotation group, or 16) [QII-abs; QII-sum "Kerninnovationen" and
 * "Quantisierung im Rueckwaertsdurchlauf"]: the randomness moves from the
 * FP4 values onto the micro-scales; a correction rescaling keeps the
 * rotated estimate unbiased, and is folded into the group scale by SR.
 * READING (textbook EDEN): deterministic RTN codes under the exact block
 * scale s_b = a_b / 6; correction c = sum z^2 / sum z*zhat over the group
 * (pairwise trees); target scale t_b = s_b * c for every block of the group.
 * Pinned by: unbiasedness under Haar-random rotations (Monte Carlo), error
 * ratio against SR above 2 [QII-abs], exact expectation of the scale SR. */
static void eden_group(const float *z, int G, uint8_t *codes_row, int64_t k0, float *tb) {
  float zz[128] = {0}, zh[128] = {0}, s_b[8] = {0};
  for (int b = 0; b < G / 16; b++) {
    const float *zb = z + 16 * b;
    float a = 0.0f;
    for (int i = 0; i < 16; i++) a = fmaxf(a, fabsf(zb[i]));
    s_b[b] = a / 6.0f;
    float r = (a > 0.0f) ? 1.0f / s_b[b] : 0.0f;
    for (int i = 0; i < 16; i++) {
      int mag = 0;
      if (a > 0.0f) mag = orc_e2m1_rne(fminf(fabsf(zb[i] * r), 6.0f));
      float q = GRID_E2M1[mag] * s_b[b];
      zh[16 * b + i] = signbit(zb[i]) ? -q : q;
      put_nibble(codes_row, k0 + 16 * b + i, (signbit(zb[i]) ? 8 : 0) | mag);
    }
  }
  for (int i = 0; i < G; i++) {
    zz[i] = z[i] * z[i];
    zh[i] = z[i] * zh[i];
  }
  float N = orc_pairwise_sum(zz, G);
  float D = orc_pairwise_sum(zh, G);
  float c = (D > 0.0f) ? N / D : 1.0f;
  for (int b = 0; b < G / 16; b++) tb[b] = s_b[b] * c;
}

/* IF4 with MS-EDEN, first half [IF4 page, Figure 4 (IF4 with MS-EDEN in
 * the backward pass); QII-abs and QII-sum "Quantisierung im
 * Rueckwaertsdurchlauf" for MS-EDEN].
 * READING: every 16-block is coded by RTN twice under its exact scales,
 * E2M1 under a/6 and integers 0..7 under a/7, and keeps the branch with the
 * smaller pairwise squared error (tie: FP4), as IF4 RTN does; the EDEN
 * correction c = sum z^2 / sum z*zhat runs over the group with the kept
 * reconstructions; t_b = (kept exact scale) * c; the INT choice goes to
 * flag[b] (bit 7 of the scale byte).  EDEN's correction makes the rotated
 * estimate unbiased for any deterministic coding of the group, so the
 * choice keeps it unbiased.
 * Pinned by: unbiasedness under Haar-random rotations and under the RHT
 * (Monte Carlo); the kept branch is the float64 minimum; lower error than
 * NVFP4 MS-EDEN on rotated Gaussian data. */
static void eden_group_if4(const float *z, int G, uint8_t *codes_row, int64_t k0, float *tb,
                           uint8_t *flag) {
  float zz[128] = {0}, zh[128] = {0}, s_b[8] = {0};
  for (int b = 0; b < G / 16; b++) {
    const float *zb = z + 16 * b;
    float a = 0.0f;
    for (int i = 0; i < 16; i++) a = fmaxf(a, fabsf(zb[i]));
    const float s_f = a / 6.0f, s_i = a / 7.0f;
    const float r_f = (a > 0.0f) ? 1.0f / s_f : 0.0f;
    const float r_i = (a > 0.0f) ? 1.0f / s_i : 0.0f;
    int mf[16], mi[16];
    float hf[16], hi[16], sqf[16], sqi[16];
    for (int i = 0; i < 16; i++) {
      mf[i] = (a > 0.0f) ? orc_e2m1_rne(fminf(fabsf(zb[i] * r_f), 6.0f)) : 0;
      mi[i] = (a > 0.0f) ? orc_int4_rne(fminf(fabsf(zb[i] * r_i), 7.0f)) : 0;
      float vf = signbit(zb[i]) ? -GRID_E2M1[mf[i]] : GRID_E2M1[mf[i]];
      float vi = signbit(zb[i]) ? -(float)mi[i] : (float)mi[i];
      hf[i] = vf * s_f;
      hi[i] = vi * s_i;
      float df = zb[i] - hf[i], di = zb[i] - hi[i];
      sqf[i] = df * df;
      sqi[i] = di * di;
    }
    const int use_int = orc_pairwise_sum(sqi, 16) < orc_pairwise_sum(sqf, 16);
    flag[b] = (uint8_t)use_int;
    s_b[b] = use_int ? s_i : s_f;
    for (int i = 0; i < 16; i++) {
      zh[16 * b + i] = use_int ? hi[i] : hf[i];
      put_nibble(codes_row, k0 + 16 * b + i, (signbit(zb[i]) ? 8 : 0) | (use_int ? mi[i] : mf[i]));
    }
  }
  for (int i = 0; i < G; i++) {
    zz[i] = z[i] * z[i];
    zh[i] = z[i] * zh[i];
  }
  float N = orc_pairwise_sum(zz, G);
  float D = orc_pairwise_sum(zh, G);
  float c = (D > 0.0f) ? N / D : 1.0f;
  for (int b = 0; b < G / 16; b++) tb[b] = s_b[b] * c;
}

/* View the input as the [rows_out x K] matrix whose rows are quantization
 * groups: axis 0 keeps rows (groups run along the contiguous dimension);
 * axis 1 transposes (groups run along the strided dimension, i.e. along the
 * reduction dimension of a row-major activation or gradient, as the
 * backward re-quantization of [QII-sum] requires). */
static void make_view(const float *x, int64_t rows, int64_t cols, int64_t ld, int axis,
                      float *Z) {
  if (axis == 0) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) memcpy(Z + r * cols, x + r * ld, sizeof(float) * cols);
  } else {
    /* Z[c][r] = x[r][c], in 64 x 64 tiles */
#pragma omp parallel for schedule(static)
    for (int64_t c0 = 0; c0 < cols; c0 += 64)
      for (int64_t r0 = 0; r0 < rows; r0 += 64)
        for (int64_t c = c0; c < c0 + 64 && c < cols; c++)
          for (int64_t r = r0; r < r0 + 64 && r < rows; r++) Z[c * rows + r] = x[r * ld + c];
  }
}

int orc_quantize(const float *x, int64_t rows, int64_t cols, int64_t ld,
                 int format, int rounding, int axis, int rht,
                 const uint32_t signs[4], uint64_t seed, uint32_t stream,
                 int eden_group_size, const float *ts_in,
                 uint8_t *codes, uint8_t *scales, float *ts_out,
                 float *z_out, float *tb_out) {
  if (!x || !codes || !scales || !ts_out) return ORC_BAD_ARG;
  if (format < 0 || format > 4 || rounding < 0 || rounding > 2 || axis < 0 || axis > 1)
    return ORC_BAD_ARG;
  if (format != ORC_FMT_NVFP4 && format != ORC_FMT_IF4 && rounding != ORC_RTN) return ORC_BAD_ARG;
  if (rows < 0 || cols < 0 || ld < cols) return ORC_BAD_SHAPE;
  const int64_t R = axis == 0 ? rows : cols;
  const int64_t K = axis == 0 ? cols : rows;
  const int G = (rounding == ORC_MSEDEN) ? eden_group_size : 16;
  if (rounding == ORC_MSEDEN && G != 16 && G != 128) return ORC_BAD_ARG;
  if (K % 16) return ORC_BAD_SHAPE;
  if ((rht || G == 128) && K % 128) return ORC_BAD_SHAPE;
  if (rht && !signs) return ORC_BAD_ARG;
  if (R == 0 || K == 0) { *ts_out = ts_in ? *ts_in : 1.0f; return ORC_OK; }

  float *Z = (float *)malloc(sizeof(float) * (size_t)(R * K));
  if (!Z) return ORC_BAD_ARG;
  make_view(x, rows, cols, ld, axis, Z);

  /* 1. rotation of every 128-group of every row */
  if (rht) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; r++)
      for (int64_t g = 0; g < K; g += 128) {
        float tmp[128];
        orc_rht128(Z + r * K + g, signs, tmp);
        memcpy(Z + r * K + g, tmp, sizeof(tmp));
      }
  }
  if (z_out) memcpy(z_out, Z, sizeof(float) * (size_t)(R * K));
  memset(codes, 0, (size_t)(R * K / 2));

  if (rounding != ORC_MSEDEN) {
    /* 2. tensor scale: absmax over the (rotated) tensor, mapped to the
     * largest representable magnitude [IF4 Table 1: 6 x 448 for NVFP4 and
     * IF4, 7 x 448 for NVINT4, 6 x 256 for NVFP4 (4/6)]; an all-zero tensor
     * takes scale 1. */
    float s_t;
    if (ts_in) {
      s_t = *ts_in;
    } else {
      float m = 0.0f;
#pragma omp parallel for reduction(max : m) schedule(static)
      for (int64_t i = 0; i < R * K; i++) m = fmaxf(m, fabsf(Z[i]));
      float top = (format == ORC_FMT_NVINT4)         ? 7.0f * 448.0f
                  : (format == ORC_FMT_NVFP4_4OVER6) ? 6.0f * 256.0f
                                                     : 6.0f * 448.0f;
      s_t = (m > 0.0f) ? m / top : 1.0f;
    }
    *ts_out = s_t;
    /* 3. per 16-block scale and codes */
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; r++)
      for (int64_t k = 0; k < K; k += 16) {
        const float *zb = Z + r * K + k;
        uint8_t *sc = scales + r * (K / 16) + k / 16;
        if (format == ORC_FMT_NVFP4)
          nvfp4_block(zb, s_t, rounding, seed, stream, (uint64_t)(r * K + k), codes + r * (K / 2),
                      k, sc);
        else if (format == ORC_FMT_IF4 && rounding == ORC_SR)
          if4_sr_block(zb, s_t, seed, stream, (uint64_t)(r * K + k), codes + r * (K / 2), k, sc);
        else if (format == ORC_FMT_NVFP4_4OVER6)
          fos_block(zb, s_t, codes + r * (K / 2), k, sc);
        else if (format == ORC_FMT_NVFP4_SEARCH)
          search_block(zb, s_t, codes + r * (K / 2), k, sc);
        else
          if4_block(zb, s_t, format, codes + r * (K / 2), k, sc);
      }
  } else {
    /* MS-EDEN: codes and target scales t_b per group, then the tensor scale
     * from the largest target, then the E4M3 scales by SR of t_b / s_t. */
    float *tb = (float *)malloc(sizeof(float) * (size_t)(R * K / 16));
    uint8_t *flag = (uint8_t *)calloc((size_t)(R * K / 16), 1);
    if (!tb || !flag) { free(tb); free(flag); free(Z); return ORC_BAD_ARG; }
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; r++)
      for (int64_t k = 0; k < K; k += G) {
        if (format == ORC_FMT_IF4)
          eden_group_if4(Z + r * K + k, G, codes + r * (K / 2), k, tb + r * (K / 16) + k / 16,
                         flag + r * (K / 16) + k / 16);
        else
          eden_group(Z + r * K + k, G, codes + r * (K / 2), k, tb + r * (K / 16) + k / 16);
      }
    float s_t;
    if (ts_in) {
      s_t = *ts_in;
    } else {
      float T = 0.0f;
#pragma omp parallel for reduction(max : T) schedule(static)
      for (int64_t i = 0; i < R * K / 16; i++) T = fmaxf(T, tb[i]);
      /* READING: the tensor scale maps the largest target scale to the
       * E4M3 maximum, so the stochastic rounding of every scale stays inside
       * the grid and keeps its expectation. */
      s_t = (T > 0.0f) ? T / 448.0f : 1.0f;
    }
    *ts_out = s_t;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < R * K / 16; b++) {
      float a = fminf(tb[b] / s_t, 448.0f);
      scales[b] = (uint8_t)(orc_sr_e4m3(a, orc_uniform16(seed, 1, stream, (uint64_t)b)) |
                            (flag[b] ? 0x80 : 0));
    }
    if (tb_out) memcpy(tb_out, tb, sizeof(float) * (size_t)(R * K / 16));
    free(tb);
    free(flag);
  }
  free(Z);
  return ORC_OK;
}

/* ======================================================================
 * Dequantization: value = sign * (v * (scale * s_t)), v the E2M1 value or,
 * for IF4 groups flagged INT (scale bit 7), the integer magnitude.  With
 * inverse-rotation signs, each 128-group is rotated back afterwards.
 * Pinned by: round trip of exactly representable tensors; Table 1 MSE.
 * ==================================================================== */
int orc_dequantize(const uint8_t *codes, const uint8_t *scales, float ts,
                   int64_t rows_out, int64_t k, int format,
                   const uint32_t *inv_signs, float *out) {
  if (!codes || !scales || !out) return ORC_BAD_ARG;
  if (k % 16 || (inv_signs && k % 128)) return ORC_BAD_SHAPE;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows_out; r++) {
    for (int64_t j = 0; j < k; j++) {
      int byte = codes[r * (k / 2) + j / 2];
      int nib = (j & 1) ? (byte >> 4) : (byte & 15);
      int e = scales[r * (k / 16) + j / 16];
      int is_int = (format == ORC_FMT_NVINT4) || (format == ORC_FMT_IF4 && (e & 0x80));
      float S = orc_e4m3_value(e & 0x7F) * ts;
      float v = is_int ? (float)(nib & 7) : GRID_E2M1[nib & 7];
      float q = v * S;
      out[r * k + j] = (nib & 8) ? -q : q;
    }
    if (inv_signs)
      for (int64_t g = 0; g < k; g += 128) {
        float tmp[128];
        orc_irht128(out + r * k + g, inv_signs, tmp);
        memcpy(out + r * k + g, tmp, sizeof(tmp));
      }
  }
  return ORC_OK;
}

/* ======================================================================
 * Block-scaled FP4 GEMM, plain definition: C = (s_A s_B) * A_hat B_hat^T
 * with A_hat[m][k] = E2M1(code) * E4M3(block scale) taken exactly, both
 * operands stored K-major.  Accumulated in fp64 (ground truth).
 * Pinned by: a dense float64 matmul (numpy) of independently dequantized
 * operands.
 * ==================================================================== */
static double operand_value(const uint8_t *codes, const uint8_t *scales, int64_t K,
                            int format, int64_t row, int64_t k) {
  int byte = codes[row * (K / 2) + k / 2];
  int nib = (k & 1) ? (byte >> 4) : (byte & 15);
  int e = scales[row * (K / 16) + k / 16];
  int is_int = (format == ORC_FMT_NVINT4) || (format == ORC_FMT_IF4 && (e & 0x80));
  double v = is_int ? (double)(nib & 7) : (double)GRID_E2M1[nib & 7];
  double q = v * (double)orc_e4m3_value(e & 0x7F);
  return (nib & 8) ? -q : q;
}

int orc_gemm_entries(const uint8_t *a_codes, const uint8_t *a_scales, float a_ts,
                     const uint8_t *b_codes, const uint8_t *b_scales, float b_ts,
                     int64_t M, int64_t N, int64_t K, int format,
                     const int64_t *im, const int64_t *in, int64_t count, double *out) {
  if (K % 16) return ORC_BAD_SHAPE;
  for (int64_t t = 0; t < count; t++)
    if (im[t] < 0 || im[t] >= M || in[t] < 0 || in[t] >= N) return ORC_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < count; t++) {
    double acc = 0.0;
    for (int64_t k = 0; k < K; k++)
      acc += operand_value(a_codes, a_scales, K, format, im[t], k) *
             operand_value(b_codes, b_scales, K, format, in[t], k);
    out[t] = (double)a_ts * (double)b_ts * acc;
  }
  return ORC_OK;
}

int orc_gemm_full(const uint8_t *a_codes, const uint8_t *a_scales, float a_ts,
                  const uint8_t *b_codes, const uint8_t *b_scales, float b_ts,
                  int64_t M, int64_t N, int64_t K, int format, double *out) {
  if (K % 16) return ORC_BAD_SHAPE;
  double *A = (double *)malloc(sizeof(double) * (size_t)(M * K));
  double *B = (double *)malloc(sizeof(double) * (size_t)(N * K));
  if (!A || !B) { free(A); free(B); return ORC_BAD_ARG; }
  for (int64_t m = 0; m < M; m++)
    for (int64_t k = 0; k < K; k++) A[m * K + k] = operand_value(a_codes, a_scales, K, format, m, k);
  for (int64_t n = 0; n < N; n++)
    for (int64_t k = 0; k < K; k++) B[n * K + k] = operand_value(b_codes, b_scales, K, format, n, k);
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; m++)
    for (int64_t n = 0; n < N; n++) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; k++) acc += A[m * K + k] * B[n * K + k];
      out[m * N + n] = (double)a_ts * (double)b_ts * acc;
    }
  free(A);
  free(B);
  return ORC_OK;
}
