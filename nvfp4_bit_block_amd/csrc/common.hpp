// common.hpp -- device helpers shared by the gfx950 kernels of libnvfp4:
// bf16 unpacking, the Philox-4x32-10 counter-based generator, E4M3 / E2M1
// conversions, fast unsigned division, wave reductions and the 8-lane
// 128-point Hadamard rotation.
//
// Arithmetic follows the library's contract: fp32, one rounding per written
// operation (built with -ffp-contract=off), correctly rounded division,
// denormals kept.  Every conversion below is an exact power-of-two scaling
// followed by a single integer rounding, so each rounding decision is taken
// on exactly representable quantities.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nv4 {

constexpr int kWave = 64;

// Word 3 of a raw (unswizzled, offset-addressed) buffer resource on gfx950.
constexpr int kRsrcWord3 = 0x00020000;

// ---------------------------------------------------------------- bits
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 2^e as an fp32 for e in [-126, 127].
__device__ __forceinline__ float pow2i(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// floor(log2(v)) for finite v >= 0, clamped from below at lo (v = 0 -> lo).
__device__ __forceinline__ int ilog2_floor_clamped(float v, int lo) {
  int e = (int)((__float_as_uint(v) >> 23) & 0xFFu) - 127;
  return e < lo ? lo : e;
}

// ---------------------------------------------------------------- division
// The operand of a fallback IEEE division, made opaque so that the compiler
// keeps the division inside its (rarely taken, wave-uniform) branch instead
// of computing it for every value and selecting.
__device__ __forceinline__ float opaque(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// a / d for the constants d = 6 and 7, correctly rounded: q0 = a * fp32(1/d),
// r = fma(-q0, d, a) (exact), q = fma(r, fp32(1/d), q0).  An exhaustive check
// over every finite fp32 a >= 2^-119 shows q equals the IEEE quotient for both
// constants; below that the IEEE division is used.
template <int D>
__device__ __forceinline__ float div_by(float a) {
  constexpr float d = (float)D;
  constexpr float inv = 1.0f / (float)D;
  const float q0 = a * inv;
  const float r = __builtin_fmaf(-q0, d, a);
  float q = __builtin_fmaf(r, inv, q0);
  // (IEEE division below the range, when some lane of the wave needs it)
  if (__builtin_amdgcn_ballot_w64(!(a >= 0x1p-119f)) != 0) q = (a >= 0x1p-119f) ? q : opaque(a) / d;
  return q;
}

// Correctly rounded reciprocal and quotient from the hardware reciprocal
// v_rcp_f32 (error below one ulp), after Markstein (P. Markstein, "IA-64 and
// Elementary Functions", Prentice Hall 2000, chapter 8):
//   e  = 1 - b*y0        one fma, exact
//   y1 = y0 + e*y0       one fma: the correctly rounded 1/b
//   q0 = a*y1            within one ulp of a/b
//   r  = a - b*q0        one fma, exact
//   q1 = q0 + r*y1       one fma: the correctly rounded a/b (Markstein's
//                        theorem, given y1 = RN(1/b))
// One Newton step from a one-ulp seed is not proven to give RN(1/b) in
// general: the device check (tests/divcheck.hip) compares y1 with the IEEE
// reciprocal for every b of the range and q1 with the IEEE quotient for
// every pair of significands.  Within [2^-60, 2^60] every intermediate is
// normal and the steps scale exactly with the exponents; outside it (and
// for NaN or infinite operands) the IEEE division runs.  Four (reciprocal)
// and six (quotient) instructions instead of about ten.
constexpr float kDivLo = 0x1p-60f, kDivHi = 0x1p60f;

__device__ __forceinline__ float rcp_refined(float b) {
  const float y0 = __builtin_amdgcn_rcpf(b);
  const float e = __builtin_fmaf(-b, y0, 1.0f);
  return __builtin_fmaf(e, y0, y0);
}

// The IEEE operation runs only when some lane of the wave is outside the
// range (one wave-uniform branch), so that the common path has no divergent
// control flow to break the schedule.

// 1/b.
__device__ __forceinline__ float rcp_rn(float b) {
  float y = rcp_refined(b);
  const bool ok = b >= kDivLo && b <= kDivHi;
  if (__builtin_amdgcn_ballot_w64(!ok) != 0) y = ok ? y : 1.0f / opaque(b);
  return y;
}

// a/b.
__device__ __forceinline__ float div_rn(float a, float b) {
  const float y = rcp_refined(b);
  const float q0 = a * y;
  const float r = __builtin_fmaf(-b, q0, a);
  float q = __builtin_fmaf(r, y, q0);
  const bool ok = b >= kDivLo && b <= kDivHi && (a == 0.0f || (a >= kDivLo && a <= kDivHi));
  if (__builtin_amdgcn_ballot_w64(!ok) != 0) q = ok ? q : opaque(a) / b;
  return q;
}

// a / b for many a and one b: the refined reciprocal of b is computed once;
// the quotients are those of div_rn(a, b).
struct Divisor {
  float b, y;
  bool ok;
};

__device__ __forceinline__ Divisor make_divisor(float b) {
  Divisor d;
  d.b = b;
  d.y = rcp_refined(b);
  d.ok = b >= kDivLo && b <= kDivHi;
  return d;
}

__device__ __forceinline__ float div_rn(float a, const Divisor &d) {
  const float q0 = a * d.y;
  const float r = __builtin_fmaf(-d.b, q0, a);
  float q = __builtin_fmaf(r, d.y, q0);
  const bool ok = d.ok && (a == 0.0f || (a >= kDivLo && a <= kDivHi));
  if (__builtin_amdgcn_ballot_w64(!ok) != 0) q = ok ? q : opaque(a) / d.b;
  return q;
}

// ---------------------------------------------------------------- E4M3
// E4M3 "FN" (bias 7, max 448, subnormals down to 2^-9).  For a value v >= 0
// with binade E = max(floor(log2 v), -6), the representable neighbours are
// integers q in [0, 16] times 2^(E-3); the byte is (E + 6) * 8 + q (q = 16
// rolls into the next binade, q <= 8 covers the subnormals).

__device__ __forceinline__ float e4m3_value(uint32_t byte) {
  uint32_t e = (byte >> 3) & 15u, m = byte & 7u;
  float sig = (float)(e ? (8u + m) : m);
  return sig * pow2i((int)(e ? e : 1u) - 10);
}

__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
  if (v >= 448.0f) return 0x7Eu;
  int E = ilog2_floor_clamped(v, -6);
  float q = rintf(v * pow2i(3 - E));
  return (uint32_t)((E + 6) * 8 + (int)q);
}

__device__ __forceinline__ uint32_t e4m3_ceil_sat(float v) {
  if (v >= 448.0f) return 0x7Eu;
  int E = ilog2_floor_clamped(v, -6);
  float q = ceilf(v * pow2i(3 - E));
  return (uint32_t)((E + 6) * 8 + (int)q);
}

// Stochastic rounding onto the E4M3 grid: up iff u16 < frac * 65536, where
// frac is the (exact) position inside the bracketing gap.
// (Written without early returns, so that the compiler selects instead of
// branching per value; for a >= 448 or a <= 0 the rounding's intermediates
// are discarded.)
__device__ __forceinline__ uint32_t e4m3_sr_sat_float(float a, uint32_t u16) {
  const int E = ilog2_floor_clamped(a, -6);
  const float y = a * pow2i(3 - E);
  const float f = floorf(y);
  const float p = y - f;
  const uint32_t up = ((float)u16 < p * 65536.0f) ? 1u : 0u;
  const uint32_t e = (uint32_t)((E + 6) * 8 + (int)f) + up;
  return (a >= 448.0f) ? 0x7Eu : ((a > 0.0f) ? e : 0u);
}

// The same rounding with one integer addition in the normal range
// [2^-6, 448].  There the gap is one unit of the fp32 mantissa's third bit,
// and frac * 2^20 is m, the 20 mantissa bits below it: u16 < m / 16 holds
// iff m >= 16 u16 + 1, iff adding 2^20 - 1 - 16 u16 to the bit pattern
// carries into bit 20.  Bits 30..20 of the sum are then (E + 127) * 8 + q
// plus the carry (which rolls q = 8 into the next binade, as the E4M3 grid
// does), 960 above the E4M3 byte (E + 6) * 8 + q; 448 itself (E = 8, q = 6,
// m = 0) gives 0x7E.  Other values (subnormal scales, zero, above 448) take
// the float form, in the lanes that hold one.
__device__ __forceinline__ uint32_t e4m3_sr_sat(float a, uint32_t u16) {
  const uint32_t b = __float_as_uint(a);
  uint32_t e = (b + ((u16 << 4) ^ 0xFFFFFu) - (960u << 20)) >> 20;  // 2^20 - 1 - 16 u16
  const bool other = !(a >= 0x1p-6f && a <= 448.0f);
  if (__builtin_amdgcn_ballot_w64(other) != 0) {
    if (other) e = e4m3_sr_sat_float(a, u16);
  }
  return e;
}

// ---------------------------------------------------------------- E2M1
// E2M1 magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}: for a in [0, 6] with binade
// E = max(floor(log2 a), 0), neighbours are integers q in [0, 4] times
// 2^(E-1) and the magnitude code is 2E + q.  Stochastic rounding: up iff
// u16 < frac * 65536 with frac the exact position inside the gap.

__device__ __forceinline__ uint32_t e2m1_sr(float a, uint32_t u16) {
  const int E = ilog2_floor_clamped(a, 0);
  const float y = a * pow2i(1 - E);
  const float f = floorf(y);
  const float p = y - f;
  const uint32_t up = ((float)u16 < p * 65536.0f) ? 1u : 0u;
  const uint32_t m = (uint32_t)(2 * E + (int)f) + up;
  return (a >= 6.0f) ? 7u : m;
}

// Stochastic rounding onto the integers 0..7 (IF4's INT branch): up iff
// u16 < frac * 65536, frac = a - floor(a) (exact); 7 and above give 7.
__device__ __forceinline__ uint32_t int4_sr(float a, uint32_t u16) {
  if (a >= 7.0f) return 7u;
  const float f = floorf(a);
  const float p = a - f;
  return (uint32_t)f + (((float)u16 < p * 65536.0f) ? 1u : 0u);
}

// Expected squared error of stochastic rounding, in grid units: (a - l)(u - a)
// with l <= a < u the neighbouring levels; 0 at the top level.  On the E2M1
// grid l = f * 2^(E-1), u = (f + 1) * 2^(E-1) (both exact) with E and f as in
// e2m1_sr; on the integers l = floor(a), u = l + 1.
__device__ __forceinline__ float e2m1_sr_err(float a) {
  const int E = ilog2_floor_clamped(a, 0);
  const float g = pow2i(E - 1);
  const float f = floorf(a * pow2i(1 - E));
  const float d = (a - f * g) * ((f + 1.0f) * g - a);
  return a >= 6.0f ? 0.0f : d;
}

__device__ __forceinline__ float int4_sr_err(float a) {
  const float f = floorf(a);
  const float d = (a - f) * ((f + 1.0f) - a);
  return a >= 7.0f ? 0.0f : d;
}

// Value of a magnitude code 0..7.
__device__ __forceinline__ float e2m1_value(uint32_t mag) {
  return (mag < 2u) ? 0.5f * (float)mag : (float)(2u + (mag & 1u)) * pow2i((int)(mag >> 1) - 2);
}

// ---------------------------------------------------------------- Philox
// Philox-4x32 with 10 rounds (Salmon et al., SC'11): per round the words 0
// and 2 are multiplied by the round multipliers; the new state is
// (hi(w2*M1) ^ w1 ^ k0, lo(w2*M1), hi(w0*M0) ^ w3 ^ k1, lo(w0*M0)), and the
// key advances by the Weyl increments between rounds.
struct Philox4 {
  uint32_t w[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // one 32x32->64 multiply (v_mad_u64_u32) gives both halves
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    // three-input exclusive or in one instruction (truth table 0x96)
    c0 = __builtin_amdgcn_bitop3_b32(hi1, c1, k0, 0x96);
    c1 = lo1;
    c2 = __builtin_amdgcn_bitop3_b32(hi0, c3, k1, 0x96);
    c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  Philox4 o;
  o.w[0] = c0;
  o.w[1] = c1;
  o.w[2] = c2;
  o.w[3] = c3;
  return o;
}

// Eight 16-bit uniforms for indices 8*call .. 8*call+7 of one stream:
// counter (call lo, call hi, tag, stream), key (seed lo, seed hi); uniform j
// is half (j & 1) of word j >> 1.
struct RngKey {
  uint32_t seed_lo, seed_hi, stream;
};

__device__ __forceinline__ Philox4 uniforms8(const RngKey &k, uint64_t call, uint32_t tag) {
  return philox4x32_10((uint32_t)call, (uint32_t)(call >> 32), tag, k.stream, k.seed_lo,
                       k.seed_hi);
}

__device__ __forceinline__ uint32_t uniform_at(const Philox4 &p, int j) {
  // (word chosen by selects, not by indexing: an index the compiler cannot
  // resolve would put the four words in scratch memory)
  const int k = j >> 1;
  const uint32_t w = k == 0 ? p.w[0] : k == 1 ? p.w[1] : k == 2 ? p.w[2] : p.w[3];
  return (w >> (16 * (j & 1))) & 0xFFFFu;
}

// ---------------------------------------------------------------- division
// Unsigned division by a runtime constant d >= 1 for numerators n < 2^31:
// q = (umulhi(n, m) + n) >> s with s = ceil(log2 d), m = 2^32 (2^s - d)/d + 1.
struct FastDiv {
  uint32_t d, m, s;
};

__host__ inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.s = s;
  f.m = (uint32_t)((((1ull << s) - d) << 32) / d + 1);
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv &f) {
  return (__umulhi(n, f.m) + n) >> f.s;
}

// ---------------------------------------------------------------- E2M1 hardware
// gfx950's v_cvt_scalef32_pk_fp4_f32 at unit scale rounds two fp32 values to
// E2M1 to nearest (ties to the even code), saturates at 6 and keeps the sign
// (also of zero): exactly the nibble sign<<3 | E2M1_RNE(min(|y|, 6)).  It
// writes byte `sel` of the packed result.
typedef float f32x2_t __attribute__((ext_vector_type(2)));

template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_rne(uint32_t old, float y0, float y1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, y0, y1, 1.0f, SEL);
}

// 16 values -> two words of packed E2M1 codes (element 2i in the low nibble
// of byte i).
__device__ __forceinline__ void e2m1x16_rne(const float y[16], uint32_t &lo, uint32_t &hi) {
  lo = e2m1x2_rne<0>(0u, y[0], y[1]);
  lo = e2m1x2_rne<1>(lo, y[2], y[3]);
  lo = e2m1x2_rne<2>(lo, y[4], y[5]);
  lo = e2m1x2_rne<3>(lo, y[6], y[7]);
  hi = e2m1x2_rne<0>(0u, y[8], y[9]);
  hi = e2m1x2_rne<1>(hi, y[10], y[11]);
  hi = e2m1x2_rne<2>(hi, y[12], y[13]);
  hi = e2m1x2_rne<3>(hi, y[14], y[15]);
}

// Signed E2M1 values of the two codes in byte SEL of w (exact).
template <int SEL>
__device__ __forceinline__ f32x2_t e2m1x2_value(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

__device__ __forceinline__ void e2m1x16_value(uint32_t lo, uint32_t hi, float v[16]) {
  f32x2_t t;
  t = e2m1x2_value<0>(lo); v[0] = t[0]; v[1] = t[1];
  t = e2m1x2_value<1>(lo); v[2] = t[0]; v[3] = t[1];
  t = e2m1x2_value<2>(lo); v[4] = t[0]; v[5] = t[1];
  t = e2m1x2_value<3>(lo); v[6] = t[0]; v[7] = t[1];
  t = e2m1x2_value<0>(hi); v[8] = t[0]; v[9] = t[1];
  t = e2m1x2_value<1>(hi); v[10] = t[0]; v[11] = t[1];
  t = e2m1x2_value<2>(hi); v[12] = t[0]; v[13] = t[1];
  t = e2m1x2_value<3>(hi); v[14] = t[0]; v[15] = t[1];
}

// ---------------------------------------------------------------- GEMM operands
// The matrix instructions take fp16 operands: an E2M1 value times an E4M3
// scale has at most 6 significant bits and lies in [2^-10, 2688], so the
// decoded operand is exact in fp16.
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

// The two E4M3 bytes in bits 0-7 and 8-15 of b as fp16 values (exact:
// every E4M3 value is an fp16 value).
__device__ __forceinline__ half2_t e4m3x2_f16(uint32_t b) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, false);
}

// 8 codes (element 2i in the low nibble of byte i) times one fp16 scale.
__device__ __forceinline__ half8_t dequant8(uint32_t w, _Float16 s) {
  const half2_t s2 = {s, s};
  const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return half8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// IF4 operands: a block whose scale byte has bit 7 set holds sign-magnitude
// integers 0..7 instead of E2M1 codes.  Every magnitude of either kind is an
// fp16 value with a zero low byte, and its high byte (below 0x80) comes from
// a 16-byte table chosen by the block's flag:
//   E2M1 {0, .5, 1, 1.5, 2, 3, 4, 6} -> 00 38 3C 3E 40 42 44 46
//   INT  {0, 1, 2, 3, 4, 5, 6, 7}    -> 00 3C 40 42 44 45 46 47
constexpr uint32_t kLutFpLo = 0x3E3C3800u, kLutFpHi = 0x46444240u;
constexpr uint32_t kLutIntLo = 0x42403C00u, kLutIntHi = 0x47464544u;

// 8 codes of one block (element 2i in the low nibble of byte i), decoded
// through the table {lut_hi:lut_lo}, times one fp16 scale.  One byte
// permute looks up the high bytes of the four even elements (magnitudes
// in the low nibbles) and one those of the four odd ones; each code's sign
// bit (bit 3 of its nibble) is then set as bit 7 of its byte, the fp16 sign;
// four more permutes spread the bytes into fp16 pairs [0, even, 0, odd].
__device__ __forceinline__ half8_t dequant8_lut(uint32_t w, _Float16 s, uint32_t lut_lo, uint32_t lut_hi) {
  const half2_t s2 = {s, s};
  const uint32_t ev = __builtin_amdgcn_perm(lut_hi, lut_lo, w & 0x07070707u) | ((w << 4) & 0x80808080u);
  const uint32_t od = __builtin_amdgcn_perm(lut_hi, lut_lo, (w >> 4) & 0x07070707u) | (w & 0x80808080u);
  half8_t out;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t v = __builtin_amdgcn_perm(od, ev, 0x000C000Cu | ((4u + k) << 24) | ((uint32_t)k << 8));
    const half2_t p = __builtin_bit_cast(half2_t, v) * s2;
    out[2 * k] = p[0];
    out[2 * k + 1] = p[1];
  }
  return out;
}

// ---------------------------------------------------------------- lanes
// A 128-point rotation group is held by 8 lanes of one 16-lane DPP row; the
// group position (0..7) of a lane is given by lane bits 0, 1 and 3 (bit 2
// tells two interleaved groups apart).  Partners in the three cross-lane
// butterfly stages are then lane ^ 1 and lane ^ 2 (quad permutations) and
// lane ^ 8 (rotation of the 16-lane row by 8): one DPP move each.
__device__ __forceinline__ uint32_t group_pos(uint32_t lane) {
  return (lane & 3u) | ((lane >> 1) & 4u);
}
// Lane index within a 64-lane wave -> rank of its block among the wave's 64
// consecutive blocks, so that 8 consecutive blocks form one group.
__device__ __forceinline__ uint32_t lane_block_rank(uint32_t lane) {
  return (lane & 0x33u) | ((lane & 4u) << 1) | ((lane & 8u) >> 1);
}

template <int S>
__device__ __forceinline__ float lane_xor(float v) {
  const int x = __float_as_int(v);
  if constexpr (S == 1) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
  } else if constexpr (S == 2) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
  } else {
    static_assert(S == 4, "lane_xor supports group bits 1, 2, 4");
    return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, true));  // row_ror:8
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v = fmaxf(v, __shfl_xor(v, s, kWave));
  return v;
}

// Max over a workgroup of `nthreads` threads (multiple of 64); result valid
// in every thread.  `red` must hold nthreads / 64 floats of LDS.
__device__ __forceinline__ float block_max(float v, float *red, int nthreads) {
  v = wave_max(v);
  const int wid = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) red[wid] = v;
  __syncthreads();
  float m = red[0];
  for (int i = 1; i < nthreads / kWave; ++i) m = fmaxf(m, red[i]);
  return m;
}

// ---------------------------------------------------------------- rotation
// In-lane stages (strides 1, 2, 4, 8) of the Sylvester fast Hadamard
// transform on 16 consecutive coordinates: (a, b) -> (a + b, a - b).
__device__ __forceinline__ void fwht16_inlane(float v[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
}

// One cross-lane stage between group positions differing in bit S: the lower
// lane needs a + b, the upper a - b (a = the lower lane's value, b = the
// upper's).  Every lane computes fma(own, k, partner) with k = +1 (lower) or
// -1 (upper): the product by +-1 is exact and the fma rounds the sum once,
// so this is exactly a + b and a - b -- signed zeros included.
template <int S>
__device__ __forceinline__ void fwht_cross(float v[16], float k) {
  float p[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) p[i] = lane_xor<S>(v[i]);
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = __builtin_fmaf(v[i], k, p[i]);
}

// The rotation of a 128-group held by 8 lanes (16 consecutive coordinates
// each, `pos` = group position): stages of stride 1, ..., 64 in that order,
// then the 1/sqrt(128) normalization.  Sign flips of the randomization are
// applied by the caller before this.
__device__ __forceinline__ void fwht128_group(float v[16], uint32_t pos) {
  fwht16_inlane(v);
  fwht_cross<1>(v, (pos & 1u) ? -1.0f : 1.0f);
  fwht_cross<2>(v, (pos & 2u) ? -1.0f : 1.0f);
  fwht_cross<4>(v, (pos & 4u) ? -1.0f : 1.0f);
  const float c = 0x1.6a09e6p-4f;  // fp32(1/sqrt(128)) = 0x3DB504F3
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = v[i] * c;
}

// The same rotation with one instruction per cross-lane stage instead of two.
// Every lane computes own + k * partner, which a DPP-sourced fused
// multiply-add does in one step: the lower lane gets a + b, the upper lane
// b - a, the negation of its a - b.  Rounding to nearest is symmetric, so the
// upper lane's value is exactly the negated result, up to the sign of an
// exact zero (x - x is +0 either way round).  Partners in the later stages
// share their negation, so k stays +1 / -1; after the three stages a lane's
// values carry the sign (-1)^popcount(pos), folded into the normalization.
// Nonzero outputs are bit-identical to fwht128_group.  A zero output may
// carry the other sign, so the function returns true -- in every lane of the
// wave -- when some lane of the wave holds a zero; the caller then
// recomputes with fwht128_group.
//
// The compiler does not fuse a DPP move into v_fmac_f32, so the stage is
// written out: v_fmac_f32_dpp d, d, k computes d + k * (d of the partner
// lane) -- every lane reads its partner's d before any lane writes.  The
// leading s_nop 1 gives the two wait states that a DPP read needs after a
// vector write of its source register; inside the block no instruction
// reads a register that an earlier one wrote.  (A DPP read also needs five
// after a vector-ALU write of EXEC, v_cmpx; the library emits none, which
// tests/test_build_invariants.py checks in the built assembly.)
#define NV4_FMAC_DPP16(CTRL)                                                                      \
  "s_nop 1\n\t"                                                                                   \
  "v_fmac_f32_dpp %0, %0, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
  "v_fmac_f32_dpp %1, %1, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
  "v_fmac_f32_dpp %2, %2, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
  "v_fmac_f32_dpp %3, %3, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
  "v_fmac_f32_dpp %4, %4, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
  "v_fmac_f32_dpp %5, %5, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
  "v_fmac_f32_dpp %6, %6, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
  "v_fmac_f32_dpp %7, %7, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
  "v_fmac_f32_dpp %8, %8, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
  "v_fmac_f32_dpp %9, %9, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
  "v_fmac_f32_dpp %10, %10, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                         \
  "v_fmac_f32_dpp %11, %11, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                         \
  "v_fmac_f32_dpp %12, %12, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                         \
  "v_fmac_f32_dpp %13, %13, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                         \
  "v_fmac_f32_dpp %14, %14, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                         \
  "v_fmac_f32_dpp %15, %15, %16 " CTRL " row_mask:0xf bank_mask:0xf"

#define NV4_V16(v)                                                                                 \
  "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]),  \
      "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]), "+v"(v[14]),     \
      "+v"(v[15])

template <int S>
__device__ __forceinline__ void fwht_cross_negating(float v[16], float k) {
  if constexpr (S == 1) {
    asm volatile(NV4_FMAC_DPP16("quad_perm:[1,0,3,2]") : NV4_V16(v) : "v"(k));
  } else if constexpr (S == 2) {
    asm volatile(NV4_FMAC_DPP16("quad_perm:[2,3,0,1]") : NV4_V16(v) : "v"(k));
  } else {
    static_assert(S == 4, "fwht_cross_negating supports group bits 1, 2, 4");
    asm volatile(NV4_FMAC_DPP16("row_ror:8") : NV4_V16(v) : "v"(k));
  }
}
#undef NV4_FMAC_DPP16
#undef NV4_V16

__device__ __forceinline__ bool fwht128_group_fast(float v[16], uint32_t pos) {
  fwht16_inlane(v);
  fwht_cross_negating<1>(v, (pos & 1u) ? -1.0f : 1.0f);
  fwht_cross_negating<2>(v, (pos & 2u) ? -1.0f : 1.0f);
  fwht_cross_negating<4>(v, (pos & 4u) ? -1.0f : 1.0f);
  const float c = (__builtin_popcount(pos) & 1) ? -0x1.6a09e6p-4f : 0x1.6a09e6p-4f;
  float m = __builtin_inff();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = v[i] * c;
    m = fminf(m, fabsf(v[i]));
  }
  return __builtin_amdgcn_ballot_w64(m == 0.0f) != 0;
}

// 16 sign bits of a lane's coordinate block within the 128-bit sign vector.
__device__ __forceinline__ uint32_t lane_sign_bits(const uint32_t sg[4], uint32_t lane_in_group) {
  const uint32_t w = sg[lane_in_group >> 1];
  return (w >> (16 * (lane_in_group & 1))) & 0xFFFFu;
}

// Pairwise tree over 16 values in natural order.
__device__ __forceinline__ float tree16(const float v[16]) {
  float s8[8], s4[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) s8[i] = v[2 * i] + v[2 * i + 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) s4[i] = s8[2 * i] + s8[2 * i + 1];
  return (s4[0] + s4[1]) + (s4[2] + s4[3]);
}

}  // namespace nv4
