// quantize.hip -- NVFP4 / MS-EDEN / IF4 quantizers for gfx950.
//
// Sources: Quartet II abstract and news summary (mind-verse.de) for the
// forward RTN scheme, stochastic rounding, the randomized Hadamard rotation
// and MS-EDEN; "Comparing INT4 and NVFP4 Palettes on Real Gradient Tensors"
// (opening paragraph) for the E2M1 grid and the SR corner; the IF4 page
// (arXiv 2603.28765: abstract, Figure 1, Table 1, Figure 3) for E4M3 ranges
// and the per-group FP4/INT4 selection.
//
// Work decomposition: one lane owns one 16-element block (one E4M3 scale) of
// the OUTPUT layout; a 128-point rotation group is 8 lanes of one 16-lane
// DPP row, holding 8 consecutive blocks.
//   axis 0: a block is 16 contiguous input elements (two 16-byte loads for
//           bf16), addressed by the flat block index.
//   axis 1: a lane loads 16 rows of one 16-byte column chunk and so holds
//           the blocks of 8 (bf16) or 4 (fp32) columns; no LDS transpose.
// A pass that needs the tensor-wide maximum writes one partial maximum per
// workgroup into the workspace; the next pass reduces those partials in every
// workgroup (no atomics, no memset, deterministic).
#include "kernels.hpp"

namespace nv4 {

// ---------------------------------------------------------------- helpers
// This thread's share of the maximum of n <= kMaxPartials partial maxima
// (all >= 0): its kMaxPartials / kThreads loads are issued together, so the
// prologue of every workgroup that needs the tensor scale waits on memory
// once rather than once per load; loads past n read 0 (range-checked).
template <int NT = kThreads>
__device__ __forceinline__ float partials_max(const float *v, uint32_t n) {
  static_assert(kMaxPartials % NT == 0, "partials per thread");
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void *)v, (short)0, (int)(4 * n), kRsrcWord3);
  float m[kMaxPartials / NT];
#pragma unroll
  for (int k = 0; k < kMaxPartials / NT; ++k)
    m[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, 4 * (threadIdx.x + k * NT), 0, 0));
  float a = 0.0f;
#pragma unroll
  for (int k = 0; k < kMaxPartials / NT; ++k) a = fmaxf(a, m[k]);
  return a;
}

template <int NT = kThreads>
__device__ __forceinline__ float tensor_scale(const QuantParams &p, float *red) {
  if (p.ts_in) return *p.ts_in;
  if (p.amax_in) {
    const float a = *p.amax_in;
    return (a > 0.0f) ? a / p.top : 1.0f;
  }
  const float m = block_max(partials_max<NT>(p.partial, p.npartial), red, NT);
  return (m > 0.0f) ? m / p.top : 1.0f;
}

// Sign masks for a lane's 16 coordinates: word w of the bf16 pairs gets bit
// 15 (element 2w) and bit 31 (element 2w+1); fp32 word i gets bit 31.
struct SignMasks {
  uint32_t m[16];
};

template <int IN_BF16>
__device__ __forceinline__ SignMasks make_masks(const QuantParams &p, uint32_t lig) {
  SignMasks s;
  const uint32_t bits = p.rht ? lane_sign_bits(p.sg, lig) : 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (IN_BF16)
      s.m[i] = (i < 8) ? ((((bits >> (2 * i)) & 1u) << 15) | (((bits >> (2 * i + 1)) & 1u) << 31))
                       : 0u;
    else
      s.m[i] = ((bits >> i) & 1u) << 31;
  }
  return s;
}

// 16 values from 8 words of bf16 pairs (low half = even element).
__device__ __forceinline__ void unpack_bf16(const uint32_t w[8], const SignMasks &sm, float z[16]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t v = w[i] ^ sm.m[i];
    z[2 * i] = bf16_lo(v);
    z[2 * i + 1] = bf16_hi(v);
  }
}

__device__ __forceinline__ void unpack_f32(const uint32_t w[16], const SignMasks &sm, float z[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = __uint_as_float(w[i] ^ sm.m[i]);
}

__device__ __forceinline__ uint32_t sign_nib(float z) { return (__float_as_uint(z) >> 28) & 8u; }

// max|x| over N raw input words (bf16 pairs or fp32): for bf16 the largest
// magnitude bits of the 16-bit halves (integer order is the order of
// magnitudes), then back to fp32.
template <int IN_BF16, int N>
__device__ __forceinline__ float raw_absmax(const uint32_t (&w)[N]) {
  if constexpr (IN_BF16) {
    typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
    u16x2_t m = {0, 0};
#pragma unroll
    for (int i = 0; i < N; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, w[i] & 0x7FFF7FFFu));
    const uint32_t hi = m[0] > m[1] ? m[0] : m[1];
    return __uint_as_float(hi << 16);
  } else {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < N; ++i) m = fmaxf(m, fabsf(__uint_as_float(w[i])));
    return m;
  }
}

// MS-EDEN with amax_out: the workgroup's maximum of |x| (the raw input)
// goes to the second partial array, which k_eden_scales reduces.
template <int NT = kThreads>
__device__ __forceinline__ void raw_partial(const QuantParams &p, float araw, float *red) {
  const float m = block_max(araw, red, NT);
  if (threadIdx.x == 0) p.rpartial[blockIdx.x] = m;
}

// ---------------------------------------------------------------- outputs
// Where one block's results go.  PtrSink: plain stores, skipped by lanes
// that hold no block.  RowSink: buffer stores over the blocks from `base` on,
// whose range check drops the stores of lanes past the last block -- no
// branch, so that every path through a loop iteration leaves the same
// memory operations pending and the compiler's waits for the next block's
// loads stay exact.
struct PtrSink {
  const QuantParams &p;
  uint32_t gb;
  bool active;
  __device__ __forceinline__ void codes(uint32_t lo, uint32_t hi) const {
    if (active) *reinterpret_cast<uint2 *>(p.codes + (size_t)gb * 8) = make_uint2(lo, hi);
  }
  __device__ __forceinline__ void scale(uint32_t e) const {
    if (active) p.scales[gb] = (uint8_t)e;
  }
  __device__ __forceinline__ void target(float t) const {
    if (active) p.tb[gb] = t;
  }
};

struct RowSink {
  __amdgpu_buffer_rsrc_t c, s, t;  // codes, scales, targets from block `base` on
  uint32_t r;                       // this lane's block - base
  bool active;
  __device__ __forceinline__ RowSink(const QuantParams &p, uint32_t base, uint32_t rank) {
    const uint64_t left = p.nblocks - base;  // blocks from base on (base < nblocks)
    const int nc = (int)(8 * left < 0x7FFFFFFFull ? 8 * left : 0x7FFFFFFFull);
    const int ns = (int)(left < 0x7FFFFFFFull ? left : 0x7FFFFFFFull);
    const int nt = (int)(4 * left < 0x7FFFFFFFull ? 4 * left : 0x7FFFFFFFull);
    c = __builtin_amdgcn_make_buffer_rsrc((void *)(p.codes + (size_t)base * 8), (short)0, nc, kRsrcWord3);
    s = __builtin_amdgcn_make_buffer_rsrc((void *)(p.scales + base), (short)0, ns, kRsrcWord3);
    t = __builtin_amdgcn_make_buffer_rsrc((void *)(p.tb ? p.tb + base : nullptr), (short)0, p.tb ? nt : 0,
                                          kRsrcWord3);
    r = rank;
    active = base + rank < p.nblocks;
  }
  __device__ __forceinline__ void codes(uint32_t lo, uint32_t hi) const {
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{lo, hi}, c, 8 * r, 0, 0);
  }
  __device__ __forceinline__ void scale(uint32_t e) const {
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)e, s, r, 0, 0);
  }
  __device__ __forceinline__ void target(float v) const {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), t, 4 * r, 0, 0);
  }
};

// ---------------------------------------------------------------- MS-EDEN
// One block's share of MS-EDEN: RTN codes under the exact scale a/6 (IF4:
// also integers under a/7, keeping the branch with the smaller pairwise
// squared error) and the block's sums for the correction
// c = sum z^2 / sum z*zhat over the group.
struct EdenBlock {
  uint32_t lo, hi;  // codes
  float s_b;        // the kept branch's exact scale
  float N, D;       // sum z^2, sum z*zhat over the block (pairwise, natural order)
  bool use_int;
};

template <int MODE>
__device__ __forceinline__ EdenBlock eden_codes(const float z[16], float a) {
  constexpr bool IF4 = MODE == kIf4Eden || MODE == kIf4EdenFused;
  EdenBlock b;
  b.s_b = div_by<6>(a);
  const float r = (a > 0.0f) ? rcp_rn(b.s_b) : 0.0f;
  float nn[16], dd[16], y[16], g[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = z[i] * r;  // r = 0 when a = 0: signed zeros
  e2m1x16_rne(y, b.lo, b.hi);
  e2m1x16_value(b.lo, b.hi, g);  // signed grid values
  b.use_int = false;
  if constexpr (IF4) {
    const float si = div_by<7>(a);
    const float ri = (a > 0.0f) ? rcp_rn(si) : 0.0f;
    // (the INT branch as in IF4 RTN: magnitudes as floats, the error from
    // |z|, codes packed per byte with the E2M1 codes' sign bits)
    float sqf[16], sqi[16], vi[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float df = z[i] - g[i] * b.s_b;
      sqf[i] = df * df;
      vi[i] = rintf(fminf(fabsf(z[i] * ri), 7.0f));
      const float di = fabsf(z[i]) - vi[i] * si;
      sqi[i] = di * di;
    }
    b.use_int = tree16(sqi) < tree16(sqf);
    if (b.use_int) {
      uint32_t ilo = 0, ihi = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ilo = __builtin_amdgcn_cvt_pk_u8_f32(vi[2 * j] + 16.0f * vi[2 * j + 1], j, ilo);
        ihi = __builtin_amdgcn_cvt_pk_u8_f32(vi[8 + 2 * j] + 16.0f * vi[9 + 2 * j], j, ihi);
      }
      b.lo = ilo | (b.lo & 0x88888888u);
      b.hi = ihi | (b.hi & 0x88888888u);
      b.s_b = si;
#pragma unroll
      for (int i = 0; i < 16; ++i) g[i] = copysignf(vi[i], z[i]);  // signed integer values
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float zh = g[i] * b.s_b;
    nn[i] = z[i] * z[i];
    dd[i] = z[i] * zh;
  }
  b.N = tree16(nn);
  b.D = tree16(dd);
  return b;
}

// The block's outputs from its group's sums N, D: target t = s_b * c
// (pass 1: codes and t, whose sign bit carries IF4's INT flag) or, with a
// known tensor scale, the scale byte by stochastic rounding of t / s_t.
template <int MODE, typename Sink>
__device__ __forceinline__ void eden_emit(const EdenBlock &b, float N, float D, uint32_t gb, const Sink &out,
                                          const QuantParams &p, float s_t, float &lmax) {
  const float c = (D > 0.0f) ? div_rn(N, D) : 1.0f;
  const float t = b.s_b * c;
  if constexpr (MODE == kEden || MODE == kIf4Eden) {
    out.codes(b.lo, b.hi);
    // the sign bit carries the INT flag (t >= +0, or NaN where the group's
    // sums overflow, whose sign is the division's)
    out.target(b.use_int ? -fabsf(t) : fabsf(t));
    if (out.active) lmax = fmaxf(lmax, t);
  } else {
    const Philox4 u = uniforms8(p.key, (uint64_t)(gb >> 3), 1u);
    const uint32_t e = e4m3_sr_sat(fminf(div_rn(t, s_t), 448.0f), uniform_at(u, (int)(gb & 7u)));
    out.codes(b.lo, b.hi);
    out.scale(b.use_int ? (e | 0x80u) : e);
  }
}

// ---------------------------------------------------------------- one block
// z: the lane's 16 (rotated) values; gb: its block index in the output
// layout (it keys the random numbers); out: where the results go.  Must be
// called by every lane of a wave (the MS-EDEN correction of a 128-group
// reduces over 8 lanes).
template <int MODE, typename Sink>
__device__ __forceinline__ void quant_block(float z[16], uint32_t gb, const Sink &out,
                                            const QuantParams &p, float s_t, float &lmax) {
  const bool active = out.active;
  if constexpr (MODE == kRot) {
    if (active) {
      float4 *o = reinterpret_cast<float4 *>(p.rot_out + (size_t)gb * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = make_float4(z[4 * i], z[4 * i + 1], z[4 * i + 2], z[4 * i + 3]);
    }
    return;
  } else {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(z[i]));

    if constexpr (MODE == kAmax) {
      if (active) lmax = fmaxf(lmax, a);
    } else if constexpr (MODE == kRtn || MODE == kSr) {
      // scale e = E4M3((a/6)/s_t), RNE (RTN) or rounded up (SR); codes of
      // min(|z| / (e * s_t), 6) on the E2M1 grid.
      const float v = div_rn(div_by<6>(a), s_t);
      const uint32_t e = (MODE == kRtn) ? e4m3_rne_sat(v) : e4m3_ceil_sat(v);
      const float r = e ? rcp_rn(e4m3_value(e) * s_t) : 0.0f;
      Philox4 u0, u1;
      if constexpr (MODE == kSr) {
        u0 = uniforms8(p.key, (uint64_t)gb * 2u, 0u);
        u1 = uniforms8(p.key, (uint64_t)gb * 2u + 1u, 0u);
      }
      uint32_t lo = 0, hi = 0;
      if constexpr (MODE == kRtn) {
        float y[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] = z[i] * r;  // r = 0 when e = 0: signed zeros
        e2m1x16_rne(y, lo, hi);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float y = fminf(fabsf(z[i] * r), 6.0f);
          const uint32_t mag = e ? e2m1_sr(y, uniform_at(i < 8 ? u0 : u1, i & 7)) : 0u;
          const uint32_t nib = sign_nib(z[i]) | mag;
          if (i < 8) lo |= nib << (4 * i);
          else hi |= nib << (4 * (i - 8));
        }
      }
      out.codes(lo, hi);
      out.scale(e);
    } else if constexpr (MODE == kIf4) {
      // both branches at their own scales; keep the smaller pairwise SSE.
      const uint32_t ef = e4m3_rne_sat(div_rn(div_by<6>(a), s_t));
      const float Sf = e4m3_value(ef) * s_t;
      const float rf = ef ? rcp_rn(Sf) : 0.0f;
      const uint32_t ei = e4m3_rne_sat(div_rn(div_by<7>(a), s_t));
      const float Si = e4m3_value(ei) * s_t;
      const float ri = ei ? rcp_rn(Si) : 0.0f;
      float sqf[16], sqi[16], y[16], vf[16], vi[16];
      uint32_t flo, fhi;
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = z[i] * rf;
      e2m1x16_rne(y, flo, fhi);
      e2m1x16_value(flo, fhi, vf);  // signed grid values
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float df = z[i] - vf[i] * Sf;
        sqf[i] = df * df;
        // the integer magnitude (0 when ei = 0: ri = 0); the error of the
        // signed value sign(z) * vi * Si is the negation of |z| - vi * Si
        // under the same rounding, so its square is the same
        vi[i] = rintf(fminf(fabsf(z[i] * ri), 7.0f));
        const float di = fabsf(z[i]) - vi[i] * Si;
        sqi[i] = di * di;
      }
      // the INT codes: magnitudes two per byte (vi[2j] + 16 vi[2j+1] is an
      // exact integer below 128), signs from the E2M1 codes, which carry
      // z's sign bit whatever they round to
      uint32_t ilo = 0, ihi = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ilo = __builtin_amdgcn_cvt_pk_u8_f32(vi[2 * j] + 16.0f * vi[2 * j + 1], j, ilo);
        ihi = __builtin_amdgcn_cvt_pk_u8_f32(vi[8 + 2 * j] + 16.0f * vi[9 + 2 * j], j, ihi);
      }
      ilo |= flo & 0x88888888u;
      ihi |= fhi & 0x88888888u;
      const bool use_int = tree16(sqi) < tree16(sqf);
      out.codes(use_int ? ilo : flo, use_int ? ihi : fhi);
      out.scale(use_int ? (ei | 0x80u) : ef);
    } else if constexpr (MODE == kIf4Sr) {
      // both branches as NVFP4 SR: scales rounded up from a/6 (E2M1) and
      // a/7 (integers); keep the smaller closed-form expected squared error
      // (S*S) * sum (y - l)(u - y), decided before any random draw; the
      // kept branch rounds with the element's uniform.
      const uint32_t ef = e4m3_ceil_sat(div_rn(div_by<6>(a), s_t));
      const float Sf = e4m3_value(ef) * s_t;
      const float rf = ef ? rcp_rn(Sf) : 0.0f;
      const uint32_t ei = e4m3_ceil_sat(div_rn(div_by<7>(a), s_t));
      const float Si = e4m3_value(ei) * s_t;
      const float ri = ei ? rcp_rn(Si) : 0.0f;
      float yf[16], yi[16], df[16], di[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // (a zero scale byte has a zero reciprocal: y = 0 without a select)
        yf[i] = fminf(fabsf(z[i] * rf), 6.0f);
        yi[i] = fminf(fabsf(z[i] * ri), 7.0f);
        df[i] = e2m1_sr_err(yf[i]);
        di[i] = int4_sr_err(yi[i]);
      }
      const bool use_int = (Si * Si) * tree16(di) < (Sf * Sf) * tree16(df);
      const Philox4 u0 = uniforms8(p.key, (uint64_t)gb * 2u, 0u);
      const Philox4 u1 = uniforms8(p.key, (uint64_t)gb * 2u + 1u, 0u);
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // one stochastic rounding, on the kept branch's grid: the integers
        // are the E2M1 rounding's binade 1 (neighbours f, f + 1) everywhere
        const uint32_t u = uniform_at(i < 8 ? u0 : u1, i & 7);
        const float y = use_int ? yi[i] : yf[i];
        const float top = use_int ? 7.0f : 6.0f;
        const int E = use_int ? 1 : ilog2_floor_clamped(y, 0);
        const float ys = y * pow2i(1 - E);
        const float f = floorf(ys);
        const uint32_t up = ((float)u < (ys - f) * 65536.0f) ? 1u : 0u;
        const uint32_t mag0 = (uint32_t)f + up + (use_int ? 0u : (uint32_t)(2 * E));
        // (y = 0 where the kept scale byte is 0, and then mag0 = 0 too)
        const uint32_t mag = y >= top ? 7u : mag0;
        const uint32_t nib = sign_nib(z[i]) | mag;
        if (i < 8) lo |= nib << (4 * i);
        else hi |= nib << (4 * (i - 8));
      }
      out.codes(lo, hi);
      out.scale(use_int ? (ei | 0x80u) : ef);
    } else if constexpr (MODE == kFos) {
      // Four Over Six: RTN with the block maximum mapped to 6 and to 4;
      // keep the smaller pairwise SSE (tie: 6).
      const uint32_t e6 = e4m3_rne_sat(div_rn(div_by<6>(a), s_t));
      const float S6 = e4m3_value(e6) * s_t;
      const float r6 = e6 ? rcp_rn(S6) : 0.0f;
      const uint32_t e4 = e4m3_rne_sat(div_rn(a * 0.25f, s_t));
      const float S4 = e4m3_value(e4) * s_t;
      const float r4 = e4 ? rcp_rn(S4) : 0.0f;
      float y[16], v[16], sq6[16], sq4[16];
      uint32_t lo6, hi6, lo4, hi4;
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = z[i] * r6;  // r = 0 when e = 0: signed zeros
      e2m1x16_rne(y, lo6, hi6);
      e2m1x16_value(lo6, hi6, v);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float d = z[i] - v[i] * S6;
        sq6[i] = d * d;
        y[i] = z[i] * r4;
      }
      e2m1x16_rne(y, lo4, hi4);
      e2m1x16_value(lo4, hi4, v);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float d = z[i] - v[i] * S4;
        sq4[i] = d * d;
      }
      const bool use4 = tree16(sq4) < tree16(sq6);
      out.codes(use4 ? lo4 : lo6, use4 ? hi4 : hi6);
      out.scale(use4 ? e4 : e6);
    } else if constexpr (MODE == kSearch) {
      // RTN at the scale bytes e0, e0-1, e0+1, ..., e0-9, e0+9 (those in
      // 1..126; e0 always); keep the first strictly smaller pairwise SSE.
      const int e0 = (int)e4m3_rne_sat(div_rn(div_by<6>(a), s_t));
      uint32_t best_e = 0, blo = 0, bhi = 0;
      float best = 0.0f;
#pragma unroll 1
      for (int t = 0; t < 19; ++t) {
        const int e = e0 + (t + 1) / 2 * ((t & 1) ? -1 : 1);
        if (t > 0 && (e < 1 || e > 126)) continue;
        const float S = e4m3_value((uint32_t)e) * s_t;
        if (t > 0) {
          // A scale with 6 S < a codes the largest element as 6: that
          // element's own term, (a - 6 S)^2 rounded as in the sum below, is
          // a lower bound of the rounded sum (every term is >= 0).  A trial
          // whose bound reaches the best sum cannot be strictly smaller.
          const float p6 = 6.0f * S;
          if (p6 < a) {
            const float d = a - p6;
            if (d * d >= best) continue;
          }
        }
        const float r = e ? rcp_rn(S) : 0.0f;
        float y[16], v[16], sq[16];
        uint32_t lo, hi;
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] = z[i] * r;  // r = 0 when e = 0: signed zeros
        e2m1x16_rne(y, lo, hi);
        e2m1x16_value(lo, hi, v);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float d = z[i] - v[i] * S;
          sq[i] = d * d;
        }
        const float sse = tree16(sq);
        if (t == 0 || sse < best) {
          best = sse;
          best_e = (uint32_t)e;
          blo = lo;
          bhi = hi;
        }
      }
      out.codes(blo, bhi);
      out.scale(best_e);
    } else if constexpr (MODE == kEden || MODE == kEdenFused || MODE == kIf4Eden || MODE == kIf4EdenFused) {
      const EdenBlock b = eden_codes<MODE>(z, a);
      float N = b.N, D = b.D;
      if (!p.group16) {
        N = N + lane_xor<1>(N);
        D = D + lane_xor<1>(D);
        N = N + lane_xor<2>(N);
        D = D + lane_xor<2>(D);
        N = N + lane_xor<4>(N);
        D = D + lane_xor<4>(D);
      }
      eden_emit<MODE>(b, N, D, gb, out, p, s_t, lmax);
    }
  }
}

// ---------------------------------------------------------------- axis 0
// Raw input words of one lane's 16-element block.
template <int IN_BF16>
struct RawBlock {
  uint4 q[IN_BF16 ? 2 : 4];
};

template <int IN_BF16>
__device__ __forceinline__ void load_row_block(const QuantParams &p, uint32_t gb, RawBlock<IN_BF16> &b) {
  const uint32_t r = fdiv(gb, p.k16div);
  const uint32_t kb = gb - r * p.K16;
  const size_t off = (size_t)r * p.ld + (size_t)kb * 16;
  if (IN_BF16) {
    const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.x) + off);
#pragma unroll
    for (int i = 0; i < 2; ++i) b.q[i] = src[i];
  } else {
    const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const float *>(p.x) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) b.q[i] = src[i];
  }
}

template <int IN_BF16>
__device__ __forceinline__ void unpack_block(const RawBlock<IN_BF16> &b, const SignMasks &sm, float z[16]) {
  uint32_t w[IN_BF16 ? 8 : 16];
#pragma unroll
  for (int i = 0; i < (IN_BF16 ? 2 : 4); ++i) {
    w[4 * i] = b.q[i].x;
    w[4 * i + 1] = b.q[i].y;
    w[4 * i + 2] = b.q[i].z;
    w[4 * i + 3] = b.q[i].w;
  }
  if (IN_BF16) unpack_bf16(w, sm, z);
  else unpack_f32(w, sm, z);
}

// Unpack and rotate one lane's block: the one-instruction cross-lane stages,
// redone with the exact two-instruction ones when the wave holds a zero
// output (whose sign the fast stages may get wrong).
template <int IN_BF16>
__device__ __forceinline__ void load_z(const RawBlock<IN_BF16> &b, const SignMasks &sm, bool rht, uint32_t lig,
                                       float z[16]) {
  unpack_block<IN_BF16>(b, sm, z);
  if (rht && fwht128_group_fast(z, lig)) {
    // (the raw words pass through an empty asm so that the compiler cannot
    // keep the in-lane stages' results alive from the fast path for reuse)
    RawBlock<IN_BF16> c = b;
#pragma unroll
    for (int i = 0; i < (IN_BF16 ? 2 : 4); ++i)
      asm volatile("" : "+v"(c.q[i].x), "+v"(c.q[i].y), "+v"(c.q[i].z), "+v"(c.q[i].w));
    unpack_block<IN_BF16>(c, sm, z);
    fwht128_group(z, lig);
  }
}

// RAW = 1 (MS-EDEN with amax_out): also the maximum of |x| over the raw input.
template <int IN_BF16, int MODE, int RAW = 0>
__global__ __launch_bounds__(kThreads) void k_quant_rows(QuantParams p) {
  __shared__ float red[kThreads / kWave];
  float s_t = 1.0f;
  if constexpr (takes_tensor_scale(MODE)) {
    s_t = tensor_scale(p, red);
    if (blockIdx.x == 0 && threadIdx.x == 0) *p.ts_out = s_t;
  }
  const uint32_t lig = group_pos(threadIdx.x & 63u);
  // this thread's block among the workgroup's 256 consecutive blocks
  const uint32_t rank = (threadIdx.x & ~63u) + lane_block_rank(threadIdx.x & 63u);
  const SignMasks sm = make_masks<IN_BF16>(p, lig);
  const uint32_t stride = gridDim.x * kThreads;
  float lmax = 0.0f, araw = 0.0f;
  // the next block's loads are issued before the current block is processed
  RawBlock<IN_BF16> cur = {}, nxt = {};
  uint32_t base = blockIdx.x * kThreads;
  // (loads past the last block re-read it, unconditionally: see RowSink)
  if (base < p.nblocks) load_row_block<IN_BF16>(p, min(base + rank, p.nblocks - 1), cur);
  for (; base < p.nblocks; base += stride) {
    const uint32_t gb = base + rank;
    const bool active = gb < p.nblocks;
    load_row_block<IN_BF16>(p, min(base + stride + rank, p.nblocks - 1), nxt);
    // lanes past the end hold stale values; they fill whole rotation groups
    // and store nothing, so they never reach an output
    float z[16];
    if constexpr (RAW) {
      // (lanes past the end hold a copy of the last block: harmless here)
      uint32_t w[IN_BF16 ? 8 : 16];
#pragma unroll
      for (int i = 0; i < (IN_BF16 ? 2 : 4); ++i) {
        w[4 * i] = cur.q[i].x;
        w[4 * i + 1] = cur.q[i].y;
        w[4 * i + 2] = cur.q[i].z;
        w[4 * i + 3] = cur.q[i].w;
      }
      araw = fmaxf(araw, raw_absmax<IN_BF16>(w));
    }
    load_z<IN_BF16>(cur, sm, p.rht, lig, z);
    if constexpr (MODE == kRot) quant_block<MODE>(z, gb, PtrSink{p, gb, active}, p, s_t, lmax);
    else quant_block<MODE>(z, gb, RowSink(p, base, rank), p, s_t, lmax);
    cur = nxt;
  }
  if constexpr (writes_partials(MODE)) {
    const float m = block_max(lmax, red, kThreads);
    if (threadIdx.x == 0) p.partial[blockIdx.x] = m;
  }
  if constexpr (RAW) raw_partial(p, araw, red);
}

// ---------------------------------------------------------------- matrix-core rotation
// For bf16 input the 128-point rotation z = c H diag(s) x (H the Sylvester
// Hadamard matrix, H[o][k] = (-1)^popcount(o & k), c = 1/sqrt(128)) is a
// product with a +-1 matrix, which bf16 holds exactly: it runs on the matrix
// cores (v_mfma_f32_32x32x16_bf16: exact products, fp32 accumulation), and
// c is applied in fp32 afterwards.  The butterfly stages cost 8 vector
// instructions per element, about 40 % of an MS-EDEN pass's vector work,
// on units that the coding needs; the matrix cores are idle in a quantizer.
// The result matches the butterflies' to fp32 rounding (both round sums of
// the same exact products), not bit for bit.
//
// MFMA D[i][j] = sum_k A[i][k] B[k][j], 32 x 32 x 16: lane l holds
// A[l % 32][8h + e] and B[8h + e][l % 32] (h = l / 32, e = 0..7), and
// D[8 (r / 4) + 4h + r % 4][l % 32] in accumulator r.  For a 128-group:
//   step t (0..7) takes input positions k = in(t, h, e),
//   chunk n (0..3) gives outputs o = 64 i2 + 16 n + 4 i[4:3] + i[1:0] of
//   A row i,
// so that lane (j, h) ends with output 64h + 16n + r in accumulator r of
// chunk n: the whole 16-block 4h + n of its group j.  Since bits 4 and 5 of
// k are bits 0 and 1 of t, A for (n, t) is (-1)^popcount(n & t & 3) times A
// for (0, t): a workgroup keeps A(0, t) and its negation, t = 0..7, in LDS
// (16 fragments x 64 lanes x 16 bytes).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kRotNorm = 0x1.6a09e6p-4f;  // fp32(1/sqrt(128)) = 0x3DB504F3

__host__ __device__ constexpr uint32_t mx_out0(uint32_t i) {
  return ((i & 4u) << 4) | ((i >> 3) << 2) | (i & 3u);
}

// Input position (0..127) of operand slot (h, e) in step t.  AXIS 0: the 8
// slots of a lane are 8 consecutive elements (one 16-byte load); AXIS 1
// (operands read from LDS one element at a time): slot bit 2 -> position
// bit 3 and the lane half -> bit 2, which puts the two lane halves' rows
// four rows apart, on disjoint LDS banks.
template <int AXIS>
__host__ __device__ constexpr uint32_t mx_in(uint32_t t, uint32_t h, uint32_t e) {
  if constexpr (AXIS == 0) return 16u * t + 8u * h + e;
  else return 16u * t + 8u * (e >> 2) + 4u * h + (e & 3u);
}

typedef uint4 RotFrags[16][64];

// Byte v of kWalsh8: bit e is the parity of v & e (e, v = 0..7).
constexpr uint64_t walsh8() {
  uint64_t c = 0;
  for (uint32_t v = 0; v < 8; ++v)
    for (uint32_t e = 0; e < 8; ++e)
      c |= (uint64_t)(__builtin_popcount(v & e) & 1) << (8 * v + e);
  return c;
}
constexpr uint64_t kWalsh8 = walsh8();
static_assert(kWalsh8 == 0x963C5AF066CCAA00ull, "Walsh patterns of 3-bit indices");

// The decomposition mx_build_frags uses, checked at compile time for every
// output row, step, lane half and slot: in(t, h, e) is the slot's base plus
// its varying bits, popcount(o & k) splits accordingly, and the sign of
// position k sits at bit sh + e (axis 0) or sh + 8 (e / 4) + e % 4 (axis 1)
// of sign word t / 2.
template <int AXIS>
constexpr bool mx_frag_rule_holds() {
  for (uint32_t i = 0; i < 32; ++i)
    for (uint32_t t = 0; t < 8; ++t)
      for (uint32_t h = 0; h < 2; ++h)
        for (uint32_t e = 0; e < 8; ++e) {
          const uint32_t o = mx_out0(i), k = mx_in<AXIS>(t, h, e), base = mx_in<AXIS>(t, h, 0);
          const uint32_t v = AXIS == 0 ? (o & 7u) : ((o & 3u) | ((o >> 1) & 4u));
          const uint32_t par = ((uint32_t)__builtin_popcount(o & base) + (uint32_t)(kWalsh8 >> (8 * v + e))) & 1u;
          if (par != ((uint32_t)__builtin_popcount(o & k) & 1u)) return false;
          const uint32_t sh = 16u * (t & 1u) + (AXIS == 0 ? 8u * h : 4u * h);
          const uint32_t bit = AXIS == 0 ? sh + e : sh + 8u * (e >> 2) + (e & 3u);
          if (32u * (t >> 1) + bit != k) return false;
        }
  return true;
}
static_assert(mx_frag_rule_holds<0>() && mx_frag_rule_holds<1>(), "fragment sign decomposition");

// Fragment f = 2t + neg of lane l holds the bf16 signs
// (-1)^(popcount(o & k) + s_k + neg), o = out(l % 32), k = in(t, l / 32, e),
// e = 0..7.  The 8 positions of a slot are one base (the bits that do not
// vary with e) plus 3 varying bits -- bits 0..2 of k on axis 0, bits 0, 1
// and 3 on axis 1 -- so popcount(o & k) is popcount(o & base) plus the
// parity of (o's varying bits) & e, one byte of kWalsh8; the random signs
// s_k of the 8 positions are one byte (axis 0) or two nibbles (axis 1) of
// the sign word.  Each wave builds whole fragments (f is wave-uniform), so
// the sign word is read from scalar registers.
template <int AXIS>
__device__ __forceinline__ void mx_build_frags(const uint32_t sg[4], RotFrags &fr) {
  const uint32_t l = threadIdx.x & 63u, h = l >> 5, o = mx_out0(l & 31u);
  const uint32_t v = AXIS == 0 ? (o & 7u) : ((o & 3u) | ((o >> 1) & 4u));
  const uint32_t walsh = (uint32_t)(kWalsh8 >> (8u * v)) & 0xFFu;
  const uint32_t nw = blockDim.x >> 6;
  for (uint32_t f = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); f < 16u; f += nw) {
    const uint32_t t = f >> 1, neg = f & 1u;
    const uint32_t word = (t >> 1) == 0u ? sg[0] : (t >> 1) == 1u ? sg[1] : (t >> 1) == 2u ? sg[2] : sg[3];
    const uint32_t base = mx_in<AXIS>(t, h, 0u);
    const uint32_t sh = 16u * (t & 1u) + (AXIS == 0 ? 8u * h : 4u * h);
    const uint32_t sbits = AXIS == 0 ? ((word >> sh) & 0xFFu)
                                     : (((word >> sh) & 0xFu) | (((word >> (sh + 8u)) & 0xFu) << 4));
    const uint32_t flip = (((uint32_t)__builtin_popcount(o & base) + neg) & 1u) ? 0xFFu : 0u;
    const uint32_t bits = walsh ^ sbits ^ flip;  // bit e set: slot e holds -1
    uint32_t w[4];
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i)  // bf16 +-1 pairs: slots 2i (low half) and 2i + 1
      w[i] = 0x3F803F80u | ((bits << (15u - 2u * i)) & 0x8000u) | ((bits << (30u - 2u * i)) & 0x80000000u);
    fr[f][l] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// The four chunks' accumulators of one group from the 8 steps' B operands.
__device__ __forceinline__ void mx_rotate(const RotFrags &fr, const uint4 (&xb)[8], uint32_t lane,
                                          f32x16_t (&acc)[4]) {
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = f32x16_t{};
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const bf16x8_t b = __builtin_bit_cast(bf16x8_t, xb[t]);
    const bf16x8_t ap = __builtin_bit_cast(bf16x8_t, fr[2 * t][lane]);
    const bf16x8_t am = __builtin_bit_cast(bf16x8_t, fr[2 * t + 1][lane]);
#pragma unroll
    for (int n = 0; n < 4; ++n)
      acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16((__builtin_popcount(n & t & 3) & 1) ? am : ap, b, acc[n],
                                                        0, 0, 0);
  }
}

// A lane's four consecutive blocks' outputs, stored together.
struct QuadOut {
  uint32_t c[8];
  uint32_t s;
  float t[4];
};

struct SlotSink {
  QuadOut &q;
  int n;
  bool active;
  __device__ __forceinline__ void codes(uint32_t lo, uint32_t hi) const {
    q.c[2 * n] = lo;
    q.c[2 * n + 1] = hi;
  }
  __device__ __forceinline__ void scale(uint32_t e) const { q.s |= (e & 0xFFu) << (8 * n); }
  __device__ __forceinline__ void target(float v) const { q.t[n] = v; }
};

// MS-EDEN (FP4 codes, no INT branch) of a lane's four blocks with the
// correction's sums as fused multiply-adds: N = sum z^2 and, per block,
// sum z g (g the signed E2M1 values), so that D = sum z zhat is
// sum_blocks s_b (sum z g) -- one instruction per element for each sum
// instead of a product, a second product and a tree of additions.  The
// codes and the block scales s_b are those of the exact rule (eden_codes);
// the sums and the quotient N / D differ from its pairwise trees only in
// rounding.  A block maximum below 2^-50 (other than zero) anywhere in the
// wave, or a sum that is not finite, leaves the wave to the exact rule: the
// function then returns false and has written nothing.  gb0 is a multiple
// of 4, so that the four blocks share one Philox call of the fused variant.
template <int MODE>
__device__ __forceinline__ bool mx_eden_fast(const f32x16_t (&acc)[4], uint32_t gb0, bool active,
                                             const QuantParams &p, float s_t, float &lmax, QuadOut &q) {
  float sb[4], nb[4], db[4];
  uint32_t lo[4], hi[4];
  bool ok = true;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    float z[16], a = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      z[r] = acc[n][r] * kRotNorm;
      a = fmaxf(a, fabsf(z[r]));
    }
    ok = ok && !(a > 0.0f && a < 0x1p-50f);
    sb[n] = div_by<6>(a);
    const float rs = (a > 0.0f) ? rcp_rn(sb[n]) : 0.0f;  // 0: signed zero codes
    float y[16], g[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) y[r] = z[r] * rs;
    e2m1x16_rne(y, lo[n], hi[n]);
    e2m1x16_value(lo[n], hi[n], g);
    float s0 = 0.0f, s1 = 0.0f, d0 = 0.0f, d1 = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      s0 = __builtin_fmaf(z[r], z[r], s0);
      s1 = __builtin_fmaf(z[r + 1], z[r + 1], s1);
      d0 = __builtin_fmaf(z[r], g[r], d0);
      d1 = __builtin_fmaf(z[r + 1], g[r + 1], d1);
    }
    nb[n] = s0 + s1;
    db[n] = sb[n] * (d0 + d1);
  }
  float c[4];  // t_b = s_b * c
  if (p.group16) {
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      ok = ok && nb[n] <= 0x1.fffffep127f && db[n] <= 0x1.fffffep127f;
      c[n] = (db[n] > 0.0f) ? nb[n] * __builtin_amdgcn_rcpf(db[n]) : 1.0f;
    }
  } else {
    float N = (nb[0] + nb[1]) + (nb[2] + nb[3]);
    float D = (db[0] + db[1]) + (db[2] + db[3]);
    const auto pn = __builtin_amdgcn_permlane32_swap(__float_as_uint(N), __float_as_uint(N), false, false);
    const auto pd = __builtin_amdgcn_permlane32_swap(__float_as_uint(D), __float_as_uint(D), false, false);
    N = __uint_as_float(pn[0]) + __uint_as_float(pn[1]);
    D = __uint_as_float(pd[0]) + __uint_as_float(pd[1]);
    ok = ok && N <= 0x1.fffffep127f && D <= 0x1.fffffep127f;
    const float cg = (D > 0.0f) ? N * __builtin_amdgcn_rcpf(D) : 1.0f;
#pragma unroll
    for (int n = 0; n < 4; ++n) c[n] = cg;
  }
  if (__builtin_amdgcn_ballot_w64(!ok) != 0) return false;
  Philox4 u;
  if constexpr (MODE == kEdenFused) u = uniforms8(p.key, (uint64_t)(gb0 >> 3), 1u);
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const float t = sb[n] * c[n];
    q.c[2 * n] = lo[n];
    q.c[2 * n + 1] = hi[n];
    if constexpr (MODE == kEden) {
      q.t[n] = t;
      if (active) lmax = fmaxf(lmax, t);
    } else {
      const uint32_t e = e4m3_sr_sat(fminf(div_rn(t, s_t), 448.0f), uniform_at(u, (int)((gb0 & 7u) + n)));
      q.s |= e << (8 * n);
    }
  }
  return true;
}

// Code the lane's four blocks (accumulators acc, first block gb0) into q
// (mx_store writes them).  MS-EDEN's group of 128 is the two lane halves' 4 + 4 blocks: the
// sums add in the same pairwise tree as the 8-lane groups of the butterfly
// kernels, ((b0 + b1) + (b2 + b3)) + ((b4 + b5) + (b6 + b7)).
template <int MODE>
__device__ __forceinline__ void mx_code4(f32x16_t (&acc)[4], uint32_t gb0, bool active, const QuantParams &p,
                                         float s_t, float &lmax, QuadOut &q) {
  constexpr bool EDEN = MODE == kEden || MODE == kEdenFused || MODE == kIf4Eden || MODE == kIf4EdenFused;
  q.s = 0u;
  if constexpr (MODE == kEden || MODE == kEdenFused) {
    if (mx_eden_fast<MODE>(acc, gb0, active, p, s_t, lmax, q)) return;
  }
  if constexpr (EDEN) {
    EdenBlock b[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      float z[16], a = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        z[r] = acc[n][r] * kRotNorm;
        a = fmaxf(a, fabsf(z[r]));
      }
      b[n] = eden_codes<MODE>(z, a);
    }
    if (p.group16) {
#pragma unroll
      for (int n = 0; n < 4; ++n) eden_emit<MODE>(b[n], b[n].N, b[n].D, gb0 + n, SlotSink{q, n, active}, p, s_t, lmax);
    } else {
      float N = (b[0].N + b[1].N) + (b[2].N + b[3].N);
      float D = (b[0].D + b[1].D) + (b[2].D + b[3].D);
      // the partner half's sums (lanes l and l ^ 32 swap)
      const auto pn = __builtin_amdgcn_permlane32_swap(__float_as_uint(N), __float_as_uint(N), false, false);
      const auto pd = __builtin_amdgcn_permlane32_swap(__float_as_uint(D), __float_as_uint(D), false, false);
      N = __uint_as_float(pn[0]) + __uint_as_float(pn[1]);
      D = __uint_as_float(pd[0]) + __uint_as_float(pd[1]);
#pragma unroll
      for (int n = 0; n < 4; ++n) eden_emit<MODE>(b[n], N, D, gb0 + n, SlotSink{q, n, active}, p, s_t, lmax);
    }
  } else {
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      float z[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) z[r] = acc[n][r] * kRotNorm;
      quant_block<MODE>(z, gb0 + n, SlotSink{q, n, active}, p, s_t, lmax);
    }
  }
}

template <int MODE>
__device__ __forceinline__ void mx_store(const QuadOut &q, uint32_t gb0, bool active, const QuantParams &p) {
  if constexpr (MODE != kAmax && MODE != kRot) {
    if (active) {
      uint4 *c = reinterpret_cast<uint4 *>(p.codes + (size_t)gb0 * 8);
      c[0] = make_uint4(q.c[0], q.c[1], q.c[2], q.c[3]);
      c[1] = make_uint4(q.c[4], q.c[5], q.c[6], q.c[7]);
      if constexpr (MODE == kEden || MODE == kIf4Eden)
        *reinterpret_cast<float4 *>(p.tb + gb0) = make_float4(q.t[0], q.t[1], q.t[2], q.t[3]);
      else
        *reinterpret_cast<uint32_t *>(p.scales + gb0) = q.s;
    }
  }
}

// The column kernel's stores: a column's two groups of a tile (128 bytes of
// codes) are held by lanes (g, h) = (j / 16, h) of that column, 32 bytes
// each.  Lanes j and j ^ 16 trade the 16-byte halves that belong to the
// other store, so that each of the two code stores writes one whole group:
// 64 contiguous bytes per column from four lanes, instead of four separate
// 16-byte pieces.  Targets and scales are already contiguous per column.
template <int MODE>
__device__ __forceinline__ void mx_store_cols(const QuadOut &q, uint32_t gb0, uint32_t g, uint32_t h, bool col_ok,
                                              bool grp1_ok, const QuantParams &p) {
  if constexpr (MODE != kAmax && MODE != kRot) {
    uint32_t send[4], recv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      send[k] = g ? q.c[k] : q.c[4 + k];
      recv[k] = (uint32_t)__shfl_xor((int)send[k], 16, kWave);
    }
    // this lane's group's codes start at byte 8 (gb0 - 4h); group 0's at 64 g
    // bytes before that
    uint8_t *const base0 = p.codes + (size_t)(gb0 - 4u * h) * 8 - 64u * g;
    if (col_ok) {
      const uint4 a = g ? make_uint4(recv[0], recv[1], recv[2], recv[3]) : make_uint4(q.c[0], q.c[1], q.c[2], q.c[3]);
      *reinterpret_cast<uint4 *>(base0 + 32u * h + 16u * g) = a;
    }
    if (col_ok && grp1_ok) {
      const uint4 b = g ? make_uint4(q.c[4], q.c[5], q.c[6], q.c[7]) : make_uint4(recv[0], recv[1], recv[2], recv[3]);
      *reinterpret_cast<uint4 *>(base0 + 64u + 32u * h + 16u * g) = b;
    }
    if (col_ok && (g == 0u || grp1_ok)) {
      if constexpr (MODE == kEden || MODE == kIf4Eden)
        *reinterpret_cast<float4 *>(p.tb + gb0) = make_float4(q.t[0], q.t[1], q.t[2], q.t[3]);
      else
        *reinterpret_cast<uint32_t *>(p.scales + gb0) = q.s;
    }
  }
}

// Axis 0, bf16 input, rotation on.  A wave tile is 32 consecutive groups of
// the row-major group order (4096 elements; contiguous in memory for a dense
// tensor); lane (j, h) rotates group j of the tile and codes its blocks
// 4h .. 4h+3, so that the tile's codes, scales and targets are contiguous
// too.  The tile is staged in the wave's 8 KB of LDS by direct-to-LDS loads:
// load i brings groups 4i .. 4i+3 (1 KB, coalesced); lane l of it takes
// 16-byte chunk c = (l % 16) ^ ((4i + l / 16) % 16) of group 4i + l / 16 and
// lands at slot 64i + l.  The MFMA operand of lane (j, h) in step t (chunk
// 2t + h of group j) is then one ds_read_b128 whose 16 lanes of a quarter
// wave hit 16 different 16-byte bank groups.  Groups past the last read
// zeros (dense: the buffer's range check) or the last group (strided), and
// store nothing.  A tile's outputs are stored in the next iteration, after
// its successor's loads were issued, so that the wait for a tile's data
// never waits for the previous tile's stores.  RAW as for k_quant_rows.
// (SR is held to three waves per SIMD, 168 VGPRs: it would take 176, and
// the few values the compiler then keeps in scratch cost less than the
// third wave gains -- the whole SR call on a 32768x11008 gradient is 4 %
// faster along rows, 7 % along columns.  MS-EDEN with max|x| out would take
// 170 and fits in 168 without spilling.)
template <int MODE, int RAW = 0>
__global__ __launch_bounds__(kMxThreads)
__attribute__((amdgpu_waves_per_eu(MODE == kSr || (MODE == kEden && RAW) ? 3 : 1)))
void k_quant_rows_mx(QuantParams p) {
  typedef __attribute__((address_space(3))) void lds_void;
  __shared__ RotFrags fr;
  __shared__ uint4 stage[kMxThreads / kWave][512];
  // (the reductions before and after the loop use the stage's first bytes)
  float *const red = reinterpret_cast<float *>(&stage[0][0]);
  const uint32_t lane = threadIdx.x & 63u, j = lane & 31u, h = lane >> 5;
  const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t G = p.K16 >> 3;  // groups per row
  const uint32_t nf = p.R * G;    // groups
  const uint32_t ntiles = (nf + 31u) >> 5;
  const uint32_t waves = gridDim.x * (kMxThreads / kWave);
  const bool dense = p.ld == (int64_t)p.K;
  // load i, lane l: group 4i + a4 (a4 = l / 16), 16-byte chunk
  // (l % 16) ^ (4i + a4) (i < 4; i + 4 alike), at byte
  // 1024 i + 256 a4 + 16 ((l % 16) ^ (4i + a4)) = 1024 i + (vbase ^ 64 i)
  const uint32_t a4 = lane >> 4;
  const uint32_t vbase = 256u * a4 + ((16u * (lane & 15u)) ^ (16u * a4));
  auto load_tile = [&](uint32_t T) {
    if (dense) {
      const uint64_t base = (uint64_t)T * 8192u, total = (uint64_t)nf * 256u;
      const uint64_t left = total - base;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(static_cast<const uint8_t *>(p.x) + base), (short)0, (int)(left < 8192u ? left : 8192u),
          kRsrcWord3);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)&stage[w][64 * i], 16,
                                                 (vbase ^ (64u * (i & 3))) + 1024u * (i & 3), 4096u * (i >> 2), 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t f = 32u * T + 4u * i + a4;
        const uint32_t fl = f < nf ? f : nf - 1u;
        const uint32_t row = fdiv(8u * fl, p.k16div);
        const uint32_t c = (lane & 15u) ^ ((4u * i + a4) & 15u);
        const uint16_t *src = static_cast<const uint16_t *>(p.x) + (size_t)row * p.ld + 128u * (fl - row * G) + 8u * c;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                         (lds_void *)&stage[w][64 * i], 16, 0, 0);
      }
    }
  };
  // this lane's operand in step t: group j, chunk 2t + h, at byte
  // 16 (64 (j / 4) + 16 (j % 4) + ((2t + h) ^ (j % 16))) = rd ^ 32t
  const uint32_t rd = 1024u * (j >> 2) + 256u * (j & 3u) + 16u * (h ^ (j & 15u));
  float lmax = 0.0f, araw = 0.0f;
  QuadOut q;
  uint32_t gbq = 0u;
  bool actq = false;
  uint32_t T = __builtin_amdgcn_readfirstlane(blockIdx.x * (kMxThreads / kWave) + (threadIdx.x >> 6));
  // Without a tensor-scale reduction (which uses the stage), the first
  // tile's loads are in flight while the fragments are built.
  float s_t = 1.0f;
  if constexpr (takes_tensor_scale(MODE)) {
    s_t = tensor_scale<kMxThreads>(p, red);
    if (blockIdx.x == 0 && threadIdx.x == 0) *p.ts_out = s_t;
  } else {
    if (T < ntiles) load_tile(T);
  }
  mx_build_frags<0>(p.sg, fr);
  __syncthreads();
  if constexpr (takes_tensor_scale(MODE)) {
    if (T < ntiles) load_tile(T);
  }
  for (; T < ntiles; T += waves) {
    // the staged tile (direct-to-LDS loads count in vmcnt only; earlier
    // stores were issued before these loads)
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    uint4 xb[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
      xb[t] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint8_t *>(&stage[w][0]) + (rd ^ (32u * t)));
    if constexpr (RAW) {
      uint32_t wd[32];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        wd[4 * t] = xb[t].x;
        wd[4 * t + 1] = xb[t].y;
        wd[4 * t + 2] = xb[t].z;
        wd[4 * t + 3] = xb[t].w;
      }
      araw = fmaxf(araw, raw_absmax<1>(wd));
    }
    f32x16_t acc[4];
    mx_rotate(fr, xb, lane, acc);
    mx_store<MODE>(q, gbq, actq, p);  // the previous tile's outputs
    // the operands are in registers (the MFMAs have read them): the stage
    // takes the next tile
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    if (T + waves < ntiles) load_tile(T + waves);
    const uint32_t f = 32u * T + j;
    gbq = 8u * f + 4u * h;
    actq = f < nf;
    mx_code4<MODE>(acc, gbq, actq, p, s_t, lmax, q);
  }
  mx_store<MODE>(q, gbq, actq, p);
  if constexpr (writes_partials(MODE)) {
    const float m = block_max(lmax, red, kMxThreads);
    if (threadIdx.x == 0) p.partial[blockIdx.x] = m;
  }
  if constexpr (RAW) raw_partial<kMxThreads>(p, araw, red);
}

// Axis 1, bf16 input (rows 16-byte aligned), rotation on.  A workgroup tile
// is two 128-row groups of 64 columns (256 rows x 128 bytes, 32 KB), staged
// in LDS by direct-to-LDS loads: wave w loads rows 64w .. 64w+63, load i
// rows 64w + 8i .. +7 (1 KB, coalesced); lane l of it takes 16-byte chunk
// (l % 8) ^ f(row) of its row, f(r) = 2 ((r / 2) % 2) + 4 (r / 128), landing
// at slot 8 row + l % 8.  Wave w then rotates columns 16w .. 16w+15 of both
// groups: lane (j, h) takes column 16w + j % 16 of group j / 16, so that its
// column's 128 bytes of codes per tile are in 4 lanes of one store.  Its
// operand in step t is the 8 elements at rows in(t, h, e) =
// 16t + 8 (e / 4) + 4h + e % 4 of its group: two transposing reads
// (ds_read_b64_tr_b16: in a group of 16 lanes, lane i receives element i % 4
// of the 8-byte vectors that lanes 4q + i / 4 point at, q = 0..3), each lane
// pointing at 4 columns of one of 4 rows; the swizzle puts the 8 rows that
// 32 lanes read on disjoint LDS banks.  Lane (j, h) codes blocks 4h .. 4h+3.
// Columns past the last read what follows in memory, rows past the last
// zeros (the buffer's range check at the tensor's end); neither is stored.
// RAW as for k_quant_cols.
template <int MODE, int RAW = 0>
__global__ __launch_bounds__(kMxThreads) __attribute__((amdgpu_waves_per_eu(MODE == kSr ? 3 : 1)))
void k_quant_cols_mx(QuantParams p) {
  typedef __attribute__((address_space(3))) void lds_void;
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
  static_assert(kMxThreads == 256, "four waves of 16 columns");
  __shared__ RotFrags fr;
  __shared__ uint4 stage[2048];  // 256 rows x 8 chunks
  // (the reductions before and after the loop use the stage's first bytes)
  float *const red = reinterpret_cast<float *>(&stage[0]);
  const uint32_t lane = threadIdx.x & 63u, j = lane & 31u, h = lane >> 5;
  const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t ngroups = p.rows >> 7;
  const uint32_t npair = p.mx_rdiv.d, nct = p.mx_cdiv.d;  // 256-row tiles, 64-column tiles
  const uint32_t ntiles = npair * nct;
  // Tile order: row pair fastest, so that consecutive tiles code the next
  // 128 bytes of the same output rows; each XCD (workgroups go round-robin to
  // the 8 XCDs: the grid is a multiple of 8) takes a contiguous eighth of the
  // tiles.
  const uint32_t xcd = blockIdx.x & 7u, per = (ntiles + 7u) >> 3;
  const uint32_t first = xcd * per, last = min(first + per, ntiles);
  const uint32_t step = gridDim.x >> 3;
  const uint32_t row_bytes = (uint32_t)p.ld * 2u;  // 256 rows of it fit in 31 bits (launch condition)
  const uint64_t end = ((uint64_t)(p.rows - 1u) * (uint64_t)p.ld + p.cols) * 2u;
  // load i, lane l: row 64w + 8i + l / 8, chunk (l % 8) ^ f(row)
  const uint32_t voff = (64u * w + (lane >> 3)) * row_bytes +
                        16u * ((lane & 7u) ^ (2u * ((lane >> 4) & 1u) + 4u * (w >> 1)));
  auto load_tile = [&](uint32_t T) {
    const uint32_t cb = fdiv(T, p.mx_rdiv), tp = T - cb * npair;
    const uint64_t base = (uint64_t)tp * 256u * row_bytes + 128u * cb;
    const uint64_t left = end > base ? end - base : 0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(static_cast<const uint8_t *>(p.x) + base), (short)0,
        (int)(left < 0x7FFFFFFFull ? left : 0x7FFFFFFFull), kRsrcWord3);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)&stage[64u * (8u * w + i)], 16,
                                               voff + 8u * i * row_bytes, 0, 0, 0);
  };
  // transposing reads: lane (G = l / 16, s = l % 16) of group g = G % 2, half
  // h = G / 2 points at row 128g + 16t + 8 e2 + 4h + s / 4, columns
  // 16w + 4 (s % 4) .. +3 (e2 = 0, 1: elements 0..3 and 4..7 of the
  // operand), at byte rdb + 2048 t + 1024 e2
  const uint32_t sl = lane & 15u, gg = (lane >> 4) & 1u;
  const uint32_t rdb = 128u * (128u * gg + 4u * h + (sl >> 2)) +
                       16u * ((2u * w + ((sl & 3u) >> 1)) ^ (2u * ((sl >> 3) & 1u) + 4u * gg)) + 8u * (sl & 1u);
  const uint8_t *const st8 = reinterpret_cast<const uint8_t *>(&stage[0]);
  float lmax = 0.0f, araw = 0.0f;
  QuadOut q;
  uint32_t gbq = 0u;
  bool colq = false, grp1q = false;
  uint32_t T = first + (blockIdx.x >> 3);
  // Without a tensor-scale reduction (which uses the stage), the first
  // tile's loads are in flight while the fragments are built.
  float s_t = 1.0f;
  if constexpr (takes_tensor_scale(MODE)) {
    s_t = tensor_scale<kMxThreads>(p, red);
    if (blockIdx.x == 0 && threadIdx.x == 0) *p.ts_out = s_t;
  } else {
    if (T < last) load_tile(T);
  }
  mx_build_frags<1>(p.sg, fr);
  __syncthreads();
  if constexpr (takes_tensor_scale(MODE)) {
    if (T < last) load_tile(T);
  }
  for (; T < last; T += step) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's part of the tile
    __builtin_amdgcn_s_barrier();        // ... and every wave's
    uint4 xb[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(st8 + rdb + 2048u * t));
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(st8 + rdb + 2048u * t + 1024u));
      const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
      xb[t] = make_uint4(a.x, a.y, b.x, b.y);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the operands are in registers
    __builtin_amdgcn_s_barrier();        // every wave's: the stage is free
    const uint32_t cb = fdiv(T, p.mx_rdiv), tp = T - cb * npair;
    const uint32_t col = 64u * cb + 16u * w + (j & 15u), grp = 2u * tp + (j >> 4);
    const bool act = col < p.cols && grp < ngroups;
    if constexpr (RAW) {
      uint32_t wd[32];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        wd[4 * t] = xb[t].x;
        wd[4 * t + 1] = xb[t].y;
        wd[4 * t + 2] = xb[t].z;
        wd[4 * t + 3] = xb[t].w;
      }
      // (columns past the last hold other data: masked)
      if (act) araw = fmaxf(araw, raw_absmax<1>(wd));
    }
    mx_store_cols<MODE>(q, gbq, j >> 4, h, colq, grp1q, p);  // the previous tile's outputs
    if (T + step < last) load_tile(T + step);
    f32x16_t acc[4];
    mx_rotate(fr, xb, lane, acc);
    gbq = col * p.K16 + 8u * grp + 4u * h;
    colq = col < p.cols;
    grp1q = 2u * tp + 1u < ngroups;
    mx_code4<MODE>(acc, gbq, act, p, s_t, lmax, q);
  }
  mx_store_cols<MODE>(q, gbq, j >> 4, h, colq, grp1q, p);
  if constexpr (writes_partials(MODE)) {
    const float m = block_max(lmax, red, kMxThreads);
    if (threadIdx.x == 0) p.partial[blockIdx.x] = m;
  }
  if constexpr (RAW) raw_partial<kMxThreads>(p, araw, red);
}

// ---------------------------------------------------------------- axis 1
// A wave's tile is 128 positions along the reduction (input rows) x 128 bytes
// of columns (64 bf16 or 32 fp32 columns).  Lane (q = lane bits 2, 4, 5;
// lig = group position) holds the rows T0 + 16 lig .. + 15 of the 16-byte
// column chunk q: the 16-element blocks of that chunk's kColCols columns, and
// the 8 lanes with the same q hold one 128-position rotation group per
// column.  Each load instruction reads 8 rows x 128 contiguous bytes (a
// buffer load whose row offset is a scalar); no LDS is used.  The rotation
// sign of a position is the same for every column: one mask per row.
template <int IN_BF16>
struct ColCfg {
  static constexpr uint32_t kEs = IN_BF16 ? 2 : 4;                        // input element bytes
  static constexpr uint32_t kColCols = IN_BF16 ? 2 * kColWords : kColWords; // columns per lane
  static constexpr uint32_t kTileCols = 8 * kColCols;                      // columns per wave tile
};
static_assert(kColWords == 4, "a lane loads one 16-byte chunk per row");

// Raw words of a lane's 16 rows x 16 bytes.
typedef uint32_t ColRaw[16][kColWords];

// Load tile (tt, tc) for this lane (zeros outside the tensor).  The buffer
// starts at the tile's first row: offsets within a 128-row tile stay below
// 2^31 for rows of up to 16 MiB.
template <int IN_BF16>
__device__ __forceinline__ void col_load(const QuantParams &p, uint32_t tt, uint32_t tc, uint32_t lig, uint32_t q,
                                         ColRaw &w) {
  using C = ColCfg<IN_BF16>;
  const uint32_t row0 = tt * 128 + 16 * lig;
  const uint32_t c0 = tc * C::kTileCols + C::kColCols * q;
  const uint64_t tile_off = (uint64_t)(tt * 128) * (uint64_t)p.ld * C::kEs;
  const uint64_t end = ((uint64_t)(p.rows - 1) * (uint64_t)p.ld + p.cols) * C::kEs;
  const uint64_t left = end > tile_off ? end - tile_off : 0;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(static_cast<const uint8_t *>(p.x) + tile_off), (short)0,
      (int)(left < 0xFFFFFFFFull ? left : 0xFFFFFFFFull), kRsrcWord3);
  const uint32_t step = (uint32_t)p.ld * C::kEs;  // bytes per input row
  const uint32_t vo = (16 * lig * (uint32_t)p.ld + c0) * C::kEs;
  const bool any = row0 < p.rows && c0 < p.cols;  // rows % 16 == 0: whole slab or nothing
  const bool full = any && p.vec && c0 + C::kColCols <= p.cols;
  // (one choice for the whole wave: were lanes to differ, the zeroing below
  // would have to wait for the other lanes' loads into the same registers)
  if (__builtin_amdgcn_ballot_w64(!full) == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, r * step, 0);
#pragma unroll
      for (int c = 0; c < kColWords; ++c) w[r][c] = v[c];
    }
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int c = 0; c < kColWords; ++c) w[r][c] = 0u;
    if (any) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
#pragma unroll
        for (uint32_t j = 0; j < C::kColCols; ++j) {
          if (c0 + j >= p.cols) continue;
          if (IN_BF16)
            w[r][j >> 1] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, vo + 2 * j, r * step, 0)
                            << (16 * (j & 1));
          else
            w[r][j] = __builtin_amdgcn_raw_buffer_load_b32(rs, vo + 4 * j, r * step, 0);
        }
      }
    }
  }
}

// One wave tile (tile row tt, tile column tc).
template <int IN_BF16, int MODE, int RAW = 0>
__device__ __forceinline__ void col_tile(const QuantParams &p, uint32_t tt, uint32_t tc, uint32_t lig, uint32_t q,
                                         uint32_t sbits, float s_t, float &lmax, float &araw) {
  using C = ColCfg<IN_BF16>;
  ColRaw w;
  col_load<IN_BF16>(p, tt, tc, lig, q, w);
  if constexpr (RAW) {
    // the raw tile before any rotation (outside the tensor it holds zeros)
    uint32_t f[16 * kColWords];
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int c = 0; c < kColWords; ++c) f[r * kColWords + c] = w[r][c];
    araw = fmaxf(araw, raw_absmax<IN_BF16>(f));
  }
  const uint32_t row0 = tt * 128 + 16 * lig;
  const uint32_t c0 = tc * C::kTileCols + C::kColCols * q;
  const bool rows_ok = row0 < p.rows;
  const uint32_t kblk = tt * 8 + lig;
  // the rotation's sign flips, once per raw word: the sign of a position is
  // the same for every column (bf16: both halves of a word)
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint32_t sflip = ((sbits >> r) & 1u) ? (IN_BF16 ? 0x80008000u : 0x80000000u) : 0u;
#pragma unroll
    for (int c = 0; c < kColWords; ++c) w[r][c] ^= sflip;
  }
#pragma unroll
  for (uint32_t j = 0; j < C::kColCols; ++j) {
    const int wi = IN_BF16 ? (int)(j >> 1) : (int)j;
    // (words taken by selects: when the compiler leaves this loop rolled, as
    // for the larger block codes, an index would move the tile to scratch)
    uint32_t cw[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
      cw[r] = wi == 0 ? w[r][0] : wi == 1 ? w[r][1] : wi == 2 ? w[r][2] : w[r][3];
    float z[16];
    auto unpack = [&]() {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        z[r] = IN_BF16 ? ((j & 1) ? bf16_hi(cw[r]) : bf16_lo(cw[r])) : __uint_as_float(cw[r]);
    };
    unpack();
    // fast stages; the exact ones when the wave holds a zero output (the raw
    // words pass through an empty asm so that the compiler recomputes the
    // in-lane stages instead of keeping them alive from the fast path)
    if (p.rht && fwht128_group_fast(z, lig)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(cw[r]));
      unpack();
      fwht128_group(z, lig);
    }
    const uint32_t col = c0 + j;
    const bool active = rows_ok && col < p.cols;
    const uint32_t gbc = active ? col * p.K16 + kblk : 0u;
    quant_block<MODE>(z, gbc, PtrSink{p, gbc, active}, p, s_t, lmax);
  }
}

// RAW as for k_quant_rows.
template <int IN_BF16, int MODE, int RAW = 0>
__global__ __launch_bounds__(kThreads) void k_quant_cols(QuantParams p) {
  __shared__ float red[kThreads / kWave];
  float s_t = 1.0f;
  if constexpr (takes_tensor_scale(MODE)) {
    s_t = tensor_scale(p, red);
    if (blockIdx.x == 0 && threadIdx.x == 0) *p.ts_out = s_t;
  }
  const uint32_t lane = threadIdx.x & 63u, lig = group_pos(lane);
  const uint32_t q = ((lane >> 2) & 1u) | ((lane >> 4) << 1);  // column chunk of this lane
  const uint32_t sbits = p.rht ? lane_sign_bits(p.sg, lig) : 0u;
  const uint32_t nct = p.ctiles_div.d;
  const uint32_t waves = gridDim.x * (kThreads / kWave);
  float lmax = 0.0f, araw = 0.0f;

  for (uint32_t t = __builtin_amdgcn_readfirstlane(blockIdx.x * (kThreads / kWave) + (threadIdx.x >> 6));
       t < p.ntiles; t += waves) {
    const uint32_t tt = fdiv(t, p.ctiles_div);
    const uint32_t tc = t - tt * nct;
    col_tile<IN_BF16, MODE, RAW>(p, tt, tc, lig, q, sbits, s_t, lmax, araw);
  }
  if constexpr (writes_partials(MODE)) {
    const float m = block_max(lmax, red, kThreads);
    if (threadIdx.x == 0) p.partial[blockIdx.x] = m;
  }
  if constexpr (RAW) raw_partial(p, araw, red);
}

// ---------------------------------------------------------------- both axes
// MS-EDEN of one tensor along both axes from one read of it (the backward
// pass re-quantizes the output gradient along its rows and along its
// reduction dimension).  A workgroup takes a tile of 128 rows x 4 wave tiles
// of columns: the row-wise pass codes its 128-element row groups, then each
// wave codes its column tile of the same rows, re-reading the tile from L2.
// pr / pc: the row-wise (axis 0) and column-wise (axis 1) outputs; each gets
// its own partial maxima and target scales.
template <int IN_BF16, int MODE>
__global__ __launch_bounds__(kThreads) void k_quant_dual(QuantParams pr, QuantParams pc) {
  constexpr uint32_t kWidth = 4 * ColCfg<IN_BF16>::kTileCols;  // tile columns
  constexpr uint32_t kBpr = kWidth / 16;     // row blocks per tile row
  __shared__ float red[kThreads / kWave];
  float s_r = 1.0f, s_c = 1.0f;
  if constexpr (MODE == kEdenFused) {
    s_r = *pr.ts_in;
    s_c = *pc.ts_in;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      *pr.ts_out = s_r;
      *pc.ts_out = s_c;
    }
  }
  const uint32_t lane = threadIdx.x & 63u, lig = group_pos(lane);
  const uint32_t rank = (threadIdx.x & ~63u) + lane_block_rank(lane);
  const uint32_t q = ((lane >> 2) & 1u) | ((lane >> 4) << 1);
  const uint32_t sbits = pc.rht ? lane_sign_bits(pc.sg, lig) : 0u;
  const SignMasks sm = make_masks<IN_BF16>(pr, lig);
  const uint32_t ntc = (pr.cols + kWidth - 1) / kWidth;   // tile columns
  const uint32_t ntiles = (pr.rows / 128) * ntc;
  float lmax_r = 0.0f, lmax_c = 0.0f;
  for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const uint32_t tt = t / ntc, tcw = t - tt * ntc;
    // row-wise: 128 x kBpr blocks, rotation groups of 8 consecutive blocks
#pragma unroll 1
    for (uint32_t i = 0; i < 128 * kBpr / kThreads; ++i) {
      const uint32_t bt = i * kThreads + rank;
      const uint32_t row = tt * 128 + bt / kBpr;
      const uint32_t kb = tcw * kBpr + bt % kBpr;
      const bool active = kb < pr.K16;
      const uint32_t gb = row * pr.K16 + kb;
      RawBlock<IN_BF16> raw = {};
      if (active) load_row_block<IN_BF16>(pr, gb, raw);
      float z[16];
      load_z<IN_BF16>(raw, sm, pr.rht, lig, z);
      quant_block<MODE>(z, active ? gb : 0u, PtrSink{pr, active ? gb : 0u, active}, pr, s_r, lmax_r);
    }
    // column-wise: wave w takes wave tile column 4 * tcw + w
    float unused = 0.0f;  // (the two-axis call takes no amax_out)
    col_tile<IN_BF16, MODE>(pc, tt, 4 * tcw + (threadIdx.x >> 6), lig, q, sbits, s_c, lmax_c, unused);
  }
  if constexpr (MODE == kEden) {
    const float mr = block_max(lmax_r, red, kThreads);
    if (threadIdx.x == 0) pr.partial[blockIdx.x] = mr;
    const float mc = block_max(lmax_c, red, kThreads);
    if (threadIdx.x == 0) pc.partial[blockIdx.x] = mc;
  }
}

// Both axes at once, bf16 input (rows 16-byte aligned), rotation on.  A
// workgroup tile is 128 rows x 128 columns: one group along each axis
// (32 KB), staged in LDS by direct-to-LDS loads from one read of the input:
// wave w loads rows 32w .. 32w+31, load i rows 32w + 4i .. +3 (1 KB); lane l
// of it takes 16-byte chunk (l % 16) ^ f(row), f(r) = 4 (r % 4) + (r / 4) % 4,
// landing at slot 16 row + l % 16.  Then wave w rotates rows 32w .. 32w+31
// (lane (j, h): two 8-byte reads per step of row 32w + j, at positions
// in(t, h, e) = 16t + 8 (e / 4) + 4h + e % 4) and columns 32w .. 32w+31
// (lane (j, h): two transposing reads per step, as in k_quant_cols_mx), with
// the same fragments.  f spreads the 4 rows of a transposing read over 4
// different 64-byte bank groups, and the 32 rows of a row read over 16
// chunk positions (two rows per bank group).  Two stages (80 KB of LDS with
// the fragments, two workgroups per CU, all resident): tile T is read from
// one while tile T + step loads into the other, issued as soon as every
// wave is done with the previous tile, so each load has a whole tile's work
// to land.  Tiles run with the column block fastest, each XCD taking a
// contiguous share, so that a row's successive 64-byte code runs are
// written by one L2.  pr / pc: the row-wise (axis 0) and column-wise
// (axis 1) outputs.
template <int MODE>
__global__ __launch_bounds__(kMxThreads) void k_quant_dual_mx(QuantParams pr, QuantParams pc) {
  typedef __attribute__((address_space(3))) void lds_void;
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
  static_assert(kMxThreads == 256, "four waves of 32 rows and 32 columns");
  __shared__ RotFrags fr;
  // two tiles of 128 rows x 16 chunks, as two objects: the compiler then
  // sees that the loads into one do not touch the operand reads of the
  // other (into one array with a variable index, it waits for the loads
  // before every LDS read)
  __shared__ uint4 stage0[2048], stage1[2048];
  float *const red = reinterpret_cast<float *>(&stage0[0]);
  float s_r = 1.0f, s_c = 1.0f;
  if constexpr (MODE == kEdenFused) {
    s_r = *pr.ts_in;
    s_c = *pc.ts_in;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      *pr.ts_out = s_r;
      *pc.ts_out = s_c;
    }
  }
  mx_build_frags<1>(pr.sg, fr);
  __syncthreads();
  const uint32_t lane = threadIdx.x & 63u, j = lane & 31u, h = lane >> 5;
  const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t ncb = pr.K16 >> 3, nrb = pr.rows >> 7;  // 128-column blocks, 128-row blocks
  const uint32_t ntiles = nrb * ncb;
  const uint32_t xcd = blockIdx.x & 7u, per = (ntiles + 7u) >> 3;
  const uint32_t first = xcd * per, last = min(first + per, ntiles);
  const uint32_t step = gridDim.x >> 3;
  const uint32_t row_bytes = (uint32_t)pr.ld * 2u;  // 128 rows of it fit in 31 bits (launch condition)
  const uint64_t end = ((uint64_t)(pr.rows - 1u) * (uint64_t)pr.ld + pr.cols) * 2u;
  auto swz = [](uint32_t r) { return 4u * (r & 3u) + ((r >> 2) & 3u); };
  // load i, lane l: row 32w + 4i + l / 16, chunk (l % 16) ^ f(row)
  uint32_t voff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t r = 32u * w + 4u * i + (lane >> 4);
    voff[i] = r * row_bytes + 16u * ((lane & 15u) ^ swz(r));
  }
  auto load_tile = [&](uint32_t T, uint4 *dst) {
    const uint32_t rb = fdiv(8u * T, pr.k16div), cb = T - rb * ncb;
    const uint64_t base = (uint64_t)rb * 128u * row_bytes + 256u * cb;
    const uint64_t left = end > base ? end - base : 0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(static_cast<const uint8_t *>(pr.x) + base), (short)0,
        (int)(left < 0x7FFFFFFFull ? left : 0x7FFFFFFFull), kRsrcWord3);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)&dst[64u * (8u * w + i)], 16, voff[i], 0, 0, 0);
  };
  // row reads: row rr = 32w + j, chunk (2t + e2) ^ f(rr), byte 8h
  const uint32_t rr = 32u * w + j, fr_r = swz(rr);
  // transposing reads: lane (G = l / 16, s = l % 16) points at row
  // 16t + 8 e2 + 4 (G / 2) + s / 4 (f of which is 4 (s / 4) + e2... taken per
  // read) and columns 32w + 16 (G % 2) + 4 (s % 4) .. +3
  const uint32_t sl = lane & 15u, g16 = lane >> 4;
  const uint32_t ccol = 32u * w + 16u * (g16 & 1u) + 4u * (sl & 3u);
  float lmax_r = 0.0f, lmax_c = 0.0f;
  // One tile: T's operands from stage cur while the next tile's loads go to
  // stage nxt.
  auto tile = [&](uint32_t T, bool later, const uint4 *cur, uint4 *nxt) {
    // This wave's part of tile T.  A later tile's loads were issued before
    // the previous tile's six output stores (two 16-byte code stores and
    // one 16-byte store of targets or scales per axis, each a single
    // instruction), so waiting for all but the last six memory operations
    // waits for the loads and leaves those stores in flight.
    if (later) __builtin_amdgcn_s_waitcnt(0x0F76);  // vmcnt(6)
    // every wave's part of tile T has landed, and every wave is done with
    // the other stage (the previous tile's operands are in registers)
    __builtin_amdgcn_s_barrier();
    if (T + step < last) load_tile(T + step, nxt);
    const uint8_t *const st8 = reinterpret_cast<const uint8_t *>(cur);
    const uint32_t rb = fdiv(8u * T, pr.k16div), cb = T - rb * ncb;
    f32x16_t acc[4];
    {
      uint4 xr[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint2 a = *reinterpret_cast<const uint2 *>(st8 + 256u * rr + 16u * ((2u * t) ^ fr_r) + 8u * h);
        const uint2 b = *reinterpret_cast<const uint2 *>(st8 + 256u * rr + 16u * ((2u * t + 1u) ^ fr_r) + 8u * h);
        xr[t] = make_uint4(a.x, a.y, b.x, b.y);
      }
      mx_rotate(fr, xr, lane, acc);
    }
    {
      QuadOut q;
      const uint32_t gb0 = (128u * rb + rr) * pr.K16 + 8u * cb + 4u * h;
      mx_code4<MODE>(acc, gb0, true, pr, s_r, lmax_r, q);
      mx_store<MODE>(q, gb0, true, pr);
    }
    {
      uint4 xc[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        uint2 v[2];
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          const uint32_t r = 16u * t + 8u * e2 + 4u * (g16 >> 1) + (sl >> 2);
          const s16x4_t x4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4 *)(st8 + 256u * r + 16u * ((ccol >> 3) ^ swz(r)) + 2u * (ccol & 7u)));
          v[e2] = __builtin_bit_cast(uint2, x4);
        }
        xc[t] = make_uint4(v[0].x, v[0].y, v[1].x, v[1].y);
      }
      mx_rotate(fr, xc, lane, acc);
      QuadOut q;
      const uint32_t gb0 = (128u * cb + 32u * w + j) * pc.K16 + 8u * rb + 4u * h;
      mx_code4<MODE>(acc, gb0, true, pc, s_c, lmax_c, q);
      mx_store<MODE>(q, gb0, true, pc);
    }
  };
  uint32_t T = first + (blockIdx.x >> 3);
  if (T < last) load_tile(T, stage0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's part of the first tile
  // tiles alternate between the stages: the loop body is written out twice
  for (bool later = false; T < last; later = true) {
    tile(T, later, stage0, stage1);
    T += step;
    if (T >= last) break;
    tile(T, true, stage1, stage0);
    T += step;
  }
  if constexpr (MODE == kEden) {
    const float mr = block_max(lmax_r, red, kMxThreads);
    if (threadIdx.x == 0) pr.partial[blockIdx.x] = mr;
    const float mc = block_max(lmax_c, red, kMxThreads);
    if (threadIdx.x == 0) pc.partial[blockIdx.x] = mc;
  }
}

// ---------------------------------------------------------------- MS-EDEN scales
// Scale byte of a target t (sign bit: IF4's INT flag, bit 7 of the byte).
__device__ __forceinline__ uint32_t eden_scale_byte(float t, const Divisor &s_t, uint32_t u16) {
  const uint32_t flag = (__float_as_uint(t) >> 24) & 0x80u;
  return e4m3_sr_sat(fminf(div_rn(fabsf(t), s_t), 448.0f), u16) | flag;
}

// The same byte where |t| and the quotient lie in their ordinary ranges --
// the refined division's fast path exact (|t| in [2^-60, 2^60], s_t too)
// and t / s_t in [2^-6, 448], where no clamp applies and the rounding is
// the integer addition of e4m3_sr_sat -- with the general form for the
// lanes outside them.  The same bytes as eden_scale_byte for every t; IF4:
// the sign bit of t is the INT flag (NVFP4 targets are never negative).
template <int IF4>
__device__ __forceinline__ uint32_t eden_scale_byte_fix(float t, const Divisor &d, uint32_t u16) {
  const float a = fabsf(t);
  const float q0 = a * d.y;
  const float r = __builtin_fmaf(-d.b, q0, a);
  const float v = __builtin_fmaf(r, d.y, q0);
  const bool fast = d.ok && a >= kDivLo && a <= kDivHi && v >= 0x1p-6f && v <= 448.0f;
  uint32_t e = (__float_as_uint(v) + ((u16 << 4) ^ 0xFFFFFu) - (960u << 20)) >> 20;
  if (__builtin_amdgcn_ballot_w64(!fast) != 0) {
    if (!fast) e = e4m3_sr_sat(fminf(div_rn(a, d), 448.0f), u16);
  }
  if constexpr (IF4) e |= (__float_as_uint(t) >> 24) & 0x80u;
  return e;
}

// s_t = max t / 448 (or the given scale); scale = SR of min(t / s_t, 448)
// onto the E4M3 grid, one Philox call per 8 consecutive blocks (tag 1).
template <int IF4>
__global__ __launch_bounds__(kThreads) void k_eden_scales(QuantParams p) {
  __shared__ float red[kThreads / kWave];
  // Whole calls (8 blocks each).  This thread's first call's targets do not
  // depend on the tensor scale: their loads are in flight during its
  // reduction (clamped to the last whole call, so they are unconditional
  // within a grid that has one).
  const uint32_t nfull = p.nblocks / 8u;
  const uint32_t stride = gridDim.x * kThreads;
  const float4 *tb = reinterpret_cast<const float4 *>(p.tb);
  uint32_t c = blockIdx.x * kThreads + threadIdx.x;
  float4 a0 = make_float4(0.0f, 0.0f, 0.0f, 0.0f), a1 = a0;
  if (nfull != 0u) {
    const uint32_t c0 = c < nfull ? c : nfull - 1u;
    a0 = tb[2 * (size_t)c0];
    a1 = tb[2 * (size_t)c0 + 1];
  }
  float s_t;
  if (p.ts_in) {
    s_t = *p.ts_in;
  } else {
    const float m = block_max(partials_max(p.partial, p.npartial), red, kThreads);
    s_t = (m > 0.0f) ? m / 448.0f : 1.0f;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *p.ts_out = s_t;
  if (p.amax_out && blockIdx.x == 0) {
    const float m = block_max(partials_max(p.rpartial, p.npartial), red, kThreads);
    if (threadIdx.x == 0) *p.amax_out = m;
  }
  const Divisor dst = make_divisor(s_t);
  // The next call's targets are loaded while this one is coded (clamped to
  // the last call, so the load is unconditional).
  auto code8 = [&](uint32_t c, const float4 &t0, const float4 &t1) {
    const Philox4 u = uniforms8(p.key, (uint64_t)c, 1u);
    const float t[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t e = eden_scale_byte_fix<IF4>(t[j], dst, uniform_at(u, j));
      if (j < 4) lo |= e << (8 * j);
      else hi |= e << (8 * (j - 4));
    }
    *reinterpret_cast<uint2 *>(p.scales + (size_t)c * 8) = make_uint2(lo, hi);
  };
  if (c < nfull) {
    for (; c < nfull; c += stride) {
      const uint32_t cn = c + stride < nfull ? c + stride : nfull - 1;
      const float4 n0 = tb[2 * (size_t)cn], n1 = tb[2 * (size_t)cn + 1];
      code8(c, a0, a1);
      a0 = n0;
      a1 = n1;
    }
  }
  // the last, partial call
  if (p.nblocks % 8u && blockIdx.x * kThreads + threadIdx.x == nfull % stride) {
    const Philox4 u = uniforms8(p.key, (uint64_t)nfull, 1u);
    for (uint32_t j = 0; nfull * 8u + j < p.nblocks; ++j)
      p.scales[nfull * 8u + j] = (uint8_t)eden_scale_byte(p.tb[nfull * 8u + j], dst, uniform_at(u, (int)j));
  }
}

// ---------------------------------------------------------------- launch
// bf16 input with the rotation: the matrix-core kernels (axis 1: rows
// 16-byte aligned, 256 of them within 2^31 bytes).
static bool use_mx(const QuantParams &p, int in_bf16, int axis) {
  return in_bf16 && p.rht && (axis == 0 || (p.vec && (uint64_t)p.ld * 2u * 256u <= 0x7FFFFFFFull));
}

uint32_t quant_grid(const QuantParams &p, int in_bf16, int axis) {
  const uint64_t waves = kThreads / kWave;
  // matrix-core rotation: axis 0, a wave per 32 groups; axis 1, a workgroup
  // per 128 rows x 128 columns
  const uint64_t mx_units = axis == 0 ? (((uint64_t)p.R * (p.K16 / 8) + 31) / 32 + waves - 1) / waves
                                      : ((uint64_t)p.mx_rdiv.d * p.mx_cdiv.d + 7) / 8 * 8;
  uint64_t units = use_mx(p, in_bf16, axis) ? mx_units
                   : axis == 0             ? ((uint64_t)p.nblocks + kThreads - 1) / kThreads
                                           : ((uint64_t)p.ntiles + waves - 1) / waves;
  if (units < 1) units = 1;
  return (uint32_t)(units < (uint64_t)kMaxPartials ? units : kMaxPartials);
}

uint32_t eden_scales_grid(const QuantParams &p) {
  uint64_t calls = ((uint64_t)p.nblocks + 7) / 8;
  uint64_t g = (calls + kThreads - 1) / kThreads;
  if (g < 1) g = 1;
  return (uint32_t)(g < (uint64_t)kMaxPartials ? g : kMaxPartials);
}

template <int IN_BF16, int MODE, int RAW = 0>
static void launch_one(const QuantParams &p, int axis, uint32_t grid, hipStream_t s) {
  if (use_mx(p, IN_BF16, axis) && axis == 0)
    hipLaunchKernelGGL((k_quant_rows_mx<MODE, RAW>), dim3(grid), dim3(kMxThreads), 0, s, p);
  else if (use_mx(p, IN_BF16, axis))
    hipLaunchKernelGGL((k_quant_cols_mx<MODE, RAW>), dim3(grid), dim3(kMxThreads), 0, s, p);
  else if (axis == 0)
    hipLaunchKernelGGL((k_quant_rows<IN_BF16, MODE, RAW>), dim3(grid), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((k_quant_cols<IN_BF16, MODE, RAW>), dim3(grid), dim3(kThreads), 0, s, p);
}

template <int IN_BF16>
static void launch_mode(const QuantParams &p, int axis, Mode mode, uint32_t grid, hipStream_t s) {
  switch (mode) {
    case kAmax: launch_one<IN_BF16, kAmax>(p, axis, grid, s); break;
    case kRtn: launch_one<IN_BF16, kRtn>(p, axis, grid, s); break;
    case kSr: launch_one<IN_BF16, kSr>(p, axis, grid, s); break;
    case kIf4: launch_one<IN_BF16, kIf4>(p, axis, grid, s); break;
    case kEden:
      if (p.amax_out) launch_one<IN_BF16, kEden, 1>(p, axis, grid, s);
      else launch_one<IN_BF16, kEden>(p, axis, grid, s);
      break;
    case kEdenFused: launch_one<IN_BF16, kEdenFused>(p, axis, grid, s); break;
    case kRot: launch_one<IN_BF16, kRot>(p, axis, grid, s); break;
    case kFos: launch_one<IN_BF16, kFos>(p, axis, grid, s); break;
    case kSearch: launch_one<IN_BF16, kSearch>(p, axis, grid, s); break;
    case kIf4Sr: launch_one<IN_BF16, kIf4Sr>(p, axis, grid, s); break;
    case kIf4Eden:
      if (p.amax_out) launch_one<IN_BF16, kIf4Eden, 1>(p, axis, grid, s);
      else launch_one<IN_BF16, kIf4Eden>(p, axis, grid, s);
      break;
    case kIf4EdenFused: launch_one<IN_BF16, kIf4EdenFused>(p, axis, grid, s); break;
  }
}

hipError_t launch_quant(const QuantParams &p, int in_bf16, int axis, Mode mode, uint32_t grid,
                        hipStream_t s) {
  if (in_bf16)
    launch_mode<1>(p, axis, mode, grid, s);
  else
    launch_mode<0>(p, axis, mode, grid, s);
  return hipGetLastError();
}

// Both axes on the matrix cores: bf16 with the rotation, rows 16-byte
// aligned, 128 of them within 2^31 bytes, whole 128-column blocks.
static bool use_dual_mx(const QuantParams &pr, int in_bf16) {
  return in_bf16 && pr.rht && pr.vec && pr.cols % 128 == 0 && (uint64_t)pr.ld * 2u * 128u <= 0x7FFFFFFFull;
}

uint32_t dual_grid(const QuantParams &pr, int in_bf16) {
  if (use_dual_mx(pr, in_bf16)) {
    // two workgroups per compute unit (80 KB of LDS each), all resident:
    // each loops over its XCD's tiles with its loads one tile ahead
    const uint64_t tiles = (uint64_t)(pr.rows / 128) * (pr.cols / 128);
    uint64_t g = (tiles + 7) / 8 * 8;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus >= 8) {
      const uint64_t resident = (uint64_t)(2 * cus / 8) * 8;
      if (g > resident) g = resident;
    }
    return (uint32_t)(g < (uint64_t)kMaxPartials ? g : kMaxPartials);
  }
  const uint32_t width = 4u * (in_bf16 ? ColCfg<1>::kTileCols : ColCfg<0>::kTileCols);
  const uint64_t tiles = (uint64_t)(pr.rows / 128) * ((pr.cols + width - 1) / width);
  uint64_t g = tiles < 1 ? 1 : tiles;
  return (uint32_t)(g < (uint64_t)kMaxPartials ? g : kMaxPartials);
}

hipError_t launch_quant_dual(const QuantParams &pr, const QuantParams &pc, int in_bf16, int fused,
                             uint32_t grid, hipStream_t s) {
  if (use_dual_mx(pr, in_bf16)) {
    if (fused) hipLaunchKernelGGL((k_quant_dual_mx<kEdenFused>), dim3(grid), dim3(kMxThreads), 0, s, pr, pc);
    else hipLaunchKernelGGL((k_quant_dual_mx<kEden>), dim3(grid), dim3(kMxThreads), 0, s, pr, pc);
  } else if (in_bf16) {
    if (fused) hipLaunchKernelGGL((k_quant_dual<1, kEdenFused>), dim3(grid), dim3(kThreads), 0, s, pr, pc);
    else hipLaunchKernelGGL((k_quant_dual<1, kEden>), dim3(grid), dim3(kThreads), 0, s, pr, pc);
  } else {
    if (fused) hipLaunchKernelGGL((k_quant_dual<0, kEdenFused>), dim3(grid), dim3(kThreads), 0, s, pr, pc);
    else hipLaunchKernelGGL((k_quant_dual<0, kEden>), dim3(grid), dim3(kThreads), 0, s, pr, pc);
  }
  return hipGetLastError();
}

// Empty tensor: the tensor scale is the given one or 1, the maximum 0 (a
// kernel rather than copies, so that nothing is staged through host memory).
__global__ void k_trivial_scale(float *ts, const float *ts_in, float *amax_out) {
  *ts = ts_in ? *ts_in : 1.0f;
  if (amax_out) *amax_out = 0.0f;
}

hipError_t launch_trivial_scale(float *ts, const float *ts_in, float *amax_out, hipStream_t s) {
  hipLaunchKernelGGL(k_trivial_scale, dim3(1), dim3(1), 0, s, ts, ts_in, amax_out);
  return hipGetLastError();
}

hipError_t launch_eden_scales(const QuantParams &p, bool if4, uint32_t grid, hipStream_t s) {
  if (if4) hipLaunchKernelGGL(k_eden_scales<1>, dim3(grid), dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL(k_eden_scales<0>, dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace nv4
