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
__device__ __forceinline__ float partials_max(const float *v, uint32_t n) {
  static_assert(kMaxPartials % kThreads == 0, "partials per thread");
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void *)v, (short)0, (int)(4 * n), kRsrcWord3);
  float m[kMaxPartials / kThreads];
#pragma unroll
  for (int k = 0; k < kMaxPartials / kThreads; ++k)
    m[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, 4 * (threadIdx.x + k * kThreads), 0, 0));
  float a = 0.0f;
#pragma unroll
  for (int k = 0; k < kMaxPartials / kThreads; ++k) a = fmaxf(a, m[k]);
  return a;
}

__device__ __forceinline__ float tensor_scale(const QuantParams &p, float *red) {
  if (p.ts_in) return *p.ts_in;
  if (p.amax_in) {
    const float a = *p.amax_in;
    return (a > 0.0f) ? a / p.top : 1.0f;
  }
  const float m = block_max(partials_max(p.partial, p.npartial), red, kThreads);
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
__device__ __forceinline__ void raw_partial(const QuantParams &p, float araw, float *red) {
  const float m = block_max(araw, red, kThreads);
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
      float sqf[16], sqi[16], y[16], vf[16];
      uint32_t flo, fhi, ilo = 0, ihi = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = z[i] * rf;
      e2m1x16_rne(y, flo, fhi);
      e2m1x16_value(flo, fhi, vf);  // signed grid values
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t sn = sign_nib(z[i]);
        const float df = z[i] - vf[i] * Sf;
        sqf[i] = df * df;
        uint32_t mi = 0;
        if (ei) mi = (uint32_t)rintf(fminf(fabsf(z[i] * ri), 7.0f));
        const float vi = (float)mi;
        const float di = z[i] - (sn ? -vi : vi) * Si;
        sqi[i] = di * di;
        if (i < 8) ilo |= (sn | mi) << (4 * i);
        else ihi |= (sn | mi) << (4 * (i - 8));
      }
      const bool use_int = tree16(sqi) < tree16(sqf);
      out.codes(use_int ? ilo : flo, use_int ? ihi : fhi);
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
    } else if constexpr (MODE == kEden || MODE == kEdenFused) {
      // RTN codes under the exact scale a/6; correction c = sum z^2 /
      // sum z*zhat over the group; target t = (a/6) * c.
      const float s_b = div_by<6>(a);
      const float r = (a > 0.0f) ? rcp_rn(s_b) : 0.0f;
      float nn[16], dd[16], y[16], g[16];
      uint32_t lo, hi;
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = z[i] * r;  // r = 0 when a = 0: signed zeros
      e2m1x16_rne(y, lo, hi);
      e2m1x16_value(lo, hi, g);  // signed grid values
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float zh = g[i] * s_b;
        nn[i] = z[i] * z[i];
        dd[i] = z[i] * zh;
      }
      float N = tree16(nn), D = tree16(dd);
      if (!p.group16) {
        N = N + lane_xor<1>(N);
        D = D + lane_xor<1>(D);
        N = N + lane_xor<2>(N);
        D = D + lane_xor<2>(D);
        N = N + lane_xor<4>(N);
        D = D + lane_xor<4>(D);
      }
      const float c = (D > 0.0f) ? div_rn(N, D) : 1.0f;
      const float t = s_b * c;
      if constexpr (MODE == kEden) {
        out.codes(lo, hi);
        out.target(t);
        if (active) lmax = fmaxf(lmax, t);
      } else {
        const Philox4 u = uniforms8(p.key, (uint64_t)(gb >> 3), 1u);
        const uint32_t e = e4m3_sr_sat(fminf(div_rn(t, s_t), 448.0f), uniform_at(u, (int)(gb & 7u)));
        out.codes(lo, hi);
        out.scale(e);
      }
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
  if constexpr (MODE == kRtn || MODE == kSr || MODE == kIf4 || MODE == kFos || MODE == kSearch ||
                MODE == kEdenFused) {
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
  if constexpr (MODE == kAmax || MODE == kEden) {
    const float m = block_max(lmax, red, kThreads);
    if (threadIdx.x == 0) p.partial[blockIdx.x] = m;
  }
  if constexpr (RAW) raw_partial(p, araw, red);
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
    uint32_t cw[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) cw[r] = w[r][wi];
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
  if constexpr (MODE == kRtn || MODE == kSr || MODE == kIf4 || MODE == kFos || MODE == kSearch ||
                MODE == kEdenFused) {
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
  if constexpr (MODE == kAmax || MODE == kEden) {
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

// ---------------------------------------------------------------- MS-EDEN scales
// s_t = max t / 448 (or the given scale); scale = SR of min(t / s_t, 448)
// onto the E4M3 grid, one Philox call per 8 consecutive blocks (tag 1).
__global__ __launch_bounds__(kThreads) void k_eden_scales(QuantParams p) {
  __shared__ float red[kThreads / kWave];
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
  // Whole calls (8 blocks each): the next call's targets are loaded while
  // this one is coded (clamped to the last call, so the load is unconditional).
  const uint32_t nfull = p.nblocks / 8u;
  const uint32_t stride = gridDim.x * kThreads;
  auto code8 = [&](uint32_t c, const float4 &t0, const float4 &t1) {
    const Philox4 u = uniforms8(p.key, (uint64_t)c, 1u);
    const float t[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t e = e4m3_sr_sat(fminf(div_rn(t[j], s_t), 448.0f), uniform_at(u, j));
      if (j < 4) lo |= e << (8 * j);
      else hi |= e << (8 * (j - 4));
    }
    *reinterpret_cast<uint2 *>(p.scales + (size_t)c * 8) = make_uint2(lo, hi);
  };
  uint32_t c = blockIdx.x * kThreads + threadIdx.x;
  if (c < nfull) {
    const float4 *tb = reinterpret_cast<const float4 *>(p.tb);
    float4 a0 = tb[2 * (size_t)c], a1 = tb[2 * (size_t)c + 1];
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
      p.scales[nfull * 8u + j] = (uint8_t)e4m3_sr_sat(fminf(div_rn(p.tb[nfull * 8u + j], s_t), 448.0f), uniform_at(u, (int)j));
  }
}

// ---------------------------------------------------------------- launch
uint32_t quant_grid(const QuantParams &p, int in_bf16, int axis) {
  (void)in_bf16;
  const uint64_t waves = kThreads / kWave;
  uint64_t units = axis == 0 ? ((uint64_t)p.nblocks + kThreads - 1) / kThreads
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

template <int IN_BF16, int MODE>
static void launch_one(const QuantParams &p, int axis, uint32_t grid, hipStream_t s) {
  if (axis == 0)
    hipLaunchKernelGGL((k_quant_rows<IN_BF16, MODE>), dim3(grid), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((k_quant_cols<IN_BF16, MODE>), dim3(grid), dim3(kThreads), 0, s, p);
}

template <int IN_BF16>
static void launch_mode(const QuantParams &p, int axis, Mode mode, uint32_t grid, hipStream_t s) {
  switch (mode) {
    case kAmax: launch_one<IN_BF16, kAmax>(p, axis, grid, s); break;
    case kRtn: launch_one<IN_BF16, kRtn>(p, axis, grid, s); break;
    case kSr: launch_one<IN_BF16, kSr>(p, axis, grid, s); break;
    case kIf4: launch_one<IN_BF16, kIf4>(p, axis, grid, s); break;
    case kEden:
      if (p.amax_out) {
        if (axis == 0)
          hipLaunchKernelGGL((k_quant_rows<IN_BF16, kEden, 1>), dim3(grid), dim3(kThreads), 0, s, p);
        else
          hipLaunchKernelGGL((k_quant_cols<IN_BF16, kEden, 1>), dim3(grid), dim3(kThreads), 0, s, p);
      } else {
        launch_one<IN_BF16, kEden>(p, axis, grid, s);
      }
      break;
    case kEdenFused: launch_one<IN_BF16, kEdenFused>(p, axis, grid, s); break;
    case kRot: launch_one<IN_BF16, kRot>(p, axis, grid, s); break;
    case kFos: launch_one<IN_BF16, kFos>(p, axis, grid, s); break;
    case kSearch: launch_one<IN_BF16, kSearch>(p, axis, grid, s); break;
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

uint32_t dual_grid(const QuantParams &pr, int in_bf16) {
  const uint32_t width = 4u * (in_bf16 ? ColCfg<1>::kTileCols : ColCfg<0>::kTileCols);
  const uint64_t tiles = (uint64_t)(pr.rows / 128) * ((pr.cols + width - 1) / width);
  uint64_t g = tiles < 1 ? 1 : tiles;
  return (uint32_t)(g < (uint64_t)kMaxPartials ? g : kMaxPartials);
}

hipError_t launch_quant_dual(const QuantParams &pr, const QuantParams &pc, int in_bf16, int fused,
                             uint32_t grid, hipStream_t s) {
  if (in_bf16) {
    if (fused) hipLaunchKernelGGL((k_quant_dual<1, kEdenFused>), dim3(grid), dim3(kThreads), 0, s, pr, pc);
    else hipLaunchKernelGGL((k_quant_dual<1, kEden>), dim3(grid), dim3(kThreads), 0, s, pr, pc);
  } else {
    if (fused) hipLaunchKernelGGL((k_quant_dual<0, kEdenFused>), dim3(grid), dim3(kThreads), 0, s, pr, pc);
    else hipLaunchKernelGGL((k_quant_dual<0, kEden>), dim3(grid), dim3(kThreads), 0, s, pr, pc);
  }
  return hipGetLastError();
}

hipError_t launch_eden_scales(const QuantParams &p, uint32_t grid, hipStream_t s) {
  hipLaunchKernelGGL(k_eden_scales, dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace nv4
