// gemm.hip -- block-scaled FP4 GEMM for gfx950:
//   C[M x N] = (ts_a * ts_b) * sum_k A[m][k] * B[n][k],
// A[m][k] = E2M1(code) * E4M3(scale of its 16-block), both operands packed
// K-major as written by the quantizers (Quartet II's NVFP4 linear-layer
// GEMMs; abstract and news summary, "Kerninnovationen").
//
// gfx950's native FP4 matrix instructions take one power-of-two (E8M0) scale
// per 32 elements; NVFP4 has an E4M3 scale per 16.  The product of an E2M1
// value and an E4M3 scale has at most 6 significant bits and lies in
// [2^-10, 2688], so it is exact in fp16: each fragment is dequantized exactly
// in registers -- v_cvt_scalef32_pk_f16_fp4 (two codes per instruction, unit
// scale) then one packed fp16 multiply by the block scale -- and multiplied
// on the fp16 matrix cores (v_mfma_f32_32x32x16_f16), accumulating in fp32.
//
// Tiling: a workgroup of 4 waves (one per SIMD) computes a 256 x 256 tile,
// each wave a 128 x 128 sub-tile as 4 x 4 MFMA tiles of 32 x 32 (256 fp32
// accumulators per lane).  Operands go straight from global memory into
// registers with buffer loads (rows past M or N read as zero): FP4 is 4x
// smaller than the fp16 it expands to, so the two waves sharing a row panel
// re-read it from L1/L2 instead of staging it through LDS.  K advances in
// chunks of 128, double-buffered in registers.
//
// K order inside a chunk: MFMA lane half h = lane / 32 holds k slots
// 8h .. 8h+7 of each 16-wide step.  A lane loads the 64 codes at
// k0 + 64h .. k0 + 64h + 63 (32 bytes) and feeds dword j of them to step j.
// A and B use the same assignment, so the permutation of k cancels.
//
// Workgroup order: workgroups are dispatched round-robin to the 8 XCDs; the
// logical tile index is remapped so that each XCD receives a contiguous run,
// and runs are laid out in groups of 4 tile-rows so that the ~32 workgroups
// resident on one XCD share A and B panels in that XCD's L2.
#include "kernels.hpp"

namespace nv4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr uint32_t kTile = 256, kWaveTile = 128, kChunk = 128, kGroupM = 4, kXcds = 8;
constexpr int kRsrcWord3 = 0x00020000;

struct Chunk {
  u32x4_t code[8][2];  // fragments 0..3 = A, 4..7 = B: 64 codes each
  uint32_t scale[8];   // the four E4M3 bytes of those 64 codes
};

struct Panels {
  __amdgpu_buffer_rsrc_t ac, as, bc, bs;  // codes / scales of this tile's rows
  uint32_t a_soff_c[4], a_soff_s[4], b_soff_c[4], b_soff_s[4];  // fragment row offsets
  uint32_t voff_c, voff_s;  // lane row offset within a fragment, + the lane half's k
  uint32_t row_c, row_s;    // lane row offset without the k part (generic loads)
  uint32_t K;
  uint32_t h;
};

__device__ __forceinline__ u32x4_t ld128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t ld32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t ld8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
}

// Whole chunk, rows 16-byte (codes) and 4-byte (scales) aligned: K % 64 == 0.
__device__ __forceinline__ void load_fast(Chunk &c, const Panels &p, uint32_t k0) {
  const uint32_t vc = p.voff_c + k0 / 2, vs = p.voff_s + k0 / 16;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    c.code[f][0] = ld128(p.ac, vc, p.a_soff_c[f]);
    c.code[f][1] = ld128(p.ac, vc + 16, p.a_soff_c[f]);
    c.scale[f] = ld32(p.as, vs, p.a_soff_s[f]);
    c.code[4 + f][0] = ld128(p.bc, vc, p.b_soff_c[f]);
    c.code[4 + f][1] = ld128(p.bc, vc + 16, p.b_soff_c[f]);
    c.scale[4 + f] = ld32(p.bs, vs, p.b_soff_s[f]);
  }
}

// Any chunk, any K % 16 == 0: dword- and byte-granular loads, zero past K.
__device__ __forceinline__ void load_generic(Chunk &c, const Panels &p, uint32_t k0) {
  const uint32_t kl = k0 + 64 * p.h;  // first k of this lane's 64
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const __amdgpu_buffer_rsrc_t rc = f < 4 ? p.ac : p.bc;
    const __amdgpu_buffer_rsrc_t rs = f < 4 ? p.as : p.bs;
    const uint32_t sc = f < 4 ? p.a_soff_c[f] : p.b_soff_c[f - 4];
    const uint32_t ss = f < 4 ? p.a_soff_s[f] : p.b_soff_s[f - 4];
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t k = kl + 8 * q;
      w[q] = (k + 8 <= p.K) ? ld32(rc, p.row_c + k / 2, sc) : 0u;
    }
    c.code[f][0] = u32x4_t{w[0], w[1], w[2], w[3]};
    c.code[f][1] = u32x4_t{w[4], w[5], w[6], w[7]};
    uint32_t s = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t k = kl + 16 * q;
      if (k < p.K) s |= ld8(rs, p.row_s + k / 16, ss) << (8 * q);
    }
    c.scale[f] = s;
  }
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

__device__ __forceinline__ uint32_t word(const Chunk &c, int f, int j) {
  const u32x4_t &v = c.code[f][j >> 2];
  return v[j & 3];
}

__device__ __forceinline__ void compute_chunk(const Chunk &c, float16_t (&acc)[4][4]) {
  // four fp16 scales per fragment (E4M3 -> fp16 is exact)
  half2_t s[8][2];
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    s[f][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.scale[f], 1.0f, false);
    s[f][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.scale[f], 1.0f, true);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = j >> 1;  // 16-block of this step
    half8_t b[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) b[n] = dequant8(word(c, 4 + n, j), s[4 + n][q >> 1][q & 1]);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const half8_t a = dequant8(word(c, m, j), s[m][q >> 1][q & 1]);
#pragma unroll
      for (int n = 0; n < 4; ++n)
        acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b[n], acc[m][n], 0, 0, 0);
    }
    // keep the scheduler from hoisting later steps' dequantization (register
    // pressure) above this step's matrix instructions
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int OUT_BF16, int FAST>
__global__ __launch_bounds__(256, 1) void k_gemm(GemmParams p) {
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t r32 = lane & 31u, h = lane >> 5;

  // ---- tile of this workgroup
  const uint32_t tiles_m = (p.M + kTile - 1) / kTile, tiles_n = (p.N + kTile - 1) / kTile;
  const uint32_t nt = tiles_m * tiles_n;
  const uint32_t bid = blockIdx.x;
  const uint32_t per = nt / kXcds, rem = nt % kXcds, xcd = bid % kXcds, idx = bid / kXcds;
  const uint32_t lid = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + idx;
  const uint32_t group = lid / (kGroupM * tiles_n);
  const uint32_t first_m = group * kGroupM;
  const uint32_t gsz = min(tiles_m - first_m, kGroupM);
  const uint32_t in_group = lid - group * kGroupM * tiles_n;
  const uint32_t tm = first_m + in_group % gsz, tn = in_group / gsz;

  const uint32_t K = p.K, K2 = K / 2, K16 = K / 16;
  const uint32_t m0 = tm * kTile, n0 = tn * kTile;
  const uint32_t rows_a = min(kTile, p.M - m0), rows_b = min(kTile, p.N - n0);
  const uint32_t wm = wave >> 1, wn = wave & 1u;

  Panels P;
  P.ac = __builtin_amdgcn_make_buffer_rsrc((void *)(p.a_codes + (size_t)m0 * K2), (short)0,
                                           (int)(rows_a * K2), kRsrcWord3);
  P.as = __builtin_amdgcn_make_buffer_rsrc((void *)(p.a_scales + (size_t)m0 * K16), (short)0,
                                           (int)(rows_a * K16), kRsrcWord3);
  P.bc = __builtin_amdgcn_make_buffer_rsrc((void *)(p.b_codes + (size_t)n0 * K2), (short)0,
                                           (int)(rows_b * K2), kRsrcWord3);
  P.bs = __builtin_amdgcn_make_buffer_rsrc((void *)(p.b_scales + (size_t)n0 * K16), (short)0,
                                           (int)(rows_b * K16), kRsrcWord3);
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const uint32_t ra = wm * kWaveTile + 32 * f, rb = wn * kWaveTile + 32 * f;
    P.a_soff_c[f] = ra * K2;
    P.a_soff_s[f] = ra * K16;
    P.b_soff_c[f] = rb * K2;
    P.b_soff_s[f] = rb * K16;
  }
  P.row_c = r32 * K2;
  P.row_s = r32 * K16;
  P.voff_c = P.row_c + 32 * h;
  P.voff_s = P.row_s + 4 * h;
  P.K = K;
  P.h = h;

  float16_t acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[m][n][e] = 0.0f;

  const uint32_t nchunks = (K + kChunk - 1) / kChunk;
  const uint32_t nfull = K / kChunk;
  auto load = [&](Chunk &c, uint32_t ci) {
    if (FAST && ci < nfull)
      load_fast(c, P, ci * kChunk);
    else
      load_generic(c, P, ci * kChunk);
  };
  Chunk c0, c1;
  load(c0, 0);
  uint32_t ci = 0;
  for (; ci + 1 < nchunks; ci += 2) {
    load(c1, ci + 1);
    compute_chunk(c0, acc);
    if (ci + 2 < nchunks) load(c0, ci + 2);
    compute_chunk(c1, acc);
  }
  if (ci < nchunks) compute_chunk(c0, acc);

  // ---- epilogue: D layout of a 32x32 tile -- lane holds column (lane % 32)
  // and rows 8*(e/4) + 4*h + (e%4), e = 0..15.
  const float alpha = (*p.a_ts) * (*p.b_ts);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const uint32_t col = n0 + wn * kWaveTile + 32 * n + r32;
      if (col >= p.N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t row = m0 + wm * kWaveTile + 32 * m + 8 * (e >> 2) + 4 * h + (e & 3);
        if (row >= p.M) continue;
        const float v = acc[m][n][e] * alpha;
        if (OUT_BF16) {
          const uint32_t u = __float_as_uint(v);
          static_cast<uint16_t *>(p.c)[(size_t)row * p.ldc + col] =
              (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
        } else {
          static_cast<float *>(p.c)[(size_t)row * p.ldc + col] = v;
        }
      }
    }
  }
}

hipError_t launch_gemm(const GemmParams &p, int out_bf16, hipStream_t s) {
  const uint32_t tiles = ((p.M + kTile - 1) / kTile) * ((p.N + kTile - 1) / kTile);
  const bool fast = (p.K % 64) == 0;
  if (out_bf16) {
    if (fast) hipLaunchKernelGGL((k_gemm<1, 1>), dim3(tiles), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((k_gemm<1, 0>), dim3(tiles), dim3(256), 0, s, p);
  } else {
    if (fast) hipLaunchKernelGGL((k_gemm<0, 1>), dim3(tiles), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((k_gemm<0, 0>), dim3(tiles), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace nv4
