// gemm.hip -- block-scaled FP4 GEMM for gfx950:
//   C[M x N] = (ts_a * ts_b) * sum_k A[m][k] * B[n][k],
// A[m][k] = E2M1(code) * E4M3(scale of its 16-block), both operands packed
// K-major as written by the quantizers (Quartet II's NVFP4 linear-layer
// GEMMs; abstract and news summary, "Kerninnovationen").
//
// gfx950's native FP4 matrix instructions take one power-of-two (E8M0) scale
// per 32 elements; NVFP4 has an E4M3 scale per 16.  The product of an E2M1
// value and an E4M3 scale has at most 6 significant bits and lies in
// [2^-10, 2688], so it is exact in fp16: each operand tile is dequantized
// exactly into fp16 registers and multiplied on the fp16 MFMA
// (v_mfma_f32_16x16x32_f16) with fp32 accumulation.
//
// Tiling: a workgroup of 4 waves computes a 256 x 256 tile; each wave a
// 128 x 128 sub-tile as 8 x 8 MFMA tiles of 16 x 16.  No LDS: every lane
// loads its fragments straight from global memory (FP4 is 4x smaller than
// the fp16 it expands to, so the redundant loads of the two waves sharing a
// row panel cost little and are served by L1/L2).
//
// K order inside a 128-wide chunk: MFMA lane group g = lane / 16 holds k
// slots 8g..8g+7 of each 32-wide step.  A lane loads 16 contiguous bytes =
// 32 codes at k = k0 + 32g .. k0 + 32g + 31 and feeds dword j of them to
// step j.  The same assignment is used for A and B, so the permutation of k
// cancels in the sum.
#include "kernels.hpp"

namespace nv4 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kTileM = 256, kTileN = 256, kChunk = 128;

struct Frag {
  uint4 codes;     // 32 codes of one row (k0 + 32g ..)
  uint32_t scales; // two E4M3 bytes (blocks k0/16 + 2g, + 1)
};

// Load one row's 32-code slice and its two scale bytes, zero beyond K or
// beyond the last row.
__device__ __forceinline__ Frag load_frag(const uint8_t *codes, const uint8_t *scales,
                                          uint32_t row, uint32_t nrows, uint32_t K, uint32_t k) {
  Frag f;
  f.codes = make_uint4(0, 0, 0, 0);
  f.scales = 0;
  if (row < nrows && k < K) {
    const uint8_t *c = codes + (size_t)row * (K / 2) + k / 2;
    const uint8_t *s = scales + (size_t)row * (K / 16) + k / 16;
    if (k + 32 <= K) {
      if ((K & 31u) == 0) {
        f.codes = *reinterpret_cast<const uint4 *>(c);
      } else {  // rows are only 8-byte aligned
        const uint2 h0 = *reinterpret_cast<const uint2 *>(c);
        const uint2 h1 = *reinterpret_cast<const uint2 *>(c + 8);
        f.codes = make_uint4(h0.x, h0.y, h1.x, h1.y);
      }
      f.scales = (uint32_t)s[0] | ((uint32_t)s[1] << 8);
    } else {  // K % 32 == 16: only the first 16 codes exist
      const uint2 h = *reinterpret_cast<const uint2 *>(c);
      f.codes = make_uint4(h.x, h.y, 0, 0);
      f.scales = (uint32_t)s[0];
    }
  }
  return f;
}

// 8 codes (element 2j in the low nibble of byte j) times one E4M3 scale,
// exactly, as 8 fp16 values.
__device__ __forceinline__ half8_t dequant8(uint32_t w, uint32_t scale_byte) {
  const float s = e4m3_value(scale_byte);
  half8_t r;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t nib = (w >> (4 * i)) & 15u;
    const float v = e2m1_value(nib & 7u) * s;
    r[i] = (_Float16)((nib & 8u) ? -v : v);
  }
  return r;
}

template <int OUT_BF16>
__global__ __launch_bounds__(256, 1) void k_gemm(GemmParams p) {
  const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63u;
  const uint32_t r16 = lane & 15u, g = lane >> 4;
  const uint32_t tiles_n = (p.N + kTileN - 1) / kTileN;
  const uint32_t tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const uint32_t a_row0 = tm * kTileM + (wave >> 1) * 128;
  const uint32_t b_row0 = tn * kTileN + (wave & 1u) * 128;

  float4_t acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  Frag fa[8], fb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    fa[i] = load_frag(p.a_codes, p.a_scales, a_row0 + 16 * i + r16, p.M, p.K, 32 * g);
    fb[i] = load_frag(p.b_codes, p.b_scales, b_row0 + 16 * i + r16, p.N, p.K, 32 * g);
  }
  for (uint32_t k0 = 0; k0 < p.K; k0 += kChunk) {
    Frag na[8], nb[8];
    const uint32_t kn = k0 + kChunk + 32 * g;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      na[i] = load_frag(p.a_codes, p.a_scales, a_row0 + 16 * i + r16, p.M, p.K, kn);
      nb[i] = load_frag(p.b_codes, p.b_scales, b_row0 + 16 * i + r16, p.N, p.K, kn);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half8_t ha[8], hb[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t wa = j == 0 ? fa[i].codes.x : j == 1 ? fa[i].codes.y : j == 2 ? fa[i].codes.z : fa[i].codes.w;
        const uint32_t wb = j == 0 ? fb[i].codes.x : j == 1 ? fb[i].codes.y : j == 2 ? fb[i].codes.z : fb[i].codes.w;
        ha[i] = dequant8(wa, (fa[i].scales >> (j < 2 ? 0 : 8)) & 0xFFu);
        hb[i] = dequant8(wb, (fb[i].scales >> (j < 2 ? 0 : 8)) & 0xFFu);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ha[i], hb[jj], acc[i][jj], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      fa[i] = na[i];
      fb[i] = nb[i];
    }
  }

  const float alpha = (*p.a_ts) * (*p.b_ts);
  // D layout of a 16x16 MFMA tile: lane holds rows 4g..4g+3 of column r16.
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const uint32_t n = b_row0 + 16 * jj + r16;
      if (n >= p.N) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t m = a_row0 + 16 * i + 4 * g + v;
        if (m >= p.M) continue;
        const float val = acc[i][jj][v] * alpha;
        if (OUT_BF16) {
          const uint32_t u = __float_as_uint(val);
          const uint16_t b = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
          static_cast<uint16_t *>(p.c)[(size_t)m * p.ldc + n] = b;
        } else {
          static_cast<float *>(p.c)[(size_t)m * p.ldc + n] = val;
        }
      }
    }
  }
}

hipError_t launch_gemm(const GemmParams &p, int out_bf16, hipStream_t s) {
  const uint32_t tiles = ((p.M + kTileM - 1) / kTileM) * ((p.N + kTileN - 1) / kTileN);
  if (out_bf16)
    hipLaunchKernelGGL(k_gemm<1>, dim3(tiles), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(k_gemm<0>, dim3(tiles), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace nv4
