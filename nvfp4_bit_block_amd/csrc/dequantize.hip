// dequantize.hip -- inverse of the NVFP4 / IF4 encodings, with the optional
// inverse 128-point rotation, for gfx950.
//
// value = sign * (v * (E4M3(scale & 0x7F) * tensor_scale)); v is the E2M1
// value of the magnitude code (grid of the palettes blog, opening paragraph)
// or, for IF4 groups whose scale has bit 7 set, the integer magnitude (IF4
// page, Figure 1).  The inverse rotation of a 128-group is
// signs * (2^-3.5 * H_128 * v), the transform being its own inverse up to
// the normalization.  One lane per 16-element block, 8 lanes per group.
#include "kernels.hpp"

namespace nv4 {

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int OUT_BF16>
__global__ __launch_bounds__(kThreads) void k_dequant(DequantParams p) {
  const float ts = *p.ts;
  const uint32_t lig = group_pos(threadIdx.x & 63u);
  const uint32_t rank = (threadIdx.x & ~63u) + lane_block_rank(threadIdx.x & 63u);
  const uint32_t sbits = p.inv_rht ? lane_sign_bits(p.sg, lig) : 0u;
  for (uint32_t base = blockIdx.x * kThreads; base < p.nblocks; base += gridDim.x * kThreads) {
    const uint32_t gb = base + rank;
    const bool active = gb < p.nblocks;
    float z[16];
    if (active) {
      const uint2 cw = *reinterpret_cast<const uint2 *>(p.codes + (size_t)gb * 8);
      const uint32_t e = p.scales[gb];
      const bool is_int = p.if4 && (e & 0x80u);
      const float S = e4m3_value(e & 0x7Fu) * ts;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t nib = ((i < 8 ? cw.x : cw.y) >> (4 * (i & 7))) & 15u;
        const float v = is_int ? (float)(nib & 7u) : e2m1_value(nib & 7u);
        const float q = v * S;
        z[i] = (nib & 8u) ? -q : q;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    }
    if (p.inv_rht) {
      fwht128_group(z, lig);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if ((sbits >> i) & 1u) z[i] = -z[i];
    }
    if (active) {
      if (OUT_BF16) {
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          w[i] = f32_to_bf16_rne(z[2 * i]) | (f32_to_bf16_rne(z[2 * i + 1]) << 16);
        uint4 *o = reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p.out) + (size_t)gb * 16);
        o[0] = make_uint4(w[0], w[1], w[2], w[3]);
        o[1] = make_uint4(w[4], w[5], w[6], w[7]);
      } else {
        float4 *o = reinterpret_cast<float4 *>(static_cast<float *>(p.out) + (size_t)gb * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[i] = make_float4(z[4 * i], z[4 * i + 1], z[4 * i + 2], z[4 * i + 3]);
      }
    }
  }
}

hipError_t launch_dequant(const DequantParams &p, int out_bf16, hipStream_t s) {
  uint64_t g = ((uint64_t)p.nblocks + kThreads - 1) / kThreads;
  if (g < 1) g = 1;
  if (g > 8192) g = 8192;
  if (out_bf16)
    hipLaunchKernelGGL(k_dequant<1>, dim3((uint32_t)g), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(k_dequant<0>, dim3((uint32_t)g), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace nv4
