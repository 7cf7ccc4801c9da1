// convcheck.hip -- device side of the exhaustive checks of the conversions the
// library's kernels use (test infrastructure; built by build() into
// tests/_build/libconvcheck.so and called from tests/test_gpu_converters.py).
// Each kernel runs the library's own device functions from common.hpp, so
// what is checked is exactly the code path the quantizers and the GEMM run:
//   - e2m1x16_rne: gfx950's packed fp32 -> E2M1 conversion (round to nearest
//     even, saturating, sign kept), over any run of fp32 bit patterns;
//   - e4m3_rne_sat / e4m3_ceil_sat: the block-scale roundings, over any run;
//   - e4m3_sr_sat: MS-EDEN's stochastic scale rounding, over given pairs
//     (value, 16-bit uniform);
//   - div_by<6> / div_by<7>: the block maximum divided by 6 and 7, against
//     the device's IEEE division, over every finite a >= 0;
//   - e2m1x16_value, e4m3x2_f16, e4m3_value, dequant8 and dequant8_lut: the
//     decoders, over every code byte and every scale byte.
// Every entry point is synchronous and returns 0 or a HIP error code;
// results go to host memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace {

// Thread i codes the 16 patterns bits_lo + 16 i .. + 15 (8 bytes).
__global__ void k_e2m1_rne(uint32_t bits_lo, uint32_t nthreads, uint2 *out) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nthreads) return;
  float y[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) y[j] = __uint_as_float(bits_lo + 16u * i + (uint32_t)j);
  uint32_t lo, hi;
  nv4::e2m1x16_rne(y, lo, hi);
  out[i] = make_uint2(lo, hi);
}

__global__ void k_e4m3(uint32_t bits_lo, uint32_t count, int ceil_mode, uint8_t *out) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  const float v = __uint_as_float(bits_lo + i);
  out[i] = (uint8_t)(ceil_mode ? nv4::e4m3_ceil_sat(v) : nv4::e4m3_rne_sat(v));
}

__global__ void k_e4m3_sr(const float *a, const uint16_t *u, uint32_t count, uint8_t *out) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  out[i] = (uint8_t)nv4::e4m3_sr_sat(a[i], u[i]);
}

struct Mismatch {
  unsigned long long count;
  uint32_t first_a;
};

// Thread i divides the 16 patterns 16 i .. 16 i + 15 (all below the first
// non-finite pattern when i < nthreads).
template <int D>
__global__ void k_div_by(uint32_t nthreads, Mismatch *res) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nthreads) return;
  unsigned long long bad = 0;
  uint32_t first = 0;
  for (uint32_t j = 0; j < 16; ++j) {
    const uint32_t bits = 16u * i + j;
    const float a = __uint_as_float(bits);
    const float got = nv4::div_by<D>(a), want = a / (float)D;
    if (__float_as_uint(got) != __float_as_uint(want)) {
      if (bad == 0) first = bits;
      ++bad;
    }
  }
  if (bad && atomicAdd(&res->count, bad) == 0) res->first_a = first;
}

// Decoders, thread b = code byte 0..255 (the word holds it four times):
// f32[b][16] from e2m1x16_value; f16 outputs from dequant8 and dequant8_lut
// at unit scale, [b][8] each.
__global__ void k_decode(float *f32, _Float16 *f16, _Float16 *lut_fp, _Float16 *lut_int) {
  const uint32_t b = threadIdx.x;
  const uint32_t w = b * 0x01010101u;
  float v[16];
  nv4::e2m1x16_value(w, w, v);
#pragma unroll
  for (int j = 0; j < 16; ++j) f32[16 * b + j] = v[j];
  const nv4::half8_t d = nv4::dequant8(w, (_Float16)1.0f);
  const nv4::half8_t lf = nv4::dequant8_lut(w, (_Float16)1.0f, nv4::kLutFpLo, nv4::kLutFpHi);
  const nv4::half8_t li = nv4::dequant8_lut(w, (_Float16)1.0f, nv4::kLutIntLo, nv4::kLutIntHi);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    f16[8 * b + j] = d[j];
    lut_fp[8 * b + j] = lf[j];
    lut_int[8 * b + j] = li[j];
  }
}

// Scale bytes, thread e = 0..255: both halves of e4m3x2_f16(e | e << 8), and
// e4m3_value(e & 0x7F) (the quantizers' software decoder).
__global__ void k_scales(_Float16 *f16, float *f32) {
  const uint32_t e = threadIdx.x;
  const nv4::half2_t h = nv4::e4m3x2_f16(e | (e << 8));
  f16[2 * e] = h[0];
  f16[2 * e + 1] = h[1];
  f32[e] = nv4::e4m3_value(e & 0x7Fu);
}

// GEMM operands as the GEMM forms them: scale byte e (blockIdx.x) through
// e4m3x2_f16, then code byte b (threadIdx.x) through dequant8 and both
// tables of dequant8_lut: out[e][b][3][8].
__global__ void k_operands(_Float16 *out) {
  const uint32_t e = blockIdx.x, b = threadIdx.x;
  const uint32_t w = b * 0x01010101u;
  const _Float16 s = nv4::e4m3x2_f16(e | (e << 8))[0];
  const nv4::half8_t d = nv4::dequant8(w, s);
  const nv4::half8_t lf = nv4::dequant8_lut(w, s, nv4::kLutFpLo, nv4::kLutFpHi);
  const nv4::half8_t li = nv4::dequant8_lut(w, s, nv4::kLutIntLo, nv4::kLutIntHi);
  _Float16 *o = out + ((size_t)e * 256 + b) * 24;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    o[j] = d[j];
    o[8 + j] = lf[j];
    o[16 + j] = li[j];
  }
}

template <typename T>
int to_host(T *host, const T *dev, size_t n) {
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(host, dev, n * sizeof(T), hipMemcpyDeviceToHost);
  return (int)e;
}

}  // namespace

extern "C" {

// Packed E2M1 codes (two per byte, even pattern low) of the fp32 bit
// patterns bits_lo .. bits_lo + count - 1; count a multiple of 16, and the
// run must not wrap past 0xFFFFFFFF.
int convcheck_e2m1_rne(uint32_t bits_lo, uint32_t count, uint8_t *host_codes) {
  if (count % 16 || (uint64_t)bits_lo + count > 0x100000000ull) return -1;
  uint2 *d = nullptr;
  const uint32_t nt = count / 16;
  hipError_t e = hipMalloc(&d, (size_t)nt * sizeof(uint2));
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(k_e2m1_rne, dim3((nt + 255) / 256), dim3(256), 0, 0, bits_lo, nt, d);
  const int st = to_host(reinterpret_cast<uint2 *>(host_codes), d, nt);
  hipFree(d);
  return st;
}

// E4M3 bytes (RNE, or rounded up) of bits_lo .. bits_lo + count - 1.
int convcheck_e4m3(uint32_t bits_lo, uint32_t count, int ceil_mode, uint8_t *host_bytes) {
  if ((uint64_t)bits_lo + count > 0x100000000ull) return -1;
  uint8_t *d = nullptr;
  hipError_t e = hipMalloc(&d, count ? count : 1);
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(k_e4m3, dim3((count + 255) / 256), dim3(256), 0, 0, bits_lo, count, ceil_mode, d);
  const int st = to_host(host_bytes, d, count);
  hipFree(d);
  return st;
}

// E4M3 bytes of the stochastic rounding of host pairs (a[i], u[i]).
int convcheck_e4m3_sr(const float *a, const uint16_t *u, uint32_t count, uint8_t *host_bytes) {
  char *d = nullptr;
  const size_t n = count ? count : 1;
  hipError_t e = hipMalloc(&d, n * 7);
  if (e != hipSuccess) return (int)e;
  float *da = reinterpret_cast<float *>(d);
  uint16_t *du = reinterpret_cast<uint16_t *>(d + n * 4);
  uint8_t *dout = reinterpret_cast<uint8_t *>(d + n * 6);
  e = hipMemcpy(da, a, (size_t)count * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(du, u, (size_t)count * 2, hipMemcpyHostToDevice);
  if (e == hipSuccess) hipLaunchKernelGGL(k_e4m3_sr, dim3((count + 255) / 256), dim3(256), 0, 0, da, du, count, dout);
  const int st = e == hipSuccess ? to_host(host_bytes, dout, count) : (int)e;
  hipFree(d);
  return st;
}

// div_by<d>(a) against a / d for every finite a >= 0 (d = 6 or 7).
int convcheck_div_by(int d, unsigned long long *mismatches, uint32_t *first_a) {
  if (d != 6 && d != 7) return -1;
  Mismatch *m = nullptr;
  hipError_t e = hipMalloc(&m, sizeof(Mismatch));
  if (e != hipSuccess) return (int)e;
  e = hipMemset(m, 0, sizeof(Mismatch));
  const uint32_t nt = 0x7F800000u / 16;  // patterns 0 .. 0x7F7FFFFF
  if (e == hipSuccess) {
    if (d == 6) hipLaunchKernelGGL(k_div_by<6>, dim3((nt + 255) / 256), dim3(256), 0, 0, nt, m);
    else hipLaunchKernelGGL(k_div_by<7>, dim3((nt + 255) / 256), dim3(256), 0, 0, nt, m);
  }
  Mismatch h{};
  const int st = e == hipSuccess ? to_host(&h, m, 1) : (int)e;
  hipFree(m);
  *mismatches = h.count;
  *first_a = h.first_a;
  return st;
}

// Decoders over every code byte and scale byte; host arrays:
// code_f32[256*16], code_f16[256*8], lut_fp[256*8], lut_int[256*8] (fp16
// as uint16 bits), scale_f16[256*2], scale_f32[256], operands[127*256*24].
int convcheck_decoders(float *code_f32, uint16_t *code_f16, uint16_t *lut_fp, uint16_t *lut_int,
                       uint16_t *scale_f16, float *scale_f32, uint16_t *operands) {
  const size_t n_ops = (size_t)127 * 256 * 24;
  char *d = nullptr;
  const size_t bytes = 256 * 16 * 4 + 3 * 256 * 8 * 2 + 256 * 2 * 2 + 256 * 4 + n_ops * 2;
  hipError_t e = hipMalloc(&d, bytes);
  if (e != hipSuccess) return (int)e;
  float *c32 = reinterpret_cast<float *>(d);
  _Float16 *c16 = reinterpret_cast<_Float16 *>(c32 + 256 * 16);
  _Float16 *lf = c16 + 256 * 8, *li = lf + 256 * 8, *s16 = li + 256 * 8;
  float *s32 = reinterpret_cast<float *>(s16 + 512);
  _Float16 *ops = reinterpret_cast<_Float16 *>(s32 + 256);
  hipLaunchKernelGGL(k_decode, dim3(1), dim3(256), 0, 0, c32, c16, lf, li);
  hipLaunchKernelGGL(k_scales, dim3(1), dim3(256), 0, 0, s16, s32);
  hipLaunchKernelGGL(k_operands, dim3(127), dim3(256), 0, 0, ops);
  int st = to_host(code_f32, c32, 256 * 16);
  if (!st) st = to_host(code_f16, reinterpret_cast<uint16_t *>(c16), 256 * 8);
  if (!st) st = to_host(lut_fp, reinterpret_cast<uint16_t *>(lf), 256 * 8);
  if (!st) st = to_host(lut_int, reinterpret_cast<uint16_t *>(li), 256 * 8);
  if (!st) st = to_host(scale_f16, reinterpret_cast<uint16_t *>(s16), 512);
  if (!st) st = to_host(scale_f32, s32, 256);
  if (!st) st = to_host(operands, reinterpret_cast<uint16_t *>(ops), n_ops);
  hipFree(d);
  return st;
}

}  // extern "C"
