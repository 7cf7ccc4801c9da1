// divcheck.hip -- device check of the refined reciprocal and quotient used by
// the quantizers (rcp_rn / div_rn in common.hpp) against the IEEE division
// the compiler emits for '/' (correctly rounded).  Built by build() into
// tests/_build/libdivcheck.so and called from tests/test_gpu_division.py and
// tests/division_exhaustive.py.  Every entry point is synchronous and
// returns 0, or a HIP error code; mismatch counts go to host memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace {

struct Result {
  unsigned long long mismatches;
  uint32_t first_a, first_b;  // bit patterns of one mismatching case (b only for reciprocals)
};

// Reciprocal: every b = 2^(e - 127) * (1 + m / 2^23), e in [e_lo, e_lo + n_exp).
__global__ void k_rcp(uint32_t e_lo, uint32_t n_exp, Result *res) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= ((uint64_t)n_exp << 23)) return;
  const uint32_t bits = ((e_lo + (uint32_t)(i >> 23)) << 23) | (uint32_t)(i & 0x7FFFFFu);
  const float b = __uint_as_float(bits);
  const float got = nv4::rcp_rn(b), want = 1.0f / b;
  if (__float_as_uint(got) != __float_as_uint(want)) {
    if (atomicAdd(&res->mismatches, 1ull) == 0) res->first_b = bits;
  }
}

// Quotient of significands: b = 1 + mb / 2^23 for every mb (one thread
// each), a = 1 + ma / 2^23 for ma = a_lo, a_lo + a_step, ... (a_count of them).
__global__ void k_div(uint32_t a_lo, uint32_t a_step, uint32_t a_count, Result *res) {
  const uint32_t mb = blockIdx.x * blockDim.x + threadIdx.x;
  if (mb >= (1u << 23)) return;
  const float b = __uint_as_float(0x3F800000u | mb);
  unsigned long long bad = 0;
  uint32_t fa = 0;
  uint32_t ma = a_lo;
  for (uint32_t k = 0; k < a_count; ++k, ma += a_step) {
    const float a = __uint_as_float(0x3F800000u | (ma & 0x7FFFFFu));
    const float got = nv4::div_rn(a, b), want = a / b;
    if (__float_as_uint(got) != __float_as_uint(want)) {
      if (bad == 0) fa = __float_as_uint(a);
      ++bad;
    }
  }
  if (bad) {
    if (atomicAdd(&res->mismatches, bad) == 0) {
      res->first_a = fa;
      res->first_b = __float_as_uint(b);
    }
  }
}

// Quotients of given pairs (for a cross-check against the host's division).
__global__ void k_div_pairs(const float *a, const float *b, float *q, float *r, uint32_t n) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    q[i] = nv4::div_rn(a[i], b[i]);
    r[i] = nv4::rcp_rn(b[i]);
  }
}

int run(Result *host, void (*launch)(Result *)) {
  Result *d = nullptr;
  hipError_t e = hipMalloc(&d, sizeof(Result));
  if (e != hipSuccess) return (int)e;
  e = hipMemset(d, 0, sizeof(Result));
  if (e == hipSuccess) {
    launch(d);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(host, d, sizeof(Result), hipMemcpyDeviceToHost);
  hipFree(d);
  return (int)e;
}

}  // namespace

extern "C" {

// Reciprocal of every b with biased exponent in [e_lo, e_lo + n_exp).
int divcheck_rcp(uint32_t e_lo, uint32_t n_exp, unsigned long long *mismatches, uint32_t *first_b) {
  if (n_exp == 0 || e_lo < 1 || e_lo + n_exp > 255) return -1;
  Result r{};
  static uint32_t s_lo, s_n;
  s_lo = e_lo;
  s_n = n_exp;
  const int st = run(&r, [](Result *d) {
    const uint64_t n = (uint64_t)s_n << 23;
    hipLaunchKernelGGL(k_rcp, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, 0, s_lo, s_n, d);
  });
  *mismatches = r.mismatches;
  *first_b = r.first_b;
  return st;
}

// Quotients a/b of significands: every b, and a_count values of a from
// a_lo in steps of a_step (ma taken modulo 2^23).
int divcheck_div(uint32_t a_lo, uint32_t a_step, uint32_t a_count, unsigned long long *mismatches,
                 uint32_t *first_a, uint32_t *first_b) {
  Result r{};
  static uint32_t s_lo, s_step, s_count;
  s_lo = a_lo;
  s_step = a_step;
  s_count = a_count;
  const int st = run(&r, [](Result *d) {
    hipLaunchKernelGGL(k_div, dim3((1u << 23) / 256), dim3(256), 0, 0, s_lo, s_step, s_count, d);
  });
  *mismatches = r.mismatches;
  *first_a = r.first_a;
  *first_b = r.first_b;
  return st;
}

// q[i] = div_rn(a[i], b[i]), r[i] = rcp_rn(b[i]) for host arrays of n pairs.
int divcheck_pairs(const float *a, const float *b, float *q, float *r, uint32_t n) {
  float *d = nullptr;
  const size_t bytes = (size_t)n * sizeof(float);
  hipError_t e = hipMalloc(&d, 4 * bytes + 4);
  if (e != hipSuccess) return (int)e;
  e = hipMemcpy(d, a, bytes, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(d + n, b, bytes, hipMemcpyHostToDevice);
  if (e == hipSuccess && n) {
    hipLaunchKernelGGL(k_div_pairs, dim3((n + 255) / 256), dim3(256), 0, 0, d, d + n, d + 2 * (size_t)n,
                       d + 3 * (size_t)n, n);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(q, d + 2 * (size_t)n, bytes, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(r, d + 3 * (size_t)n, bytes, hipMemcpyDeviceToHost);
  hipFree(d);
  return (int)e;
}

}  // extern "C"
