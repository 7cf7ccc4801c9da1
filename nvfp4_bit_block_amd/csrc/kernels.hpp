// kernels.hpp -- launch interface between the C ABI (api.cpp) and the gfx950
// kernels.  Internal to libnvfp4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace nv4 {

enum Mode : int {
  kAmax = 0,       // rotated-or-raw absmax only -> per-workgroup partial maxima
  kRtn = 1,        // NVFP4 round-to-nearest
  kSr = 2,         // NVFP4 stochastic rounding
  kIf4 = 3,        // IF4 selection (RTN in both branches)
  kEden = 4,       // MS-EDEN pass 1: codes + target scales + partial maxima
  kEdenFused = 5,  // MS-EDEN with a given tensor scale: codes + scales in one pass
  kRot = 6,        // rotation only: rotated fp32 values
  kFos = 7,        // NVFP4 RTN, Four Over Six block scale (maximum -> 6 or 4)
  kSearch = 8,     // NVFP4 RTN, block scale searched over 19 E4M3 bytes
  kIf4Sr = 9,      // IF4 with stochastic rounding (branch by expected error)
  kIf4Eden = 10,   // IF4 MS-EDEN pass 1: codes + flagged target scales + partials
  kIf4EdenFused = 11  // IF4 MS-EDEN with a given tensor scale
};

// Passes that code with a known tensor scale, and passes that end with
// per-workgroup partial maxima for the next pass.
constexpr bool takes_tensor_scale(int m) {
  return m == kRtn || m == kSr || m == kIf4 || m == kFos || m == kSearch || m == kEdenFused || m == kIf4Sr ||
         m == kIf4EdenFused;
}
constexpr bool writes_partials(int m) { return m == kAmax || m == kEden || m == kIf4Eden; }

constexpr int kThreads = 256;      // threads per workgroup of the quantizers
constexpr int kMxThreads = 256;    // ... of the matrix-core rotation kernels
constexpr int kMaxPartials = 2048; // workgroups of a pass that writes partials
// Axis-1 kernels: each lane loads kColWords 32-bit words of each of its 16
// rows (bf16: 2 columns per word, fp32: 1), so a wave tile is 128 rows x
// 8 * kColWords words of columns.
constexpr int kColWords = 4;
constexpr size_t kPartialBytes = 16384;  // partial maxima: two arrays of kMaxPartials floats

struct QuantParams {
  const void *x;
  int64_t ld;         // input leading dimension (elements)
  int vec;            // rows are 16-byte aligned: vector loads allowed
  uint32_t rows, cols;  // input shape
  uint32_t R, K;        // output rows, output row length
  uint32_t K16;         // K / 16
  uint32_t nblocks;     // R * K16
  FastDiv k16div;       // division by K16 (axis 0)
  FastDiv ctiles_div;   // division by the number of column tiles (axis 1)
  uint32_t ntiles;      // axis 1 tile count
  FastDiv mx_cdiv;      // axis 1, matrix-core rotation: division by the 64-column tiles
  FastDiv mx_rdiv;      // ... by the 256-row tiles
  uint8_t *codes;
  uint8_t *scales;
  float *ts_out;
  float *partial;       // kMaxPartials floats of workspace
  uint32_t npartial;    // partial maxima written by the previous pass
  float *tb;            // MS-EDEN target scales, nblocks floats of workspace (IF4: sign bit = INT flag)
  const float *ts_in;   // given tensor scale or nullptr
  const float *amax_in; // given max|x| (tensor scale amax_in / top) or nullptr
  float *amax_out;      // MS-EDEN: max|x| of the raw input written here, or nullptr
  float *rpartial;      // kMaxPartials floats of workspace: partial max|x| for amax_out
  float *rot_out;       // kRot output
  uint32_t sg[4];       // rotation sign words
  int rht;
  int group16;          // MS-EDEN correction group of 16 instead of 128
  float top;            // largest magnitude times 448 (tensor scale divisor)
  RngKey key;
};

// in_bf16: 1 = bf16 input, 0 = fp32 input.
hipError_t launch_quant(const QuantParams &p, int in_bf16, int axis, Mode mode, uint32_t grid,
                        hipStream_t s);
// if4: the targets' sign bits are IF4's INT flags.
hipError_t launch_eden_scales(const QuantParams &p, bool if4, uint32_t grid, hipStream_t s);
// Empty tensor: *ts = *ts_in (or 1), *amax_out = 0 if given.
hipError_t launch_trivial_scale(float *ts, const float *ts_in, float *amax_out, hipStream_t s);
// MS-EDEN along both axes from one read (fused = given tensor scales).
hipError_t launch_quant_dual(const QuantParams &pr, const QuantParams &pc, int in_bf16, int fused,
                             uint32_t grid, hipStream_t s);
uint32_t dual_grid(const QuantParams &pr, int in_bf16);
uint32_t quant_grid(const QuantParams &p, int in_bf16, int axis);
uint32_t eden_scales_grid(const QuantParams &p);

struct DequantParams {
  const uint8_t *codes;
  const uint8_t *scales;
  const float *ts;
  void *out;
  uint32_t R, K, K16, nblocks;
  uint32_t sg[4];
  int inv_rht;
  int if4;
};
hipError_t launch_dequant(const DequantParams &p, int out_bf16, hipStream_t s);

enum GemmOut : int {
  kOutF32 = 0,    // C in fp32 at c (leading dimension ldc)
  kOutBf16 = 1,   // C in bf16, nearest even
  kOutNvfp4 = 2   // C coded as NVFP4 RTN along N (q_* fields)
};

struct GemmParams {
  const uint8_t *a_codes, *a_scales;
  const uint8_t *b_codes, *b_scales;
  const float *a_ts, *b_ts;
  void *c;
  int64_t ldc;
  // kOutNvfp4: codes [M][N/2] and scales [M][N/16] of C with the tensor
  // scale *q_ts; q_amax, if not null, receives max |C| (the launch clears it
  // first).
  uint8_t *q_codes, *q_scales;
  const float *q_ts;
  float *q_amax;
  uint32_t M, N, K;
};
// out: a GemmOut; if4: operands may hold IF4 blocks (scale bit 7 = INT
// flag), 0: NVFP4 only (kOutNvfp4 is built for NVFP4 operands only).
hipError_t launch_gemm(const GemmParams &p, int out, int if4, hipStream_t s);

}  // namespace nv4
