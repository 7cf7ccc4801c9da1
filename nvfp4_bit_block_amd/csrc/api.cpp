// api.cpp -- the C ABI of libnvfp4 (declared in include/nvfp4.h): argument
// validation, workspace layout and the launch sequence of each entry point.
// Every check happens on the host before anything is enqueued; a failing
// call returns a negative status and leaves a thread-local message.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/nvfp4.h"
#include "kernels.hpp"

using namespace nv4;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return NVFP4_OK;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_size(int dtype) { return dtype == NVFP4_BF16 ? 2 : 4; }

// Blocks (of 16 output elements) a quantizer writes; limits of this build.
constexpr uint64_t kMaxBlocks = (1ull << 31) - 1;
constexpr uint64_t kMaxDim = (1ull << 31) - 1;
constexpr uint64_t kMaxColStride = 1ull << 24;  // bytes per input row, axis 1

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Shape {
  uint32_t R, K;
  uint64_t nblocks;
};

// Validation of the input tensor, the options and the shape.
int check_input(const void *x, int in_dtype, int64_t rows, int64_t cols, int64_t ld,
                const nvfp4_opts *o, bool if4, Shape *sh) {
  if (!o) return fail(NVFP4_INVALID_ARG, "opts is NULL");
  if (in_dtype != NVFP4_F32 && in_dtype != NVFP4_BF16)
    return fail(NVFP4_INVALID_ARG, "in_dtype %d is not NVFP4_F32 or NVFP4_BF16", in_dtype);
  if (o->rounding < NVFP4_RTN || o->rounding > NVFP4_MSEDEN)
    return fail(NVFP4_INVALID_ARG, "rounding %d is not RTN, SR or MSEDEN", o->rounding);
  if (o->axis != 0 && o->axis != 1) return fail(NVFP4_INVALID_ARG, "axis %d is not 0 or 1", o->axis);
  if (o->rht != 0 && o->rht != 1) return fail(NVFP4_INVALID_ARG, "rht %d is not 0 or 1", o->rht);
  if (o->scale_rule != NVFP4_SCALE_MAX6 && o->scale_rule != NVFP4_SCALE_4OVER6 &&
      o->scale_rule != NVFP4_SCALE_SEARCH)
    return fail(NVFP4_INVALID_ARG, "scale_rule %d is not MAX6, 4OVER6 or SEARCH", o->scale_rule);
  if (o->scale_rule != NVFP4_SCALE_MAX6 && (if4 || o->rounding != NVFP4_RTN))
    return fail(NVFP4_INVALID_ARG, "scale rules other than MAX6 take NVFP4 with rounding RTN only");
  if (o->rounding == NVFP4_MSEDEN && o->eden_group != 128 && o->eden_group != 16)
    return fail(NVFP4_INVALID_ARG, "eden_group %d is not 128 or 16", o->eden_group);
  if (o->amax_out && (o->rounding != NVFP4_MSEDEN || o->tensor_scale_in))
    return fail(NVFP4_UNSUPPORTED, "amax_out is written by MS-EDEN with a computed tensor scale only");
  if (o->amax_in && (o->rounding == NVFP4_MSEDEN || o->rht || o->tensor_scale_in))
    return fail(NVFP4_UNSUPPORTED, "amax_in is taken by calls without rotation, MS-EDEN or tensor_scale_in only");
  if ((o->amax_out && !aligned(o->amax_out, 4)) || (o->amax_in && !aligned(o->amax_in, 4)))
    return fail(NVFP4_MISALIGNED, "amax_out / amax_in must be 4-byte aligned");
  if (rows < 0 || cols < 0)
    return fail(NVFP4_INVALID_ARG, "negative shape %lld x %lld", (long long)rows, (long long)cols);
  if ((uint64_t)rows > kMaxDim || (uint64_t)cols > kMaxDim)
    return fail(NVFP4_UNSUPPORTED, "dimension above 2^31 - 1");
  if (ld < cols) return fail(NVFP4_BAD_SHAPE, "ld %lld < cols %lld", (long long)ld, (long long)cols);
  // the column-wise kernels address a 128-row tile with 32-bit offsets
  if (o->axis == 1 && (uint64_t)ld * elem_size(in_dtype) > kMaxColStride)
    return fail(NVFP4_UNSUPPORTED, "axis 1: a row stride of %llu bytes is above 16 MiB",
                (unsigned long long)((uint64_t)ld * elem_size(in_dtype)));
  const int64_t R = o->axis == 0 ? rows : cols;
  const int64_t K = o->axis == 0 ? cols : rows;
  if (K % 16)
    return fail(NVFP4_BAD_SHAPE, "quantized dimension %lld is not a multiple of 16", (long long)K);
  const bool need128 = o->rht || (o->rounding == NVFP4_MSEDEN && o->eden_group == 128);
  if (need128 && K % 128)
    return fail(NVFP4_BAD_SHAPE, "quantized dimension %lld is not a multiple of 128 (rotation or "
                "MS-EDEN group 128)", (long long)K);
  const uint64_t nblocks = (uint64_t)R * (uint64_t)(K / 16);
  if (nblocks > kMaxBlocks) return fail(NVFP4_UNSUPPORTED, "more than 2^31 - 1 blocks");
  if (nblocks > 0) {
    if (!x) return fail(NVFP4_INVALID_ARG, "x is NULL");
    const bool rows16 = aligned(x, 16) && ((uint64_t)ld * elem_size(in_dtype)) % 16 == 0;
    if (o->axis == 0 && !rows16)
      return fail(NVFP4_MISALIGNED, "axis 0: x must be 16-byte aligned with ld * elem_size a "
                  "multiple of 16");
    if (!aligned(x, elem_size(in_dtype)))
      return fail(NVFP4_MISALIGNED, "x is not aligned to its element size");
  }
  sh->R = (uint32_t)R;
  sh->K = (uint32_t)K;
  sh->nblocks = nblocks;
  return NVFP4_OK;
}

// Validation of the quantizer outputs and workspace.
int check_outputs(int64_t rows, int64_t cols, const nvfp4_opts *o, const Shape &sh,
                  const uint8_t *codes, const uint8_t *scales, const float *tensor_scale,
                  const void *ws, size_t ws_bytes) {
  if (!tensor_scale) return fail(NVFP4_INVALID_ARG, "tensor_scale is NULL");
  if (!aligned(tensor_scale, 4)) return fail(NVFP4_MISALIGNED, "tensor_scale must be 4-byte aligned");
  if (sh.nblocks == 0) return NVFP4_OK;
  if (!codes || !scales || !ws) return fail(NVFP4_INVALID_ARG, "null device pointer");
  if (!aligned(codes, 16) || !aligned(scales, 16))
    return fail(NVFP4_MISALIGNED, "codes and scales must be 16-byte aligned");
  if (!aligned(ws, 256)) return fail(NVFP4_MISALIGNED, "workspace must be 256-byte aligned");
  const size_t need = nvfp4_workspace_size(rows, cols, o);
  if (ws_bytes < need)
    return fail(NVFP4_WS_TOO_SMALL, "workspace of %zu bytes is below the %zu required", ws_bytes, need);
  return NVFP4_OK;
}

void fill_common(QuantParams &p, const void *x, int in_dtype, int64_t rows, int64_t cols,
                 int64_t ld, const nvfp4_opts *o, const Shape &sh, uint8_t *codes,
                 uint8_t *scales, float *tensor_scale, void *ws) {
  std::memset(&p, 0, sizeof(p));
  p.x = x;
  p.ld = ld;
  p.vec = aligned(x, 16) && ((uint64_t)ld * elem_size(in_dtype)) % 16 == 0;
  p.rows = (uint32_t)rows;
  p.cols = (uint32_t)cols;
  p.R = sh.R;
  p.K = sh.K;
  p.K16 = sh.K / 16;
  p.nblocks = (uint32_t)sh.nblocks;
  p.k16div = make_fastdiv(p.K16 ? p.K16 : 1);
  // axis 1 tiles: 128 rows x 8 * kColWords words of columns (one tile per wave)
  const uint32_t tc = 8u * (in_dtype == NVFP4_BF16 ? 2u * kColWords : (uint32_t)kColWords);
  const uint32_t nct = (uint32_t)((cols + tc - 1) / tc);
  const uint32_t ntt = (uint32_t)((rows + 127) / 128);
  p.ctiles_div = make_fastdiv(nct ? nct : 1);
  p.ntiles = nct * ntt;
  const uint32_t mx_nct = (uint32_t)((cols + 63) / 64), mx_npair = (uint32_t)((rows + 255) / 256);
  p.mx_cdiv = make_fastdiv(mx_nct ? mx_nct : 1);
  p.mx_rdiv = make_fastdiv(mx_npair ? mx_npair : 1);
  p.codes = codes;
  p.scales = scales;
  p.ts_out = tensor_scale;
  if (ws) {
    p.partial = static_cast<float *>(ws);
    p.rpartial = p.partial + kMaxPartials;
    p.tb = reinterpret_cast<float *>(static_cast<char *>(ws) + kPartialBytes);
  }
  p.ts_in = o->tensor_scale_in;
  p.amax_in = o->amax_in;
  p.amax_out = o->amax_out;
  for (int i = 0; i < 4; ++i) p.sg[i] = o->rht_signs[i];
  p.rht = o->rht;
  p.group16 = o->eden_group == 16;
  p.top = o->scale_rule == NVFP4_SCALE_4OVER6 ? 6.0f * 256.0f : 6.0f * 448.0f;
  p.key.seed_lo = (uint32_t)o->seed;
  p.key.seed_hi = (uint32_t)(o->seed >> 32);
  p.key.stream = o->stream;
}

// Zero-size tensor: only the tensor scale is defined (the given one, or 1),
// and the maximum (0) if it is asked for.
int write_trivial_scale(const nvfp4_opts *o, float *tensor_scale, hipStream_t s) {
  const hipError_t e = launch_trivial_scale(tensor_scale, o->tensor_scale_in, o->amax_out, s);
  if (e != hipSuccess) return fail(NVFP4_HIP_ERROR, "%s", hipGetErrorString(e));
  return ok();
}

int quantize_impl(const void *x, int in_dtype, int64_t rows, int64_t cols, int64_t ld,
                  const nvfp4_opts *o, uint8_t *codes, uint8_t *scales, float *tensor_scale,
                  void *ws, size_t ws_bytes, void *stream, bool if4) {
  Shape sh;
  int st = check_input(x, in_dtype, rows, cols, ld, o, if4, &sh);
  if (!st) st = check_outputs(rows, cols, o, sh, codes, scales, tensor_scale, ws, ws_bytes);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (sh.nblocks == 0) return write_trivial_scale(o, tensor_scale, s);
  QuantParams p;
  fill_common(p, x, in_dtype, rows, cols, ld, o, sh, codes, scales, tensor_scale, ws);
  const int bf = in_dtype == NVFP4_BF16;
  const uint32_t grid = quant_grid(p, bf, o->axis);
  hipError_t e = hipSuccess;
  if (o->rounding == NVFP4_MSEDEN) {
    if (o->tensor_scale_in) {
      e = launch_quant(p, bf, o->axis, if4 ? kIf4EdenFused : kEdenFused, grid, s);
    } else {
      e = launch_quant(p, bf, o->axis, if4 ? kIf4Eden : kEden, grid, s);
      if (e == hipSuccess) {
        p.npartial = grid;
        e = launch_eden_scales(p, if4, eden_scales_grid(p), s);
      }
    }
  } else {
    const Mode m = if4 ? (o->rounding == NVFP4_SR ? kIf4Sr : kIf4)
                   : o->rounding == NVFP4_SR ? kSr
                   : o->scale_rule == NVFP4_SCALE_4OVER6 ? kFos
                   : o->scale_rule == NVFP4_SCALE_SEARCH ? kSearch
                                                         : kRtn;
    if (!o->tensor_scale_in && !o->amax_in) {
      e = launch_quant(p, bf, o->axis, kAmax, grid, s);
      p.npartial = grid;
    }
    if (e == hipSuccess) e = launch_quant(p, bf, o->axis, m, grid, s);
  }
  if (e != hipSuccess) return fail(NVFP4_HIP_ERROR, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int quantize_dual_impl(const void *x, int in_dtype, int64_t rows, int64_t cols, int64_t ld,
                       const nvfp4_opts *o, uint8_t *codes_r, uint8_t *scales_r, float *ts_r,
                       uint8_t *codes_c, uint8_t *scales_c, float *ts_c, void *ws, size_t ws_bytes,
                       void *stream) {
  if (!o) return fail(NVFP4_INVALID_ARG, "opts is NULL");
  if (o->rounding != NVFP4_MSEDEN)
    return fail(NVFP4_INVALID_ARG, "the two-axis quantization takes rounding MSEDEN only");
  if (o->amax_out || o->amax_in)
    return fail(NVFP4_UNSUPPORTED, "the two-axis quantization takes no amax_out / amax_in");
  nvfp4_opts orow = *o, ocol = *o;
  orow.axis = 0;
  ocol.axis = 1;
  Shape shr, shc;
  int st = check_input(x, in_dtype, rows, cols, ld, &orow, false, &shr);
  if (!st) st = check_input(x, in_dtype, rows, cols, ld, &ocol, false, &shc);
  if (st) return st;
  if (rows % 128)  // the kernel works on tiles of 128 whole rows
    return fail(NVFP4_BAD_SHAPE, "the two-axis quantization needs rows %% 128 == 0 (rows = %lld)",
                (long long)rows);
  const size_t wr = nvfp4_workspace_size(rows, cols, &orow);
  if (ws_bytes < wr) return fail(NVFP4_WS_TOO_SMALL, "workspace of %zu bytes is below the %zu required",
                                 ws_bytes, nvfp4_workspace_size_dual(rows, cols, o));
  void *ws_c = ws ? static_cast<char *>(ws) + wr : nullptr;
  st = check_outputs(rows, cols, &orow, shr, codes_r, scales_r, ts_r, ws, wr);
  if (!st) st = check_outputs(rows, cols, &ocol, shc, codes_c, scales_c, ts_c, ws_c, ws_bytes - wr);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (shr.nblocks == 0) {
    st = write_trivial_scale(o, ts_r, s);
    return st ? st : write_trivial_scale(o, ts_c, s);
  }
  QuantParams pr, pc;
  fill_common(pr, x, in_dtype, rows, cols, ld, &orow, shr, codes_r, scales_r, ts_r, ws);
  fill_common(pc, x, in_dtype, rows, cols, ld, &ocol, shc, codes_c, scales_c, ts_c, ws_c);
  const int bf = in_dtype == NVFP4_BF16;
  const uint32_t grid = dual_grid(pr, bf);
  hipError_t e = launch_quant_dual(pr, pc, bf, o->tensor_scale_in != nullptr, grid, s);
  if (e == hipSuccess && !o->tensor_scale_in) {
    pr.npartial = grid;
    pc.npartial = grid;
    e = launch_eden_scales(pr, false, eden_scales_grid(pr), s);
    if (e == hipSuccess) e = launch_eden_scales(pc, false, eden_scales_grid(pc), s);
  }
  if (e != hipSuccess) return fail(NVFP4_HIP_ERROR, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

void nvfp4_opts_init(nvfp4_opts *o) {
  if (!o) return;
  std::memset(o, 0, sizeof(*o));
  o->rounding = NVFP4_RTN;
  o->eden_group = 128;
}

size_t nvfp4_workspace_size(int64_t rows, int64_t cols, const nvfp4_opts *o) {
  if (!o || rows < 0 || cols < 0) return 0;
  size_t bytes = kPartialBytes;
  if (o->rounding == NVFP4_MSEDEN && !o->tensor_scale_in) {
    const int64_t R = o->axis == 0 ? rows : cols;
    const int64_t K = o->axis == 0 ? cols : rows;
    bytes += (size_t)R * (size_t)(K / 16) * sizeof(float);
  }
  return round_up(bytes, 256);
}

size_t nvfp4_workspace_size_dual(int64_t rows, int64_t cols, const nvfp4_opts *o) {
  if (!o) return 0;
  nvfp4_opts orow = *o, ocol = *o;
  orow.axis = 0;
  ocol.axis = 1;
  const size_t a = nvfp4_workspace_size(rows, cols, &orow), b = nvfp4_workspace_size(rows, cols, &ocol);
  return (a && b) ? a + b : 0;
}

int nvfp4_quantize_nvfp4_dual(const void *x, int in_dtype, int64_t rows, int64_t cols, int64_t ld,
                              const nvfp4_opts *o, uint8_t *codes_r, uint8_t *scales_r, float *ts_r,
                              uint8_t *codes_c, uint8_t *scales_c, float *ts_c, void *ws,
                              size_t ws_bytes, void *stream) {
  return quantize_dual_impl(x, in_dtype, rows, cols, ld, o, codes_r, scales_r, ts_r, codes_c, scales_c,
                            ts_c, ws, ws_bytes, stream);
}

int nvfp4_quantize_nvfp4(const void *x, int in_dtype, int64_t rows, int64_t cols, int64_t ld,
                         const nvfp4_opts *o, uint8_t *codes, uint8_t *scales,
                         float *tensor_scale, void *ws, size_t ws_bytes, void *stream) {
  return quantize_impl(x, in_dtype, rows, cols, ld, o, codes, scales, tensor_scale, ws, ws_bytes,
                       stream, false);
}

int nvfp4_quantize_if4(const void *x, int in_dtype, int64_t rows, int64_t cols, int64_t ld,
                       const nvfp4_opts *o, uint8_t *codes, uint8_t *scales,
                       float *tensor_scale, void *ws, size_t ws_bytes, void *stream) {
  return quantize_impl(x, in_dtype, rows, cols, ld, o, codes, scales, tensor_scale, ws, ws_bytes,
                       stream, true);
}

int nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales, const float *tensor_scale,
                     int64_t rows_out, int64_t k, int format, const uint32_t *inv_rht_signs,
                     int out_dtype, void *out, void *stream) {
  if (format != NVFP4_FORMAT_NVFP4 && format != NVFP4_FORMAT_IF4)
    return fail(NVFP4_INVALID_ARG, "format %d is not NVFP4 or IF4", format);
  if (out_dtype != NVFP4_F32 && out_dtype != NVFP4_BF16)
    return fail(NVFP4_INVALID_ARG, "out_dtype %d is not NVFP4_F32 or NVFP4_BF16", out_dtype);
  if (rows_out < 0 || k < 0) return fail(NVFP4_INVALID_ARG, "negative shape");
  if (k % 16) return fail(NVFP4_BAD_SHAPE, "k %lld is not a multiple of 16", (long long)k);
  if (inv_rht_signs && k % 128)
    return fail(NVFP4_BAD_SHAPE, "k %lld is not a multiple of 128 (inverse rotation)", (long long)k);
  const uint64_t nblocks = (uint64_t)rows_out * (uint64_t)(k / 16);
  if (nblocks > kMaxBlocks) return fail(NVFP4_UNSUPPORTED, "more than 2^31 - 1 blocks");
  if (nblocks == 0) return ok();
  if (!codes || !scales || !tensor_scale || !out) return fail(NVFP4_INVALID_ARG, "null device pointer");
  if (!aligned(codes, 16) || !aligned(scales, 16) || !aligned(out, 16))
    return fail(NVFP4_MISALIGNED, "codes, scales and out must be 16-byte aligned");
  if (!aligned(tensor_scale, 4)) return fail(NVFP4_MISALIGNED, "tensor_scale must be 4-byte aligned");
  DequantParams p;
  std::memset(&p, 0, sizeof(p));
  p.codes = codes;
  p.scales = scales;
  p.ts = tensor_scale;
  p.out = out;
  p.R = (uint32_t)rows_out;
  p.K = (uint32_t)k;
  p.K16 = (uint32_t)(k / 16);
  p.nblocks = (uint32_t)nblocks;
  p.inv_rht = inv_rht_signs != nullptr;
  if (inv_rht_signs)
    for (int i = 0; i < 4; ++i) p.sg[i] = inv_rht_signs[i];
  p.if4 = format == NVFP4_FORMAT_IF4;
  hipError_t e = launch_dequant(p, out_dtype == NVFP4_BF16, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(NVFP4_HIP_ERROR, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

namespace {
// Shape and operand checks shared by the GEMM entry points; fills the
// operand fields of p.  Returns NVFP4_OK or the failure's status.
int gemm_operands(GemmParams &p, const uint8_t *a_codes, const uint8_t *a_scales, const float *a_ts,
                  const uint8_t *b_codes, const uint8_t *b_scales, const float *b_ts, int64_t M, int64_t N,
                  int64_t K) {
  if (M < 0 || N < 0 || K < 0) return fail(NVFP4_INVALID_ARG, "negative shape");
  if ((uint64_t)M > kMaxDim || (uint64_t)N > kMaxDim || (uint64_t)K > kMaxDim)
    return fail(NVFP4_UNSUPPORTED, "dimension above 2^31 - 1");
  if (K % 16) return fail(NVFP4_BAD_SHAPE, "K %lld is not a multiple of 16", (long long)K);
  // a 256-row operand panel (256 * K/2 code bytes) is addressed through one
  // buffer resource with a 32-bit byte range
  if ((uint64_t)K * 128u > 0x7FFFFFFFull)
    return fail(NVFP4_UNSUPPORTED, "K %lld above 16777200", (long long)K);
  p = GemmParams{};
  p.M = (uint32_t)M;
  p.N = (uint32_t)N;
  p.K = (uint32_t)K;
  if (M == 0 || N == 0) return ok();
  if (!a_codes || !a_scales || !a_ts || !b_codes || !b_scales || !b_ts)
    return fail(NVFP4_INVALID_ARG, "null device pointer");
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(a_scales, 16) ||
      !aligned(b_scales, 16))
    return fail(NVFP4_MISALIGNED, "codes and scales must be 16-byte aligned");
  if (!aligned(a_ts, 4) || !aligned(b_ts, 4)) return fail(NVFP4_MISALIGNED, "a tensor scale is misaligned");
  p.a_codes = a_codes;
  p.a_scales = a_scales;
  p.b_codes = b_codes;
  p.b_scales = b_scales;
  p.a_ts = a_ts;
  p.b_ts = b_ts;
  return ok();
}

int gemm_impl(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_ts,
              const uint8_t *b_codes, const uint8_t *b_scales, const float *b_ts, int64_t M,
              int64_t N, int64_t K, void *c, int out_dtype, int64_t ldc, void *stream, int if4) {
  if (out_dtype != NVFP4_F32 && out_dtype != NVFP4_BF16)
    return fail(NVFP4_INVALID_ARG, "out_dtype %d is not NVFP4_F32 or NVFP4_BF16", out_dtype);
  GemmParams p;
  int rc = gemm_operands(p, a_codes, a_scales, a_ts, b_codes, b_scales, b_ts, M, N, K);
  if (rc != NVFP4_OK) return rc;
  if (ldc < N) return fail(NVFP4_BAD_SHAPE, "ldc %lld < N %lld", (long long)ldc, (long long)N);
  if (M == 0 || N == 0) return ok();
  if (!c) return fail(NVFP4_INVALID_ARG, "null device pointer");
  if (!aligned(c, out_dtype == NVFP4_BF16 ? 2 : 4)) return fail(NVFP4_MISALIGNED, "c is misaligned");
  p.c = c;
  p.ldc = ldc;
  hipError_t e = launch_gemm(p, out_dtype == NVFP4_BF16 ? kOutBf16 : kOutF32, if4,
                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(NVFP4_HIP_ERROR, "launch failed: %s", hipGetErrorString(e));
  return ok();
}
}  // namespace

int nvfp4_gemm_nvfp4(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_ts,
                     const uint8_t *b_codes, const uint8_t *b_scales, const float *b_ts,
                     int64_t M, int64_t N, int64_t K, void *c, int out_dtype, int64_t ldc,
                     void *stream) {
  return gemm_impl(a_codes, a_scales, a_ts, b_codes, b_scales, b_ts, M, N, K, c, out_dtype, ldc,
                   stream, 0);
}

int nvfp4_gemm_if4(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_ts,
                   const uint8_t *b_codes, const uint8_t *b_scales, const float *b_ts,
                   int64_t M, int64_t N, int64_t K, void *c, int out_dtype, int64_t ldc,
                   void *stream) {
  return gemm_impl(a_codes, a_scales, a_ts, b_codes, b_scales, b_ts, M, N, K, c, out_dtype, ldc,
                   stream, 1);
}

int nvfp4_gemm_nvfp4_rtn(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_ts,
                         const uint8_t *b_codes, const uint8_t *b_scales, const float *b_ts,
                         int64_t M, int64_t N, int64_t K, const float *c_ts, uint8_t *c_codes,
                         uint8_t *c_scales, float *c_amax, void *stream) {
  GemmParams p;
  int rc = gemm_operands(p, a_codes, a_scales, a_ts, b_codes, b_scales, b_ts, M, N, K);
  if (rc != NVFP4_OK) return rc;
  if (N % 16) return fail(NVFP4_BAD_SHAPE, "N %lld is not a multiple of 16", (long long)N);
  if (c_amax && !aligned(c_amax, 4)) return fail(NVFP4_MISALIGNED, "c_amax is misaligned");
  if (M > 0 && N > 0) {
    if (!c_ts || !c_codes || !c_scales) return fail(NVFP4_INVALID_ARG, "null device pointer");
    if (!aligned(c_codes, 16) || !aligned(c_scales, 16))
      return fail(NVFP4_MISALIGNED, "c_codes and c_scales must be 16-byte aligned");
    if (!aligned(c_ts, 4)) return fail(NVFP4_MISALIGNED, "c_ts is misaligned");
  }
  if ((M == 0 || N == 0) && !c_amax) return ok();  // nothing to write
  p.q_codes = c_codes;
  p.q_scales = c_scales;
  p.q_ts = c_ts;
  p.q_amax = c_amax;
  hipError_t e = launch_gemm(p, kOutNvfp4, 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(NVFP4_HIP_ERROR, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int nvfp4_rht(const void *x, int in_dtype, int64_t rows, int64_t cols, int64_t ld, int axis,
              const uint32_t *rht_signs, float *out, void *stream) {
  if (!rht_signs) return fail(NVFP4_INVALID_ARG, "rht_signs is NULL");
  nvfp4_opts o;
  nvfp4_opts_init(&o);
  o.axis = axis;
  o.rht = 1;
  for (int i = 0; i < 4; ++i) o.rht_signs[i] = rht_signs[i];
  Shape sh;
  const int st = check_input(x, in_dtype, rows, cols, ld, &o, false, &sh);
  if (st) return st;
  if (sh.nblocks == 0) return ok();
  if (!out) return fail(NVFP4_INVALID_ARG, "out is NULL");
  if (!aligned(out, 16)) return fail(NVFP4_MISALIGNED, "out must be 16-byte aligned");
  QuantParams p;
  fill_common(p, x, in_dtype, rows, cols, ld, &o, sh, nullptr, nullptr, nullptr, nullptr);
  p.rot_out = out;
  const int bf = in_dtype == NVFP4_BF16;
  hipError_t e = launch_quant(p, bf, axis, kRot, quant_grid(p, bf, axis), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(NVFP4_HIP_ERROR, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free entry point
// The workspace of nvfp4_quantize_nvfp4_noalloc: a file-scope device array,
// one copy per GPU, held until the process ends.  Host code never uses the
// array's name as an address (on the host it is a stand-in, not device
// memory): the device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address reaches kernels.
constexpr size_t kScratchBytes = NVFP4_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0 && kScratchBytes > kPartialBytes, "scratch layout");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

// This device's copy of the scratch array (looked up on its first use).
int device_scratch(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(NVFP4_HIP_ERROR, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(NVFP4_UNSUPPORTED, "device %d above the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(NVFP4_HIP_ERROR, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return NVFP4_OK;
}
}  // namespace

extern "C" {

int nvfp4_quantize_nvfp4_noalloc(const void *x, int in_dtype, int64_t rows, int64_t cols, int64_t ld,
                                 const nvfp4_opts *o, uint8_t *codes, uint8_t *scales, float *tensor_scale,
                                 void *stream) {
  if (!o) return fail(NVFP4_INVALID_ARG, "opts is NULL");
  if (rows < 0 || cols < 0) return fail(NVFP4_INVALID_ARG, "negative shape");
  const size_t need = nvfp4_workspace_size(rows, cols, o);
  if (need > kScratchBytes)
    return fail(NVFP4_UNSUPPORTED, "this call needs %zu bytes of workspace, above the %zu bytes of the "
                "allocation-free entry point's scratch (use nvfp4_quantize_nvfp4 with a workspace)",
                need, kScratchBytes);
  void *ws = nullptr;
  const int st = device_scratch(&ws);
  if (st) return st;
  return quantize_impl(x, in_dtype, rows, cols, ld, o, codes, scales, tensor_scale, ws, kScratchBytes, stream,
                       false);
}

const char *nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_INVALID_ARG: return "invalid argument";
    case NVFP4_BAD_SHAPE: return "bad shape";
    case NVFP4_MISALIGNED: return "misaligned pointer or stride";
    case NVFP4_WS_TOO_SMALL: return "workspace too small";
    case NVFP4_HIP_ERROR: return "HIP error";
    case NVFP4_UNSUPPORTED: return "unsupported";
    default: return "unknown status";
  }
}

const char *nvfp4_last_error(void) { return g_last_error.c_str(); }

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

}  // extern "C"
