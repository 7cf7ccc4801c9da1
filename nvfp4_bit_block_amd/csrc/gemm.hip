// gemm.hip -- block-scaled FP4 GEMM for gfx950:
//   C[M x N] = (ts_a * ts_b) * sum_k A[m][k] * B[n][k],
// A[m][k] = E2M1(code) * E4M3(scale of its 16-block), both operands packed
// K-major as written by the quantizers (Quartet II's NVFP4 linear-layer
// GEMMs; abstract and news summary, "Kerninnovationen").
//
// gfx950's native FP4 matrix instructions take one power-of-two (E8M0) scale
// per 32 elements; NVFP4 has an E4M3 scale per 16.  The product of an E2M1
// value and an E4M3 scale has at most 6 significant bits and lies in
// [2^-10, 2688], so it is exact in fp16: each operand fragment is
// dequantized exactly -- v_cvt_scalef32_pk_f16_fp4 (two codes per
// instruction, unit scale) then one packed fp16 multiply by the block scale
// -- and multiplied on the fp16 matrix cores (v_mfma_f32_32x32x16_f16) with
// fp32 accumulation.
//
// Tiling: a workgroup of 16 waves (four per SIMD, so that others can issue
// while one waits on LDS or the barrier) computes a 256 x 256 tile; wave
// (wm, wn) a 64 x 64 sub-tile as 2 x 2 MFMA tiles of 32 x 32 (64 fp32
// accumulators per lane, about 125 VGPRs in all).  K advances in chunks of 64
// (four 16-wide MFMA steps).  The tile's 16 row fragments per chunk (8 of A,
// 8 of B, 32 rows each) are split between the waves: wave w loads fragment w
// (A for w < 8, B after; buffer loads, rows past M or N read as zero),
// dequantizes it once, and writes the fp16 MFMA operands to LDS in operand
// order (lane l's 16 bytes at slot l: conflict-free).  Every wave then reads
// its 2 + 2 operands per step from LDS.  So each fragment is loaded and
// dequantized once per workgroup, not once per wave that uses it -- the
// dequantization is the vector-ALU cost that competes with the matrix
// cores.  LDS is double-buffered (2 x 64 KB):
// chunk c+1 is dequantized, one step at a time, between the MFMA steps of
// chunk c, and the raw codes of chunk c+3 are loaded as soon as a register
// buffer frees up; one barrier per chunk.
//
// K order inside a chunk: MFMA lane half h = lane / 32 holds k slots
// 8h .. 8h+7 of each 16-wide step.  A lane loads the 32 codes at
// k0 + 32h .. k0 + 32h + 31 and feeds dword j of them to step j.  A and B use
// the same assignment, so the permutation of k cancels.
//
// Workgroup order: the grid holds one workgroup per compute unit (a
// multiple of 8), each looping over tiles bid, bid + grid, ...; workgroups
// are dispatched round-robin to the 8 XCDs, so a workgroup's tiles all
// belong to its XCD.  The tile index is remapped so that each XCD receives
// a contiguous run, laid out in groups of 4 tile-rows so that the 32
// workgroups resident on one XCD share A and B panels in that XCD's L2.
//
// Epilogue: the accumulators go through LDS (each wave's 64 x 64 tile in
// its own 8 KB of the stage) so that the output is written in 16-byte row
// segments; the next tile's first operand loads are issued before it.  The
// output is fp32, bf16, or NVFP4: each 16-column block of a row coded with
// round-to-nearest under a given tensor scale, the forward pass's coding of
// the next layer's input (Quartet II news summary, "Quantisierung im
// Vorwaertsdurchlauf").
#include "kernels.hpp"

namespace nv4 {

typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr uint32_t kTile = 256, kWaveCols = 64, kChunk = 64, kSteps = 4, kGroupM = 4, kXcds = 8;

// Raw codes of this wave's fragment for one chunk: the lane's 32 codes and
// the chunk's four E4M3 scale bytes of its row -- bytes 2h, 2h+1 are the
// lane half's.
struct Raw {
  u32x4_t code;
  uint32_t scale;
};

struct Panels {
  __amdgpu_buffer_rsrc_t c, s;  // codes / scales of the panel (A or B) of this wave's fragment
  // vo_c: byte offset of this lane's row of its fragment plus its lane
  // half's first code byte; vo_s: that row's first scale byte.  The whole row offset is in the vector offset, so
  // rows past M or N fall outside the buffer's range and read as zero; the
  // chunk's k offset (< one row) is the scalar offset.
  uint32_t vo_c, vo_s;
  uint32_t K, h;
};

// Whole chunk at k0 < K, K % 64 == 0.
__device__ __forceinline__ void load_fast(Raw &r, const Panels &p, uint32_t k0) {
  r.code = __builtin_amdgcn_raw_buffer_load_b128(p.c, p.vo_c, k0 / 2, 0);
  r.scale = __builtin_amdgcn_raw_buffer_load_b32(p.s, p.vo_s, k0 / 16, 0);
}

// Any chunk at k0 < K, K % 16 == 0: dword- and byte-granular loads, zero past K.
__device__ __forceinline__ void load_generic(Raw &r, const Panels &p, uint32_t k0) {
  const uint32_t kl = k0 + 32 * p.h;  // first k of this lane's 32
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    w[q] = (kl + 8 * q + 8 <= p.K) ? __builtin_amdgcn_raw_buffer_load_b32(p.c, p.vo_c + 4 * q, k0 / 2, 0) : 0u;
  r.code = u32x4_t{w[0], w[1], w[2], w[3]};
  uint32_t s = 0;
#pragma unroll
  for (int q = 0; q < 2; ++q)
    if (kl + 16 * q < p.K)
      s |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(p.s, p.vo_s + 2 * p.h + q, k0 / 16, 0)
           << (8 * (q + 2 * p.h));
  r.scale = s;
}

// LDS stage: [buffer][fragment 0..15 (A 0..7, B 8..15)][step][lane] x 16 bytes.
typedef half8_t Stage[2][16][kSteps][64];
static_assert(sizeof(Stage) == 16 * 8192, "the epilogue gives each of the 16 waves 8 KB of the stage");

// The two fp16 block scales of this lane half (bytes 2h, 2h+1 of the word)
// and, for IF4 operands, their INT flags (bits 7 and 15 of f).
template <int IF4>
struct Scales {
  half2_t s;
  uint32_t f;
};

template <int IF4>
__device__ __forceinline__ void scales16(const Raw &r, uint32_t h, Scales<IF4> &sc) {
  const uint32_t b = r.scale >> (16 * h);
  if (IF4) {
    sc.f = b;
    sc.s = e4m3x2_f16(b & 0x7F7Fu);
  } else {
    sc.s = e4m3x2_f16(b);
  }
}

// Dequantize step j of this wave's fragment (fragment w: A 0..7, B 8..15)
// for one chunk into buffer b.
template <int IF4>
__device__ __forceinline__ void dequant_item(Stage &st, int b, const Raw &r, const Scales<IF4> &sc, uint32_t w,
                                             uint32_t lane, int j) {
  if (IF4) {
    const bool is_int = (sc.f >> (8 * (j >> 1) + 7)) & 1u;
    st[b][w][j][lane] = dequant8_lut(r.code[j], sc.s[j >> 1], is_int ? kLutIntLo : kLutFpLo,
                                     is_int ? kLutIntHi : kLutFpHi);
  } else {
    st[b][w][j][lane] = dequant8(r.code[j], sc.s[j >> 1]);
  }
}

struct Ops {
  half8_t a[2], b[2];
};

__device__ __forceinline__ void read_ops(Ops &op, const Stage &st, int b, uint32_t wm, uint32_t wn, uint32_t lane,
                                         int j) {
#pragma unroll
  for (int n = 0; n < 2; ++n) op.b[n] = st[b][8 + 2 * wn + n][j][lane];
#pragma unroll
  for (int m = 0; m < 2; ++m) op.a[m] = st[b][2 * wm + m][j][lane];
}

// B is the first MFMA operand: the 32 x 32 result is the transposed tile,
// so that a lane holds one output row and, for each group of four
// accumulators, four adjacent output columns (see the epilogue).
__device__ __forceinline__ void mfma16(const Ops &op, float16_t (&acc)[2][2]) {
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
      acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(op.b[n], op.a[m], acc[m][n], 0, 0, 0);
}

// Interleave one step: each MFMA followed by up to NV vector-ALU instructions
// and one LDS access.
template <int NV>
__device__ __forceinline__ void interleave_step() {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);  // VALU
    __builtin_amdgcn_sched_group_barrier(0x080, 1, 0);   // LDS
  }
}

// One chunk of the steady state.  On entry `op` holds step 0 of chunk c (in
// buffer c&1) and `rd` the raw codes of chunk c+1.  Steps 0-2 dequantize
// chunk c+1 (two, one and one of its four steps) into the other buffer while
// computing; the barrier after step 2 publishes it (and retires every read
// of this chunk's buffer), so step 3 can already fetch chunk c+1's first
// operands.  `rd` is then reloaded with
// chunk `k_next` (clamped into range by the caller).
template <int IF4>
__device__ __forceinline__ void chunk(Stage &st, uint32_t c, uint32_t k_next, Raw &rd, Ops &op, const Panels &p,
                                      uint32_t w, uint32_t wm, uint32_t wn, uint32_t lane,
                                      float16_t (&acc)[2][2]) {
  const int cur = c & 1, nxt = cur ^ 1;
  Scales<IF4> s;
  scales16<IF4>(rd, p.h, s);
  Ops nx;
  // step 0
  read_ops(nx, st, cur, wm, wn, lane, 1);
#pragma unroll
  for (int j = 0; j < 2; ++j) dequant_item<IF4>(st, nxt, rd, s, w, lane, j);
  mfma16(op, acc);
  interleave_step<IF4 ? 10 : 8>();
  __builtin_amdgcn_sched_barrier(0);
  // step 1
  read_ops(op, st, cur, wm, wn, lane, 2);
  dequant_item<IF4>(st, nxt, rd, s, w, lane, 2);
  mfma16(nx, acc);
  interleave_step<IF4 ? 10 : 8>();
  __builtin_amdgcn_sched_barrier(0);
  // step 2
  read_ops(nx, st, cur, wm, wn, lane, 3);
  dequant_item<IF4>(st, nxt, rd, s, w, lane, 3);
  mfma16(op, acc);
  interleave_step<IF4 ? 10 : 8>();
  __builtin_amdgcn_sched_barrier(0);
  load_fast(rd, p, k_next);
  __syncthreads();
  // step 3
  read_ops(op, st, nxt, wm, wn, lane, 0);
  mfma16(nx, acc);
  interleave_step<0>();
  __builtin_amdgcn_sched_barrier(0);
}

// NVFP4 round-to-nearest of one 16-block z of C with tensor scale s_t (the
// quantizer's RTN step: the E4M3 scale e = RNE((max |z| / 6) / s_t), codes
// of z / (E4M3(e) * s_t) on the E2M1 grid, signed zeros when e = 0).
// Returns e; folds max |z| into amax.
__device__ __forceinline__ uint32_t rtn_block16(const float z[16], float s_t, uint32_t &lo, uint32_t &hi,
                                                float &amax) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(z[i]));
  amax = fmaxf(amax, a);
  const uint32_t e = e4m3_rne_sat(div_rn(div_by<6>(a), s_t));
  const float r = e ? rcp_rn(e4m3_value(e) * s_t) : 0.0f;
  float y[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = z[i] * r;
  e2m1x16_rne(y, lo, hi);
  return e;
}

// Epilogue.  With B as the first MFMA operand, lane (r32, h) of tile
// (m, n) holds output row 32m + r32 of the wave tile and, in accumulators
// 4q .. 4q+3, its columns 32n + 8q + 4h .. +3.  The wave scales and
// rounds them, writes its tile to its own 8 KB of the (now idle) stage,
// and reads it back by rows, so that every lane stores 16 contiguous
// bytes and eight (bf16) or sixteen (fp32) lanes cover a whole row of the
// wave tile.  The 16-byte column chunks of a row are XOR-swizzled by the
// row so that both the writes and the reads spread over all LDS banks.
// The bf16 and fp32 rows are written with non-temporal stores: an output of
// this size is not read again while it could still be in the caches, and
// dirty lines left in L2 and the memory-side cache would be written back
// while the next kernel runs, at that kernel's expense.
template <int OUT>
__device__ __forceinline__ void store_tile(Stage &st, const float16_t (&acc)[2][2], const GemmParams &p, uint32_t m0,
                                           uint32_t n0, uint32_t w, float &qmax) {
  constexpr bool OUT_BF16 = OUT == kOutBf16;
  const uint32_t wm = w >> 2, wn = w & 3u;
  const float alpha = (*p.a_ts) * (*p.b_ts);
  // (the lane index is re-derived opaquely, so that the compiler does not
  // hoist the epilogue's addresses out of the tile loop and keep them live
  // through the main loop)
  uint32_t lane = threadIdx.x;
  asm volatile("" : "+v"(lane));
  lane &= 63u;
  const uint32_t r32 = lane & 31u, h = lane >> 5;
  uint8_t *const wbuf = reinterpret_cast<uint8_t *>(&st) + w * 8192u;
  const uint32_t row0 = m0 + wm * 64, col0 = n0 + wn * kWaveCols;
  const uint32_t esz = OUT_BF16 ? 2 : 4;
  // 16-byte stores need a 16-byte aligned row start in every row
  const bool vec = ((reinterpret_cast<uintptr_t>(p.c) | (uintptr_t)(p.ldc * esz)) & 15u) == 0;
  if (OUT_BF16) {
    // the whole 64 x 64 wave tile, rows of 128 bytes (8 chunks)
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint32_t rl = 32 * m + r32;
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t b[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t u = __float_as_uint(acc[m][n][4 * q + t] * alpha);
            b[t] = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // bf16, nearest even
          }
          const uint32_t chunk = (4 * n + q) ^ ((rl >> 1) & 7u);
          *reinterpret_cast<uint2 *>(wbuf + rl * 128 + chunk * 16 + 8 * h) =
              uint2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t rl = 8 * i + (lane >> 3), cc = lane & 7u;
      const uint4 v = *reinterpret_cast<const uint4 *>(wbuf + rl * 128 + ((cc ^ ((rl >> 1) & 7u)) * 16));
      const uint32_t row = row0 + rl, col = col0 + 8 * cc;
      if (row >= p.M || col >= p.N) continue;
      uint16_t *dst = static_cast<uint16_t *>(p.c) + (size_t)row * p.ldc + col;
      if (vec && col + 8 <= p.N) {
        __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t *>(dst));
      } else {
        const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (col + t < p.N) dst[t] = (uint16_t)(vv[t >> 1] >> (16 * (t & 1)));
      }
    }
  } else {
    // fp32 and NVFP4: one 32 x 64 half (m) of the wave tile at a time, as
    // fp32 rows of 256 bytes (16 chunks)
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (m) __syncthreads();  // the reads of the first half are done
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t chunk = (8 * n + 2 * q + h) ^ (r32 & 15u);
          *reinterpret_cast<float4 *>(wbuf + r32 * 256 + chunk * 16) =
              float4{acc[m][n][4 * q] * alpha, acc[m][n][4 * q + 1] * alpha, acc[m][n][4 * q + 2] * alpha,
                     acc[m][n][4 * q + 3] * alpha};
        }
      __syncthreads();
      if (OUT == kOutNvfp4) {
        // one 16-column block per lane and pass: 32 rows x 4 blocks
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint32_t rl = 16 * i + (lane >> 2), b = lane & 3u;
          float z[16];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float4 v = *reinterpret_cast<const float4 *>(wbuf + rl * 256 + (((4 * b + c) ^ (rl & 15u)) * 16));
            z[4 * c] = v.x;
            z[4 * c + 1] = v.y;
            z[4 * c + 2] = v.z;
            z[4 * c + 3] = v.w;
          }
          const uint32_t row = row0 + 32 * m + rl, col = col0 + 16 * b;
          if (row >= p.M || col >= p.N) continue;  // N % 16 == 0: blocks are whole
          uint32_t lo, hi;
          const uint32_t e = rtn_block16(z, *p.q_ts, lo, hi, qmax);
          *reinterpret_cast<uint2 *>(p.q_codes + (size_t)row * (p.N / 2) + col / 2) = make_uint2(lo, hi);
          p.q_scales[(size_t)row * (p.N / 16) + col / 16] = (uint8_t)e;
        }
        continue;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t rl = 4 * i + (lane >> 4), cc = lane & 15u;
        const float4 v = *reinterpret_cast<const float4 *>(wbuf + rl * 256 + ((cc ^ (rl & 15u)) * 16));
        const uint32_t row = row0 + 32 * m + rl, col = col0 + 4 * cc;
        if (row >= p.M || col >= p.N) continue;
        float *dst = static_cast<float *>(p.c) + (size_t)row * p.ldc + col;
        if (vec && col + 4 <= p.N) {
          __builtin_nontemporal_store(f32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4_t *>(dst));
        } else {
          const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (col + t < p.N) dst[t] = vv[t];
        }
      }
    }
  }
}

// Placement of workgroup-order tile `bid`: workgroups are dispatched
// round-robin to the XCDs, so tile bid is remapped such that each XCD
// receives a contiguous run, laid out in groups of kGroupM tile-rows.
__device__ __forceinline__ void tile_at(uint32_t bid, uint32_t tiles_m, uint32_t tiles_n, uint32_t &m0, uint32_t &n0) {
  const uint32_t nt = tiles_m * tiles_n;
  const uint32_t per = nt / kXcds, rem = nt % kXcds, xcd = bid % kXcds, idx = bid / kXcds;
  const uint32_t lid = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + idx;
  const uint32_t group = lid / (kGroupM * tiles_n);
  const uint32_t first_m = group * kGroupM;
  const uint32_t gsz = min(tiles_m - first_m, kGroupM);
  const uint32_t in_group = lid - group * kGroupM * tiles_n;
  m0 = (first_m + in_group % gsz) * kTile;
  n0 = (in_group / gsz) * kTile;
}

// Wave w's operand panel (A rows m0.., or B rows n0..) of a tile.
__device__ __forceinline__ void make_panels(Panels &P, const GemmParams &p, uint32_t m0, uint32_t n0, uint32_t w,
                                            uint32_t r32, uint32_t h) {
  const uint32_t K2 = p.K / 2, K16 = p.K / 16;
  if (w < 8) {
    const uint32_t rows = min(kTile, p.M - m0);
    P.c = __builtin_amdgcn_make_buffer_rsrc((void *)(p.a_codes + (size_t)m0 * K2), (short)0, (int)(rows * K2),
                                            kRsrcWord3);
    P.s = __builtin_amdgcn_make_buffer_rsrc((void *)(p.a_scales + (size_t)m0 * K16), (short)0, (int)(rows * K16),
                                            kRsrcWord3);
  } else {
    const uint32_t rows = min(kTile, p.N - n0);
    P.c = __builtin_amdgcn_make_buffer_rsrc((void *)(p.b_codes + (size_t)n0 * K2), (short)0, (int)(rows * K2),
                                            kRsrcWord3);
    P.s = __builtin_amdgcn_make_buffer_rsrc((void *)(p.b_scales + (size_t)n0 * K16), (short)0, (int)(rows * K16),
                                            kRsrcWord3);
  }
  const uint32_t row = 32 * (w & 7u) + r32;  // this lane's row of its fragment
  P.vo_c = row * K2 + 16 * h;
  P.vo_s = row * K16;
  P.K = p.K;
  P.h = h;
}

template <int OUT, int FAST, int IF4>
__global__ __launch_bounds__(1024, 1) void k_gemm(GemmParams p) {
  __shared__ Stage st;
  const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t r32 = lane & 31u, h = lane >> 5;
  const uint32_t wm = w >> 2, wn = w & 3u;  // wave tile: rows 64 wm.., columns 64 wn..

  // Tiles of this workgroup: bid, bid + gridDim.x, ...  The grid is a
  // multiple of the XCD count (or covers every tile at once), so all of a
  // workgroup's tiles map to the XCD it runs on.  The next tile's first two
  // chunks are loaded before this tile's epilogue, so that their latency
  // overlaps the output stores.
  const uint32_t tiles_m = (p.M + kTile - 1) / kTile, tiles_n = (p.N + kTile - 1) / kTile;
  const uint32_t nt = tiles_m * tiles_n;
  const uint32_t K = p.K;
  const uint32_t nfull = FAST ? K / kChunk : 0;
  const uint32_t klast = nfull > 0 ? (nfull - 1) * kChunk : 0;
  uint32_t bid = blockIdx.x, m0, n0;
  tile_at(bid, tiles_m, tiles_n, m0, n0);
  Panels P;
  make_panels(P, p, m0, n0, w, r32, h);
  // chunk 0 in r0, chunk 1 in r1 (loads of chunks past the end re-read the
  // last chunk, unused); sched barriers keep the loads in this order
  Raw r0, r1;
  float qmax = 0.0f;  // kOutNvfp4: max |C| over this lane's blocks
  if (nfull > 0) {
    load_fast(r0, P, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_fast(r1, P, min(kChunk, klast));
    __builtin_amdgcn_sched_barrier(0);
  }
  for (;;) {
    float16_t acc[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[m][n][e] = 0.0f;

    if (nfull > 0) {
      // Prologue: chunk 0 into buffer 0, then chunk 2 into r0.
      {
        Scales<IF4> s;
        scales16<IF4>(r0, P.h, s);
#pragma unroll
        for (int j = 0; j < 4; ++j) dequant_item<IF4>(st, 0, r0, s, w, lane, j);
      }
      __builtin_amdgcn_sched_barrier(0);
      load_fast(r0, P, min(2 * kChunk, klast));
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      Ops op;
      read_ops(op, st, 0, wm, wn, lane, 0);
      // Steady state: chunk c+1's codes are in r1 (c even) or r0 (c odd).
      // The chunk after the last dequantizes stale codes into the idle buffer.
      uint32_t c = 0;
      for (; c + 1 < nfull; c += 2) {
        chunk<IF4>(st, c, min((c + 3) * kChunk, klast), r1, op, P, w, wm, wn, lane, acc);
        chunk<IF4>(st, c + 1, min((c + 4) * kChunk, klast), r0, op, P, w, wm, wn, lane, acc);
      }
      if (c < nfull) chunk<IF4>(st, c, klast, r1, op, P, w, wm, wn, lane, acc);
      __syncthreads();  // every wave is done with both buffers before any reuse below
    }
    // remaining K (K % 64 != 0): one chunk at a time through buffer 0
    for (uint32_t k0 = nfull * kChunk; k0 < K; k0 += kChunk) {
      Raw r;
      load_generic(r, P, k0);
      Scales<IF4> s;
      scales16<IF4>(r, P.h, s);
#pragma unroll
      for (int j = 0; j < 4; ++j) dequant_item<IF4>(st, 0, r, s, w, lane, j);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < (int)kSteps; ++j) {
        Ops op;
        read_ops(op, st, 0, wm, wn, lane, j);
        mfma16(op, acc);
      }
      __syncthreads();
    }

    const uint32_t nbid = bid + gridDim.x;
    const uint32_t cm0 = m0, cn0 = n0;
    if (nbid < nt) {
      tile_at(nbid, tiles_m, tiles_n, m0, n0);
      make_panels(P, p, m0, n0, w, r32, h);
      if (nfull > 0) {
        load_fast(r0, P, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_fast(r1, P, min(kChunk, klast));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    store_tile<OUT>(st, acc, p, cm0, cn0, w, qmax);
    if (nbid >= nt) break;
    __syncthreads();  // every wave has read its output back before the next tile's stage writes
    bid = nbid;
  }
  if (OUT == kOutNvfp4 && p.q_amax) {
    // |C| >= 0, so its fp32 bits order as unsigned integers: one atomic
    // maximum per wave, whose result does not depend on their order
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, d));
    if (lane == 0) atomicMax(reinterpret_cast<unsigned int *>(p.q_amax), __float_as_uint(qmax));
  }
}

// Clears the maximum that k_gemm<kOutNvfp4> accumulates (a kernel rather
// than a memset node, so that the call can be captured in a graph).
__global__ void k_clear_amax(float *amax) { *amax = 0.0f; }

template <int OUT, int IF4>
static void launch_out(const GemmParams &p, uint32_t grid, hipStream_t s) {
  if ((p.K % 64) == 0) hipLaunchKernelGGL((k_gemm<OUT, 1, IF4>), dim3(grid), dim3(1024), 0, s, p);
  else hipLaunchKernelGGL((k_gemm<OUT, 0, IF4>), dim3(grid), dim3(1024), 0, s, p);
}

// One workgroup per compute unit (the stage takes most of a CU's LDS), a
// multiple of the XCD count; fewer when there are fewer tiles.
static uint32_t gemm_grid(uint32_t tiles) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return tiles;
  const uint32_t g = ((uint32_t)(cus > 0 ? cus : 0) / kXcds) * kXcds;
  return (g == 0 || tiles <= g) ? tiles : g;
}

hipError_t launch_gemm(const GemmParams &p, int out, int if4, hipStream_t s) {
  if (out == kOutNvfp4 && p.q_amax) hipLaunchKernelGGL(k_clear_amax, dim3(1), dim3(1), 0, s, p.q_amax);
  if (p.M == 0 || p.N == 0) return hipGetLastError();
  const uint32_t grid = gemm_grid(((p.M + kTile - 1) / kTile) * ((p.N + kTile - 1) / kTile));
  if (out == kOutNvfp4) {
    if (if4) return hipErrorInvalidValue;
    launch_out<kOutNvfp4, 0>(p, grid, s);
  } else if (out == kOutBf16) {
    if (if4) launch_out<kOutBf16, 1>(p, grid, s);
    else launch_out<kOutBf16, 0>(p, grid, s);
  } else {
    if (if4) launch_out<kOutF32, 1>(p, grid, s);
    else launch_out<kOutF32, 0>(p, grid, s);
  }
  return hipGetLastError();
}

}  // namespace nv4
