// RMSNorm forward for gfx950.
//
// y[m,k] = x[m,k] * r_m * g[k],  r_m = 1 / sqrt(sum_k x[m,k]^2 / d + eps)
// ("When to hand-write a GPU kernel on Apple Silicon", Rung 2: one reduction
// per row, eps inside the root; Rung 4: wide vector loads and a hardware
// cross-lane reduction instead of a shared-memory tree).
//
// gfx950 design: one 64-lane wavefront owns one row.  Each lane loads
// 16-byte chunks (8 bf16 or 4 fp32) with lane-consecutive addresses, so one
// wave instruction moves 1 KiB contiguous.  The chunks stay in VGPRs between
// the reduction and the scaling pass, so x is read from HBM exactly once.
// The row sum is a 64-lane butterfly; no LDS and no barrier.  Rows too long
// for the register cache fall back to a two-sweep variant that re-reads x.
#include "common.h"
#include "launch.h"

namespace ffn {

template <int EB>
struct Chunk;  // 16-byte chunk helpers per element size
template <>
struct Chunk<2> {
  static constexpr int E = 8;
  __device__ static float sumsq(const uint4& v) {
    float f[8];
    unpack8(v, f);
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = __builtin_fmaf(f[i], f[i], a);
    return a;
  }
  __device__ static uint4 scale(const uint4& v, const uint4& gv, float r) {
    float f[8], gg[8];
    unpack8(v, f);
    unpack8(gv, gg);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (f[i] * r) * gg[i];
    return pack8(f);
  }
};
template <>
struct Chunk<4> {
  static constexpr int E = 4;
  __device__ static float sumsq(const uint4& v) {
    float a = __uint_as_float(v.x) * __uint_as_float(v.x);
    a = __builtin_fmaf(__uint_as_float(v.y), __uint_as_float(v.y), a);
    a = __builtin_fmaf(__uint_as_float(v.z), __uint_as_float(v.z), a);
    a = __builtin_fmaf(__uint_as_float(v.w), __uint_as_float(v.w), a);
    return a;
  }
  __device__ static uint4 scale(const uint4& v, const uint4& gv, float r) {
    return make_uint4(__float_as_uint((__uint_as_float(v.x) * r) * __uint_as_float(gv.x)),
                      __float_as_uint((__uint_as_float(v.y) * r) * __uint_as_float(gv.y)),
                      __float_as_uint((__uint_as_float(v.z) * r) * __uint_as_float(gv.z)),
                      __float_as_uint((__uint_as_float(v.w) * r) * __uint_as_float(gv.w)));
  }
};

constexpr int kRowsPerBlock = 4;  // 4 wavefronts, one row each
// Launches of many rows stream x in and y out with non-temporal (streaming)
// loads and stores: 16384 x 4096 bf16 50.3 -> 46.9 us (interleaved A/B,
// bitwise identical; the prefill block, whose GEMM then reads n, unchanged).
// Launches of a few rows keep plain accesses: their output is read at once
// by the next kernel.
#ifndef FFN_RMS_NT
#define FFN_RMS_NT 1
#endif
#ifndef FFN_RMS_PREG_ROWS
#define FFN_RMS_PREG_ROWS 64
#endif

// CACHE = 16-byte chunks per lane kept in registers; requires
// nchunk <= 64 * CACHE.  PREG: the gain chunks are loaded together with x
// instead of after the reduction (one dependent memory round trip less; for
// launches of a few rows, where that latency is the kernel's length).
template <int EB, int CACHE, bool PREG>
__global__ __launch_bounds__(256) void rmsnorm_cached(const uint4* __restrict__ x,
                                                      const uint4* __restrict__ g,
                                                      uint4* __restrict__ y, int64_t rows,
                                                      int nchunk, float inv_d, float eps) {
  constexpr bool NT = !PREG && FFN_RMS_NT;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint4* xr = x + row * nchunk;
  uint4 v[CACHE], gv[PREG ? CACHE : 1];
#pragma unroll
  for (int i = 0; i < CACHE; ++i) {
    const int c = lane + 64 * i;
    v[i] = c < nchunk ? (NT ? ld_nt(xr + c) : xr[c]) : make_uint4(0, 0, 0, 0);
    if (PREG) gv[PREG ? i : 0] = c < nchunk ? g[c] : make_uint4(0, 0, 0, 0);
  }
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < CACHE; ++i) acc += Chunk<EB>::sumsq(v[i]);
  acc = wave_sum(acc);
  const float r = 1.0f / __builtin_sqrtf(acc * inv_d + eps);
  uint4* yr = y + row * nchunk;
#pragma unroll
  for (int i = 0; i < CACHE; ++i) {
    const int c = lane + 64 * i;
    if (c < nchunk) st16<NT>(yr + c, Chunk<EB>::scale(v[i], PREG ? gv[PREG ? i : 0] : g[c], r));
  }
}

// Any row length: sum of squares in one sweep, scaling in a second sweep.
template <int EB>
__global__ __launch_bounds__(256) void rmsnorm_stream(const uint4* __restrict__ x,
                                                      const uint4* __restrict__ g,
                                                      uint4* __restrict__ y, int64_t rows,
                                                      int nchunk, float inv_d, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint4* xr = x + row * nchunk;
  float acc = 0.f;
  for (int c = lane; c < nchunk; c += 64) acc += Chunk<EB>::sumsq(xr[c]);
  acc = wave_sum(acc);
  const float r = 1.0f / __builtin_sqrtf(acc * inv_d + eps);
  uint4* yr = y + row * nchunk;
  for (int c = lane; c < nchunk; c += 64) yr[c] = Chunk<EB>::scale(xr[c], g[c], r);
}

template <int EB>
static hipError_t launch_eb(const void* x, const void* g, void* y, int64_t rows, int64_t d,
                            float eps, hipStream_t s) {
  const int nchunk = (int)(d / Chunk<EB>::E);
  const float inv_d = 1.0f / (float)d;
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(256);
  const uint4* xx = (const uint4*)x;
  const uint4* gg = (const uint4*)g;
  uint4* yy = (uint4*)y;
  // a few rows: latency-bound, gain fetched with x; many rows: the gain
  // (L2-resident) is fetched after the reduction, keeping registers free
  const bool few = rows <= FFN_RMS_PREG_ROWS;
#define FFN_RMS_CACHED(C)                                                                              \
  if (few)                                                                                           \
    FFN_DISPATCH((rmsnorm_cached<EB, C, true>), grid, block, 0, s, xx, gg, yy, rows, nchunk, inv_d, eps); \
  else                                                                                               \
    FFN_DISPATCH((rmsnorm_cached<EB, C, false>), grid, block, 0, s, xx, gg, yy, rows, nchunk, inv_d, eps);
  if (nchunk <= 64 * 2) {
    FFN_RMS_CACHED(2)
  } else if (nchunk <= 64 * 4) {
    FFN_RMS_CACHED(4)
  } else if (nchunk <= 64 * 8) {
    FFN_RMS_CACHED(8)
  } else if (nchunk <= 64 * 16) {
    FFN_RMS_CACHED(16)
  } else
    FFN_DISPATCH((rmsnorm_stream<EB>), grid, block, 0, s, xx, gg, yy, rows, nchunk, inv_d, eps);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int elem_bytes, const void* x, const void* g, void* y, int64_t rows,
                          int64_t d, float eps, hipStream_t s) {
  return elem_bytes == 2 ? launch_eb<2>(x, g, y, rows, d, eps, s)
                         : launch_eb<4>(x, g, y, rows, d, eps, s);
}

}  // namespace ffn
