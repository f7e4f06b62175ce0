// Second passes of the split-K projections: y = x + the fp32 partial sums
// of the K ranges of a down projection, or h = silu(G) * U from those of a
// fused gate/up GEMM, added in range order (deterministic; no atomics).  The
// deeper K split of the FFN-down projection is the experiment of "Megakernels
// on Mac", "Projection shape changes the achieved rate"; here the split
// spreads the few hundred 16-row output tiles of a decode down projection
// evenly over all compute units.
//
// One thread per 8 consecutive outputs of a token row: 16-byte loads of x and
// stores of y, 32-byte loads of each partial.  The range count is a template
// argument, so every load of a thread (x and all S partials) is issued before
// the first add: one memory round trip per thread instead of one per range.
#include "common.h"
#include "launch.h"

namespace ffn {

// x and y rows are ld8 groups of 8 elements apart (a column block of a wider
// output when ld8 > n8, the block's width in groups)
template <int S>
__global__ __launch_bounds__(256) void splitk_residual(const float4* __restrict__ part,
                                                       const uint4* __restrict__ x,
                                                       uint4* __restrict__ y, int groups,
                                                       size_t split_stride, int n8, int ld8) {
  const int i = blockIdx.x * 256 + threadIdx.x;  // 8-output group
  if (i >= groups) return;
  const size_t io = ld8 == n8 ? (size_t)i : (size_t)(i / n8) * ld8 + i % n8;
  const uint4 xv = x[io];
  float4 a[S], b[S];
#pragma unroll
  for (int z = 0; z < S; ++z) {
    const float4* p = part + z * split_stride + 2 * (size_t)i;
    a[z] = p[0];
    b[z] = p[1];
  }
  // ranges added in order from zero, then x
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int z = 0; z < S; ++z) {
    v[0] += a[z].x; v[1] += a[z].y; v[2] += a[z].z; v[3] += a[z].w;
    v[4] += b[z].x; v[5] += b[z].y; v[6] += b[z].z; v[7] += b[z].w;
  }
  float xf[8];
  unpack8(xv, xf);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = xf[e] + v[e];
  y[io] = pack8(v);
}

template <int S>
static void splitk_go(const float* part, const void* x, void* y, int groups, size_t stride,
                      int n8, int ld8, hipStream_t s) {
  const dim3 grid((unsigned)((groups + 255) / 256)), block(256);
  FFN_DISPATCH(splitk_residual<S>, grid, block, 0, s, (const float4*)part, (const uint4*)x,
               (uint4*)y, groups, stride, n8, ld8);
}

// h = silu(sum_z G_z) * sum_z U_z for the split-K fused gate/up GEMM: gate
// planes 0..S-1, up planes S..2S-1 of [M, f] each; one thread per 8 outputs.
template <int S>
__global__ __launch_bounds__(256) void splitk_swiglu(const float4* __restrict__ part,
                                                     uint4* __restrict__ h, int groups,
                                                     size_t plane, int n8, int ld8) {
  const int i = blockIdx.x * 256 + threadIdx.x;  // 8-output group
  if (i >= groups) return;
  float4 ga[S], gb[S], ua[S], ub[S];
#pragma unroll
  for (int z = 0; z < S; ++z) {
    const float4* pg = part + z * plane + 2 * (size_t)i;
    const float4* pu = part + (S + z) * plane + 2 * (size_t)i;
    ga[z] = pg[0];
    gb[z] = pg[1];
    ua[z] = pu[0];
    ub[z] = pu[1];
  }
  float g[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, u[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int z = 0; z < S; ++z) {
    g[0] += ga[z].x; g[1] += ga[z].y; g[2] += ga[z].z; g[3] += ga[z].w;
    g[4] += gb[z].x; g[5] += gb[z].y; g[6] += gb[z].z; g[7] += gb[z].w;
    u[0] += ua[z].x; u[1] += ua[z].y; u[2] += ua[z].z; u[3] += ua[z].w;
    u[4] += ub[z].x; u[5] += ub[z].y; u[6] += ub[z].z; u[7] += ub[z].w;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) g[e] = silu_mul(g[e], u[e]);
  h[ld8 == n8 ? (size_t)i : (size_t)(i / n8) * ld8 + i % n8] = pack8(g);
}

template <int S>
static void swiglu_go(const float* part, void* h, int groups, size_t plane, int n8, int ld8,
                      hipStream_t s) {
  const dim3 grid((unsigned)((groups + 255) / 256)), block(256);
  FFN_DISPATCH(splitk_swiglu<S>, grid, block, 0, s, (const float4*)part, (uint4*)h, groups, plane,
               n8, ld8);
}

// one instantiation per range count, 1..kPrefillMaxSplits
template <template <int> class F, class... A>
static bool by_splits(int splits, A... args) {
  static_assert(kPrefillMaxSplits == 16 && kQuantMaxSplits <= kPrefillMaxSplits, "");
  switch (splits) {
    case 1: F<1>::go(args...); return true;
    case 2: F<2>::go(args...); return true;
    case 3: F<3>::go(args...); return true;
    case 4: F<4>::go(args...); return true;
    case 5: F<5>::go(args...); return true;
    case 6: F<6>::go(args...); return true;
    case 7: F<7>::go(args...); return true;
    case 8: F<8>::go(args...); return true;
    case 9: F<9>::go(args...); return true;
    case 10: F<10>::go(args...); return true;
    case 11: F<11>::go(args...); return true;
    case 12: F<12>::go(args...); return true;
    case 13: F<13>::go(args...); return true;
    case 14: F<14>::go(args...); return true;
    case 15: F<15>::go(args...); return true;
    case 16: F<16>::go(args...); return true;
  }
  return false;
}
template <int S>
struct ResidualGo {
  static void go(const float* part, const void* x, void* y, int groups, size_t stride, int n8,
                 int ld8, hipStream_t s) {
    splitk_go<S>(part, x, y, groups, stride, n8, ld8, s);
  }
};
template <int S>
struct SwigluGo {
  static void go(const float* part, void* h, int groups, size_t plane, int n8, int ld8,
                 hipStream_t s) {
    swiglu_go<S>(part, h, groups, plane, n8, ld8, s);
  }
};

hipError_t launch_splitk_residual(const float* part, int splits, const void* x, void* y, int M,
                                  int N, hipStream_t s, int ldo) {
  if (ldo <= 0) ldo = N;
  const int groups = M * (N / 8);
  const size_t stride = (size_t)M * N / 4;
  if (!by_splits<ResidualGo>(splits, part, x, y, groups, stride, N / 8, ldo / 8, s))
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_splitk_swiglu(const float* part, int splits, void* h, int M, int f,
                                hipStream_t s, int ldo) {
  if (ldo <= 0) ldo = f;
  const int groups = M * (f / 8);
  const size_t plane = (size_t)M * f / 4;
  if (!by_splits<SwigluGo>(splits, part, h, groups, plane, f / 8, ldo / 8, s))
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ffn
