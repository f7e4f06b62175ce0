// Second pass of the split-K down projections: y = x + the fp32 partial sums
// of the K ranges, added in range order (deterministic; no atomics).  The
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

template <int S>
__global__ __launch_bounds__(256) void splitk_residual(const float4* __restrict__ part,
                                                       const uint4* __restrict__ x,
                                                       uint4* __restrict__ y, int groups,
                                                       size_t split_stride) {
  const int i = blockIdx.x * 256 + threadIdx.x;  // 8-output group
  if (i >= groups) return;
  const uint4 xv = x[i];
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
  y[i] = pack8(v);
}

template <int S>
static void splitk_go(const float* part, const void* x, void* y, int groups, size_t stride,
                      hipStream_t s) {
  const dim3 grid((unsigned)((groups + 255) / 256)), block(256);
  FFN_DISPATCH(splitk_residual<S>, grid, block, 0, s, (const float4*)part, (const uint4*)x,
               (uint4*)y, groups, stride);
}

hipError_t launch_splitk_residual(const float* part, int splits, const void* x, void* y, int M,
                                  int N, hipStream_t s) {
  static_assert(kQuantMaxSplits == 8, "one instantiation per range count");
  const int groups = M * (N / 8);
  const size_t stride = (size_t)M * N / 4;
  switch (splits) {
    case 1: splitk_go<1>(part, x, y, groups, stride, s); break;
    case 2: splitk_go<2>(part, x, y, groups, stride, s); break;
    case 3: splitk_go<3>(part, x, y, groups, stride, s); break;
    case 4: splitk_go<4>(part, x, y, groups, stride, s); break;
    case 5: splitk_go<5>(part, x, y, groups, stride, s); break;
    case 6: splitk_go<6>(part, x, y, groups, stride, s); break;
    case 7: splitk_go<7>(part, x, y, groups, stride, s); break;
    case 8: splitk_go<8>(part, x, y, groups, stride, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ffn
