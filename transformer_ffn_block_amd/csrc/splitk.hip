// Second pass of the split-K down projections: y = x + the fp32 partial sums
// of the K ranges, added in range order (deterministic; no atomics).  The
// deeper K split of the FFN-down projection is the experiment of "Megakernels
// on Mac", "Projection shape changes the achieved rate"; here the split
// spreads the few hundred 16-row output tiles of a decode down projection
// evenly over all compute units.
//
// One thread per 8 consecutive outputs of a token row: 16-byte loads of x and
// stores of y, 32-byte loads of each partial.
#include "common.h"
#include "launch.h"

namespace ffn {

__global__ __launch_bounds__(256) void splitk_residual(const float4* __restrict__ part, int splits,
                                                       const uint4* __restrict__ x,
                                                       uint4* __restrict__ y, int groups,
                                                       size_t split_stride) {
  const int i = blockIdx.x * 256 + threadIdx.x;  // 8-output group
  if (i >= groups) return;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int z = 0; z < splits; ++z) {
    const float4* p = part + z * split_stride + 2 * (size_t)i;
    const float4 a = p[0], b = p[1];
    v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w;
    v[4] += b.x; v[5] += b.y; v[6] += b.z; v[7] += b.w;
  }
  float xf[8];
  unpack8(x[i], xf);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = xf[e] + v[e];
  y[i] = pack8(v);
}

hipError_t launch_splitk_residual(const float* part, int splits, const void* x, void* y, int M,
                                  int N, hipStream_t s) {
  const int groups = M * (N / 8);
  const dim3 grid((unsigned)((groups + 255) / 256)), block(256);
  FFN_DISPATCH(splitk_residual, grid, block, 0, s, (const float4*)part, splits,
                     (const uint4*)x, (uint4*)y, groups, (size_t)M * N / 4);
  return hipGetLastError();
}

}  // namespace ffn
