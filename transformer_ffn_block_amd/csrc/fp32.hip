// fp32 path of the block (all arithmetic in fp32), for small models and
// for checking the bf16 path's roundings.  Plain SIMT tiles: it is a
// correctness path, not a throughput path.
//
//   STORE    : C[m][n] = sum_k A[m][k] W0[n][k]
//   SWIGLU   : C[m][n] = silu(sum_k A W0) * (sum_k A W1)     (gate/up, fused)
//   RESIDUAL : C[m][n] = R[m][n] + sum_k A[m][k] W0[n][k]   (down + residual)
// (SwiGLU activation in fp32: "When to hand-write a GPU kernel on Apple
// Silicon", Rung 1; gate/up: "Unfusing a Kernel Made It 1.63x Faster",
// Finding 1; FFN-down: "Megakernels on Mac".)
#include "common.h"
#include "launch.h"

namespace ffn {

constexpr int FT = 64;   // output tile 64 x 64
constexpr int FKT = 16;  // k per LDS stage

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32(const float* __restrict__ A,
                                                const float* __restrict__ W0,
                                                const float* __restrict__ W1,
                                                const float* __restrict__ R,
                                                float* __restrict__ C, int M, int N, int K) {
  constexpr int NW = EPI == F32_SWIGLU ? 2 : 1;
  __shared__ float As[FKT][FT + 1];
  __shared__ float Ws[NW][FKT][FT + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * FT, n0 = blockIdx.x * FT;
  float acc[NW][4][4] = {};
  for (int k0 = 0; k0 < K; k0 += FKT) {
    for (int i = threadIdx.x; i < FT * FKT; i += 256) {
      const int r = i / FKT, kk = i % FKT;
      const int m = m0 + r, n = n0 + r, k = k0 + kk;
      As[kk][r] = (m < M && k < K) ? A[(size_t)m * K + k] : 0.f;
      Ws[0][kk][r] = (n < N && k < K) ? W0[(size_t)n * K + k] : 0.f;
      if (NW == 2) Ws[NW - 1][kk][r] = (n < N && k < K) ? W1[(size_t)n * K + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FKT; ++kk) {
      float a[4], w[NW][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int v = 0; v < NW; ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j) w[v][j] = Ws[v][kk][tx * 4 + j];
#pragma unroll
      for (int v = 0; v < NW; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[v][i][j] = __builtin_fmaf(a[i], w[v][j], acc[v][i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      float v = acc[0][i][j];
      if (EPI == F32_SWIGLU) v = silu_mul(v, acc[NW - 1][i][j]);
      if (EPI == F32_RESIDUAL) v += R[(size_t)m * N + n];
      C[(size_t)m * N + n] = v;
    }
  }
}

hipError_t launch_gemm_f32(int epi, const float* a, const float* w0, const float* w1,
                           const float* resid, float* c, int M, int N, int K, hipStream_t s) {
  const dim3 grid((unsigned)((N + FT - 1) / FT), (unsigned)((M + FT - 1) / FT)), block(256);
  if (epi == F32_SWIGLU)
    FFN_DISPATCH(gemm_f32<F32_SWIGLU>, grid, block, 0, s, a, w0, w1, resid, c, M, N, K);
  else if (epi == F32_RESIDUAL)
    FFN_DISPATCH(gemm_f32<F32_RESIDUAL>, grid, block, 0, s, a, w0, w1, resid, c, M, N, K);
  else
    FFN_DISPATCH(gemm_f32<F32_STORE>, grid, block, 0, s, a, w0, w1, resid, c, M, N, K);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void swiglu_f32(const float* __restrict__ G,
                                                  const float* __restrict__ U,
                                                  float* __restrict__ h, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * 256)
    h[i] = silu_mul(G[i], U[i]);
}

hipError_t launch_swiglu_f32(const float* G, const float* U, float* h, int64_t count,
                             hipStream_t s) {
  int64_t blocks = (count + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  FFN_DISPATCH(swiglu_f32, dim3((unsigned)blocks), dim3(256), 0, s, G, U, h, count);
  return hipGetLastError();
}

}  // namespace ffn
