// Q8_0 weight-streaming projections with in-register dequantisation.
//
// A Q8_0 weight w[j,k] = q[j,k] * s[j, k/32]: 32 int8 quants along the
// reduction axis share one fp16 scale (the format named in "Unfusing a
// Kernel Made It 1.63x Faster", Finding 2).  Activations stay bf16.
//
//   gate/up : h[m,j] = silu(sum_k Wg[j,k] n[m,k]) * (sum_k Wu[j,k] n[m,k])
//   down    : y[m,i] = x[m,i] + sum_j Wd[i,j] h[m,j]
//
// gfx950 mapping.  Because a block of 32 quants is exactly one K step of
// v_mfma_f32_16x16x32_bf16, the scale factors out of the block's dot product:
//   sum_{k in b} q[j,k] s[j,b] n[m,k] = s[j,b] * sum_{k in b} q[j,k] n[m,k].
// The quants themselves are exact in bf16 (|q| <= 128 needs 8 significant
// bits), so the MFMA runs on the raw integers with a zero accumulator and the
// lane then adds s[j,b] * partial in fp32: the dequantisation adds no
// rounding at all.  Operands: A = 16 tokens x 32 k (bf16 activations), B =
// 32 k x 16 weight rows (converted quants); lane l's result is D[4(l/16)+e][l%16]
// = 4 tokens of weight row l%16, the same row whose quants and scale the
// lane loaded, so no cross-lane exchange is needed.  Quants are streamed
// straight into VGPRs (LDS staging of streamed quantised weights lost every
// pair in "Megakernels on Mac", "Threadgroup staging").
#include "common.h"
#include "launch.h"

namespace ffn {

// 8 int8 quants -> 8 bf16 (exact)
__device__ __forceinline__ uint4 q8x8_to_bf16(uint2 v) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = (float)(((int)(v.x << (24 - 8 * i))) >> 24);
    f[4 + i] = (float)(((int)(v.y << (24 - 8 * i))) >> 24);
  }
  return pack8(f);
}

__device__ __forceinline__ float f16bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

template <int NMAT, int MT, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void q8_proj(
    const uint16_t* __restrict__ act,                      // [M, K] bf16
    const int8_t* __restrict__ q0, const uint16_t* __restrict__ s0,  // [N, K], [N, K/32]
    const int8_t* __restrict__ q1, const uint16_t* __restrict__ s1,
    const uint16_t* __restrict__ resid,                    // [M, N] (NMAT == 1)
    uint16_t* __restrict__ out,                            // [M, N]
    int M, int K, int N) {
  constexpr int U = 8;  // blocks per unrolled step
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int j0 = blockIdx.x * 16;
  const int jrow = min(j0 + r, N - 1);
  const int nb = K >> 5;  // blocks per row
  const int K8 = K >> 3;

  const uint2* pq0 = reinterpret_cast<const uint2*>(q0 + (size_t)jrow * K);
  const uint2* pq1 = reinterpret_cast<const uint2*>((NMAT == 2 ? q1 : q0) + (size_t)jrow * K);
  const uint16_t* ps0 = s0 + (size_t)jrow * nb;
  const uint16_t* ps1 = (NMAT == 2 ? s1 : s0) + (size_t)jrow * nb;
  const uint4* pa[MT];
  bool av[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int tok = t * 16 + r;
    av[t] = tok < M;
    pa[t] = reinterpret_cast<const uint4*>(act) + (size_t)min(tok, M - 1) * K8;
  }
  f32x4 acc0[MT], acc1[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    acc0[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};

  const int bb = (int)(((long)nb * wave) / WAVES);
  const int be = (int)(((long)nb * (wave + 1)) / WAVES);
  auto step = [&](int b, uint2 w0v, uint2 w1v, uint16_t s0v, uint16_t s1v, const uint4* av4) {
    const uint4 B0 = q8x8_to_bf16(w0v);
    const float sc0 = f16bits_to_f32(s0v);
    uint4 B1;
    float sc1 = 0.f;
    if (NMAT == 2) {
      B1 = q8x8_to_bf16(w1v);
      sc1 = f16bits_to_f32(s1v);
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const f32x4 p0 = mfma16(av4[t], B0, z4);
      acc0[t] += sc0 * p0;
      if (NMAT == 2) {
        const f32x4 p1 = mfma16(av4[t], B1, z4);
        acc1[t] += sc1 * p1;
      }
    }
    (void)b;
  };

  int b = bb;
  for (; b + U <= be; b += U) {
    uint2 w0v[U], w1v[U];
    uint16_t s0v[U], s1v[U];
    uint4 a[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c8 = (b + u) * 4 + q;  // 8-byte unit index within the row
      w0v[u] = ld_nt(pq0 + c8);
      s0v[u] = ps0[b + u];
      if (NMAT == 2) {
        w1v[u] = ld_nt(pq1 + c8);
        s1v[u] = ps1[b + u];
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const uint4 v = pa[t][c8];
        a[u][t] = keep_or_zero(av[t], v);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) step(b + u, w0v[u], NMAT == 2 ? w1v[u] : w0v[u], s0v[u],
                                     NMAT == 2 ? s1v[u] : s0v[u], a[u]);
  }
  for (; b < be; ++b) {
    const int c8 = b * 4 + q;
    uint4 a[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const uint4 v = pa[t][c8];
      a[t] = keep_or_zero(av[t], v);
    }
    step(b, pq0[c8], pq1[c8], ps0[b], ps1[b], a);
  }

  __shared__ float red[WAVES][MT][NMAT][4][64];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      red[wave][t][0][e][lane] = acc0[t][e];
      if (NMAT == 2) red[wave][t][NMAT - 1][e][lane] = acc1[t][e];
    }
  }
  __syncthreads();
  for (int t = wave; t < MT; t += WAVES) {
    const int col = j0 + r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v0 = 0.f, v1 = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        v0 += red[w][t][0][e][lane];
        if (NMAT == 2) v1 += red[w][t][NMAT - 1][e][lane];
      }
      const int tok = t * 16 + 4 * q + e;
      if (tok < M && col < N) {
        const size_t off = (size_t)tok * N + col;
        float o;
        if (NMAT == 2)
          o = silu_mul(v0, v1);
        else
          o = bf2f(resid[off]) + v0;
        out[off] = f2bf(o);
      }
    }
  }
}

int q8_max_tokens() { return 64; }

template <int NMAT, int WAVES>
static hipError_t launch_q8(const void* act, const int8_t* q0, const uint16_t* s0,
                            const int8_t* q1, const uint16_t* s1, const void* resid, void* out,
                            int M, int K, int N, hipStream_t s) {
  const dim3 grid((unsigned)((N + 15) / 16)), block(WAVES * 64);
  const uint16_t* a = (const uint16_t*)act;
  const uint16_t* rr = (const uint16_t*)resid;
  uint16_t* o = (uint16_t*)out;
  if (M <= 16)
    hipLaunchKernelGGL((q8_proj<NMAT, 1, WAVES>), grid, block, 0, s, a, q0, s0, q1, s1, rr, o, M, K, N);
  else if (M <= 32)
    hipLaunchKernelGGL((q8_proj<NMAT, 2, WAVES>), grid, block, 0, s, a, q0, s0, q1, s1, rr, o, M, K, N);
  else
    hipLaunchKernelGGL((q8_proj<NMAT, 4, WAVES>), grid, block, 0, s, a, q0, s0, q1, s1, rr, o, M, K, N);
  return hipGetLastError();
}

hipError_t launch_q8_gateup(const void* n, const int8_t* qg, const uint16_t* sg,
                            const int8_t* qu, const uint16_t* su, void* h, int M, int d, int f,
                            hipStream_t s) {
  return launch_q8<2, 4>(n, qg, sg, qu, su, nullptr, h, M, d, f, s);
}

hipError_t launch_q8_down(const void* h, const int8_t* qd, const uint16_t* sd, const void* x,
                          void* y, int M, int d, int f, hipStream_t s) {
  return launch_q8<1, 8>(h, qd, sd, nullptr, nullptr, x, y, M, f, d, s);
}

}  // namespace ffn
