// Decode-regime projections (few tokens): weight streaming on bf16 MFMA.
//
//   gate/up : h[m,j] = silu(sum_k Wg[j,k] n[m,k]) * (sum_k Wu[j,k] n[m,k])
//   down    : y[m,i] = x[m,i] + sum_j Wd[i,j] h[m,j]
// (gate and up projections of the SwiGLU MLP: "Unfusing a Kernel Made It
// 1.63x Faster", Finding 1; FFN-down: "Megakernels on Mac", "Projection
// shape changes the achieved rate"; the FFN weights are the bulk of a decode
// pass's payload: "Megakernels on Mac", "The 27.65 ms estimate".)
//
// With M <= 64 tokens every weight is used M times, far below the chip's
// flop:byte ridge, so the kernels are bound by streaming W from HBM once.
// gfx950 mapping: v_mfma_f32_16x16x32_bf16 with the A operand = 16 weight
// rows x 32 k and the B operand = 32 k x 16 tokens (tokens past M are zero),
// so the matrix core does the multiply-adds and the VALU stays free for
// address and epilogue work.  Lane l holds A[l%16][8(l/16)..+8] and
// B[8(l/16)..+8][l%16]; the result lane l holds D[4(l/16)+e][l%16], i.e. four
// consecutive weight rows of one token, which the epilogue stores as one
// 8-byte write.  Each workgroup owns 16 weight rows; its W waves split K
// into contiguous slices, each lane keeping 8 16-byte weight loads in flight;
// the W partial tiles are summed in a fixed order through LDS (deterministic,
// no atomics).  Weights are read straight into VGPRs: staging a streamed
// weight through threadgroup memory lost every pair in "Megakernels on Mac",
// "Threadgroup staging", and nothing here is re-read.
#include "common.h"
#include "launch.h"

namespace ffn {

// NMAT = 2: gate+up with the silu epilogue; NMAT = 1: down with residual.
// MT = token tiles of 16 (M <= 16*MT). WAVES = K-split waves per workgroup.
template <int NMAT, int MT, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void decode_proj(
    const uint16_t* __restrict__ act,  // [M, K]
    const uint16_t* __restrict__ w0,   // [N, K]
    const uint16_t* __restrict__ w1,   // [N, K] (NMAT == 2)
    const uint16_t* __restrict__ resid,  // [M, N] (NMAT == 1)
    uint16_t* __restrict__ out,        // [M, N]
    int M, int K, int N) {
  constexpr int U = 8 / NMAT;  // 16-byte weight loads in flight per matrix per lane
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int j0 = blockIdx.x * 16;
  const int jrow = min(j0 + r, N - 1);  // clamped: rows past N load row N-1, never stored
  const int K8 = K >> 3;                // 16-byte chunks per row
  const int nsteps = K8 >> 2;           // full 32-wide k steps

  const uint4* p0 = reinterpret_cast<const uint4*>(w0) + (size_t)jrow * K8;
  const uint4* p1 = reinterpret_cast<const uint4*>(NMAT == 2 ? w1 : w0) + (size_t)jrow * K8;
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

  // contiguous K slice of this wave, in 32-wide steps
  const int sb = (int)(((long)nsteps * wave) / WAVES);
  const int se = (int)(((long)nsteps * (wave + 1)) / WAVES);
  int s = sb;
  for (; s + U <= se; s += U) {
    uint4 a0[U], a1[U], b[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = (s + u) * 4 + q;
      a0[u] = ld_nt(p0 + c);
      if (NMAT == 2) a1[u] = ld_nt(p1 + c);
#pragma unroll
      for (int t = 0; t < MT; ++t) b[u][t] = pa[t][c];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const uint4 bb = keep_or_zero(av[t], b[u][t]);
        acc0[t] = mfma16(a0[u], bb, acc0[t]);
        if (NMAT == 2) acc1[t] = mfma16(a1[u], bb, acc1[t]);
      }
    }
  }
  for (; s < se; ++s) {
    const int c = s * 4 + q;
    const uint4 a0 = p0[c];
    const uint4 a1 = p1[c];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const uint4 bb = keep_or_zero(av[t], pa[t][c]);
      acc0[t] = mfma16(a0, bb, acc0[t]);
      if (NMAT == 2) acc1[t] = mfma16(a1, bb, acc1[t]);
    }
  }
  // ragged K (K % 32 != 0, K % 8 == 0): one masked step on the last wave
  if (wave == WAVES - 1 && (K8 & 3)) {
    const int c = nsteps * 4 + q;
    const bool kin = c < K8;
    const int cc = kin ? c : K8 - 1;
    const uint4 a0 = keep_or_zero(kin, p0[cc]);
    const uint4 a1 = keep_or_zero(kin, p1[cc]);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const uint4 bb = keep_or_zero(av[t] && kin, pa[t][cc]);
      acc0[t] = mfma16(a0, bb, acc0[t]);
      if (NMAT == 2) acc1[t] = mfma16(a1, bb, acc1[t]);
    }
  }

  // fixed-order cross-wave sum through LDS: red[w][t][mat][e][lane]
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
  // wave w finishes token tiles t = w, w + WAVES, ...
  for (int t = wave; t < MT; t += WAVES) {
    const int tok = t * 16 + r;
    const int col = j0 + 4 * q;  // four consecutive output columns col..col+3
    float v0[4], v1[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        s0 += red[w][t][0][e][lane];
        if (NMAT == 2) s1 += red[w][t][NMAT - 1][e][lane];
      }
      v0[e] = s0;
      v1[e] = s1;
    }
    if (tok < M && col < N) {
      uint2 o;
      const size_t off = (size_t)tok * N + col;
      if (NMAT == 2) {
        o.x = pack_bf16x2(silu_mul(v0[0], v1[0]), silu_mul(v0[1], v1[1]));
        o.y = pack_bf16x2(silu_mul(v0[2], v1[2]), silu_mul(v0[3], v1[3]));
      } else {
        const uint2 xr = *reinterpret_cast<const uint2*>(resid + off);
        o.x = pack_bf16x2(bf2f(xr.x & 0xFFFFu) + v0[0], bf2f(xr.x >> 16) + v0[1]);
        o.y = pack_bf16x2(bf2f(xr.y & 0xFFFFu) + v0[2], bf2f(xr.y >> 16) + v0[3]);
      }
      *reinterpret_cast<uint2*>(out + off) = o;
    }
  }
}

int decode_max_tokens() { return 64; }

template <int NMAT, int WAVES>
static hipError_t launch_mt(const void* act, const void* w0, const void* w1, const void* resid,
                            void* out, int M, int K, int N, hipStream_t s) {
  const dim3 grid((unsigned)((N + 15) / 16)), block(WAVES * 64);
  const uint16_t* a = (const uint16_t*)act;
  const uint16_t* p0 = (const uint16_t*)w0;
  const uint16_t* p1 = (const uint16_t*)w1;
  const uint16_t* rr = (const uint16_t*)resid;
  uint16_t* o = (uint16_t*)out;
  if (M <= 16)
    hipLaunchKernelGGL((decode_proj<NMAT, 1, WAVES>), grid, block, 0, s, a, p0, p1, rr, o, M, K, N);
  else if (M <= 32)
    hipLaunchKernelGGL((decode_proj<NMAT, 2, WAVES>), grid, block, 0, s, a, p0, p1, rr, o, M, K, N);
  else
    hipLaunchKernelGGL((decode_proj<NMAT, 4, WAVES>), grid, block, 0, s, a, p0, p1, rr, o, M, K, N);
  return hipGetLastError();
}

hipError_t launch_decode_gateup(const void* n, const void* wg, const void* wu, void* h, int M,
                                int d, int f, hipStream_t s) {
  return launch_mt<2, 4>(n, wg, wu, nullptr, h, M, d, f, s);
}

hipError_t launch_decode_down(const void* h, const void* wd, const void* x, void* y, int M,
                              int d, int f, hipStream_t s) {
  return launch_mt<1, 8>(h, wd, nullptr, x, y, M, f, d, s);
}

}  // namespace ffn
