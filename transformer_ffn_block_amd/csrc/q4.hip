// Q4_0 weight-streaming projections with in-register dequantisation.
//
// A Q4_0 block holds 32 weights along the reduction axis as one fp16 scale
// and 16 bytes whose low and high nibbles carry different weights (the
// 18-byte blocks of "Unfusing a Kernel Made It 1.63x Faster", "The finding
// that keeps us honest about microbenchmarks").  Taken here: byte i holds
// weight i (low nibble) and weight i + 16 (high nibble); w = (nibble - 8) * s.
// The library stores the nibble bytes and the scales in separate arrays
// (the repacked layout: a row's bytes are contiguous, so a 256-k stage of a
// row is 128 consecutive bytes).  Activations stay bf16.
//
//   gate/up : h[m,j] = silu(sum_k Wg[j,k] n[m,k]) * (sum_k Wu[j,k] n[m,k])
//   down    : y[m,i] = x[m,i] + sum_j Wd[i,j] h[m,j]
//
// gfx950 mapping (as the Q8_0 kernels).  A block is one K step of
// v_mfma_f32_16x16x32_bf16, so the scale factors out of the block's dot
// product.  Lane (r, q) feeds weights 8q..8q+7 of a block of row r: the low
// nibbles (q < 2) or high nibbles (q >= 2) of bytes 8(q & 1) .. 8(q & 1) + 7.
// Converting nibbles one by one through integer-to-float instructions costs
// about three VALU operations per weight, which made the kernel VALU-bound.
// Instead the lane masks its nibbles into the low four bits of each byte and
// byte-permutes them under the constant 0x43: the bf16 pattern 0x430n is
// exactly 128 + n (bf16 128.0 with n in the last mantissa bits), four
// operations per four weights.  The offset goes into the MFMA's initial
// accumulator: C = sum_k a_k * (-136), one extra MFMA per block shared by the
// gate and up matrices, so the MFMA returns sum_k a_k (n_k - 8).  Every
// product is exact in fp32; the fp32 sums run ~30x larger than the result,
// costing ~5 of fp32's 24 bits (relative error ~2^-19 of the partial, far
// below the bf16 rounding of the activations).
//
// Streaming: a workgroup owns 16 weight rows (per matrix); its waves split K
// into 256-k stages (128 bytes per row).  Each matrix's stage is 16 rows x 8
// chunks of 16 bytes in a per-wave 2 KiB LDS buffer, fetched by two
// instructions of 8 rows x 128 B; chunk c of row R sits at position
// (c + R/2) & 7 of the row, so the 8-byte fragment reads of a block (16 rows
// x two halves) hit all 64 banks once.  Prefetches past a wave's K slice use
// an out-of-range buffer offset and read nothing.  Scales, activations, the
// software pipeline and the fixed-order cross-wave reduction are those of
// the Q8_0 kernels.
//
// For narrow projections with up to 8 tokens the norm is folded into the
// gate/up kernel (FOLD, as for Q8_0): the block then skips the norm launch,
// which at f = 2176 takes the block from 23.5 to 21.0 us; at f = 17408 the
// fold's staging work (and two more VGPRs than the three-waves-per-SIMD
// budget) made the block slower (58.1 vs 55.5 us), so there n comes from the
// norm kernel.
//
// Split-K down projection.  With d = 5120 outputs the down projection has
// only 320 row tiles for 256 compute units: a quarter of the units get two
// tiles and set the kernel's length.  The K axis is therefore split into a
// few contiguous ranges (enough for ~1024 workgroups); each workgroup writes
// its fp32 partial tile and a second kernel adds the ranges in order, plus
// the residual (deterministic, no atomics).  Measured per-wave timelines
// show these kernels limited by the latency of each stage's dependent chain
// (loads, LDS staging, conversion, MFMA, scaling) at one to four waves per
// SIMD rather than by HBM: with every global load removed a 5120 x 17408
// projection still takes ~14 us.  A dword-interleaved nibble layout that
// skipped the LDS stage (16 rows x 64 B per load) was slower, as were two
// row tiles per wave, more or fewer waves per workgroup and rotated stage
// orders.
#include "common.h"
#include "launch.h"

#ifndef FFN_Q4_GU_WAVES
#define FFN_Q4_GU_WAVES 4
#endif
// The 8-token gate/up kernel (norm not folded): waves per SIMD it is
// register-allocated for (three: 165 VGPRs, no AGPRs, no spills), and the
// 32-nibble blocks whose MFMAs are issued before their scale FMAs.
#ifndef FFN_Q4_DEEP_DN8
#define FFN_Q4_DEEP_DN8 0
#endif
#ifndef FFN_Q4_GU8_WPE
#define FFN_Q4_GU8_WPE 3
#endif
// 17..32 tokens with both token tiles staged through LDS in two-wave
// workgroups, as for Q8_0 (0: activations read straight from L2).
// Interleaved A/B, d = 5120, f = 17408: block 106 / 122 / 139 -> 92 / 96 /
// 100 us at 17 / 24 / 32 tokens, 197 / 270 -> 160 / 194 us at 48 / 64;
// d = 4096, f = 11008 at 32 tokens 78 -> 52 us.
#ifndef FFN_Q4_STAGE32
#define FFN_Q4_STAGE32 1
#endif
#ifndef FFN_Q4_S32_WAVES
#define FFN_Q4_S32_WAVES 2
#endif
#ifndef FFN_Q4_S32_GB
#define FFN_Q4_S32_GB 1
#endif
#ifndef FFN_Q4_GU8_GB
#define FFN_Q4_GU8_GB 4
#endif
#ifndef FFN_Q4_DN_WAVES
#define FFN_Q4_DN_WAVES 4
#endif
#ifndef FFN_Q4_DN_SPLIT_TARGET
#define FFN_Q4_DN_SPLIT_TARGET 1024
#endif
// Down projections of up to FFN_Q4_DN_WHOLE tokens whose 16-row tiles fill
// whole rounds of the compute units (d = 4096 on 256 CUs) run unsplit.
// Interleaved A/B, d = 4096, f = 11008: block 29.5 / 33.6 / 39.8 -> 28.2 /
// 31.1 / 37.9 us at 1 / 8 / 16 tokens; at 32 tokens the split stays faster
// (50.6 -> 57.3 us unsplit).
#ifndef FFN_Q4_DN_WHOLE
#define FFN_Q4_DN_WHOLE 16
#endif

namespace ffn {

// 8 nibbles of bytes lo (0..3), hi (4..7), the low ones (shift 0) or the
// high ones (shift 4) -> 8 bf16 of value 128 + nibble, in byte order.
// v_perm_b32(s0, s1, sel): result byte i = byte sel_i of the 8-byte value
// s0:s1 (selectors 0..3 pick s1, 4..7 pick s0).
__device__ __forceinline__ uint4 q4x8_to_bf16_biased(uint32_t lo, uint32_t hi, uint32_t shift) {
  constexpr uint32_t kExp = 0x43434343u;  // high byte of bf16 128.0
  const uint32_t a = (lo >> shift) & 0x0F0F0F0Fu;
  const uint32_t b = (hi >> shift) & 0x0F0F0F0Fu;
  uint4 o;
  o.x = __builtin_amdgcn_perm(kExp, a, 0x04010400u);  // {0x43, n1, 0x43, n0} -> 128+n0, 128+n1
  o.y = __builtin_amdgcn_perm(kExp, a, 0x04030402u);
  o.z = __builtin_amdgcn_perm(kExp, b, 0x04010400u);
  o.w = __builtin_amdgcn_perm(kExp, b, 0x04030402u);
  return o;
}

// 8 copies of bf16 -136.0 (0xC308): the MFMA B operand of the offset term
constexpr uint32_t kNegOffsetPair = 0xC308C308u;

__device__ __forceinline__ float q4_f16bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// PART: split-K pass (NMAT == 1): workgroup (tile, z) covers the z-th of
// gridDim.y contiguous ranges of stages and writes its fp32 partial sums to
// part[z][M][N] (no residual); a fixed-order reduce adds them up.
// FOLD (gate/up, up to 8 tokens): the RMSNorm is folded in, as in the Q8_0
// and bf16 decode kernels: act is x, the staged activations are multiplied
// by the gain while the sums of squares of x accumulate, and the epilogue
// scales both projections by r_m.
template <int NMAT, int MT, int WAVES, bool SALIGN, int ASTAGE, bool PART, bool FOLD>
__global__ __launch_bounds__(WAVES * 64)
__attribute__((amdgpu_waves_per_eu(NMAT == 2 && ASTAGE == 8 && !FOLD ? FFN_Q4_GU8_WPE : 1)))
void q4_stream(
    const uint16_t* __restrict__ act,     // [M, K] bf16: x (FOLD), n or h
    const uint16_t* __restrict__ gain,    // [K] (FOLD)
    const uint8_t* __restrict__ q0, const uint16_t* __restrict__ s0,  // [N, K/2], [N, K/32]
    const uint8_t* __restrict__ q1, const uint16_t* __restrict__ s1,
    const uint16_t* __restrict__ resid,   // [M, N] (NMAT == 1, !PART)
    uint16_t* __restrict__ out,           // [M, N] (!PART)
    float* __restrict__ part,             // [gridDim.y, M, N] (PART)
    int M, int K, int N, float eps) {
  static_assert(!FOLD || (NMAT == 2 && !PART && ASTAGE == 8), "the norm folds into the 8-token gate/up kernel only");
  // SALIGN is only chosen when K % 256 == 0: every stage is then whole, so
  // the clamps and masks of a partial last stage compile away.  Measured
  // (interleaved A/B, bitwise identical): block 70.4 -> 66.4 us at 16
  // tokens and 146 -> 140 us at 32, but 55.4 -> 56.9 us at 8 (both 8-token
  // kernels ~2.5% slower: scheduling, same occupancy), so the 8-token
  // kernels keep the general form.
  constexpr bool KFULL = SALIGN && ASTAGE != 8;
  auto cl = [](int v, int hi) { return KFULL ? v : min(v, hi); };
  constexpr int SB = 8;        // 32-weight blocks per stage (256 k, 128 B per row)
  constexpr int NU = 2;        // nibble load instructions per matrix per stage (8 rows each)
  __shared__ uint4 wb[WAVES][NMAT][128];           // per-wave nibble stage (2 KiB per matrix)
  __shared__ float red[WAVES][MT][NMAT][4][64];
  __shared__ uint4 abuf[WAVES][ASTAGE ? ASTAGE * 32 : 1];  // per-wave activation stage [rows][32]
  __shared__ float ssq[FOLD ? WAVES : 1][8];  // per-wave partial sums of squares (FOLD)

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  // workgroup b of G (gridDim.x) owns output rows [b N / G, (b + 1) N / G),
  // at most 16; tile rows past row1 load nothing and are never stored
  const int j0 = (int)(((long)blockIdx.x * N) / gridDim.x);
  const int row1 = (int)(((long)(blockIdx.x + 1) * N) / gridDim.x);
  const int nb = K >> 5;                // blocks per row
  const int K32 = K >> 5;               // 16-byte nibble chunks per row (one per block)
  const int K8 = K >> 3;                // 16-byte activation chunks per row
  const int nst = (nb + SB - 1) / SB;
  const int zs = PART ? (int)(((long)nst * blockIdx.y) / gridDim.y) : 0;        // this split's stages
  const int ze = PART ? (int)(((long)nst * (blockIdx.y + 1)) / gridDim.y) : nst;
  const int sb = zs + (int)(((long)(ze - zs) * wave) / WAVES);
  const int se = zs + (int)(((long)(ze - zs) * (wave + 1)) / WAVES);

  // staged loads: instruction u covers rows 8u..8u+7; lane -> row 8u + lane/8,
  // LDS slot u*64 + lane, which holds chunk (lane%8 - row/2) & 7 of the row's
  // 128-byte stage segment; chunk c of row R therefore sits at slot
  // R*8 + ((c + R/2) & 7)
  __amdgpu_buffer_rsrc_t rq[NMAT];  // nibbles through buffer resources (< 2 GiB)
  rq[0] = make_rsrc(q0, (long)N * (K / 2));
  if (NMAT == 2) rq[NMAT - 1] = make_rsrc(q1, (long)N * (K / 2));
  unsigned gq[NU];  // byte offset of this lane's row in each instruction
  int cst[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int rr = 8 * u + (lane >> 3);
    const int row = j0 + rr;
    cst[u] = ((lane & 7) - (rr >> 1)) & 7;
    // kOutOfRange plus any in-row offset (< 2^31) stays past the resource
    gq[u] = row < row1 ? (unsigned)row * (unsigned)(K / 2) : kOutOfRange;
  }
  // this lane's weight row (MFMA B operand) and its scales
  const int jr = min(j0 + r, row1 - 1);  // scale row (rows past row1: a valid row's, cached)
  const uint16_t* ps[NMAT];
  ps[0] = s0 + (size_t)jr * nb;
  if (NMAT == 2) ps[NMAT - 1] = s1 + (size_t)jr * nb;
  // SALIGN: both matrices' scale rows at the same byte offset of their own
  // buffer resources
  __amdgpu_buffer_rsrc_t rs[NMAT];
  rs[0] = make_rsrc(s0, (long)N * nb * 2);
  if (NMAT == 2) rs[NMAT - 1] = make_rsrc(s1, (long)N * nb * 2);
  const unsigned srow = (unsigned)jr * (unsigned)nb * 2u;

  // direct activations: token t*16 + r; staged: instruction v covers token
  // rows 2v, 2v+1 (lane -> row 2v + lane/32, LDS slot v*64 + lane holding
  // chunk ((lane & 31) - row) & 31 of the row's 512-byte stage segment)
  constexpr int NA = ASTAGE ? ASTAGE / 2 : SB * MT;  // activation loads per batch
  // the gate/up kernels address staged rows and scale rows through buffer
  // resources with 32-bit offsets (fewer VGPRs); the down kernels keep plain
  // pointers (the freed registers raised their occupancy and measured slower)
  constexpr bool kBuf = NMAT == 2;
  // (32 staged rows: both kinds form the row offset at each load instead)
  constexpr bool kRow = ASTAGE >= 32;
  const uint4* pa[ASTAGE && (kBuf || kRow) ? 1 : (ASTAGE ? NA : MT)];
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(act, (long)M * K * 2);
  unsigned aro[ASTAGE && kBuf && !kRow ? NA : 1];
  if (ASTAGE && !kRow) {
#pragma unroll
    for (int v = 0; v < NA; ++v) {
      const int row = min(2 * v + (lane >> 5), M - 1);
      if (kBuf)
        aro[kBuf ? v : 0] = (unsigned)row * (unsigned)K8 * 16u;
      else
        pa[kBuf ? 0 : v] = reinterpret_cast<const uint4*>(act) + (size_t)row * K8;
    }
  } else if (!ASTAGE) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
      pa[t] = reinterpret_cast<const uint4*>(act) + (size_t)min(t * 16 + r, M - 1) * K8;
  }

  f32x4 acc[NMAT][MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  const uint4 negoff = make_uint4(kNegOffsetPair, kNegOffsetPair, kNegOffsetPair, kNegOffsetPair);
  const uint32_t nib_shift = (uint32_t)(q >> 1) * 4u;  // lanes q >= 2 take the high nibbles

  // FOLD: lane -> chunk lane & 31 of every row it stages (one gain chunk per
  // stage), written to slot v*64 + (lane/32)*32 + ((lane & 31) + row) & 31,
  // the same LDS layout; sums of squares of x per staged row in ss[v]
  const uint4* G4 = reinterpret_cast<const uint4*>(gain);
  float ss[FOLD ? NA : 1];
#pragma unroll
  for (int i = 0; i < (FOLD ? NA : 1); ++i) ss[i] = 0.f;
  auto fold = [&](const uint4& xa, const uint4& gv, float& s2) -> uint4 {
    float xf[8], gf[8];
    unpack8(xa, xf);
    unpack8(gv, gf);
    s2 = sumsq8(xa, s2);
#pragma unroll
    for (int e = 0; e < 8; ++e) xf[e] *= gf[e];
    return pack8(xf);
  };

  struct Batch {
    uint4 w[NMAT][NU];
    uint4 s[NMAT];  // SALIGN: the stage's 8 scales of row r; else .x = blocks 2q, 2q+1
    uint4 a[NA];
    uint4 g;        // the stage's gain chunk lane & 31 (FOLD)
  };
  // st < 0 marks a prefetch past the slice end: the nibble loads then read
  // nothing (out-of-range offset) and the small loads hit cache
  auto load_w = [&](Batch& B, int st_req) {
    const int st = st_req < 0 ? se - 1 : st_req;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int c = cl(st * 8 + cst[u], K32 - 1);
      const unsigned o = st_req < 0 ? kOutOfRange : gq[u] + (unsigned)c * 16u;
#pragma unroll
      for (int m = 0; m < NMAT; ++m) B.w[m][u] = buf_ld_nt(rq[m], o);
    }
  };
  auto load_s = [&](Batch& B, int st_req) {
    const int st = st_req < 0 ? se - 1 : st_req;
    if (SALIGN) {
      const int c = cl(st, (nb >> 3) - 1);
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
        B.s[m] = kBuf ? buf_ld16(rs[m], srow + (unsigned)c * 16u) : reinterpret_cast<const uint4*>(ps[m])[c];
    } else {
      const int b0 = cl(st * SB + 2 * q, nb - 1), b1 = cl(st * SB + 2 * q + 1, nb - 1);
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
        B.s[m].x = (uint32_t)ps[m][b0] | ((uint32_t)ps[m][b1] << 16);
    }
  };
  auto load_a = [&](Batch& B, int st_req) {
    const int st = st_req < 0 ? se - 1 : st_req;
    if (ASTAGE) {
#pragma unroll
      for (int v = 0; v < NA; ++v) {
        const int c = FOLD ? (lane & 31) : ((lane & 31) - (2 * v + (lane >> 5))) & 31;
        const int cc = cl(st * 32 + c, K8 - 1);
        if (kRow) {
          const unsigned ro = (unsigned)min(2 * v + (lane >> 5), M - 1) * (unsigned)K8 * 16u;
          B.a[v] = buf_ld16(ra, ro + (unsigned)cc * 16u);
        } else {
          B.a[v] = kBuf ? buf_ld16(ra, aro[kBuf && !kRow ? v : 0] + (unsigned)cc * 16u) : pa[kBuf ? 0 : v][cc];
        }
      }
      if (FOLD) B.g = G4[cl(st * 32 + (lane & 31), K8 - 1)];
    } else {
#pragma unroll
      for (int b = 0; b < SB; ++b) {
        const int c = cl(st * SB + b, nb - 1) * 4 + q;
#pragma unroll
        for (int t = 0; t < MT; ++t) B.a[b * MT + t] = pa[t][c];
      }
    }
  };
  auto load = [&](Batch& B, int st_req) {
    load_w(B, st_req);
    load_s(B, st_req);
    load_a(B, st_req);
  };
  // the nibbles (W) and the staged activations (B) of a stage go to LDS
  auto stage = [&](const Batch& W, const Batch& B, int st) {
    const bool ragged = !KFULL && (st + 1) * SB > nb;  // only a row's last stage can be partial
#pragma unroll
    for (int u = 0; u < NU; ++u) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        uint4 x = W.w[m][u];
        if (ragged) x = keep_or_zero(st * 8 + cst[u] < K32, x);
        wb[wave][m][u * 64 + lane] = x;
      }
    }
    if (ASTAGE) {
#pragma unroll
      for (int v = 0; v < NA; ++v) {
        const int row = 2 * v + (lane >> 5);
        uint4 a = B.a[v];
        if (ragged) {
          const int c = FOLD ? (lane & 31) : ((lane & 31) - row) & 31;
          a = keep_or_zero(st * 32 + c < K8, a);
        }
        if (FOLD) {
          a = fold(a, B.g, ss[FOLD ? v : 0]);
          abuf[wave][ASTAGE ? v * 64 + (lane & 32) + (((lane & 31) + row) & 31) : 0] = a;
        } else {
          abuf[wave][ASTAGE ? v * 64 + lane : 0] = a;
        }
      }
    }
  };
  // the MFMAs and scale FMAs of a stage: W supplies the scales, B the direct
  // activations (ASTAGE == 0)
  auto compute = [&](const Batch& W, const Batch& B, int st) {
    const bool ragged = !KFULL && (st + 1) * SB > nb;
    // the MFMAs of a group of blocks first, then their scale FMAs
    constexpr int GB = ASTAGE == 32 ? FFN_Q4_S32_GB : NMAT == 2 && ASTAGE == 8 && !FOLD ? FFN_Q4_GU8_GB : 4;
#pragma unroll
    for (int b0 = 0; b0 < SB; b0 += GB) {
      f32x4 p[GB][NMAT][MT];
      float scv[GB][NMAT];
#pragma unroll
      for (int bb = 0; bb < GB; ++bb) {
        const int b = b0 + bb;
        uint4 aa[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if (ASTAGE) {
            // token r, chunk 4b + q of the stage; with 8 staged rows, lanes of
            // rows 8..15 re-read rows 0..7 (those outputs are never stored)
            const int ar = ASTAGE >= 32 ? t * 16 + r : r & (ASTAGE ? ASTAGE - 1 : 0);
            aa[t] = abuf[wave][ASTAGE ? ar * 32 + ((4 * b + q + ar) & 31) : 0];
          } else {
            aa[t] = B.a[b * MT + t];
            if (ragged) aa[t] = keep_or_zero(st * SB + b < nb, aa[t]);
          }
        }
        // offset term -136 * sum_k a_k of each token, shared by the matrices
        f32x4 c0[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) c0[t] = mfma16(aa[t], negoff, z4);
        const int src_lane = r + 16 * (b >> 1);  // the lane of row r holding block b's scale
        // block b of row r: chunk b of the row's stage segment, bytes 8(q & 1) .. +8
        const int slot = r * 8 + ((b + (r >> 1)) & 7);
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          const uint2 qv = reinterpret_cast<const uint2*>(&wb[wave][m][slot])[q & 1];
          const uint4 Bq = q4x8_to_bf16_biased(qv.x, qv.y, nib_shift);
          uint32_t pair;
          if (SALIGN) {
            pair = (b >> 1) == 0 ? W.s[m].x : (b >> 1) == 1 ? W.s[m].y : (b >> 1) == 2 ? W.s[m].z : W.s[m].w;
          } else {
            pair = (uint32_t)__shfl((int)W.s[m].x, src_lane, 64);
          }
          scv[bb][m] = q4_f16bits_to_f32((b & 1) ? (pair >> 16) : (pair & 0xFFFFu));
#pragma unroll
          for (int t = 0; t < MT; ++t) p[bb][m][t] = mfma16(aa[t], Bq, c0[t]);
        }
      }
#pragma unroll
      for (int bb = 0; bb < GB; ++bb)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int t = 0; t < MT; ++t) acc[m][t] += scv[bb][m] * p[bb][m][t];
    }
  };

  auto stage_and_compute = [&](const Batch& B, int st) {
    stage(B, B, st);
    compute(B, B, st);
  };

  const int n = se - sb;
  // the deeper pipeline below, except in the 8-token down projection unless
  // FFN_Q4_DEEP_DN8 is set (measured slower there)
  constexpr bool kDeep = ASTAGE != 0 && !(NMAT == 1 && ASTAGE == 8 && !FFN_Q4_DEEP_DN8);
  if (kDeep && n >= 2) {
    // staged activations single-buffered, nibbles of two stages in flight
    // during the MFMAs, scales reloaded after the MFMA loop that reads them
    Batch X, Y, A;
    load_w(X, sb);
    load_s(X, sb);
    load_a(A, sb);
    load_w(Y, sb + 1);
    load_s(Y, sb + 1);
    for (int s = sb;;) {
      __builtin_amdgcn_sched_barrier(0);
      stage(X, A, s);
      __builtin_amdgcn_sched_barrier(0);
      load_a(A, s + 1 < se ? s + 1 : -1);
      load_w(X, s + 2 < se ? s + 2 : -1);
      __builtin_amdgcn_sched_barrier(0);
      compute(X, A, s);
      __builtin_amdgcn_sched_barrier(0);
      load_s(X, s + 2 < se ? s + 2 : -1);
      if (++s >= se) break;
      __builtin_amdgcn_sched_barrier(0);
      stage(Y, A, s);
      __builtin_amdgcn_sched_barrier(0);
      load_a(A, s + 1 < se ? s + 1 : -1);
      load_w(Y, s + 2 < se ? s + 2 : -1);
      __builtin_amdgcn_sched_barrier(0);
      compute(Y, A, s);
      __builtin_amdgcn_sched_barrier(0);
      load_s(Y, s + 2 < se ? s + 2 : -1);
      if (++s >= se) break;
    }
  } else if (n >= 2) {
    Batch X, Y;
    load(X, sb);
    load(Y, sb + 1);
    for (int s = sb;;) {
      __builtin_amdgcn_sched_barrier(0);
      stage_and_compute(X, s);
      __builtin_amdgcn_sched_barrier(0);
      load(X, s + 2 < se ? s + 2 : -1);
      if (++s >= se) break;
      __builtin_amdgcn_sched_barrier(0);
      stage_and_compute(Y, s);
      __builtin_amdgcn_sched_barrier(0);
      load(Y, s + 2 < se ? s + 2 : -1);
      if (++s >= se) break;
    }
  } else if (n == 1) {
    Batch X;
    load(X, sb);
    stage_and_compute(X, sb);
  }

  // ---- fixed-order reduction over the WAVES K slices
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave][t][m][e][lane] = acc[m][t][e];
  if (FOLD) {
    // token 2v + h: the 32 lanes of half h hold its partial sums
#pragma unroll
    for (int v = 0; v < (FOLD ? NA : 1); ++v) {
      float sv = ss[v];
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) sv += __shfl_xor(sv, o, 64);
      if ((lane & 31) == 0) ssq[FOLD ? wave : 0][2 * v + (lane >> 5)] = sv;
    }
  }
  __syncthreads();
  for (int t = wave; t < MT; t += WAVES) {
    const int col = j0 + r;  // lane's weight row = output column
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tok = t * 16 + 4 * q + e;
      float v0 = 0.f, v1 = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        v0 += red[w][t][0][e][lane];
        if (NMAT == 2) v1 += red[w][t][NMAT - 1][e][lane];
      }
      if (tok < M && col < row1) {
        const size_t off = (size_t)tok * N + col;
        if (PART) {
          part[(size_t)blockIdx.y * M * N + off] = v0;
        } else {
          if (FOLD) {
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) sum += ssq[FOLD ? w : 0][tok & 7];
            const float rs = 1.0f / __builtin_sqrtf(sum / (float)K + eps);
            v0 *= rs;
            v1 *= rs;
          }
          const float o = NMAT == 2 ? silu_mul(v0, v1) : bf2f(resid[off]) + v0;
          out[off] = f2bf(o);
        }
      }
    }
  }
}

// Tokens per launch; the API walks larger M in chunks of this size.
int q4_max_tokens() { return 32; }

// Gate/up grid policy (stream_groups): 1 = fill a single round evenly when
// the tiles fit one.  Whole rounds past one (policy 2: 1536 workgroups of
// 11-12 rows instead of 1088 tiles at f = 17408) measured slower in
// interleaved A/B (Q8_0 block 73.1 -> 78.0 us, Q4_0 55.6 -> 56.9 us at 8
// tokens): the extra workgroups cost more than the partial last round.
// Policy 3 (a whole multiple of the compute units: 1280 workgroups of 13-14
// rows at f = 17408, five per CU) measured slightly faster (Q8_0 71.9 ->
// 71.6 us at 8 tokens, 64.5 -> 63.9 at 1; Q4_0 55.5 -> 55.0 and 48.1 ->
// 47.6; bitwise identical).
#ifndef FFN_Q4_BALANCE
#define FFN_Q4_BALANCE 3
#endif

template <class Kern>
static void q4_go(Kern kern, bool gateup, int splits, int N, int threads, const uint16_t* a,
                     const uint16_t* gn, const uint8_t* q0, const uint16_t* s0,
                     const uint8_t* q1, const uint16_t* s1, const uint16_t* rr,
                     uint16_t* o, float* part, int M, int K, float eps, int slots, hipStream_t s) {
  static const int cus = device_cus();
  const int groups = gateup ? stream_groups(N, slots, FFN_Q4_BALANCE, cus) : (N + 15) / 16;
  FFN_DISPATCH(kern, dim3((unsigned)groups, (unsigned)splits), dim3(threads), 0, s, a, gn, q0, s0, q1,
               s1, rr, o, part, M, K, N, eps);
}

template <int NMAT, int WAVES, bool SALIGN, bool PART, bool FOLD = false>
static void launch_q4_mt(const uint16_t* a, const uint16_t* gn, float eps, const uint8_t* q0,
                         const uint16_t* s0, const uint8_t* q1, const uint16_t* s1,
                         const uint16_t* rr, uint16_t* o, float* part, int splits, int M, int K,
                         int N, hipStream_t s) {
  constexpr int T = WAVES * 64;
  constexpr bool GU = NMAT == 2;
  // each kernel's occupancy is fixed: computed once (the library assumes
  // every device it runs on is the same model)
  if constexpr (FOLD) {
    auto k = q4_stream<NMAT, 1, WAVES, SALIGN, 8, PART, true>;
    static const int slots = GU ? resident_slots(k, T) : 0;
    q4_go(k, GU, splits, N, T, a, gn, q0, s0, q1, s1, rr, o, part, M, K, eps, slots, s);
  } else {
    if (M <= 8) {
      auto k = q4_stream<NMAT, 1, WAVES, SALIGN, 8, PART, false>;
      static const int slots = GU ? resident_slots(k, T) : 0;
      q4_go(k, GU, splits, N, T, a, gn, q0, s0, q1, s1, rr, o, part, M, K, eps, slots, s);
    } else if (M <= 16) {
      auto k = q4_stream<NMAT, 1, WAVES, SALIGN, 16, PART, false>;
      static const int slots = GU ? resident_slots(k, T) : 0;
      q4_go(k, GU, splits, N, T, a, gn, q0, s0, q1, s1, rr, o, part, M, K, eps, slots, s);
    } else if (FFN_Q4_STAGE32) {
      // 17..32 tokens: both token tiles staged through LDS (as for Q8_0)
      constexpr int W2 = FFN_Q4_S32_WAVES;
      auto k = q4_stream<NMAT, 2, W2, SALIGN, 32, PART, false>;
      static const int slots = GU ? resident_slots(k, W2 * 64) : 0;
      q4_go(k, GU, splits, N, W2 * 64, a, gn, q0, s0, q1, s1, rr, o, part, M, K, eps, slots, s);
    } else {
      auto k = q4_stream<NMAT, 2, WAVES, SALIGN, 0, PART, false>;
      static const int slots = GU ? resident_slots(k, T) : 0;
      q4_go(k, GU, splits, N, T, a, gn, q0, s0, q1, s1, rr, o, part, M, K, eps, slots, s);
    }
  }
}

// 16-byte scale loads need every row of scales (K/16 bytes) and the base
// pointers 16-byte aligned
static bool q4_scales_aligned(int K, const uint16_t* s0, const uint16_t* s1) {
  return K % 256 == 0 && ((uintptr_t)s0 % 16) == 0 && (s1 == nullptr || ((uintptr_t)s1 % 16) == 0);
}

hipError_t launch_q4_gateup(const void* act, const void* gain, float eps, const uint8_t* qg,
                            const uint16_t* sg, const uint8_t* qu, const uint16_t* su, void* h,
                            int M, int d, int f, hipStream_t s) {
  constexpr int W = FFN_Q4_GU_WAVES;
  const uint16_t* a = (const uint16_t*)act;
  const uint16_t* gn = (const uint16_t*)gain;
  const bool al = q4_scales_aligned(d, sg, su);
  if (gain) {
    if (M > 8) return hipErrorInvalidValue;  // the folded kernel stages at most 8 token rows
    if (al) launch_q4_mt<2, W, true, false, true>(a, gn, eps, qg, sg, qu, su, nullptr, (uint16_t*)h, nullptr, 1, M, d, f, s);
    else launch_q4_mt<2, W, false, false, true>(a, gn, eps, qg, sg, qu, su, nullptr, (uint16_t*)h, nullptr, 1, M, d, f, s);
  } else {
    if (al) launch_q4_mt<2, W, true, false>(a, nullptr, 0.f, qg, sg, qu, su, nullptr, (uint16_t*)h, nullptr, 1, M, d, f, s);
    else launch_q4_mt<2, W, false, false>(a, nullptr, 0.f, qg, sg, qu, su, nullptr, (uint16_t*)h, nullptr, 1, M, d, f, s);
  }
  return hipGetLastError();
}

// Split-K factor of the down projection: enough (row tile, K range) workgroups
// for about FFN_Q4_DN_SPLIT_TARGET of them in total (4 per compute unit on
// 256 compute units), at most 8 ranges and no more than the 256-k stages.
int q4_down_splits(int M, int N, int K) {
  const int target = FFN_Q4_DN_SPLIT_TARGET;
  const int tiles = (N + 15) / 16;
  if (M <= FFN_Q4_DN_WHOLE && tiles % device_cus() == 0) return 1;
  const int nst = (K / 32 + 7) / 8;
  int sp = target > 0 ? (target + tiles - 1) / tiles : 1;
  sp = sp < 1 ? 1 : sp > kQuantMaxSplits ? kQuantMaxSplits : sp;
  return sp > nst ? (nst > 0 ? nst : 1) : sp;
}

hipError_t launch_q4_down(const void* h, const uint8_t* qd, const uint16_t* sd, const void* x,
                          void* y, float* part, int M, int d, int f, hipStream_t s) {
  constexpr int W = FFN_Q4_DN_WAVES;
  const uint16_t* a = (const uint16_t*)h;
  const int sp = q4_down_splits(M, d, f);
  const bool al = q4_scales_aligned(f, sd, nullptr);
  if (sp == 1) {
    if (al) launch_q4_mt<1, W, true, false>(a, nullptr, 0.f, qd, sd, nullptr, nullptr, (const uint16_t*)x, (uint16_t*)y, nullptr, 1, M, f, d, s);
    else launch_q4_mt<1, W, false, false>(a, nullptr, 0.f, qd, sd, nullptr, nullptr, (const uint16_t*)x, (uint16_t*)y, nullptr, 1, M, f, d, s);
    return hipGetLastError();
  }
  if (al) launch_q4_mt<1, W, true, true>(a, nullptr, 0.f, qd, sd, nullptr, nullptr, nullptr, nullptr, part, sp, M, f, d, s);
  else launch_q4_mt<1, W, false, true>(a, nullptr, 0.f, qd, sd, nullptr, nullptr, nullptr, nullptr, part, sp, M, f, d, s);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_splitk_residual(part, sp, x, y, M, d, s);
}

}  // namespace ffn
