// Q8_0 weight-streaming projections with in-register dequantisation.
//
// A Q8_0 weight w[j,k] = q[j,k] * s[j, k/32]: 32 int8 quants along the
// reduction axis share one fp16 scale (the format named in "Unfusing a
// Kernel Made It 1.63x Faster", Finding 2).  Activations stay bf16.
//
//   gate/up : h[m,j] = silu(sum_k Wg[j,k] n[m,k]) * (sum_k Wu[j,k] n[m,k])
//   down    : y[m,i] = x[m,i] + sum_j Wd[i,j] h[m,j]
// n = rmsnorm(x) * g normally comes from the norm kernel.  With up to 8
// tokens the norm is folded into the gate/up kernel instead (FOLD, as in the
// bf16 decode kernels: x * g where the activations are staged, r_m in the
// epilogue): the fold saves the norm launch for some staging work (measured:
// block 10% faster at f = 2176 and 2% faster at f = 17408; 3-17% slower at
// 16 and 32 tokens, which keep the norm kernel).
//
// gfx950 mapping.  A block of 32 quants is exactly one K step of
// v_mfma_f32_16x16x32_bf16, so the scale factors out of the block's dot
// product:  sum_{k in b} q[j,k] s[j,b] a[m,k] = s[j,b] * sum_{k in b} q[j,k] a[m,k].
// The quants are exact in bf16 (|q| <= 128 needs 8 significant bits), so the
// MFMA runs on the raw integers with a zero accumulator and the lane adds
// s[j,b] * partial in fp32: the dequantisation adds no rounding at all.
// Operands: A = 16 tokens x 32 k (bf16 activations), B = 32 k x 16 weight
// rows (quants converted to bf16); lane l's result D[4(l/16)+e][l%16] holds 4
// tokens of weight row l%16, so the lane needs the scales of one row only.
//
// Streaming: a workgroup owns 16 weight rows (per matrix); its waves split K
// into 256-k stages.  Quants are fetched as 256-byte row segments (4 rows x
// 256 B per wave instruction) into a per-wave 4 KiB LDS stage whose 16-byte
// chunks are rotated per row so the 8-byte fragment reads are bank-conflict
// free; prefetches past a wave's K slice use an out-of-range buffer offset
// and read nothing.  The 8 scales a row needs per stage are fetched by one 16-byte load
// per lane when rows of scales are 16-byte aligned (K % 256 == 0); otherwise
// lane (r, q) takes blocks 2q, 2q+1 of row r and hands them to the other lanes
// of the row with cross-lane permutes.  Scale loads from 16 rows touch 16
// cache lines each, so their count, not their bytes, is what costs.  The K
// loop is software-pipelined: with staged activations the quants of two
// stages are in flight while a stage's MFMAs run (quants and scales
// double-buffered in registers, activations single-buffered: reloaded as soon
// as they are in LDS; the scales, which the MFMA loop reads, are reloaded
// after it); partial tiles are reduced across waves in a fixed order.
// Activation rows past M are clamped copies of row M-1: they only feed
// output rows that are never stored, so they need no masking.
// The down projection (320 row tiles at d = 5120) splits its K axis into a
// few ranges with two waves per workgroup, as the Q4_0 one does; the ranges'
// fp32 partials are added in order by launch_splitk_residual.
#include "common.h"
#include "launch.h"

#ifndef FFN_Q8_GU_WAVES
#define FFN_Q8_GU_WAVES 4
#endif
#ifndef FFN_Q8_DN_WAVES
#define FFN_Q8_DN_WAVES 2
#endif
#ifndef FFN_Q8_DN_SPLIT_TARGET
#define FFN_Q8_DN_SPLIT_TARGET 1024
#endif
// Down projections of up to FFN_Q8_DN_WHOLE tokens whose 16-row tiles fill
// whole rounds of the compute units (d = 4096 on 256 CUs) run unsplit in
// four-wave workgroups.  Interleaved A/B, d = 4096, f = 11008: block 38.7 /
// 41.1 / 42.8 / 48.5 -> 36.9 / 39.0 / 39.9 / 46.4 us at 1 / 4 / 8 / 16
// tokens; at 32 and 64 tokens the split stays faster (58.4 -> 62.3 and
// 111.5 -> 120.2 us unsplit).
#ifndef FFN_Q8_DN_WHOLE
#define FFN_Q8_DN_WHOLE 16
#endif

// The 8-token gate/up kernel (two matrices, 8 staged token rows, norm not
// folded): waves per SIMD it is register-allocated for, and the 32-quant
// blocks whose MFMAs are issued before their scale FMAs (GB partial tiles
// stay live).  At three waves (166 VGPRs, no AGPRs) the other waves cover the
// wait of each FMA on its MFMA; GB = 2 or 4 at three waves spills.
#ifndef FFN_Q8_DEEP_DN8
#define FFN_Q8_DEEP_DN8 0
#endif
#ifndef FFN_Q8_GU8_WPE
#define FFN_Q8_GU8_WPE 3
#endif
// 17..32 tokens with both token tiles staged through LDS in two-wave
// workgroups (0: activations read straight from L2 in the MFMA operand
// layout, 256 VGPRs at four waves).  Interleaved A/B, d = 5120, f = 17408:
// block 121 / 137 / 154 -> 107 / 111 / 116 us at 17 / 24 / 32 tokens, 230 /
// 303 -> 191 / 226 us at 48 / 64 (two chunks); d = 4096, f = 11008 at 32
// tokens 85 -> 59 us.  Then the waves per workgroup (four: 4-8% slower) and
// the blocks per MFMA group of that kernel (two spills into AGPRs).
#ifndef FFN_Q8_STAGE32
#define FFN_Q8_STAGE32 1
#endif
#ifndef FFN_Q8_S32_WAVES
#define FFN_Q8_S32_WAVES 2
#endif
#ifndef FFN_Q8_S32_GB
#define FFN_Q8_S32_GB 1
#endif
#ifndef FFN_Q8_GU8_GB
#define FFN_Q8_GU8_GB 1
#endif

namespace ffn {

// 8 int8 quants (two dwords) -> 8 bf16 (exact)
__device__ __forceinline__ uint4 q8x8_to_bf16(uint32_t lo, uint32_t hi) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = (float)(((int)(lo << (24 - 8 * i))) >> 24);
    f[4 + i] = (float)(((int)(hi << (24 - 8 * i))) >> 24);
  }
  return pack8(f);
}

__device__ __forceinline__ float f16bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}


// ASTAGE: 0 = activations read straight from L2 in the MFMA operand layout;
// 8 = 8 token rows, 16 = 16 token rows fetched as 512-byte token segments and
// staged through LDS (fewer, fuller cache-line requests).
// PART: split-K pass (NMAT == 1): workgroup (tile, z) covers the z-th of
// gridDim.y contiguous ranges of stages and writes fp32 partial sums to
// part[z][M][N]; launch_splitk_residual adds the ranges in order.
// FOLD (gate/up, up to 8 tokens): the RMSNorm is folded in, as in the bf16
// decode kernels: act is x, the staged activations are multiplied by the
// gain while the sums of squares of x accumulate, and the epilogue scales
// both projections by r_m.
template <int NMAT, int MT, int WAVES, bool SALIGN, int ASTAGE, bool PART, bool FOLD>
__global__ __launch_bounds__(WAVES * 64)
__attribute__((amdgpu_waves_per_eu(NMAT == 2 && ASTAGE == 8 && !FOLD ? FFN_Q8_GU8_WPE : 1)))
void q8_stream(
    const uint16_t* __restrict__ act,     // [M, K] bf16: x (FOLD), n or h
    const uint16_t* __restrict__ gain,    // [K] (FOLD)
    const int8_t* __restrict__ q0, const uint16_t* __restrict__ s0,  // [N, K], [N, K/32]
    const int8_t* __restrict__ q1, const uint16_t* __restrict__ s1,
    const uint16_t* __restrict__ resid,   // [M, N] (NMAT == 1)
    uint16_t* __restrict__ out,           // [M, N] (!PART)
    float* __restrict__ part,             // [gridDim.y, M, N] (PART)
    int M, int K, int N, float eps) {
  static_assert(!FOLD || (NMAT == 2 && !PART && ASTAGE == 8), "the norm folds into the 8-token gate/up kernel only");
  // SALIGN is only chosen when K % 256 == 0: every stage is then whole, so
  // the clamps and masks of a partial last stage compile away (10% fewer
  // VALU instructions in the folded gate/up kernel; interleaved A/B,
  // bitwise identical: block 73.8 -> 72.7 us at 8 tokens, 84.1 -> 82.2 at
  // 16, 165 -> 156 at 32)
  constexpr bool KFULL = SALIGN;
  auto cl = [](int v, int hi) { return KFULL ? v : min(v, hi); };
  constexpr int SB = 8;  // 32-quant blocks per stage (256 k, 256 B per row)
  __shared__ uint4 wb[WAVES][NMAT][256];           // per-wave quant stage (4 KiB per matrix)
  __shared__ uint4 abuf[WAVES][ASTAGE ? ASTAGE * 32 : 1];  // per-wave activation stage [rows][32]
  __shared__ float ssq[FOLD ? WAVES : 1][8];  // per-wave partial sums of squares (FOLD)
  // the cross-wave partial tiles reuse each wave's own quant stage once its
  // K loop is done (MT * NMAT KiB <= NMAT * 4 KiB)
  static_assert(MT <= 4, "partial tiles must fit the quant stage");
  auto red = [&](int w, int t, int m, int e) -> float* {
    return reinterpret_cast<float*>(&wb[w][0][0]) + ((t * NMAT + m) * 4 + e) * 64;
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar loop control
  const int r = lane & 15, q = lane >> 4;
  // workgroup b of G (gridDim.x) owns output rows [b N / G, (b + 1) N / G),
  // at most 16; tile rows past row1 load nothing and are never stored
  const int j0 = (int)(((long)blockIdx.x * N) / gridDim.x);
  const int row1 = (int)(((long)(blockIdx.x + 1) * N) / gridDim.x);
  const int nb = K >> 5;                // blocks per row
  const int K16 = K >> 4;               // 16-byte quant chunks per row
  const int K8 = K >> 3;                // 16-byte activation chunks per row
  const int nst = (nb + SB - 1) / SB;
  const int zs = PART ? (int)(((long)nst * blockIdx.y) / gridDim.y) : 0;  // this split's stages
  const int ze = PART ? (int)(((long)nst * (blockIdx.y + 1)) / gridDim.y) : nst;
  const int sb = zs + (int)(((long)(ze - zs) * wave) / WAVES);
  const int se = zs + (int)(((long)(ze - zs) * (wave + 1)) / WAVES);

  // staged loads: instruction u covers tile rows 4u..4u+3; lane -> row
  // 4u + q, LDS slot u*64 + lane, which holds chunk (r - (4u + q)) & 15 of the
  // row's 256-byte stage segment; so chunk c of tile row R sits at slot
  // (R >> 2)*64 + (R & 3)*16 + ((c + R) & 15)
  __amdgpu_buffer_rsrc_t rq[NMAT];  // quants through buffer resources (< 2 GiB)
  rq[0] = make_rsrc(q0, (long)N * K);
  if (NMAT == 2) rq[NMAT - 1] = make_rsrc(q1, (long)N * K);
  unsigned gq[4];  // byte offset of this lane's quant row in each instruction
  int cst[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = j0 + 4 * u + q;
    cst[u] = (r - (4 * u + q)) & 15;
    // kOutOfRange plus any in-row offset (< 2^31) stays past the resource
    gq[u] = row < row1 ? (unsigned)row * (unsigned)K : kOutOfRange;
  }
  // this lane's weight row (MFMA B operand) and its scales; lane (r, q)
  // fetches blocks 2q, 2q+1 of each stage for row r
  const int jr = min(j0 + r, row1 - 1);  // scale row (rows past row1: a valid row's, cached)
  const uint16_t* ps[NMAT];
  ps[0] = s0 + (size_t)jr * nb;
  if (NMAT == 2) ps[NMAT - 1] = s1 + (size_t)jr * nb;
  // SALIGN: both matrices' scale rows at the same byte offset of their own
  // buffer resources (one 32-bit offset instead of two 64-bit pointers)
  __amdgpu_buffer_rsrc_t rs[NMAT];
  rs[0] = make_rsrc(s0, (long)N * nb * 2);
  if (NMAT == 2) rs[NMAT - 1] = make_rsrc(s1, (long)N * nb * 2);
  const unsigned srow = (unsigned)jr * (unsigned)nb * 2u;
  const int rd_base = (r >> 2) * 64 + (r & 3) * 16;

  // direct activations: token t*16 + r; staged: instruction v covers token
  // rows 2v, 2v+1 (lane -> row 2v + lane/32, LDS slot v*64 + lane holding
  // chunk ((lane & 31) - row) & 31 of the row's 512-byte stage segment).
  // FOLD: lane -> chunk lane & 31 of every row it stages (one gain chunk per
  // stage), written to slot v*64 + (lane/32)*32 + ((lane & 31) + row) & 31:
  // the same LDS layout (chunk c of row R at R*32 + ((c + R) & 31)).
  constexpr int NA = ASTAGE ? ASTAGE / 2 : SB * MT;  // activation loads per batch
  const uint4* pa[ASTAGE ? 1 : MT];
  // staged rows through a buffer resource: 32-bit byte offsets per row
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(act, (long)M * K * 2);
  unsigned aro[ASTAGE && ASTAGE < 32 ? NA : 1];
  if (ASTAGE) {
#pragma unroll
    for (int v = 0; v < NA; ++v)
      if (ASTAGE < 32) aro[ASTAGE && ASTAGE < 32 ? v : 0] = (unsigned)min(2 * v + (lane >> 5), M - 1) * (unsigned)K8 * 16u;
  } else {
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
  const uint4* G4 = reinterpret_cast<const uint4*>(gain);
  // FOLD: sums of squares of x per staged row (ss[v], token 2v + lane/32)
  float ss[FOLD ? NA : 1];
#pragma unroll
  for (int i = 0; i < (FOLD ? NA : 1); ++i) ss[i] = 0.f;
  // x * g in fp32, rounded once to bf16, and the sum of squares of x
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
    uint4 w[NMAT][4];
    uint4 s[NMAT];  // SALIGN: the stage's 8 scales of row r; else .x = blocks 2q, 2q+1
    uint4 a[NA];
    uint4 g;  // the stage's gain chunk lane & 31 (FOLD)
  };
  // st < 0 marks a prefetch past the slice end: the quant loads then read
  // nothing (out-of-range offset) and the small loads hit cache
  auto load_w = [&](Batch& B, int st_req) {
    const int st = st_req < 0 ? se - 1 : st_req;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = cl(st * 16 + cst[u], K16 - 1);
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
      for (int m = 0; m < NMAT; ++m) B.s[m] = buf_ld16(rs[m], srow + (unsigned)c * 16u);
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
        // row 2v + (lane>>5): chunk (lane&31 - row) & 31 of its stage
        // segment, or chunk lane & 31 when folding
        const int c = FOLD ? (lane & 31) : ((lane & 31) - (2 * v + (lane >> 5))) & 31;
        // 32 staged rows: the row offset is formed here (16 offsets held for
        // the whole K loop would cost 16 VGPRs)
        const unsigned ro = ASTAGE >= 32 ? (unsigned)min(2 * v + (lane >> 5), M - 1) * (unsigned)K8 * 16u
                                         : aro[ASTAGE ? v : 0];
        B.a[v] = buf_ld16(ra, ro + (unsigned)cl(st * 32 + c, K8 - 1) * 16u);
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
  // the quants (W) and the staged activations (A) of a stage go to LDS
  auto stage = [&](const Batch& W, const Batch& B, int st) {
    const bool ragged = !KFULL && (st + 1) * SB > nb;  // only a row's last stage can be partial
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        uint4 v = W.w[m][u];
        if (ragged) v = keep_or_zero(st * 16 + cst[u] < K16, v);
        wb[wave][m][u * 64 + lane] = v;
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
    // per block: the MFMAs of a group of blocks first, then their scale FMAs,
    // so the FMAs do not wait on each MFMA in turn
    constexpr int GB = ASTAGE == 32 ? FFN_Q8_S32_GB : NMAT == 2 && ASTAGE == 8 && !FOLD ? FFN_Q8_GU8_GB : 4;
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
            // token r of tile t, chunk 4b + q of the stage; with 8 staged
            // rows, lanes of rows 8..15 re-read rows 0..7 (those outputs are
            // never stored); 32 staged rows hold both token tiles
            const int ar = ASTAGE >= 32 ? t * 16 + r : r & (ASTAGE ? ASTAGE - 1 : 0);
            aa[t] = abuf[wave][ASTAGE ? ar * 32 + ((4 * b + q + ar) & 31) : 0];
          } else {
            aa[t] = B.a[b * MT + t];
            if (ragged) aa[t] = keep_or_zero(st * SB + b < nb, aa[t]);
          }
        }
        // quants k = 32b + 8q .. +8 of row r: chunk 2b + q/2 of the stage, half q & 1
        const int slot = rd_base + ((2 * b + (q >> 1) + r) & 15);
        const int src_lane = r + 16 * (b >> 1);  // the lane of row r holding block b's scale
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          const uint2 qv = reinterpret_cast<const uint2*>(&wb[wave][m][slot])[q & 1];
          const uint4 Bq = q8x8_to_bf16(qv.x, qv.y);
          uint32_t pair;
          if (SALIGN) {
            pair = (b >> 1) == 0 ? W.s[m].x : (b >> 1) == 1 ? W.s[m].y : (b >> 1) == 2 ? W.s[m].z : W.s[m].w;
          } else {
            pair = (uint32_t)__shfl((int)W.s[m].x, src_lane, 64);
          }
          scv[bb][m] = f16bits_to_f32((b & 1) ? (pair >> 16) : (pair & 0xFFFFu));
#pragma unroll
          for (int t = 0; t < MT; ++t) p[bb][m][t] = mfma16(aa[t], Bq, z4);
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
  // FFN_Q8_DEEP_DN8 is set (measured slower there)
  constexpr bool kDeep = ASTAGE != 0 && !(NMAT == 1 && ASTAGE == 8 && !FFN_Q8_DEEP_DN8);
  if (kDeep && n >= 2) {
    // staged activations are single-buffered: the next stage's are loaded as
    // soon as this stage's are in LDS, and the quants two stages out right
    // after them, so two stages of quants are in flight during the MFMAs;
    // the scales, still read by the MFMA loop, are reloaded after it
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
      for (int e = 0; e < 4; ++e) red(wave, t, m, e)[lane] = acc[m][t][e];
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
        v0 += red(w, t, 0, e)[lane];
        if (NMAT == 2) v1 += red(w, t, NMAT - 1, e)[lane];
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

// Tokens per launch; the API walks larger M in chunks of this size (two
// token tiles keep the kernels free of register spills).
int q8_max_tokens() { return 32; }

// Gate/up grid policy (stream_groups): 1 = fill a single round evenly when
// the tiles fit one.  Whole rounds past one (policy 2: 1536 workgroups of
// 11-12 rows instead of 1088 tiles at f = 17408) measured slower in
// interleaved A/B (Q8_0 block 73.1 -> 78.0 us, Q4_0 55.6 -> 56.9 us at 8
// tokens): the extra workgroups cost more than the partial last round.
// Policy 3 (a whole multiple of the compute units: 1280 workgroups of 13-14
// rows at f = 17408, five per CU) measured slightly faster (Q8_0 71.9 ->
// 71.6 us at 8 tokens, 64.5 -> 63.9 at 1; Q4_0 55.5 -> 55.0 and 48.1 ->
// 47.6; bitwise identical).
#ifndef FFN_Q8_BALANCE
#define FFN_Q8_BALANCE 3
#endif

#ifndef FFN_Q8_DN_BALANCE
#define FFN_Q8_DN_BALANCE 0
#endif
template <class Kern>
static void q8_go(Kern kern, bool gateup, int splits, int N, int threads, const uint16_t* a,
                     const uint16_t* gn, const int8_t* q0, const uint16_t* s0,
                     const int8_t* q1, const uint16_t* s1, const uint16_t* rr,
                     uint16_t* o, float* part, int M, int K, float eps, int slots, hipStream_t s) {
  static const int cus = device_cus();
  const int groups = gateup ? stream_groups(N, slots, FFN_Q8_BALANCE, cus)
                     : FFN_Q8_DN_BALANCE ? stream_groups(N, 1, 3, cus) : (N + 15) / 16;
  FFN_DISPATCH(kern, dim3((unsigned)groups, (unsigned)splits), dim3(threads), 0, s, a, gn, q0, s0, q1,
               s1, rr, o, part, M, K, N, eps);
}

template <int NMAT, int WAVES, bool SALIGN, bool PART, bool FOLD = false>
static void launch_q8_mt(const uint16_t* a, const uint16_t* gn, float eps, const int8_t* q0,
                         const uint16_t* s0, const int8_t* q1, const uint16_t* s1,
                         const uint16_t* rr, uint16_t* o, float* part, int splits, int M, int K,
                         int N, hipStream_t s) {
  constexpr int T = WAVES * 64;
  constexpr bool GU = NMAT == 2;
  // each kernel's occupancy is fixed: computed once (the library assumes
  // every device it runs on is the same model)
  if constexpr (FOLD) {
    auto k = q8_stream<NMAT, 1, WAVES, SALIGN, 8, PART, true>;
    static const int slots = GU ? resident_slots(k, T) : 0;
    q8_go(k, GU, splits, N, T, a, gn, q0, s0, q1, s1, rr, o, part, M, K, eps, slots, s);
  } else {
    if (M <= 8) {
      auto k = q8_stream<NMAT, 1, WAVES, SALIGN, 8, PART, false>;
      static const int slots = GU ? resident_slots(k, T) : 0;
      q8_go(k, GU, splits, N, T, a, gn, q0, s0, q1, s1, rr, o, part, M, K, eps, slots, s);
    } else if (M <= 16) {
      auto k = q8_stream<NMAT, 1, WAVES, SALIGN, 16, PART, false>;
      static const int slots = GU ? resident_slots(k, T) : 0;
      q8_go(k, GU, splits, N, T, a, gn, q0, s0, q1, s1, rr, o, part, M, K, eps, slots, s);
    } else if (FFN_Q8_STAGE32) {
      // 17..32 tokens: both token tiles staged through LDS, in workgroups of
      // FFN_Q8_S32_WAVES waves (32 staged rows take 16 KiB per wave)
      constexpr int W2 = FFN_Q8_S32_WAVES;
      auto k = q8_stream<NMAT, 2, W2, SALIGN, 32, PART, false>;
      static const int slots = GU ? resident_slots(k, W2 * 64) : 0;
      q8_go(k, GU, splits, N, W2 * 64, a, gn, q0, s0, q1, s1, rr, o, part, M, K, eps, slots, s);
    } else {
      auto k = q8_stream<NMAT, 2, WAVES, SALIGN, 0, PART, false>;
      static const int slots = GU ? resident_slots(k, T) : 0;
      q8_go(k, GU, splits, N, T, a, gn, q0, s0, q1, s1, rr, o, part, M, K, eps, slots, s);
    }
  }
}

// 16-byte scale loads need every row of scales (K/16 bytes) and the base
// pointers 16-byte aligned
static bool q8_scales_aligned(int K, const uint16_t* s0, const uint16_t* s1) {
  return K % 256 == 0 && ((uintptr_t)s0 % 16) == 0 && (s1 == nullptr || ((uintptr_t)s1 % 16) == 0);
}

hipError_t launch_q8_gateup(const void* act, const void* gain, float eps, const int8_t* qg,
                            const uint16_t* sg, const int8_t* qu, const uint16_t* su, void* h,
                            int M, int d, int f, hipStream_t s) {
  constexpr int W = FFN_Q8_GU_WAVES;
  const uint16_t* a = (const uint16_t*)act;
  const uint16_t* gn = (const uint16_t*)gain;
  const bool al = q8_scales_aligned(d, sg, su);
  if (gain) {
    if (M > 8) return hipErrorInvalidValue;  // the folded kernel stages at most 8 token rows
    if (al) launch_q8_mt<2, W, true, false, true>(a, gn, eps, qg, sg, qu, su, nullptr, (uint16_t*)h, nullptr, 1, M, d, f, s);
    else launch_q8_mt<2, W, false, false, true>(a, gn, eps, qg, sg, qu, su, nullptr, (uint16_t*)h, nullptr, 1, M, d, f, s);
  } else {
    if (al) launch_q8_mt<2, W, true, false>(a, nullptr, 0.f, qg, sg, qu, su, nullptr, (uint16_t*)h, nullptr, 1, M, d, f, s);
    else launch_q8_mt<2, W, false, false>(a, nullptr, 0.f, qg, sg, qu, su, nullptr, (uint16_t*)h, nullptr, 1, M, d, f, s);
  }
  return hipGetLastError();
}

// Split-K factor of the down projection, as for Q4_0: about
// FFN_Q8_DN_SPLIT_TARGET workgroups in total, at most kQuantMaxSplits ranges
// and no more than the 256-k stages.
int q8_down_splits(int M, int N, int K) {
  const int target = FFN_Q8_DN_SPLIT_TARGET;
  const int tiles = (N + 15) / 16;
  if (M <= FFN_Q8_DN_WHOLE && tiles % device_cus() == 0) return 1;
  const int nst = (K / 32 + 7) / 8;
  int sp = target > 0 ? (target + tiles - 1) / tiles : 1;
  sp = sp < 1 ? 1 : sp > kQuantMaxSplits ? kQuantMaxSplits : sp;
  return sp > nst ? (nst > 0 ? nst : 1) : sp;
}

hipError_t launch_q8_down(const void* h, const int8_t* qd, const uint16_t* sd, const void* x,
                          void* y, float* part, int M, int d, int f, hipStream_t s) {
  constexpr int W = FFN_Q8_DN_WAVES;
  const uint16_t* a = (const uint16_t*)h;
  const int sp = q8_down_splits(M, d, f);
  const bool al = q8_scales_aligned(f, sd, nullptr);
  if (sp == 1) {
    constexpr int W1 = FFN_Q8_DN_WHOLE > 0 ? 4 : W;
    if (al) launch_q8_mt<1, W1, true, false>(a, nullptr, 0.f, qd, sd, nullptr, nullptr, (const uint16_t*)x, (uint16_t*)y, nullptr, 1, M, f, d, s);
    else launch_q8_mt<1, W1, false, false>(a, nullptr, 0.f, qd, sd, nullptr, nullptr, (const uint16_t*)x, (uint16_t*)y, nullptr, 1, M, f, d, s);
    return hipGetLastError();
  }
  if (al) launch_q8_mt<1, W, true, true>(a, nullptr, 0.f, qd, sd, nullptr, nullptr, nullptr, nullptr, part, sp, M, f, d, s);
  else launch_q8_mt<1, W, false, true>(a, nullptr, 0.f, qd, sd, nullptr, nullptr, nullptr, nullptr, part, sp, M, f, d, s);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_splitk_residual(part, sp, x, y, M, d, s);
}

}  // namespace ffn
