// Decode-regime projections (few tokens), weight streaming through LDS on
// bf16 MFMA, with the RMSNorm folded into the gate/up kernel.
//
//   gate/up : h[m,j] = silu(r_m (Wg (x_m * g))_j) * (r_m (Wu (x_m * g))_j),
//             r_m = 1 / sqrt(sum_k x[m,k]^2 / d + eps)
//   down    : y[m,i] = x[m,i] + sum_j Wd[i,j] h[m,j]
// (RMSNorm: "When to hand-write a GPU kernel on Apple Silicon", Rung 2;
// gate/up of the SwiGLU MLP: "Unfusing a Kernel Made It 1.63x Faster",
// Finding 1; FFN-down: "Megakernels on Mac", "Projection shape changes the
// achieved rate"; the FFN weights dominate a decode pass's payload:
// "Megakernels on Mac", "The 27.65 ms estimate".)
//
// The norm folds because W n_m = r_m W (x_m * g): the K loop multiplies
// the weights with bf16(x * g) and accumulates sum x^2 from the same loads,
// and the epilogue scales by r_m once the whole row's sum is known (the
// full-row dependency of the norm, "Megakernels on Mac", "Dependencies and
// synchronization", is respected: r_m is applied only after every K slice
// has been reduced).  This removes the separate norm launch and the n round
// trip.
//
// With M <= 64 tokens every weight is used M times, far below the flop:byte
// ridge, so the kernels are bound by reading W from HBM once.  gfx950 design:
//  * a workgroup owns at most 16 weight rows (per matrix; an equal share of
//    the rows when the grid is balanced, below); its W waves split K into
//    contiguous slices of 128-k stages;
//  * weights are fetched in 256-byte row segments (4 rows x 256 B per wave
//    instruction), which streams markedly faster on this chip than the
//    16-rows x 64-B pattern of the MFMA operand layout, then staged in a
//    per-wave 4 KiB LDS buffer and read back in MFMA layout.  Within a row
//    the 16-byte chunks are rotated by the row index, so both the stores and
//    the ds_read_b128 fragment reads are bank-conflict free;
//  * the activation stage (16 tokens x 128 k) is fetched and staged the same
//    way (tokens in place of rows): fetching it in the MFMA operand layout
//    (16 tokens x 64 B per instruction) cost about 11 us of a 58 us decode
//    call at 16 tokens; tokens past M repeat token M-1 and only feed output
//    columns that are never stored;
//  * v_mfma_f32_16x16x32_bf16: A = 16 weight rows x 32 k, B = 32 k x 16
//    tokens, both read from the LDS stages;
//  * the K loop is software-pipelined over two register batches (the next
//    stage's loads are in flight while the current one is staged and
//    multiplied); every iteration issues the same loads (uniform wait
//    counts): past the slice end the weight loads get an out-of-range buffer
//    offset, which returns zeros without touching memory;
//  * the W partial tiles (and partial sums of squares) are reduced in a fixed
//    order through LDS: deterministic, no atomics;
//  * h, which only these two kernels see, is kept in the down projection's
//    MFMA operand order (blocked layout below): the gate/up epilogue scatters
//    its 8-byte groups there, and the down kernel reads each 32-k operand of
//    16 tokens as one contiguous 1 KiB wave load straight into registers, with
//    no LDS stage for the activations (down projection at 16 tokens 19.2 ->
//    18.6 us, bitwise identical to the row-major form);
//  * up to 64 tokens (four 16-token tiles) go through each projection in one
//    launch, so every weight is streamed once per call.
#include "common.h"
#include "launch.h"

#ifndef FFN_DS_GU_WAVES
#define FFN_DS_GU_WAVES 4
#endif
#ifndef FFN_DS_DN_WAVES
#define FFN_DS_DN_WAVES 8
#endif

// Waves per SIMD the 16-token gate/up kernel is register-allocated for: at
// 3 (168 VGPRs, no spills; 49 KiB LDS) all 688 workgroups of an f = 11008
// projection are resident at once instead of 512 plus a second round.
#ifndef FFN_DS_GU_STAGED_WPE
#define FFN_DS_GU_STAGED_WPE 3
#endif

namespace ffn {

// 8-byte store written through to the coherence point shared by all XCDs
__device__ __forceinline__ void coh_st8(void* p, uint32_t lo, uint32_t hi) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), ((uint64_t)hi << 32) | lo, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Blocked layout of h for the decode kernels: token tile T (16 tokens), 128-k
// stage S, 32-k step t, 8-k group q, token r of the tile, 8 values, i.e.
// element ((((T * nst + S) * 4 + t) * 64 + q * 16 + r) * 8 + e) holds
// h[16 T + r, 128 S + 32 t + 8 q + e], nst = ceil(f / 128).  The 64 lanes
// (r, q) of a wave then read the 16-byte MFMA B-operand fragments of one
// 32-k step as one contiguous 1 KiB.  A buffer of T token tiles takes
// T * 16 * nst * 128 elements; slots of tokens past M or columns past f are
// never written and never used unmasked.
__device__ __forceinline__ size_t hblk_index(int tok, int col, int nst) {
  return ((((size_t)(tok >> 4) * nst + (col >> 7)) * 4 + ((col >> 5) & 3)) * 64 + ((col >> 3) & 3) * 16 +
          (tok & 15)) * 8 + (col & 7);
}

// Epilogue of a tile: gate/up (h = silu(G) * U, with the folded norm),
// down (y = x + acc) or an fp32 partial tile of a split reduction axis.
enum { DS_EPI_GATEUP = 0, DS_EPI_DOWN = 1, DS_EPI_PARTIAL = 2 };

// LDS of a tile body, in uint4 / float units
template <int NMAT, int MT, int WAVES, bool ASTAGE>
struct DsLds {
  static constexpr int wb = WAVES * NMAT * 256;                 // per-wave weight stages
  static constexpr int ab = ASTAGE ? WAVES * MT * 256 : 1;      // per-wave activation stages
  static constexpr int ssq = WAVES * MT * 16;                   // partial sums of squares
};

// Output rows [row0, row1) (at most 16: one MFMA tile) over stages [zs, ze)
// of the reduction axis (ze < 0: all of it), split over the workgroup's WAVES
// waves.  Tile rows past row1 are loaded with an out-of-range buffer offset
// (zeros, no memory access) and never stored.
// ASTAGE: activations fetched in 256-byte token segments and staged through
// LDS (pays off from about 8 tokens); otherwise read straight from L2 in the
// MFMA operand layout (for one token every lane reads the same 64 bytes).
// COH: the output is written through to the coherence point shared by all
// XCDs (it is read by other workgroups of the same launch).
// KFULL: K is a multiple of the 128-k stage, so every stage is whole and the
// clamps and masks of a partial last stage compile away.
// HBLK: h is in the blocked layout (hblk_index): the gate/up epilogue writes
// it so, and a down tile reads it directly (requires !ASTAGE).
template <int NMAT, int MT, int WAVES, bool FOLD, bool ASTAGE, int EPI, bool COH, bool KFULL = false,
          bool HBLK = false>
__device__ __forceinline__ void ds_tile(
    const uint16_t* __restrict__ act,    // [M, K]: x (FOLD) or h
    const uint16_t* __restrict__ gain,   // [K] (FOLD)
    const uint16_t* __restrict__ w0,     // [N, K]
    const uint16_t* __restrict__ w1,     // [N, K] (NMAT == 2)
    const uint16_t* __restrict__ resid,  // [M, N] (DS_EPI_DOWN)
    uint16_t* __restrict__ out,          // [M, N] bf16 (GATEUP, DOWN)
    float* __restrict__ part,            // [M, N] fp32 (PARTIAL)
    int M, int K, int N, float eps, int row0, int row1, int zs, int ze,
    uint4* __restrict__ wbs, uint4* __restrict__ abs_, float* __restrict__ ssqs) {
  constexpr int ST = 16;  // 16-byte chunks per row per stage (128 k)
  auto cl = [](int v, int hi) { return KFULL ? v : min(v, hi); };
  auto lds_w = [&](int w, int m, int i) -> uint4& { return wbs[(w * NMAT + m) * 256 + i]; };
  auto lds_a = [&](int w, int mt, int i) -> uint4& { return abs_[ASTAGE ? (w * MT + mt) * 256 + i : 0]; };
  auto lds_ssq = [&](int w, int t, int i) -> float& { return ssqs[(w * MT + t) * 16 + i]; };
  // the cross-wave partial tiles reuse each wave's own weight stage once its
  // K loop is done (MT * NMAT * 1 KiB <= NMAT * 4 KiB)
  static_assert(MT <= 4, "partial tiles must fit the weight stage");
  auto red = [&](int w, int t, int m, int e) -> float* {
    return reinterpret_cast<float*>(&lds_w(w, 0, 0)) + ((t * NMAT + m) * 4 + e) * 64;
  };

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int j0 = row0;
  const int K8 = K >> 3;
  const int nst = (K8 + ST - 1) / ST;
  const int z0 = zs, z1 = ze < 0 ? nst : ze;
  const int sb = z0 + (int)(((long)(z1 - z0) * wave) / WAVES);
  const int se = z0 + (int)(((long)(z1 - z0) * (wave + 1)) / WAVES);

  // staged loads: instruction u fetches rows 4u..4u+3, lane -> (row 4u + q,
  // chunk (r - (4u + q)) & 15) and lands at LDS slot u*64 + lane, so chunk c
  // of tile row R sits at slot (R>>2)*64 + (R&3)*16 + ((c + R) & 15)
  // weights through buffer resources: 32-bit byte offsets (matrices < 2 GiB)
  __amdgpu_buffer_rsrc_t rw[NMAT];
  rw[0] = make_rsrc(w0, (long)N * K * 2);
  if (NMAT == 2) rw[NMAT - 1] = make_rsrc(w1, (long)N * K * 2);
  unsigned gw[4];  // byte offset of this lane's row in each instruction
  int cst[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = j0 + 4 * u + q;  // rows past row1 (<= N): nothing loaded, never stored
    cst[u] = (r - (4 * u + q)) & 15;
    // kOutOfRange plus any in-row offset (< 2^31) stays past the resource
    gw[u] = row < row1 ? (unsigned)row * (unsigned)K * 2u : kOutOfRange;
  }
  const int rd_base = (r >> 2) * 64 + (r & 3) * 16;

  // activations are staged the same way: tile "row" = token, instruction u
  // fetches tokens 4u..4u+3 of each 16-token tile (tokens past M are clamped
  // copies of row M-1 that only feed output columns never stored)
  const uint4* pa[MT][4];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int tok = ASTAGE ? t * 16 + 4 * u + q : t * 16 + r;
      pa[t][u] = reinterpret_cast<const uint4*>(act) + (size_t)min(tok, M - 1) * K8;
    }
  const uint4* G4 = reinterpret_cast<const uint4*>(gain);
  // blocked h: this lane's fragment of token tile mt (tokens past M repeat
  // token M-1, as above), in 16-byte units, before the stage and step terms
  static_assert(!HBLK || (!COH && (EPI == DS_EPI_GATEUP || (EPI == DS_EPI_DOWN && !ASTAGE))),
                "blocked h: written by a gate/up tile, read directly by a down tile");
  const uint4* H4 = reinterpret_cast<const uint4*>(act);
  size_t hb[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
    hb[t] = (size_t)t * nst * 256 + q * 16 + (min(t * 16 + r, M - 1) & 15);

  f32x4 acc[NMAT][MT];
  // sums of squares of x: direct layout, token r of tile t (ss[t][0]);
  // staged layout, token 4u + q of tile t (ss[t][u])
  float ss[MT][ASTAGE ? 4 : 1];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
#pragma unroll
    for (int u = 0; u < (ASTAGE ? 4 : 1); ++u) ss[t][u] = 0.f;
#pragma unroll
    for (int m = 0; m < NMAT; ++m) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  struct WB {
    uint4 w[NMAT][4];
  };
  struct AB {
    uint4 a[MT][4];
    uint4 g[FOLD ? 4 : 1];
  };
  // st < 0 marks a prefetch past the slice end: the weight loads then read
  // nothing (out-of-range offset) and the activation loads hit cache
  auto load_w = [&](WB& B, int st_req) {
    const int st = st_req < 0 ? se - 1 : st_req;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = cl(st * ST + cst[u], K8 - 1);
      const unsigned o = st_req < 0 ? kOutOfRange : gw[u] + (unsigned)c * 16u;
#pragma unroll
      for (int m = 0; m < NMAT; ++m) B.w[m][u] = buf_ld_nt(rw[m], o);
    }
  };
  auto load_a = [&](AB& B, int st_req) {
    const int st = st_req < 0 ? se - 1 : st_req;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // staged: chunk cst[u] of token 4u+q; direct: chunk 4u+q of token r
      const int c = cl(st * ST + (ASTAGE ? cst[u] : 4 * u + q), K8 - 1);
      if (HBLK && EPI == DS_EPI_DOWN) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) B.a[mt][u] = H4[hb[mt] + (size_t)(st * 4 + u) * 64];
      } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) B.a[mt][u] = pa[mt][u][c];
      }
      if (FOLD) B.g[u] = G4[c];  // the gain of the same chunk
    }
  };
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
  // the weights of a stage go to LDS first, which frees their registers for
  // the next prefetch before the MFMAs of this stage run; staged activations
  // go to LDS already multiplied by the gain
  auto stage = [&](const WB& B, const AB& A, int st) {
    const bool ragged = !KFULL && (st + 1) * ST > K8;  // only the last stage of a row can be partial
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        uint4 v = B.w[m][u];
        if (ragged) v = keep_or_zero(st * ST + cst[u] < K8, v);
        lds_w(wave, m, u * 64 + lane) = v;
      }
      if (ASTAGE) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          uint4 v = A.a[mt][u];
          if (ragged) v = keep_or_zero(st * ST + cst[u] < K8, v);
          if (FOLD) v = fold(v, A.g[u], ss[mt][ASTAGE ? u : 0]);
          lds_a(wave, mt, u * 64 + lane) = v;
        }
      }
    }
  };
  auto compute = [&](const AB& A, int st) {
    const bool ragged = !KFULL && (st + 1) * ST > K8;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int slot = rd_base + ((4 * t + q + r) & 15);
      uint4 bb[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (ASTAGE) {
          bb[mt] = lds_a(wave, mt, slot);  // chunks past K zeroed when staged
        } else {
          uint4 xa = A.a[mt][t];
          if (ragged) xa = keep_or_zero(st * ST + 4 * t + q < K8, xa);
          bb[mt] = FOLD ? fold(xa, A.g[t], ss[mt][0]) : xa;
        }
      }
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const uint4 af = lds_w(wave, m, slot);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[m][mt] = mfma16(af, bb[mt], acc[m][mt]);
      }
    }
  };

  const int n = se - sb;
  if (ASTAGE && n >= 2) {
    // activations single-buffered: the next stage's are loaded as soon as
    // this stage's are in LDS, ahead of the weights two stages out (loads
    // complete in order, so the wait before a stage leaves those in flight)
    WB X, Y;
    AB A;
    load_w(X, sb);
    load_a(A, sb);
    load_w(Y, sb + 1);
    for (int s = sb;;) {
      __builtin_amdgcn_sched_barrier(0);
      stage(X, A, s);
      __builtin_amdgcn_sched_barrier(0);
      load_a(A, s + 1 < se ? s + 1 : -1);
      load_w(X, s + 2 < se ? s + 2 : -1);
      __builtin_amdgcn_sched_barrier(0);
      compute(A, s);
      if (++s >= se) break;
      __builtin_amdgcn_sched_barrier(0);
      stage(Y, A, s);
      __builtin_amdgcn_sched_barrier(0);
      load_a(A, s + 1 < se ? s + 1 : -1);
      load_w(Y, s + 2 < se ? s + 2 : -1);
      __builtin_amdgcn_sched_barrier(0);
      compute(A, s);
      if (++s >= se) break;
    }
  } else if (n >= 2) {
    // direct activations are read by the MFMA loop: two full batches
    WB X, Y;
    AB XA, YA;
    load_w(X, sb);
    load_a(XA, sb);
    load_w(Y, sb + 1);
    load_a(YA, sb + 1);
    for (int s = sb;;) {
      __builtin_amdgcn_sched_barrier(0);
      stage(X, XA, s);
      __builtin_amdgcn_sched_barrier(0);
      load_w(X, s + 2 < se ? s + 2 : -1);
      __builtin_amdgcn_sched_barrier(0);
      compute(XA, s);
      __builtin_amdgcn_sched_barrier(0);
      load_a(XA, s + 2 < se ? s + 2 : -1);
      if (++s >= se) break;
      __builtin_amdgcn_sched_barrier(0);
      stage(Y, YA, s);
      __builtin_amdgcn_sched_barrier(0);
      load_w(Y, s + 2 < se ? s + 2 : -1);
      __builtin_amdgcn_sched_barrier(0);
      compute(YA, s);
      __builtin_amdgcn_sched_barrier(0);
      load_a(YA, s + 2 < se ? s + 2 : -1);
      if (++s >= se) break;
    }
  } else if (n == 1) {
    WB X;
    AB A;
    load_w(X, sb);
    load_a(A, sb);
    stage(X, A, sb);
    compute(A, sb);
  }

  // ---- fixed-order reduction over the WAVES K slices
#pragma unroll
  for (int t = 0; t < MT; ++t) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) red(wave, t, m, e)[lane] = acc[m][t][e];
    if (FOLD) {
      if (ASTAGE) {
        // token 4u + q: sum over the 16 lanes of group q (r = 0..15)
#pragma unroll
        for (int u = 0; u < (ASTAGE ? 4 : 1); ++u) {
          float v = ss[t][u];
          v += __shfl_xor(v, 1, 64);
          v += __shfl_xor(v, 2, 64);
          v += __shfl_xor(v, 4, 64);
          v += __shfl_xor(v, 8, 64);
          if (r == 0) lds_ssq(wave, t, 4 * u + q) = v;
        }
      } else {
        // token r: sum over the four lane groups q
        float v = ss[t][0];
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        if (q == 0) lds_ssq(wave, t, r) = v;
      }
    }
  }
  __syncthreads();
  for (int t = wave; t < MT; t += WAVES) {
    const int tok = t * 16 + r;
    const int col = j0 + 4 * q;  // four consecutive output columns
    float v0[4], v1[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        s0 += red(w, t, 0, e)[lane];
        if (NMAT == 2) s1 += red(w, t, NMAT - 1, e)[lane];
      }
      v0[e] = s0;
      v1[e] = s1;
    }
    if (tok < M && col < row1) {
      const size_t off = (size_t)tok * N + col;
      // four columns inside the range and 4-element aligned: vector access;
      // otherwise (the edge of an unaligned row range) element by element
      const bool whole = col + 4 <= row1 && (off & 3) == 0;
      const int nc = min(4, row1 - col);
      if (EPI == DS_EPI_PARTIAL) {
        float* pp = part + off;
        if (COH) {
          coh_st8(pp, __float_as_uint(v0[0]), __float_as_uint(v0[1]));
          coh_st8(pp + 2, __float_as_uint(v0[2]), __float_as_uint(v0[3]));
        } else if (whole) {
          *reinterpret_cast<float4*>(pp) = make_float4(v0[0], v0[1], v0[2], v0[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (e < nc) pp[e] = v0[e];
        }
        continue;
      }
      if (NMAT == 2) {
        float rs = 1.f;
        if (FOLD) {
          float sum = 0.f;
#pragma unroll
          for (int w = 0; w < WAVES; ++w) sum += lds_ssq(w, t, r);
          rs = 1.0f / __builtin_sqrtf(sum / (float)K + eps);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) v0[e] = silu_mul(v0[e] * rs, v1[e] * rs);
      } else if (whole) {
        const uint2 xr = *reinterpret_cast<const uint2*>(resid + off);
        v0[0] += bf2f(xr.x & 0xFFFFu);
        v0[1] += bf2f(xr.x >> 16);
        v0[2] += bf2f(xr.y & 0xFFFFu);
        v0[3] += bf2f(xr.y >> 16);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e < nc) v0[e] += bf2f(resid[off + e]);
      }
      uint2 o;
      o.x = pack_bf16x2(v0[0], v0[1]);
      o.y = pack_bf16x2(v0[2], v0[3]);
      if (HBLK && NMAT == 2) {
        // blocked h: four columns starting at a multiple of 4 share one
        // 8-byte group; otherwise element by element
        const int nstN = (N + 127) >> 7;
        if (col + 4 <= row1 && (col & 3) == 0) {
          *reinterpret_cast<uint2*>(out + hblk_index(tok, col, nstN)) = o;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (e < nc) {
              const uint32_t w = e < 2 ? o.x : o.y;
              out[hblk_index(tok, col + e, nstN)] = (uint16_t)(e & 1 ? w >> 16 : w & 0xFFFFu);
            }
        }
      } else if (COH) {
        coh_st8(out + off, o.x, o.y);
      } else if (whole) {
        *reinterpret_cast<uint2*>(out + off) = o;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e < nc) {
            const uint32_t w = e < 2 ? o.x : o.y;
            out[off + e] = (uint16_t)(e & 1 ? w >> 16 : w & 0xFFFFu);
          }
      }
    }
  }
}

template <int NMAT, int MT, int WAVES, bool FOLD, bool ASTAGE, bool KFULL, bool HBLK>
__global__ __launch_bounds__(WAVES * 64)
__attribute__((amdgpu_waves_per_eu(NMAT == 2 && MT == 1 && ASTAGE ? FFN_DS_GU_STAGED_WPE : 1)))
void decode_stream(
    const uint16_t* __restrict__ act,    // [M, K]: x (FOLD) or h
    const uint16_t* __restrict__ gain,   // [K] (FOLD)
    const uint16_t* __restrict__ w0,     // [N, K]
    const uint16_t* __restrict__ w1,     // [N, K] (NMAT == 2)
    const uint16_t* __restrict__ resid,  // [M, N] (NMAT == 1)
    uint16_t* __restrict__ out,          // [M, N]
    int M, int K, int N, float eps) {
  using L = DsLds<NMAT, MT, WAVES, ASTAGE>;
  __shared__ uint4 wb[L::wb];
  __shared__ uint4 ab[L::ab];
  __shared__ float ssq[L::ssq];
  // workgroup b of G owns rows [b N / G, (b + 1) N / G): at most 16 rows
  // (G >= N / 16), as even a share of the rows as the grid allows
  const int row0 = (int)(((long)blockIdx.x * N) / gridDim.x);
  const int row1 = (int)(((long)(blockIdx.x + 1) * N) / gridDim.x);
  ds_tile<NMAT, MT, WAVES, FOLD, ASTAGE, NMAT == 2 ? DS_EPI_GATEUP : DS_EPI_DOWN, false, KFULL, HBLK>(
      act, gain, w0, w1, resid, out, nullptr, M, K, N, eps, row0, row1, 0, -1, wb, ab, ssq);
}

// Tokens per launch with row-major h (two 16-token tiles keep the LDS
// stages within budget): the API walks larger decode batches in chunks of
// this size.  With blocked h the gate/up kernel takes up to
// decode_gateup_tokens() and the down kernel every token.
int decode_chunk_tokens() { return 32; }
int decode_max_tokens() { return 64; }

// Balanced grids.  A 16-row tile per workgroup leaves the compute
// units unevenly loaded when the tile count is not a multiple of the
// workgroups that fit at once (f = 11008: 688 tiles on 768 slots, three
// tiles on 176 CUs and two on 80; the kernel lasts as long as the busiest
// CU).  Instead the grid is sized to whole rounds of resident workgroups and
// each takes an equal share (<= 16) of the rows.  Past one round, the grid
// is a whole multiple of the compute units (policy 3 of stream_groups), so
// every CU still gets the same number of rows: 1.5 rounds of 14-15 rows
// instead of 1.34 rounds of 16 (M = 1 / 8 / 24 / 48 / 64 at f = 11008:
// 0.4-1.7% faster; d = 5120, f = 13824 at 16 tokens 89.2 -> 85.6 us;
// bitwise identical).  FFN_DS_BALANCE 0 keeps one workgroup per 16-row
// tile, 1 balances single rounds only.
#ifndef FFN_DS_BALANCE
#define FFN_DS_BALANCE 3
#endif
// The down projections too: at d = 5120 its 320 row tiles on 512 slots
// (two 8-wave workgroups per CU) left 64 CUs with two tiles; balanced, every
// CU takes 20 rows (block 93.4 -> 88.8 us at 16 tokens, d = 6144 120.9 ->
// 116.1 us; bitwise identical, other shapes unchanged).
#ifndef FFN_DS_DN_BALANCE
#define FFN_DS_DN_BALANCE 1
#endif

template <int NMAT, int MT, int WAVES, bool FOLD, bool ASTAGE, bool KFULL, bool HBLK>
static void launch_one(const uint16_t* a, const uint16_t* gg, const uint16_t* p0,
                       const uint16_t* p1, const uint16_t* rr, uint16_t* o, int M, int K, int N,
                       float eps, hipStream_t s) {
  auto kern = decode_stream<NMAT, MT, WAVES, FOLD, ASTAGE, KFULL, HBLK>;
  // the occupancy of a kernel is fixed: computed once (the library assumes
  // every device it runs on is the same model)
  static const int slots = NMAT == 2 || FFN_DS_DN_BALANCE ? resident_slots(kern, WAVES * 64) : 0;
  static const int cus = device_cus();
  const int groups = NMAT == 2 || FFN_DS_DN_BALANCE ? stream_groups(N, slots, FFN_DS_BALANCE, cus) : (N + 15) / 16;
  FFN_DISPATCH(kern, dim3((unsigned)groups), dim3(WAVES * 64), 0, s, a, gg, p0, p1, rr, o, M, K, N, eps);
}

// Blocked h (see hblk_index) between the decode gate/up and down kernels;
// FFN_DS_HBLK 0 keeps h row-major (the down kernel then stages 9..32-token
// activations through LDS).
#ifndef FFN_DS_HBLK
#define FFN_DS_HBLK 1
#endif

int decode_h_blocked() { return FFN_DS_HBLK; }

// With blocked h the gate/up kernel also takes 33..64 tokens (three or four
// 16-token tiles) in one launch, so the weights stream once per call.
// FFN_DS_GU64 0 keeps 32-token launches.
#ifndef FFN_DS_GU64
#define FFN_DS_GU64 1
#endif
int decode_gateup_tokens() { return FFN_DS_HBLK && FFN_DS_GU64 ? 64 : 32; }

template <int NMAT, int MT, int WAVES, bool FOLD, bool ASTAGE, bool HBLK>
static void launch_k(const uint16_t* a, const uint16_t* gg, const uint16_t* p0, const uint16_t* p1,
                     const uint16_t* rr, uint16_t* o, int M, int K, int N, float eps, hipStream_t s) {
  if (K % 128 == 0)  // whole 128-k stages
    launch_one<NMAT, MT, WAVES, FOLD, ASTAGE, true, HBLK>(a, gg, p0, p1, rr, o, M, K, N, eps, s);
  else
    launch_one<NMAT, MT, WAVES, FOLD, ASTAGE, false, HBLK>(a, gg, p0, p1, rr, o, M, K, N, eps, s);
}

// Token-count dispatch: activations read directly for up to 8 tokens and
// staged through LDS for 9..16 (one token tile) and 17..32 (two).
template <int NMAT, int WAVES, bool FOLD, bool HBLK>
static void launch_by_m(const uint16_t* a, const uint16_t* gg, const uint16_t* p0, const uint16_t* p1,
                        const uint16_t* rr, uint16_t* o, int M, int K, int N, float eps, hipStream_t s) {
  if (M <= 8) launch_k<NMAT, 1, WAVES, FOLD, false, HBLK>(a, gg, p0, p1, rr, o, M, K, N, eps, s);
  else if (M <= 16) launch_k<NMAT, 1, WAVES, FOLD, true, HBLK>(a, gg, p0, p1, rr, o, M, K, N, eps, s);
  else launch_k<NMAT, 2, WAVES, FOLD, true, HBLK>(a, gg, p0, p1, rr, o, M, K, N, eps, s);
}

// hblk: a gate/up kernel writes h blocked; a down kernel reads blocked h,
// directly at every token count, up to four token tiles (64 tokens) per
// launch.
template <int NMAT, int WAVES, bool FOLD>
static hipError_t launch_ds(const void* act, const void* gain, const void* w0, const void* w1,
                            const void* resid, void* out, int M, int K, int N, float eps, bool hblk,
                            hipStream_t s) {
  const uint16_t* a = (const uint16_t*)act;
  const uint16_t* gg = (const uint16_t*)gain;
  const uint16_t* p0 = (const uint16_t*)w0;
  const uint16_t* p1 = (const uint16_t*)w1;
  const uint16_t* rr = (const uint16_t*)resid;
  uint16_t* o = (uint16_t*)out;
  if constexpr (NMAT == 1) {
    if (!hblk) launch_by_m<NMAT, WAVES, FOLD, false>(a, gg, p0, p1, rr, o, M, K, N, eps, s);
    else if (M <= 16) launch_k<NMAT, 1, WAVES, FOLD, false, true>(a, gg, p0, p1, rr, o, M, K, N, eps, s);
    else if (M <= 32) launch_k<NMAT, 2, WAVES, FOLD, false, true>(a, gg, p0, p1, rr, o, M, K, N, eps, s);
    else if (M <= 48) launch_k<NMAT, 3, WAVES, FOLD, false, true>(a, gg, p0, p1, rr, o, M, K, N, eps, s);
    else launch_k<NMAT, 4, WAVES, FOLD, false, true>(a, gg, p0, p1, rr, o, M, K, N, eps, s);
  } else {
    if (hblk && M > 32) {
      // 33..64 tokens in one launch.  Every workgroup stages all the tokens'
      // activations (M/32 bytes per weight byte it streams), so the choice
      // rests on how many 16-row tiles there are per compute unit (measured
      // at d = 2048..8192, f = 1376..14336): below one, two 32-token
      // launches keep more waves in flight; up to 2.5, two-wave workgroups
      // (the K range split over both); past that, one wave per workgroup.
      const int tiles = (N + 15) / 16, cus = device_cus();
      if (tiles < cus) {
        // tokens 32.. start at token tile 2 of blocked h
        const size_t h2 = (size_t)32 * ((N + 127) / 128) * 128;
        launch_by_m<NMAT, WAVES, FOLD, true>(a, gg, p0, p1, rr, o, 32, K, N, eps, s);
        launch_by_m<NMAT, WAVES, FOLD, true>(a + (size_t)32 * K, gg, p0, p1, rr, o + h2, M - 32, K, N, eps, s);
      } else if (2 * tiles < 5 * cus) {
        if (M > 48) launch_k<NMAT, 4, 2, FOLD, true, true>(a, gg, p0, p1, rr, o, M, K, N, eps, s);
        else launch_k<NMAT, 3, 2, FOLD, true, true>(a, gg, p0, p1, rr, o, M, K, N, eps, s);
      } else {
        if (M > 48) launch_k<NMAT, 4, 1, FOLD, true, true>(a, gg, p0, p1, rr, o, M, K, N, eps, s);
        else launch_k<NMAT, 3, 1, FOLD, true, true>(a, gg, p0, p1, rr, o, M, K, N, eps, s);
      }
    } else if (hblk) {
      launch_by_m<NMAT, WAVES, FOLD, true>(a, gg, p0, p1, rr, o, M, K, N, eps, s);
    } else {
      launch_by_m<NMAT, WAVES, FOLD, false>(a, gg, p0, p1, rr, o, M, K, N, eps, s);
    }
  }
  return hipGetLastError();
}

hipError_t launch_decode_gateup_norm(const void* x, const void* g, const void* wg, const void* wu,
                                     void* h, int M, int d, int f, float eps, hipStream_t s) {
  return launch_ds<2, FFN_DS_GU_WAVES, true>(x, g, wg, wu, nullptr, h, M, d, f, eps, FFN_DS_HBLK != 0, s);
}

hipError_t launch_decode_down(const void* h, const void* wd, const void* x, void* y, int M,
                              int d, int f, bool h_blocked, hipStream_t s) {
  return launch_ds<1, FFN_DS_DN_WAVES, false>(h, nullptr, wd, nullptr, x, y, M, f, d, 0.f, h_blocked, s);
}

// ---------------------------------------------------------------------------
// Single-dispatch decode block: the megakernel schedule of "Megakernels on
// Mac" ("The 27.65 ms estimate" onward: one launch, work items that wait on
// completion flags instead of dispatch boundaries), for 1..16 tokens.
//
// Workgroups take work items from a ticket counter: first the f/16 gate/up
// tiles (norm folded, as in decode_stream), then the down projection as
// (tile, K range) items, range-major.  A down item for K range z needs the h
// columns of z, i.e. the gate/up tiles of z: their count is kept per range.
// Every dependency points to a smaller ticket, and tickets are handed out in
// order, so the items waited for are already owned by running workgroups and
// never wait themselves: no deadlock whatever the residency.  The waits are
// bounded: past spin_limit polls a workgroup records an error in counter 1
// and stops waiting (the result is then wrong, but the kernel ends).
// h and the fp32 partials cross XCDs: they are written with agent-scope
// atomic stores (written through to the coherence point, so no cache
// write-back is needed), each workgroup waits for its stores to complete
// before it increments a counter; a down item, once its range is complete,
// invalidates its caches (agent-scope acquire) and then reads h through
// them, and the partials are read with agent-scope atomic loads.  The last of a down tile's S items adds the S partials
// in range order and the residual: the same order as the two-pass
// split-K reduce, deterministic.
// Counters (caller's workspace, cleared by a preceding launch): [0] ticket,
// [1] error, [2, 2+S) gate/up tiles done per range, [2+S, 2+S+d/16) down
// items done per output tile.
constexpr int kPersistWaves = 4;

__global__ void clear_u32(unsigned* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Two waves per SIMD: at three the two tile bodies together spill.
#ifndef FFN_DS_PERSIST_WPE
#define FFN_DS_PERSIST_WPE 2
#endif

__global__ __launch_bounds__(kPersistWaves * 64) __attribute__((amdgpu_waves_per_eu(FFN_DS_PERSIST_WPE)))
void decode_persistent(const uint16_t* __restrict__ x, const uint16_t* __restrict__ g,
                       const uint16_t* __restrict__ wg, const uint16_t* __restrict__ wu,
                       const uint16_t* __restrict__ wd, uint16_t* __restrict__ h,
                       float* __restrict__ part, uint16_t* __restrict__ y,
                       unsigned* __restrict__ ctr, int M, int d, int f, float eps, int splits,
                       unsigned spin_limit) {
  constexpr int W = kPersistWaves;
  using LG = DsLds<2, 1, W, true>;  // the gate/up body needs the most LDS
  static_assert(DsLds<1, 1, W, true>::wb <= LG::wb && DsLds<1, 1, W, true>::ab <= LG::ab, "");
  __shared__ uint4 wb[LG::wb];
  __shared__ uint4 ab[LG::ab];
  __shared__ float ssq[LG::ssq];
  __shared__ int s_item, s_last;

  const int n_gu = (f + 15) / 16, n_dt = (d + 15) / 16;
  const int n_items = n_gu + n_dt * splits;
  const int nst_f = (f / 8 + 15) / 16;  // 128-k stages of the down projection
  unsigned* done_gu = ctr + 2;
  unsigned* done_dt = ctr + 2 + splits;
  auto range_lo = [&](int z) { return (int)(((long)nst_f * z) / splits); };

  // (fetching the next ticket ahead of time was measured slower: it binds
  // the last gate/up tiles to workgroups before they are free)
  for (;;) {
    if (threadIdx.x == 0)
      s_item = (int)__hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int item = s_item;
    if (item >= n_items) break;
    if (item < n_gu) {
      ds_tile<2, 1, W, true, true, DS_EPI_GATEUP, true>(x, g, wg, wu, nullptr, h, nullptr, M, d, f,
                                                         eps, item * 16, min(item * 16 + 16, f), 0, -1,
                                                         wb, ab, ssq);
      // h stores complete (written through) before the tile is counted
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      if (threadIdx.x == 0) {
        const int st = item / 8;  // the 128-k stage of h this tile's 16 columns fall in
        int z = 0;
        while (z + 1 < splits && range_lo(z + 1) <= st) ++z;
        __hip_atomic_fetch_add(done_gu + z, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      const int dn = item - n_gu;
      const int z = dn / n_dt, tile = dn % n_dt;  // range-major: early ranges first
      const int zs = range_lo(z), ze = range_lo(z + 1);
      if (threadIdx.x == 0) {
        const unsigned need = (unsigned)(min(ze * 8, n_gu) - min(zs * 8, n_gu));
        unsigned spins = 0;
        while (__hip_atomic_load(done_gu + z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
          if (++spins > spin_limit) {
            __hip_atomic_store(ctr + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(8);
        }
        // acquire: drop possibly stale cached lines of h (an earlier call's)
        // before this workgroup reads it through the caches
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      }
      __syncthreads();
      ds_tile<1, 1, W, false, true, DS_EPI_PARTIAL, true>(h, nullptr, wd, nullptr, nullptr, nullptr,
                                                         part + (size_t)z * M * d, M, f, d, 0.f,
                                                         tile * 16, min(tile * 16 + 16, d), zs, ze,
                                                         wb, ab, ssq);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // partial stores complete before counting
      __syncthreads();
      if (threadIdx.x == 0) {
        const unsigned old =
            __hip_atomic_fetch_add(done_dt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = old == (unsigned)(splits - 1);
      }
      __syncthreads();
      if (s_last) {
        // y = x + sum_z partial[z], one output per thread (16 columns x M tokens)
        for (int i = threadIdx.x; i < 16 * M; i += W * 64) {
          const int tok = i >> 4, col = tile * 16 + (i & 15);
          if (col < d) {
            const size_t off = (size_t)tok * d + col;
            float v = 0.f;
            for (int zz = 0; zz < splits; ++zz)
              v += __hip_atomic_load(part + (size_t)zz * M * d + off, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
            y[off] = f2bf(bf2f(x[off]) + v);
          }
        }
      }
    }
    __syncthreads();  // s_item and s_last are rewritten by the next item
  }
}

#ifndef FFN_DS_PERSIST_SPLITS
#define FFN_DS_PERSIST_SPLITS 1
#endif

int decode_persistent_splits(int d, int f) {
  (void)d;
  const int nst_f = (f / 8 + 15) / 16;
  const int sp = FFN_DS_PERSIST_SPLITS;
  return nst_f < sp ? (nst_f > 0 ? nst_f : 1) : sp;
}

size_t decode_persistent_counters(int d, int splits) { return 2 + (size_t)splits + (d + 15) / 16; }

hipError_t launch_decode_persistent(const void* x, const void* g, const void* wg, const void* wu,
                                    const void* wd, void* h, float* part, unsigned* ctr, void* y,
                                    int M, int d, int f, float eps, hipStream_t s) {
  const int splits = decode_persistent_splits(d, f);
  const int nc = (int)decode_persistent_counters(d, splits);
  FFN_DISPATCH(clear_u32, dim3((unsigned)((nc + 255) / 256)), dim3(256), 0, s, ctr, nc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int cus = device_cus();
  const int n_items = (f + 15) / 16 + ((d + 15) / 16) * splits;
  const int grid = n_items < FFN_DS_PERSIST_WPE * cus ? n_items : FFN_DS_PERSIST_WPE * cus;
  FFN_DISPATCH(decode_persistent, dim3((unsigned)grid), dim3(kPersistWaves * 64), 0, s,
                     (const uint16_t*)x, (const uint16_t*)g, (const uint16_t*)wg,
                     (const uint16_t*)wu, (const uint16_t*)wd, (uint16_t*)h, part, (uint16_t*)y,
                     ctr, M, d, f, eps, splits, 1u << 20);
  return hipGetLastError();
}

}  // namespace ffn
