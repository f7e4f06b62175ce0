// Prefill-regime projections (thousands of tokens) on bf16 MFMA with
// LDS-staged tiles.
//
//   C[m][n] = sum_k A[m][k] * W[n][k]      A = activations [M,K], W = weights [N,K]
// with three epilogues:
//   STORE    : C -> bf16                                  (split gate / split up)
//   SWIGLU   : h = silu(A Wg^T) * (A Wu^T) -> bf16         (fused gate/up)
//   RESIDUAL : y = resid + C -> bf16                       (down projection)
// The fused-vs-split choice for gate/up is the subject of "Unfusing a Kernel
// Made It 1.63x Faster", Finding 1 (fusion saves a memory pass but cost the
// original kernel 64 extra accumulators per thread); "Finding 3" shows
// threadgroup memory as the binding resource on that chip.
//
// gfx950 design (not the page's): the fused kernel is register-neutral.
// A workgroup's weight tile holds BN/2 gate rows and the SAME BN/2 up rows,
// and each wave's sub-tile covers matching gate and up rows, so a lane ends
// the K loop with G and U for the same (token, column) pairs and applies
// silu(G)*U in registers; the accumulator count equals the split GEMM's.
//
//  * v_mfma_f32_16x16x32_bf16, A operand = 16 weight rows, B operand = 16
//    tokens; a lane's result is 4 consecutive output columns of one token.
//    (A 32x32x16 variant of this kernel measured slower in interleaved A/B
//    runs on gfx950, so the 16x16 shape stays.)
//  * BK = 64: every LDS row is 128 B = 8 chunks of 16 B; chunk c of row r is
//    stored at c ^ (r & 7).  Measured on gfx950 with the LDS bank-conflict
//    counter: the fragment reads (16 rows x one chunk column) and the tile
//    writes are then conflict free, a ds_read_b128 takes 4 cycles; adding
//    row bit 3 to the XOR doubles the read time.
//  * two LDS stages and a register prefetch two K tiles ahead; the writes of
//    the next tile into the free stage are interleaved with the MFMAs of the
//    current one; one barrier per K tile.  When K is a multiple of 64 the
//    tiles instead go from memory straight into LDS (gemm_dma below): no
//    staging registers and no LDS write instructions, measured 2-3% faster
//    on the prefill block; BK = 32 with 3-5 stages measured slower (twice
//    the barriers).
//  * for whole tiles (M % 256, N % tile width, K % 128 all zero) the eight
//    waves run as two groups of four, one wave of each group per SIMD, half
//    a k-step apart: while one wave of a SIMD issues its k-step's MFMAs the
//    other reads its next fragments from LDS (ping-pong), with a barrier
//    between phases.  Each lane's fragment addresses are one base register
//    per k-step plus immediate offsets, and the DMA sources one register per
//    operand plus a scalar offset, so the kernel fits two waves per SIMD
//    without spills.  Measured against the one-group schedule: fused gate/up
//    GEMM 3-5% faster, down GEMM within +-2%.  With the tile DMA removed the
//    same loop runs at ~2.07 PFLOP/s (MFMAs alone ~2.2): the time left is the
//    wait for the next tile's global->LDS loads, which two 64 KB stages
//    cannot hide further (a third does not fit in 160 KB of LDS).
//  * the residual epilogue issues all of a lane's residual loads before the
//    first add, one wait per tile instead of one per 16x16 sub-tile.
//  * workgroups are dispatched round-robin over the 8 XCDs; tile ids are
//    remapped so each XCD works on a contiguous range of tiles, grouped 8
//    token tiles deep (2 for the down projection), so concurrently running
//    tiles share operands in the XCD's own L2.
#include "common.h"
#include "launch.h"

#include <type_traits>
#include <utility>

namespace ffn {

enum { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_RESIDUAL = 2 };

__device__ __forceinline__ int swz(int row) { return row & 7; }

// FOLD (SWIGLU only): the RMSNorm is folded in.  act is x; every token
// chunk is multiplied by the gain on its way from registers to LDS (the
// operand is bf16(x * g), as in the decode kernels) while the thread sums
// the squares of x; the epilogue scales G and U by r_m = 1/sqrt(sum/K + eps)
// once the whole row's sum is known (W n = r_m W (x * g)).
template <int BM, int BN, int WM, int WN, int EPI, bool FOLD = false>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bf16(
    const uint16_t* __restrict__ act,    // [M, K]: n, or x (FOLD)
    const uint16_t* __restrict__ w0,     // [N, K]  (gate for SWIGLU)
    const uint16_t* __restrict__ w1,     // [N, K]  (up for SWIGLU)
    const uint16_t* __restrict__ resid,  // [M, N]  (RESIDUAL)
    uint16_t* __restrict__ out,          // [M, N]
    int M, int N, int K, const uint16_t* __restrict__ gain = nullptr, float eps = 0.f) {
  static_assert(!FOLD || EPI == EPI_SWIGLU, "the norm folds into the fused gate/up GEMM only");
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM;  // tokens per wave
  constexpr int TN = BN / WN;  // weight rows per wave (half gate, half up for SWIGLU)
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int BNO = EPI == EPI_SWIGLU ? BN / 2 : BN;  // output columns per tile
  constexpr int ROWS = BN + BM;                           // LDS rows per stage
  constexpr int CH = ROWS * 8 / NT;                       // 16-byte chunks per thread per stage
  static_assert(ROWS * 8 % NT == 0 && (BN * 8) % NT == 0, "tile/thread mismatch");
  static_assert(TM % 16 == 0 && TN % 16 == 0 && (EPI != EPI_SWIGLU || FN % 2 == 0), "bad wave tile");
  static_assert((NT / 8) % 8 == 0, "row stride per chunk must keep the swizzle");
  static_assert(EPI != EPI_SWIGLU || (BN / 2) % (NT / 8) == 0, "gate/up rows must split on chunk boundaries");

  extern __shared__ uint4 lds[];  // [2][ROWS][8]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int K8 = K >> 3;
  const int nkt = (K8 + 7) >> 3;

  // ---- tile coordinates: XCD-contiguous, then grouped 8 token tiles deep
  const int ntm = (M + BM - 1) / BM, ntn = (N + BNO - 1) / BNO;
  const int T = ntm * ntn;
  int L = blockIdx.x;
  if ((T & 7) == 0) L = (L & 7) * (T >> 3) + (L >> 3);
  constexpr int GM = 8;
  const int group = L / (GM * ntn);
  const int first_m = group * GM;
  const int gm = min(ntm - first_m, GM);
  const int inner = L - group * GM * ntn;
  const int tm = first_m + inner % gm;
  const int tn = inner / gm;
  const int m0 = tm * BM, n0 = tn * BNO;

  // ---- per-thread global chunk sources (fixed over K).  Chunk i of this
  // thread is LDS row i*(NT/8) + tid/8, 16-byte column tid%8; since NT/8 is a
  // multiple of 8 the swizzle of every such row is swz(tid/8).  Rows past M
  // or N are clamped to the last valid row: they only feed output rows or
  // columns that are never stored, so they need no zeroing.  Only the ragged
  // last K tile is masked (in store_tile, after the MFMAs of the previous
  // tile, so the loads' latency stays hidden behind them).
  constexpr int CW = BN * 8 / NT;  // chunks per thread that come from weights
  const int crow = tid >> 3, ccol = tid & 7;
  const int sw_st = ccol ^ swz(crow);
  int off[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int row = i * (NT / 8) + crow;
    if (i < CW) {
      int wr = n0 + row;
      if (EPI == EPI_SWIGLU && row >= BN / 2) wr = n0 + row - BN / 2;
      off[i] = min(wr, N - 1) * K8;
    } else {
      off[i] = min(m0 + row - BN, M - 1) * K8;
    }
  }
  const uint4* A4 = reinterpret_cast<const uint4*>(act);
  const uint4* W0 = reinterpret_cast<const uint4*>(w0);
  const uint4* W1 = reinterpret_cast<const uint4*>(EPI == EPI_SWIGLU ? w1 : w0);

  uint4 pre[CH];
  uint4 gpre;                        // FOLD: the gain chunk of the prefetched tile
  float ssq[FOLD ? CH - CW : 1];     // FOLD: sums of squares of this thread's token rows
#pragma unroll
  for (int i = 0; i < (FOLD ? CH - CW : 1); ++i) ssq[i] = 0.f;
  const uint4* G4 = reinterpret_cast<const uint4*>(gain);
  auto load_tile = [&](int kt) {
    const int kc = min(kt * 8 + ccol, K8 - 1);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const uint4* base = i < CW ? ((EPI == EPI_SWIGLU && i >= CW / 2) ? W1 : W0) : A4;
      pre[i] = base[off[i] + kc];
    }
    if (FOLD) gpre = G4[kc];
  };
  auto store_tile = [&](int stage, int kt) {
    uint4* L0 = lds + stage * ROWS * 8 + crow * 8 + sw_st;
    if ((kt + 1) * 8 > K8) {  // ragged last K tile: zero the chunks past K
      const bool kin = kt * 8 + ccol < K8;
#pragma unroll
      for (int i = 0; i < CH; ++i) pre[i] = keep_or_zero(kin, pre[i]);
    }
    if (FOLD) {
      // token chunks: x * g in fp32, rounded once to bf16; sum of x^2
      float gf[8];
      unpack8(gpre, gf);
#pragma unroll
      for (int i = CW; i < CH; ++i) {
        float xf[8];
        unpack8(pre[i], xf);
        ssq[FOLD ? i - CW : 0] = sumsq8(pre[i], ssq[FOLD ? i - CW : 0]);
#pragma unroll
        for (int e = 0; e < 8; ++e) xf[e] *= gf[e];
        pre[i] = pack8(xf);
      }
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) L0[i * (NT / 8) * 8] = pre[i];
  };

  // LDS rows read by this lane's fragments; all are congruent to fr mod 16,
  // so they share the swizzle swz(fr).
  const int fr = lane & 15, fq = lane >> 4;
  const int sw_ld = swz(fr);
  int arow[FN], brow[FM];
#pragma unroll
  for (int t = 0; t < FN; ++t) {
    if (EPI == EPI_SWIGLU) {
      const int half = t / (FN / 2), tt = t % (FN / 2);
      arow[t] = half * (BN / 2) + wn * (TN / 2) + tt * 16 + fr;
    } else {
      arow[t] = wn * TN + t * 16 + fr;
    }
  }
#pragma unroll
  for (int t = 0; t < FM; ++t) brow[t] = BN + wm * TM + t * 16 + fr;

  f32x4 acc[FN][FM];
#pragma unroll
  for (int a = 0; a < FN; ++a)
#pragma unroll
    for (int b = 0; b < FM; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Pipeline: LDS stage kt&1 holds tile kt, registers `pre` hold tile kt+1.
  // Iteration kt: fragment reads of k-step 0, then its MFMAs interleaved with
  // the LDS writes of tile kt+1 into the other stage (read by everyone in
  // iteration kt-1, which ended with a barrier), then the global loads of
  // tile kt+2 (a whole iteration to land), then k-step 1, then one barrier.
  auto compute_ks = [&](const uint4* L0, int ks, uint4 (&af)[FN], uint4 (&bfr)[FM]) {
    const int ch = ks * 4 + fq;
#pragma unroll
    for (int t = 0; t < FN; ++t) af[t] = L0[arow[t] * 8 + (ch ^ sw_ld)];
#pragma unroll
    for (int t = 0; t < FM; ++t) bfr[t] = L0[brow[t] * 8 + (ch ^ sw_ld)];
  };
  auto mfmas = [&](const uint4 (&af)[FN], const uint4 (&bfr)[FM]) {
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
      for (int b = 0; b < FM; ++b) acc[a][b] = mfma16(af[a], bfr[b], acc[a][b]);
  };
  auto iter = [&](int kt, auto do_store, auto do_load) {
    const uint4* L0 = lds + (kt & 1) * ROWS * 8;
    uint4 af[FN], bfr[FM];
    // FOLD: the gain multiply needs registers of its own, so its tile goes
    // to LDS before the fragments are live rather than between the MFMAs
    if (FOLD && decltype(do_store)::value) store_tile((kt + 1) & 1, kt + 1);
    compute_ks(L0, 0, af, bfr);
    if (!FOLD && decltype(do_store)::value) store_tile((kt + 1) & 1, kt + 1);
    mfmas(af, bfr);
    if (!FOLD && decltype(do_store)::value) {
      // 12 fragment reads, then 4 MFMAs per LDS write
      __builtin_amdgcn_sched_group_barrier(0x100, FN + FM, 0);
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, FN * FM / CH, 0);
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      }
    }
    if (decltype(do_load)::value) load_tile(kt + 2);
    compute_ks(L0, 1, af, bfr);
    mfmas(af, bfr);
    __syncthreads();
  };
  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;
  load_tile(0);
  store_tile(0, 0);
  if (nkt > 1) load_tile(1);
  __syncthreads();
  int kt = 0;
  for (; kt + 2 < nkt; ++kt) iter(kt, T_{}, T_{});
  if (kt + 1 < nkt) iter(kt++, T_{}, F_{});
  iter(kt, F_{}, F_{});

  // ---- FOLD: r_m of the tile's token rows.  A row's chunks are held by the
  // 8 consecutive threads with its crow (ccol = 0..7); the last K loop
  // iteration ended with a barrier, so the stages are free for the r table.
  float* rtab = reinterpret_cast<float*>(lds);
  if (FOLD) {
#pragma unroll
    for (int i = 0; i < (FOLD ? CH - CW : 1); ++i) {
      float v = ssq[i];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      if (ccol == 0) rtab[i * (NT / 8) + crow] = 1.0f / __builtin_sqrtf(v / (float)K + eps);
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds D[4*fq + e][fr] of every (a, b) sub-tile
  if (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int a = 0; a < FN / 2; ++a) {
      const int col = n0 + wn * (TN / 2) + a * 16 + 4 * fq;
#pragma unroll
      for (int b = 0; b < FM; ++b) {
        const int tok = m0 + wm * TM + b * 16 + fr;
        if (tok < M && col < N) {
          f32x4 gg = acc[a][b], uu = acc[a + FN / 2][b];
          if (FOLD) {
            const float rs = rtab[wm * TM + b * 16 + fr];
            gg *= rs;
            uu *= rs;
          }
          uint2 o;
          o.x = pack_bf16x2(silu_mul(gg[0], uu[0]), silu_mul(gg[1], uu[1]));
          o.y = pack_bf16x2(silu_mul(gg[2], uu[2]), silu_mul(gg[3], uu[3]));
          *reinterpret_cast<uint2*>(out + (size_t)tok * N + col) = o;
        }
      }
    }
  } else {
    // residual: every load is issued before the first add (an address
    // outside the output reads element 0 and is never stored), so the
    // tile waits for memory once rather than once per sub-tile
    uint2 xr[FN][FM];
    if (EPI == EPI_RESIDUAL) {
#pragma unroll
      for (int a = 0; a < FN; ++a) {
        const int col = n0 + wn * TN + a * 16 + 4 * fq;
#pragma unroll
        for (int b = 0; b < FM; ++b) {
          const int tok = m0 + wm * TM + b * 16 + fr;
          const size_t off = (tok < M && col < N) ? (size_t)tok * N + col : 0;
          xr[a][b] = *reinterpret_cast<const uint2*>(resid + off);
        }
      }
    }
#pragma unroll
    for (int a = 0; a < FN; ++a) {
      const int col = n0 + wn * TN + a * 16 + 4 * fq;
#pragma unroll
      for (int b = 0; b < FM; ++b) {
        const int tok = m0 + wm * TM + b * 16 + fr;
        if (tok < M && col < N) {
          const size_t off = (size_t)tok * N + col;
          f32x4 v = acc[a][b];
          if (EPI == EPI_RESIDUAL) {
            v[0] += bf2f(xr[a][b].x & 0xFFFFu);
            v[1] += bf2f(xr[a][b].x >> 16);
            v[2] += bf2f(xr[a][b].y & 0xFFFFu);
            v[3] += bf2f(xr[a][b].y >> 16);
          }
          uint2 o;
          o.x = pack_bf16x2(v[0], v[1]);
          o.y = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<uint2*>(out + off) = o;
        }
      }
    }
  }
}

// Variant fed by buffer loads straight into LDS (no register staging, no
// LDS write instructions): S stages of BK-deep tiles, each stage its own LDS
// array so the compiler waits for exactly the stage being read.  Iteration kt
// waits for this thread's loads of tile kt, meets the other waves at one
// barrier (their loads of tile kt are then complete too, and everyone has
// finished reading tile kt-1), issues tile kt+S-1 into tile kt-1's stage and
// computes tile kt.  Used when K is a multiple of BK (no ragged K tile).
// Tile kt's LDS layout matches the register-staged kernel: row R holds its
// CPR = BK/8 chunks, chunk c at position c ^ sw(R), so each load instruction
// fills 1 KiB of consecutive LDS positions from lane-permuted sources.
// Compile-time choices: FFN_PF_BK / FFN_PF_S configure the schedule in which
// all eight waves read and multiply together; FFN_PF_PP selects the two-group
// (ping-pong) schedule for whole tiles, FFN_PF_PP_BK / FFN_PF_PP_S its tile
// depth and stage count.  Measured on gfx950 (prefill block): 64-deep tiles
// in two stages are fastest for both; 32-deep tiles (two or four stages)
// were 25% slower, and more than two stages of 32-deep tiles also make the
// compiler wait for the newest DMA before some fragment reads.
#ifndef FFN_PF_BK
#define FFN_PF_BK 64
#endif
#ifndef FFN_PF_S
#define FFN_PF_S 2
#endif
#ifndef FFN_PF_PP
#define FFN_PF_PP 1
#endif
constexpr int kDmaBK = FFN_PF_BK, kDmaS = FFN_PF_S;
// Token tiles per tile group (see the tile coordinates in gemm_dma).  With
// XCD-contiguous ranges and one workgroup per CU, a round of the whole chip
// covers every token tile and a few weight tiles when groups are 8 deep:
// right when the activations fit the 256 MB memory-side cache and the
// weights are streamed once (fused gate/up: n is 64 MB at M = 8192; 4 / 8
// deep measured alike, 2 and 16 slower).  The down projection's activations
// (h, 235 MB at M = 8192, f = 14336) do not fit: with 2-deep groups a round
// covers half the token tiles and every weight tile, so h is read once and
// the 117 MB of W_down is what repeats (down GEMM 0.772 -> 0.753 ms,
// bitwise identical; a mapping that also kept 4 x 8 tile blocks per XCD
// round measured the same as 2-deep groups).
#ifndef FFN_PF_GM
#define FFN_PF_GM 8
#endif
#ifndef FFN_PF_PERSIST
#define FFN_PF_PERSIST 1
#endif
#ifndef FFN_PF_GM_RES
#define FFN_PF_GM_RES 2
#endif
#ifndef FFN_PF_PP_BK
#define FFN_PF_PP_BK 64
#endif
#ifndef FFN_PF_PP_S
#define FFN_PF_PP_S 2
#endif
constexpr bool kPingPong = FFN_PF_PP != 0;
constexpr int kPpBK = FFN_PF_PP_BK, kPpS = FFN_PF_PP_S;

constexpr std::integral_constant<int, 0> I0{};
constexpr std::integral_constant<int, 1> I1{};
// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>), unrolled
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int BK>
__device__ __forceinline__ int dswz(int row) {
  return BK == 64 ? (row & 7) : ((row >> 2) & 3);
}

// Epilogue of a gemm_dma tile at (m0, n0): the lane holds D[4*fq + e][fr] of
// every (a, b) MFMA sub-tile of its wave's (wm, wn) block.  WIDE (whole
// tiles): the lanes of a pair (fq, fq ^ 1) trade the packed outputs of two
// neighbouring sub-tiles, so that each lane stores 8 consecutive columns
// (16 bytes) instead of 4, and a wave's store covers 16 rows x 64 bytes
// (interleaved A/B, bitwise identical: fused gate/up GEMM 1.380 -> 1.357 ms,
// prefill block fused 2.143 -> 2.114 ms, split 2.429 -> 2.316 ms).
#ifndef FFN_PF_WIDE
#define FFN_PF_WIDE 1
#endif
template <int EPI, int FN, int FM, int TM, int TN, bool WIDE = false>
__device__ __forceinline__ void dma_epilogue(const f32x4 (&acc)[FN][FM],
                                             const uint16_t* __restrict__ resid,
                                             uint16_t* __restrict__ out, int M, int N, int ldo,
                                             int m0, int n0, int wm, int wn, int fr, int fq) {
  if constexpr (WIDE) {
    constexpr int NA = EPI == EPI_SWIGLU ? FN / 2 : FN;  // output sub-tiles across n
    static_assert(NA % 2 == 0, "sub-tiles pair up");
    const int cw = n0 + wn * (EPI == EPI_SWIGLU ? TN / 2 : TN);
    const bool odd = fq & 1;
    // residual loads all issued before the first add, as below
    uint2 xr[EPI == EPI_RESIDUAL ? NA : 1][EPI == EPI_RESIDUAL ? FM : 1];
    if constexpr (EPI == EPI_RESIDUAL) {
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b)
          xr[a][b] = *reinterpret_cast<const uint2*>(resid + (size_t)(m0 + wm * TM + b * 16 + fr) * ldo +
                                                     cw + a * 16 + 4 * fq);
    }
#pragma unroll
    for (int b = 0; b < FM; ++b) {
      const int tok = m0 + wm * TM + b * 16 + fr;
#pragma unroll
      for (int pr = 0; pr < NA / 2; ++pr) {
        uint2 o[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int a = 2 * pr + h;
          if constexpr (EPI == EPI_SWIGLU) {
            const f32x4 gg = acc[a][b], uu = acc[a + FN / 2][b];
            o[h].x = pack_bf16x2(silu_mul(gg[0], uu[0]), silu_mul(gg[1], uu[1]));
            o[h].y = pack_bf16x2(silu_mul(gg[2], uu[2]), silu_mul(gg[3], uu[3]));
          } else {
            f32x4 v = acc[a][b];
            if constexpr (EPI == EPI_RESIDUAL) {
              const uint2 x2 = xr[EPI == EPI_RESIDUAL ? a : 0][EPI == EPI_RESIDUAL ? b : 0];
              v[0] += bf2f(x2.x & 0xFFFFu);
              v[1] += bf2f(x2.x >> 16);
              v[2] += bf2f(x2.y & 0xFFFFu);
              v[3] += bf2f(x2.y >> 16);
            }
            o[h].x = pack_bf16x2(v[0], v[1]);
            o[h].y = pack_bf16x2(v[2], v[3]);
          }
        }
        // even lanes keep sub-tile 2pr and receive its next four columns;
        // odd lanes keep sub-tile 2pr+1 and receive its previous four
        const uint2 send = odd ? o[0] : o[1];
        const uint2 keep = odd ? o[1] : o[0];
        const uint32_t rx = (uint32_t)__shfl_xor((int)send.x, 16, 64);
        const uint32_t ry = (uint32_t)__shfl_xor((int)send.y, 16, 64);
        const uint4 v = odd ? make_uint4(rx, ry, keep.x, keep.y) : make_uint4(keep.x, keep.y, rx, ry);
        const int col = cw + (2 * pr + (odd ? 1 : 0)) * 16 + 4 * (fq & 2);
        *reinterpret_cast<uint4*>(out + (size_t)tok * ldo + col) = v;
      }
    }
    return;
  }
  if (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int a = 0; a < FN / 2; ++a) {
      const int col = n0 + wn * (TN / 2) + a * 16 + 4 * fq;
#pragma unroll
      for (int b = 0; b < FM; ++b) {
        const int tok = m0 + wm * TM + b * 16 + fr;
        if (tok < M && col < N) {
          const f32x4 gg = acc[a][b], uu = acc[a + FN / 2][b];
          uint2 o;
          o.x = pack_bf16x2(silu_mul(gg[0], uu[0]), silu_mul(gg[1], uu[1]));
          o.y = pack_bf16x2(silu_mul(gg[2], uu[2]), silu_mul(gg[3], uu[3]));
          *reinterpret_cast<uint2*>(out + (size_t)tok * ldo + col) = o;
        }
      }
    }
  } else {
    // residual: every load is issued before the first add (an address
    // outside the output reads element 0 and is never stored), so the
    // tile waits for memory once rather than once per sub-tile
    uint2 xr[FN][FM];
    if (EPI == EPI_RESIDUAL) {
#pragma unroll
      for (int a = 0; a < FN; ++a) {
        const int col = n0 + wn * TN + a * 16 + 4 * fq;
#pragma unroll
        for (int b = 0; b < FM; ++b) {
          const int tok = m0 + wm * TM + b * 16 + fr;
          const size_t off = (tok < M && col < N) ? (size_t)tok * ldo + col : 0;
          xr[a][b] = *reinterpret_cast<const uint2*>(resid + off);
        }
      }
    }
#pragma unroll
    for (int a = 0; a < FN; ++a) {
      const int col = n0 + wn * TN + a * 16 + 4 * fq;
#pragma unroll
      for (int b = 0; b < FM; ++b) {
        const int tok = m0 + wm * TM + b * 16 + fr;
        if (tok < M && col < N) {
          const size_t off = (size_t)tok * ldo + col;
          f32x4 v = acc[a][b];
          if (EPI == EPI_RESIDUAL) {
            v[0] += bf2f(xr[a][b].x & 0xFFFFu);
            v[1] += bf2f(xr[a][b].x >> 16);
            v[2] += bf2f(xr[a][b].y & 0xFFFFu);
            v[3] += bf2f(xr[a][b].y >> 16);
          }
          uint2 o;
          o.x = pack_bf16x2(v[0], v[1]);
          o.y = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<uint2*>(out + off) = o;
        }
      }
    }
  }
}

// PERSIST (ping-pong schedule only): the grid is at most one workgroup per
// resident slot and each workgroup walks tiles blockIdx.x, + gridDim.x, ...;
// as soon as a tile's K loop has read its last stage, the first S K tiles
// of the workgroup's next tile go out, so their latency overlaps the
// epilogue instead of opening the next tile.
// PART (split K): workgroup (tile, z) covers the z-th of gridDim.y contiguous
// ranges of K tiles (whole groups of S tiles on the ping-pong schedule) and
// writes its fp32 partial sums instead of the epilogue: plane z of part
// ([planes][M][N]; SWIGLU: the gate sums in plane z, the up sums in plane
// gridDim.y + z), which a second pass adds up in range order.
template <int BM, int BN, int WM, int WN, int EPI, int BK, int S, bool PP, bool PERSIST = false,
          bool PART = false>
__global__ __launch_bounds__(WM * WN * 64) void gemm_dma(
    const uint16_t* __restrict__ act,    // [M, K]
    const uint16_t* __restrict__ w0,     // [N, K]  (gate for SWIGLU)
    const uint16_t* __restrict__ w1,     // [N, K]  (up for SWIGLU)
    const uint16_t* __restrict__ resid,  // [M, N]  (RESIDUAL)
    uint16_t* __restrict__ out,          // [M, N]
    int M, int N, int K, int ldo, float* __restrict__ part) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int BNO = EPI == EPI_SWIGLU ? BN / 2 : BN;
  constexpr int ROWS = BN + BM;
  constexpr int CPR = BK / 8;                  // 16-byte chunks per LDS row
  constexpr int SZ = ROWS * CPR;               // chunks per stage
  constexpr int J = SZ / NT;                   // load instructions per thread per tile
  constexpr int KS = BK / 32;                  // MFMA k-steps per tile
  static_assert(SZ % NT == 0 && NT % CPR == 0, "tile/thread mismatch");
  static_assert(S >= 2 && S <= 5, "stages");
  __shared__ uint4 st0[SZ];
  __shared__ uint4 st1[SZ];
  __shared__ uint4 st2[S > 2 ? SZ : 1];
  __shared__ uint4 st3[S > 3 ? SZ : 1];
  __shared__ uint4 st4[S > 4 ? SZ : 1];
  auto stage = [&](int i) -> uint4* {  // i is a compile-time constant after unrolling
    return i == 0 ? st0 : i == 1 ? st1 : i == 2 ? st2 : i == 3 ? st3 : st4;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int K8 = K >> 3;
  static_assert(!(PART && PERSIST), "split-K grids hold one tile per workgroup");
  // this workgroup's K tiles [kt0, kt0 + nkt): ranges in whole groups of S
  // K tiles whenever the tile count allows (always on the ping-pong
  // schedule), so both schedules cut K at the same places
  const int unit = (K / BK) % S == 0 ? S : 1;
  const int units = (K / BK) / unit;
  const int zr = PART ? (int)blockIdx.y : 0, Zr = PART ? (int)gridDim.y : 1;
  const int u0 = (int)(((long)units * zr) / Zr), u1 = (int)(((long)units * (zr + 1)) / Zr);
  const int kt0 = PART ? u0 * unit : 0;
  const int nkt = PART ? (u1 - u0) * unit : K / BK;
  const unsigned kbyte0 = (unsigned)kt0 * (unsigned)BK * 2u;  // byte offset of the range in a row
  (void)K8;

  // ---- tile coordinates: XCD-contiguous, then grouped GM token tiles deep
  // (a persistent grid is a multiple of 8 workgroups or one per tile, so a
  // workgroup's tiles stay on its XCD)
  static_assert(!PERSIST || PP, "the persistent walk uses the ping-pong schedule");
  const int ntm = (M + BM - 1) / BM, ntn = (N + BNO - 1) / BNO;
  const int T = ntm * ntn;
  auto coords = [&](int tile, int& m0_, int& n0_) {
    int L = tile;
    if ((T & 7) == 0) L = (L & 7) * (T >> 3) + (L >> 3);
    constexpr int GM = EPI == EPI_RESIDUAL ? FFN_PF_GM_RES : FFN_PF_GM;
    const int group = L / (GM * ntn);
    const int first_m = group * GM;
    const int gm = min(ntm - first_m, GM);
    const int inner = L - group * GM * ntn;
    m0_ = (first_m + inner % gm) * BM;
    n0_ = (inner / gm) * BNO;
  };
  int m0i, n0i;
  coords(blockIdx.x, m0i, n0i);
  const int m0 = m0i, n0 = n0i;

  // ---- load sources: instruction j of this thread fills LDS position
  // p = j*NT + tid = row p / CPR, stored chunk p % CPR, which holds global
  // chunk (p % CPR) ^ sw(row) of that row.  Instruction j covers rows
  // [j*NT/CPR, (j+1)*NT/CPR), and the region boundaries (gate / up / tokens at
  // BN/2 and BN) are multiples of NT/CPR, so the source of instruction j is
  // fixed at compile time.  Rows past M or N are clamped: they only feed
  // outputs that are never stored.
  constexpr int RJ = NT / CPR;  // rows per load instruction
  static_assert((BN / 2) % RJ == 0 && BN % RJ == 0, "regions must align to load instructions");
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(act, (long)M * K * 2);
  const __amdgpu_buffer_rsrc_t rw0 = make_rsrc(w0, (long)N * K * 2);
  const __amdgpu_buffer_rsrc_t rw1 = make_rsrc(EPI == EPI_SWIGLU ? w1 : w0, (long)N * K * 2);
  unsigned soff[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int row = j * RJ + tid / CPR, cs = tid % CPR;
    const int cg = cs ^ dswz<BK>(row);
    int src_row;
    if (j * RJ < BN) {
      src_row = (EPI == EPI_SWIGLU && j * RJ >= BN / 2) ? n0 + row - BN / 2 : n0 + row;
      src_row = min(src_row, N - 1);
    } else {
      src_row = min(m0 + row - BN, M - 1);
    }
    soff[j] = (unsigned)src_row * (unsigned)K * 2u + (unsigned)cg * 16u + kbyte0;
  }
  // tile kt into stage i; tiles past the end read nothing (out-of-range
  // offset, or-ed in: a branch here would cost the exact load waits)
  auto issue = [&](int i, int kt) {
    uint4* Ls = stage(i);
    const unsigned ko = (unsigned)kt * (unsigned)BK * 2u | (kt < nkt ? 0u : kOutOfRange);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      uint4* dst = Ls + j * NT + wave * 64;  // wave-uniform; lane l lands at +l
      if (j * RJ < BN / 2 || (EPI != EPI_SWIGLU && j * RJ < BN)) buf_ld_lds16<0>(rw0, dst, soff[j] + ko);
      else if (j * RJ < BN) buf_ld_lds16<0>(rw1, dst, soff[j] + ko);
      else buf_ld_lds16<0>(ra, dst, soff[j] + ko);
    }
  };

  // LDS rows read by this lane's fragments: fr plus a multiple of 16 (the
  // rows of fragment t are a compile-time offset from those of fragment 0),
  // so every fragment of the lane shares one swizzle, and its address is a
  // per-lane base per k-step plus an immediate offset.
  const int fr = lane & 15, fq = lane >> 4;
  const int xo = dswz<BK>(fr);
  const int arow0 = (EPI == EPI_SWIGLU ? wn * (TN / 2) : wn * TN) + fr;
  const int brow0 = BN + wm * TM + fr;
  static_assert(TN % 32 == 0 && TM % 16 == 0 && BN % 32 == 0, "fragment rows must stay congruent mod 16");
  auto aoff = [](int t) {  // row offset of A fragment t (compile-time after unrolling)
    return EPI == EPI_SWIGLU ? (t / (FN / 2)) * (BN / 2) + (t % (FN / 2)) * 16 : t * 16;
  };
  int abase[KS], bbase[KS];  // uint4 index within a stage
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    abase[ks] = arow0 * CPR + ((ks * 4 + fq) ^ xo);
    bbase[ks] = brow0 * CPR + ((ks * 4 + fq) ^ xo);
  }

  f32x4 acc[FN][FM];
#pragma unroll
  for (int a = 0; a < FN; ++a)
#pragma unroll
    for (int b = 0; b < FM; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int i) {
    const uint4* Ls = stage(i);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 af[FN], bfr[FM];
#pragma unroll
      for (int t = 0; t < FN; ++t) af[t] = Ls[abase[ks] + aoff(t) * CPR];
#pragma unroll
      for (int t = 0; t < FM; ++t) bfr[t] = Ls[bbase[ks] + t * 16 * CPR];
#pragma unroll
      for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b) acc[a][b] = mfma16(af[a], bfr[b], acc[a][b]);
    }
  };
  // wait until at most `pending` tiles of this thread's loads are in flight,
  // then meet the other waves
  auto meet = [&](int pending) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (pending >= 3) __builtin_amdgcn_s_waitcnt(0x0F70 | ((3 * J) & 15) | (((3 * J) >> 4) << 14));
    else if (pending == 2) __builtin_amdgcn_s_waitcnt(0x0F70 | ((2 * J) & 15) | (((2 * J) >> 4) << 14));
    else if (pending == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | (J & 15) | ((J >> 4) << 14));
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };

  if constexpr (PP) {
    // Ping-pong schedule.  The waves with wm = 0 (group 0, one per SIMD) and
    // those with wm = 1 (group 1, the other wave of each SIMD) run the same
    // sequence -- read the fragments of one 32-deep k-step into registers,
    // barrier, multiply them, barrier -- with group 1 one barrier behind, so
    // that on every SIMD one wave multiplies while the other reads.  With
    // h = KS kt + ks the k-step index, group g reads step h in phase 2h+g
    // and multiplies it in phase 2h+1+g.  The S stages start full (tiles
    // 0..S-1); tile kt+S-1 (kt >= 1) goes into the stage of tile kt-1 as each
    // wave starts reading tile kt, after both groups' reads of tile kt-1
    // (last in phase 2 KS kt - 1).  Tile kt+1 must be in LDS before group 0
    // reads it in phase 2 KS (kt+1): every wave waits for its own loads of
    // it in its last phase before that (group 0 after multiplying the last
    // k-step of tile kt, group 1 after reading it), leaving its later tiles
    // in flight.  Group 1 starts with one extra barrier and skips the last
    // one, so both execute 2 KS nkt + 1 barriers.  nkt must be a multiple
    // of S and the tiles whole.
    static_assert(WM == 2, "ping-pong layout: two wave rows");
    uint4 af[FN], bfr[FM];
    auto readf = [&](int i, int ks) {
      const uint4* Ls = stage(i);
#pragma unroll
      for (int t = 0; t < FN; ++t) af[t] = Ls[abase[ks] + aoff(t) * CPR];
#pragma unroll
      for (int t = 0; t < FM; ++t) bfr[t] = Ls[bbase[ks] + t * 16 * CPR];
    };
    auto mma = [&]() {
#pragma unroll
      for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b) acc[a][b] = mfma16(af[a], bfr[b], acc[a][b]);
    };
    auto bar = [&]() {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };
    // waits stay where they are written (not hoisted above the MFMAs)
    auto wait_lds = [&]() {  // lgkmcnt(0)
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0xC07F);
    };
    // wait until tile kt+1 has landed: this wave's loads of the tiles after
    // it (at most S-2 of them, fewer near the end) may stay in flight
    auto wait_next = [&](int kt) {
      const int after = min(S - 2, nkt - 2 - kt);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_sched_barrier(0);
      if (S >= 4 && after >= 2) __builtin_amdgcn_s_waitcnt(0x0F70 | ((2 * J) & 15) | (((2 * J) >> 4) << 14));
      else if (S >= 3 && after >= 1) __builtin_amdgcn_s_waitcnt(0x0F70 | (J & 15) | ((J >> 4) << 14));
      else __builtin_amdgcn_s_waitcnt(0x0F70);
    };
    static_assert(S >= 2 && S <= 4, "wait_next covers up to two tiles in flight");
    // DMA of tile kt (always < nkt here) into stage i, half of it by each
    // group.  Tiles are whole (M % BM == 0, N % BNO == 0), so no row is
    // clamped: every load's source is one of two per-lane offsets (weight
    // rows, token rows) plus a wave-uniform row-block and K offset in the
    // scalar operand.
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int rr = tid / CPR;
    const unsigned cgp = (unsigned)((tid % CPR) ^ dswz<BK>(rr)) * 16u;
    const unsigned vw0 = (unsigned)(n0 + rr) * (unsigned)K * 2u + cgp + kbyte0;
    const unsigned va0 = (unsigned)(m0 + rr) * (unsigned)K * 2u + cgp + kbyte0;
    const int blk = RJ * K * 2;  // bytes of one load instruction's row block
    // vw, va: this lane's weight-row and token-row source offsets of the tile
    auto issue_pp = [&](int i, int kt, unsigned vw, unsigned va) {
      uint4* Ls = stage(i);
      const int ko = kt * BK * 2;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        uint4* dst = Ls + j * NT + wave_s * 64;
        if (j * RJ < BN) {
          const int rb = (EPI == EPI_SWIGLU ? j % (BN / 2 / RJ) : j);
          if (EPI != EPI_SWIGLU || j * RJ < BN / 2) buf_ld_lds16s<0>(rw0, dst, vw, ko + rb * blk);
          else buf_ld_lds16s<0>(rw1, dst, vw, ko + rb * blk);
        } else {
          buf_ld_lds16s<0>(ra, dst, va, ko + (j - BN / RJ) * blk);
        }
      }
    };
    static_for<S>([&](auto si) { issue_pp(decltype(si)::value, decltype(si)::value, vw0, va0); });
    // S tiles per iteration keep every stage index a compile-time constant,
    // and no path reaches a read of one stage with a DMA into that same
    // stage pending: the compiler then adds no wait for the DMA before the
    // reads.  body(i, ks, kt): k-step ks of tile kt, in stage i.  The group
    // is a compile-time constant in each copy of the loop.
    auto run = [&](auto gi, unsigned vw, unsigned va) {
      constexpr int G = decltype(gi)::value;
      auto body = [&](auto si, auto ki, int kt) {
        constexpr int i = decltype(si)::value, ks = decltype(ki)::value;
        if (ks == 0 && kt >= 1 && kt + S - 1 < nkt) issue_pp((i + S - 1) % S, kt + S - 1, vw, va);
        readf(i, ks);
        wait_lds();
        if (ks == KS - 1 && G == 1) wait_next(kt);
        bar();
        mma();
        if (ks == KS - 1 && G == 0) wait_next(kt);
        if (ks < KS - 1 || G == 0 || kt + 1 < nkt) bar();
      };
      if (G == 1) bar();
      for (int kt = 0; kt < nkt; kt += S) {
        static_for<S>([&](auto si) {
          static_for<KS>([&](auto ki) { body(si, ki, kt + decltype(si)::value); });
        });
      }
    };
    if constexpr (!PERSIST) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0x0F70 | (((S - 1) * J) & 15) | ((((S - 1) * J) >> 4) << 14));  // tile 0
      bar();
      if (__builtin_amdgcn_readfirstlane(wm) == 0) run(I0, vw0, va0);
      else run(I1, vw0, va0);
    } else {
      int pm0 = m0, pn0 = n0;
      unsigned vw = vw0, va = va0;
      for (int tile = blockIdx.x;;) {
        // K tile 0 of this tile has landed (the S - 1 after it and the
        // previous tile's output stores may still be in flight: loads
        // complete in order, and at most (S - 1) J operations remain)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0x0F70 | (((S - 1) * J) & 15) | ((((S - 1) * J) >> 4) << 14));
        bar();
        if (__builtin_amdgcn_readfirstlane(wm) == 0) run(I0, vw, va);
        else run(I1, vw, va);
        // every wave has passed the K loop's last barrier, after which no
        // stage is read: the next tile's first S K tiles can go out
        const int next = tile + (int)gridDim.x;
        int m1 = 0, n1 = 0;
        if (next < T) {
          coords(next, m1, n1);
          vw = (unsigned)(n1 + rr) * (unsigned)K * 2u + cgp;
          va = (unsigned)(m1 + rr) * (unsigned)K * 2u + cgp;
          static_for<S>([&](auto si) { issue_pp(decltype(si)::value, decltype(si)::value, vw, va); });
        }
        dma_epilogue<EPI, FN, FM, TM, TN, FFN_PF_WIDE != 0>(acc, resid, out, M, N, ldo, pm0, pn0, wm, wn, fr, fq);
        if (next >= T) return;
#pragma unroll
        for (int a = 0; a < FN; ++a)
#pragma unroll
          for (int b = 0; b < FM; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        tile = next;
        pm0 = m1;
        pn0 = n1;
      }
    }
  } else {
#pragma unroll
  for (int i = 0; i < S - 1; ++i) issue(i, i);
  // main loop: whole groups of S tiles, no early exit
  const int ngroups = nkt >= S - 1 ? (nkt - (S - 1)) / S : 0;
  int kt = 0;
  for (int g = 0; g < ngroups; ++g) {
#pragma unroll
    for (int i = 0; i < S; ++i, ++kt) {
      meet(S - 2);                        // tiles kt+1 .. kt+S-2 may stay in flight
      issue((i + S - 1) % S, kt + S - 1);  // into tile kt-1's stage
      __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the MFMAs
      compute(i);
    }
  }
  // tail: tiles kt .. nkt-1, at most 2S-2 of them; loads for those not yet
  // issued go out as before while in-flight ones drain
#pragma unroll
  for (int i = 0; i < 2 * S - 1; ++i) {
    if (kt + i < nkt) {
      const int left = nkt - 1 - (kt + i);           // tiles after this one
      const int inflight = min(left, S - 2);
      meet(inflight);
      if (kt + i + S - 1 < nkt) issue((i + S - 1) % S, kt + i + S - 1);
      compute(i % S);
    }
  }
  }

  if constexpr (PART) {
    // fp32 partial sums: lane (fr, fq) holds 4 consecutive columns of token
    // row fr of every sub-tile
    constexpr int NA = EPI == EPI_SWIGLU ? FN / 2 : FN;
#pragma unroll
    for (int a = 0; a < FN; ++a) {
      const int col = n0 + wn * (EPI == EPI_SWIGLU ? TN / 2 : TN) + (a % NA) * 16 + 4 * fq;
      const int plane = a < NA ? zr : Zr + zr;  // SWIGLU: gate, then up
#pragma unroll
      for (int b = 0; b < FM; ++b) {
        const int tok = m0 + wm * TM + b * 16 + fr;
        if (tok < M && col < N)
          *reinterpret_cast<float4*>(part + ((size_t)plane * M + tok) * N + col) =
              make_float4(acc[a][b][0], acc[a][b][1], acc[a][b][2], acc[a][b][3]);
      }
    }
    return;
  }
  // whole tiles (the ping-pong schedule) store 16 bytes per lane
  dma_epilogue<EPI, FN, FM, TM, TN, PP && FFN_PF_WIDE != 0>(acc, resid, out, M, N, ldo, m0, n0, wm, wn, fr, fq);
}

// Tile configuration: 256 tokens x 256 weight rows, 8 waves as 2 x 4, each
// wave 128 tokens x 64 weight rows (32 MFMA tiles, 128 fp32 accumulators).
constexpr int kBM = 256, kBN = 256, kWM = 2, kWN = 4;
constexpr int kLdsBytes = 2 * (kBM + kBN) * 128;


// FFN_PF_FORCE_REG 1 routes every GEMM to the register-staged kernel (for
// measurements that compare the schedules).
#ifndef FFN_PF_FORCE_REG
#define FFN_PF_FORCE_REG 0
#endif

template <int EPI, bool FOLD = false>
static hipError_t launch_reg(const void* act, const void* w0, const void* w1, const void* resid,
                             void* out, int M, int N, int K, const void* gain, float eps,
                             hipStream_t s) {
  constexpr int BNO = EPI == EPI_SWIGLU ? kBN / 2 : kBN;
  const long tiles = (long)((M + kBM - 1) / kBM) * ((N + BNO - 1) / BNO);
  auto kern = gemm_bf16<kBM, kBN, kWM, kWN, EPI, FOLD>;
  // allow more than the default dynamic LDS (per device, so done per launch)
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     kLdsBytes);
  if (e != hipSuccess) return e;
  FFN_DISPATCH(kern, dim3((unsigned)tiles), dim3(kWM * kWN * 64), kLdsBytes, s,
               (const uint16_t*)act, (const uint16_t*)w0, (const uint16_t*)w1,
               (const uint16_t*)resid, (uint16_t*)out, M, N, K, (const uint16_t*)gain, eps);
  return hipGetLastError();
}

// Token tile of the LDS-fed kernels: 256, or 128 for batches of at most
// FFN_PF_BM128 tokens (0 = off).  Up to 128 tokens the tile count is the same
// either way and the 128-token tile skips the MFMA work and LDS traffic of
// the padded rows (interleaved A/B, d = 4096, f = 11008: block 98.4 / 105.3 /
// 112.5 -> 94.9 / 101.6 / 105.8 us at 65 / 100 / 128 tokens).  Above that it
// multiplies the tiles, which costs whole rounds (300 tokens: 258 instead of
// 172 gate/up tiles, 163 -> 213 us).
#ifndef FFN_PF_BM128
#define FFN_PF_BM128 128
#endif
static int tile_m(int M) { return M <= FFN_PF_BM128 ? kBM / 2 : kBM; }

// Workgroups of the persistent ping-pong kernel resident at once (a multiple
// of 8, one per XCD slot; one per compute unit if the runtime cannot tell:
// its LDS stages take 96-128 KB).
template <int EPI, int BM>
static int pp_slots() {
  static const int slots = [] {
    const int r = resident_slots(gemm_dma<BM, kBN, kWM, kWN, EPI, kPpBK, kPpS, true, true>, kWM * kWN * 64);
    return (r > 0 ? r : device_cus()) / 8 * 8;
  }();
  return slots;
}
template <int EPI>
static int pp_slots(int bm) {
  return bm == kBM ? pp_slots<EPI, kBM>() : pp_slots<EPI, kBM / 2>();
}

// ldo: row stride of out and resid in elements (N unless the GEMM covers a
// column block of a wider output)
template <int EPI, int BM>
static void launch_dma(const void* act, const void* w0, const void* w1, const void* resid,
                       void* out, int M, int N, int K, hipStream_t s, int ldo) {
  constexpr int BNO = EPI == EPI_SWIGLU ? kBN / 2 : kBN;
  const long tiles = (long)((M + BM - 1) / BM) * ((N + BNO - 1) / BNO);
  // whole tiles and an even number of K tiles: the ping-pong schedule,
  // walked persistently when the tiles take more than one round
  if (kPingPong && M % BM == 0 && N % BNO == 0 && K % (kPpS * kPpBK) == 0) {
    auto pers = gemm_dma<BM, kBN, kWM, kWN, EPI, kPpBK, kPpS, true, true>;
    const int slots = pp_slots<EPI, BM>();
    if (FFN_PF_PERSIST && slots >= 8 && tiles > slots)
      FFN_DISPATCH(pers, dim3((unsigned)slots), dim3(kWM * kWN * 64), 0, s, (const uint16_t*)act,
                   (const uint16_t*)w0, (const uint16_t*)w1, (const uint16_t*)resid, (uint16_t*)out, M,
                   N, K, ldo, nullptr);
    else
      FFN_DISPATCH((gemm_dma<BM, kBN, kWM, kWN, EPI, kPpBK, kPpS, true>), dim3((unsigned)tiles),
                   dim3(kWM * kWN * 64), 0, s, (const uint16_t*)act, (const uint16_t*)w0,
                   (const uint16_t*)w1, (const uint16_t*)resid, (uint16_t*)out, M, N, K, ldo, nullptr);
  } else
    FFN_DISPATCH((gemm_dma<BM, kBN, kWM, kWN, EPI, kDmaBK, kDmaS, false>), dim3((unsigned)tiles),
                 dim3(kWM * kWN * 64), 0, s, (const uint16_t*)act, (const uint16_t*)w0,
                 (const uint16_t*)w1, (const uint16_t*)resid, (uint16_t*)out, M, N, K, ldo, nullptr);
}

template <int EPI>
static hipError_t launch_cfg(const void* act, const void* w0, const void* w1, const void* resid,
                             void* out, int M, int N, int K, hipStream_t s, int ldo = 0) {
  if (ldo <= 0) ldo = N;
  // whole K tiles and every operand addressable by a buffer resource: LDS-fed kernel
  if (!FFN_PF_FORCE_REG && K % kDmaBK == 0 && (size_t)M * K * 2 < ((size_t)1 << 31) &&
      (size_t)N * K * 2 < ((size_t)1 << 31)) {
    if (tile_m(M) == kBM)
      launch_dma<EPI, kBM>(act, w0, w1, resid, out, M, N, K, s, ldo);
    else
      launch_dma<EPI, kBM / 2>(act, w0, w1, resid, out, M, N, K, s, ldo);
    return hipGetLastError();
  }
  return launch_reg<EPI>(act, w0, w1, resid, out, M, N, K, nullptr, 0.f, s);
}

// Split K for GEMMs whose tiles leave compute units idle (fewer than one per
// CU: a down projection below 4096 tokens at d = 4096 has 16 per 256 tokens,
// the fused gate/up 86 at f = 11008).  floor(CUs / tiles) ranges, at most
// kPrefillMaxSplits and at least one group of K tiles each; 1 = no split.
// Only the LDS-fed kernels split (K a multiple of the K tile).
#ifndef FFN_PF_SPLITK
#define FFN_PF_SPLITK 1
#endif
static bool dma_ok(int M, int N, int K) {
  return !FFN_PF_FORCE_REG && K % kDmaBK == 0 && (size_t)M * K * 2 < ((size_t)1 << 31) &&
         (size_t)N * K * 2 < ((size_t)1 << 31);
}
static bool pp_ok(int M, int N, int K, int bno) {
  return kPingPong && M % tile_m(M) == 0 && N % bno == 0 && K % (kPpS * kPpBK) == 0;
}
static int splits_for(int M, int N, int K, int bno) {
  if (!FFN_PF_SPLITK || !dma_ok(M, N, K)) return 1;
  const int bm = tile_m(M);
  const long tiles = (long)((M + bm - 1) / bm) * ((N + bno - 1) / bno);
  const int cus = device_cus();
  long z = tiles > 0 ? cus / tiles : 1;
  // the kernels' range unit: whole groups of S K tiles when they divide K
  const int nk = pp_ok(M, N, K, bno) ? K / kPpBK : K / kDmaBK;
  const int sg = pp_ok(M, N, K, bno) ? kPpS : kDmaS;
  const int units = nk % sg == 0 ? nk / sg : nk;
  if (z > kPrefillMaxSplits) z = kPrefillMaxSplits;
  if (z > units) z = units;
  return z > 1 ? (int)z : 1;
}

// Past one round, a tile count just above a whole number of rounds leaves
// the last round nearly empty (258 fused gate/up tiles at 768 tokens and
// f = 11008 take two rounds of 256).  Then the columns that fill the rounds
// before it run unsplit, and the rest -- at most half a round of tiles --
// split over K into as many ranges as fill one round; FFN_PF_TAIL is the
// least number of ranges worth the partial sums' extra traffic (0: off).
#ifndef FFN_PF_TAIL
#define FFN_PF_TAIL 2
#endif
template <int EPI>
static PrefillPlan plan_for(int M, int N, int K) {
  constexpr int BNO = EPI == EPI_SWIGLU ? kBN / 2 : kBN;
  PrefillPlan p;
  p.main = N;
  const int z = splits_for(M, N, K, BNO);
  if (z > 1) {
    p.main = 0;
    p.z = z;
    return p;
  }
  if (!FFN_PF_SPLITK || FFN_PF_TAIL < 2 || !dma_ok(M, N, K) || !pp_ok(M, N, K, BNO)) return p;
  const int bm = tile_m(M);
  const long mt = M / bm, nt = N / BNO, tiles = mt * nt, slots = pp_slots<EPI>(bm);
  if (slots < 8 || tiles <= slots) return p;
  const long rounds = (tiles + slots - 1) / slots;
  const long nm = (rounds - 1) * slots / mt;  // column tiles filling the earlier rounds
  if (nm < 1 || nm >= nt) return p;
  const long tail = mt * (nt - nm);
  const long units = K / kPpBK % kPpS == 0 ? K / kPpBK / kPpS : K / kPpBK;
  long zt = slots / tail;
  if (zt > kPrefillMaxSplits) zt = kPrefillMaxSplits;
  if (zt > units) zt = units;
  if (zt < FFN_PF_TAIL) return p;
  p.main = (int)(nm * BNO);
  p.z = (int)zt;
  return p;
}
PrefillPlan prefill_gateup_plan(int M, int d, int f) { return plan_for<EPI_SWIGLU>(M, f, d); }
PrefillPlan prefill_down_plan(int M, int d, int f) { return plan_for<EPI_RESIDUAL>(M, d, f); }

template <int EPI, int BM>
static void launch_part_bm(const void* act, const void* w0, const void* w1, float* part, int Z,
                           int M, int N, int K, hipStream_t s) {
  constexpr int BNO = EPI == EPI_SWIGLU ? kBN / 2 : kBN;
  const long tiles = (long)((M + BM - 1) / BM) * ((N + BNO - 1) / BNO);
  const dim3 grid((unsigned)tiles, (unsigned)Z), block(kWM * kWN * 64);
  if (pp_ok(M, N, K, BNO))
    FFN_DISPATCH((gemm_dma<BM, kBN, kWM, kWN, EPI, kPpBK, kPpS, true, false, true>), grid, block, 0, s,
                 (const uint16_t*)act, (const uint16_t*)w0, (const uint16_t*)w1, nullptr, nullptr, M,
                 N, K, N, part);
  else
    FFN_DISPATCH((gemm_dma<BM, kBN, kWM, kWN, EPI, kDmaBK, kDmaS, false, false, true>), grid, block,
                 0, s, (const uint16_t*)act, (const uint16_t*)w0, (const uint16_t*)w1, nullptr,
                 nullptr, M, N, K, N, part);
}

template <int EPI>
static hipError_t launch_part(const void* act, const void* w0, const void* w1, float* part, int Z,
                              int M, int N, int K, hipStream_t s) {
  if (Z < 1 || Z > kPrefillMaxSplits || !dma_ok(M, N, K)) return hipErrorInvalidValue;
  if (tile_m(M) == kBM)
    launch_part_bm<EPI, kBM>(act, w0, w1, part, Z, M, N, K, s);
  else
    launch_part_bm<EPI, kBM / 2>(act, w0, w1, part, Z, M, N, K, s);
  return hipGetLastError();
}

hipError_t launch_gemm_gateup_fused_part(const void* n, const void* wg, const void* wu, float* part,
                                         int Z, int M, int d, int f, hipStream_t s) {
  return launch_part<EPI_SWIGLU>(n, wg, wu, part, Z, M, f, d, s);
}
hipError_t launch_gemm_down_part(const void* h, const void* wd, float* part, int Z, int M, int d,
                                 int f, hipStream_t s) {
  return launch_part<EPI_RESIDUAL>(h, wd, nullptr, part, Z, M, d, f, s);
}

hipError_t launch_gemm_gateup_fused(const void* n, const void* wg, const void* wu, void* h,
                                    int M, int d, int f, hipStream_t s, int ldo) {
  return launch_cfg<EPI_SWIGLU>(n, wg, wu, nullptr, h, M, f, d, s, ldo);
}
hipError_t launch_gemm_gateup_fused_norm(const void* x, const void* g, const void* wg,
                                         const void* wu, void* h, int M, int d, int f, float eps,
                                         hipStream_t s) {
  return launch_reg<EPI_SWIGLU, true>(x, wg, wu, nullptr, h, M, f, d, g, eps, s);
}
hipError_t launch_gemm_store(const void* a, const void* w, void* c, int M, int N, int K,
                             hipStream_t s) {
  return launch_cfg<EPI_STORE>(a, w, nullptr, nullptr, c, M, N, K, s);
}
hipError_t launch_gemm_residual(const void* a, const void* w, const void* resid, void* y,
                                int M, int N, int K, hipStream_t s, int ldo) {
  return launch_cfg<EPI_RESIDUAL>(a, w, nullptr, resid, y, M, N, K, s, ldo);
}

// ---- split-variant activation: h = silu(G) * U, 8 bf16 per 16-byte chunk
__global__ __launch_bounds__(256) void swiglu_bf16(const uint4* __restrict__ G,
                                                   const uint4* __restrict__ U,
                                                   uint4* __restrict__ h, int64_t nchunk) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nchunk;
       i += (int64_t)gridDim.x * 256) {
    float gg[8], uu[8];
    unpack8(G[i], gg);
    unpack8(U[i], uu);
#pragma unroll
    for (int e = 0; e < 8; ++e) gg[e] = silu_mul(gg[e], uu[e]);
    h[i] = pack8(gg);
  }
}

hipError_t launch_swiglu_bf16(const void* G, const void* U, void* h, int64_t count,
                              hipStream_t s) {
  const int64_t nchunk = count / 8;
  int64_t blocks = (nchunk + 255) / 256;
  if (blocks > 256 * 16) blocks = 256 * 16;  // grid-stride beyond 16 workgroups per CU
  if (blocks < 1) blocks = 1;
  FFN_DISPATCH(swiglu_bf16, dim3((unsigned)blocks), dim3(256), 0, s, (const uint4*)G,
                     (const uint4*)U, (uint4*)h, nchunk);
  return hipGetLastError();
}

}  // namespace ffn
