// Host-side launchers of the gfx950 kernels (internal to libffn; the public
// C ABI is include/ffn.h).  Each launcher assumes its arguments were already
// validated by the API layer and only enqueues kernels on `s`.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ffn {

// Per-dispatch timing.  While the API layer's per-kernel timing is on for
// the calling thread, dispatch_events() hands out a fresh (start, stop)
// event pair for the next kernel, which hipExtLaunchKernel binds to the
// dispatch itself (the kernel's own begin and end timestamps, not event
// records around it); otherwise both are null and the launch is plain.
void dispatch_events(hipEvent_t* start, hipEvent_t* stop);

// Compute units of the current device (256 if the runtime cannot tell).
int device_cus();

// Workgroups of `kern` (block threads, no dynamic LDS) resident at once on
// the device; 0 if the runtime cannot tell.
template <class Kern>
inline int resident_slots(Kern kern, int block) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, block, 0) != hipSuccess || per_cu < 1)
    return 0;
  return per_cu * device_cus();
}

// Grid of a weight-streaming projection of N output rows whose workgroups
// each own an equal share (at most 16: one MFMA tile) of the rows, given
// `slots` resident workgroups.  policy 0: one workgroup per 16-row tile;
// 1: if the tiles fit one round, fill that round (every compute unit gets an
// equal number of rows); 2: also, past one round, whole rounds; 3: with at
// least one tile per compute unit (`cus` of them), the same number of
// workgroups on every compute unit, in as many rounds as that takes (fewer
// tiles: as policy 1).
inline int stream_groups(int N, int slots, int policy, int cus = 0) {
  const int t0 = (N + 15) / 16;
  if (policy <= 0 || slots < 1) return t0;
  if (policy >= 3 && cus > 0 && t0 >= cus) return (t0 + cus - 1) / cus * cus;
  if (t0 <= slots) return 2 * t0 > slots ? slots : t0;
  return policy >= 2 ? (t0 + slots - 1) / slots * slots : t0;
}

// RMSNorm, one wavefront per row ("When to hand-write a GPU kernel on Apple
// Silicon", Rung 2 / Rung 4).  elem_bytes 2 = bf16, 4 = fp32.
hipError_t launch_rmsnorm(int elem_bytes, const void* x, const void* g, void* y,
                          int64_t rows, int64_t d, float eps, hipStream_t s);

// Decode (few tokens) weight-streaming projections on bf16 MFMA.
//   gate/up: h[M,f] = silu(n Wg^T) * (n Wu^T) with n = rmsnorm(x) * g folded in
//   down   : y[M,d] = x + h Wd^T
int decode_max_tokens();    // largest M routed to the decode kernels
int decode_chunk_tokens();  // tokens per decode launch (row-major h)
int decode_gateup_tokens(); // tokens per decode gate/up launch writing blocked h
hipError_t launch_decode_gateup_norm(const void* x, const void* g, const void* wg, const void* wu,
                                     void* h, int M, int d, int f, float eps, hipStream_t s);
// 1 if the decode gate/up kernel writes h in the blocked layout (token tile,
// 128-k stage, MFMA operand order; T token tiles take T * 16 * ceil(f/128) *
// 128 elements), which the down kernel then reads with h_blocked = true;
// h from any other producer is row-major [M, f] (h_blocked = false).
int decode_h_blocked();
hipError_t launch_decode_down(const void* h, const void* wd, const void* x, void* y,
                              int M, int d, int f, bool h_blocked, hipStream_t s);
// Single-dispatch block for 1..16 tokens: gate/up tiles, then (tile, K range)
// down items in one launch ordered by completion counters (ctr: caller's
// workspace, cleared by a preceding launch; part: [splits, M, d] fp32).
int decode_persistent_splits(int d, int f);
size_t decode_persistent_counters(int d, int splits);
hipError_t launch_decode_persistent(const void* x, const void* g, const void* wg, const void* wu,
                                    const void* wd, void* h, float* part, unsigned* ctr, void* y,
                                    int M, int d, int f, float eps, hipStream_t s);

// Prefill (many tokens) LDS-tiled bf16 MFMA GEMMs, C[m][n] = sum_k A[m][k] W[n][k].
// ldo (0: the output width): row stride of h / y and the residual, for a
// GEMM over a column block of a wider output (pointers at the block).
hipError_t launch_gemm_gateup_fused(const void* n, const void* wg, const void* wu, void* h,
                                    int M, int d, int f, hipStream_t s, int ldo = 0);
// The same with the RMSNorm folded in: x (not n) and the gain g go in, and
// r_m scales the accumulators in the epilogue (register-staged kernel).
hipError_t launch_gemm_gateup_fused_norm(const void* x, const void* g, const void* wg,
                                         const void* wu, void* h, int M, int d, int f, float eps,
                                         hipStream_t s);
hipError_t launch_gemm_store(const void* a, const void* w, void* c, int M, int N, int K,
                             hipStream_t s);
hipError_t launch_gemm_residual(const void* a, const void* w, const void* resid, void* y,
                                int M, int N, int K, hipStream_t s, int ldo = 0);
// Split K for prefill GEMMs whose tiles leave compute units idle.  A plan
// runs output columns [0, main) with the launchers above and splits the
// columns [main, N) over K into z ranges (z = 1: no split, main = N; main =
// 0: the whole GEMM splits), with the GEMMs below that write fp32 partial
// sums instead of their epilogue -- fused gate/up: gate sums in
// part[z][M][f], up sums in part[Z + z][M][f]; down: part[z][M][d], f and d
// being the split block's width -- for launch_splitk_swiglu /
// launch_splitk_residual.
constexpr int kPrefillMaxSplits = 16;
struct PrefillPlan {
  int main = 0, z = 1;
};
PrefillPlan prefill_gateup_plan(int M, int d, int f);
PrefillPlan prefill_down_plan(int M, int d, int f);
hipError_t launch_gemm_gateup_fused_part(const void* n, const void* wg, const void* wu, float* part,
                                         int Z, int M, int d, int f, hipStream_t s);
hipError_t launch_gemm_down_part(const void* h, const void* wd, float* part, int Z, int M, int d,
                                 int f, hipStream_t s);
// h[m,j] = bf16(silu(sum_z G_z[m,j]) * sum_z U_z[m,j]), ranges added in z
// order, from the partial planes above (f % 8 == 0).  ldo (0: f): row
// stride of h in elements, a multiple of 8, when the planes cover a column
// block of a wider h (h then points at the block's first column).
hipError_t launch_splitk_swiglu(const float* part, int splits, void* h, int M, int f,
                                hipStream_t s, int ldo = 0);
// h = silu(G) * U elementwise over `count` bf16 values (count % 8 == 0).
hipError_t launch_swiglu_bf16(const void* G, const void* U, void* h, int64_t count,
                              hipStream_t s);

// fp32 path (all fp32 arithmetic, SIMT tiles).
enum F32Epi { F32_STORE = 0, F32_SWIGLU = 1, F32_RESIDUAL = 2 };
hipError_t launch_gemm_f32(int epi, const float* a, const float* w0, const float* w1,
                           const float* resid, float* c, int M, int N, int K, hipStream_t s);
hipError_t launch_swiglu_f32(const float* G, const float* U, float* h, int64_t count,
                             hipStream_t s);

// Most K ranges of a split-K down projection (quantised blocks).
constexpr int kQuantMaxSplits = 8;

// Q8_0 weight-streaming projections (bf16 activations, in-register dequant).
//   gate/up: h = silu(n Wg^T) * (n Wu^T); with gain != nullptr (M <= 8) act
//            is x and n = rmsnorm(x) * gain is folded in (eps inside the
//            root), otherwise act is n
//   down   : y = x + h Wd^T
hipError_t launch_q8_gateup(const void* act, const void* gain, float eps, const int8_t* qg,
                            const uint16_t* sg, const int8_t* qu, const uint16_t* su, void* h,
                            int M, int d, int f, hipStream_t s);
// Down projection, split over K into q8_down_splits(M, d, f) ranges when that
// is above 1 (partials in part[splits][M][d], as for Q4_0 below).
int q8_down_splits(int M, int N, int K);
hipError_t launch_q8_down(const void* h, const int8_t* qd, const uint16_t* sd, const void* x,
                          void* y, float* part, int M, int d, int f, hipStream_t s);
int q8_max_tokens();

// Q4_0 weight-streaming projections (split nibble / scale arrays, bf16
// activations, in-register dequant); same roles as the Q8_0 launchers.
hipError_t launch_q4_gateup(const void* act, const void* gain, float eps, const uint8_t* qg,
                            const uint16_t* sg, const uint8_t* qu, const uint16_t* su, void* h,
                            int M, int d, int f, hipStream_t s);
// Down projection, split over K into q4_down_splits(M, d, f) ranges when that
// is above 1: the fp32 partial sums go to part[splits][M][d] (caller's
// workspace) and launch_splitk_residual adds them to x in range order.
int q4_down_splits(int M, int N, int K);
hipError_t launch_q4_down(const void* h, const uint8_t* qd, const uint16_t* sd, const void* x,
                          void* y, float* part, int M, int d, int f, hipStream_t s);
int q4_max_tokens();

// y[m,i] = bf16(x[m,i] + sum_{z < splits} part[z][m][i]), summed in z order
// (N % 8 == 0; splits <= kPrefillMaxSplits).  ldo (0: N): row stride of x
// and y in elements, a multiple of 8, when the partials cover a column block
// of a wider output (the pointers then point at the block's first column).
hipError_t launch_splitk_residual(const float* part, int splits, const void* x, void* y, int M,
                                  int N, hipStream_t s, int ldo = 0);

// Bandwidth probes.
int probe_read_groups(int waves_per_cu);
hipError_t launch_probe_read(const void* src, size_t bytes, void* sink, int waves_per_cu,
                             hipStream_t s);
// groups_per_cu > 0: grid-stride copy with that many 256-thread workgroups
// per CU; 0: one workgroup per contiguous 16 KiB chunk.
int probe_copy_groups(size_t bytes, int groups_per_cu);
hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, int groups_per_cu,
                             bool nontemporal, hipStream_t s);
// Matrix-core loop: probe_mfma_groups(waves_per_cu) workgroups of 4 waves,
// each wave 8 * iters bf16 16x16x32 MFMAs (16384 flop each).
int probe_mfma_groups(int waves_per_cu);
hipError_t launch_probe_mfma(int iters, int waves_per_cu, float* sink, hipStream_t s);

}  // namespace ffn

// Every kernel of the library is enqueued through this macro.
#define FFN_DISPATCH(kernel, grid, block, lds, stream, ...)                                     \
  do {                                                                                          \
    hipEvent_t ffn_e0_ = nullptr, ffn_e1_ = nullptr;                                            \
    ::ffn::dispatch_events(&ffn_e0_, &ffn_e1_);                                                 \
    hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, ffn_e0_, ffn_e1_, 0u, __VA_ARGS__); \
  } while (0)
