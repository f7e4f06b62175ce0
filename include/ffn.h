/*
 * ffn.h - C ABI of libffn.so, the MI355X (gfx950) pre-norm SwiGLU
 * feed-forward block:
 *
 *     n = rmsnorm(x) * g                 r_m = 1 / sqrt(mean_k x[m,k]^2 + eps)
 *     y = x + (silu(n W_gate^T) * (n W_up^T)) W_down^T,   silu(v) = v / (1 + e^-v)
 *
 * Sources of the operations (page title, section):
 *   - RMSNorm, one reduction per row, eps inside the root:
 *       "When to hand-write a GPU kernel on Apple Silicon", Rung 2 and Rung 4.
 *   - SwiGLU silu(gate) * up, activation evaluated in fp32:
 *       "When to hand-write a GPU kernel on Apple Silicon", Rung 1.
 *   - gate and up projections of the SwiGLU MLP, fused in one kernel or
 *     dispatched as two GEMMs plus the activation:
 *       "Unfusing a Kernel Made It 1.63x Faster", Finding 1.
 *   - the FFN-down projection:
 *       "Megakernels on Mac", "Projection shape changes the achieved rate".
 *   - Q8_0 weights (32 int8 quants share one fp16 scale):
 *       "Unfusing a Kernel Made It 1.63x Faster", Finding 2 (format name).
 *   - Q4_0 weights (18-byte blocks: one fp16 scale and 16 bytes whose low
 *     and high nibbles are different weights), stored repacked:
 *       "Unfusing a Kernel Made It 1.63x Faster", "The finding that keeps us
 *       honest about microbenchmarks".
 *   - explicit supported shapes and failure behaviour, ownership of buffers
 *     that submitted work still reads:
 *       "Megakernels on Mac", "Choosing a fusion boundary" and
 *       "Dependencies and synchronization".
 * The pages do not place the norm or the residual; this library takes the
 * pre-norm reading: the residual adds the un-normalised x.
 *
 * Conventions for every entry point:
 *   - Tensors are DEVICE pointers to contiguous row-major arrays. Weights are
 *     [out, in]: W_gate, W_up are [f, d], W_down is [d, f].
 *   - The caller owns every buffer and keeps it alive until the work queued
 *     on `stream` has completed. The library never allocates device memory,
 *     never synchronises and never prints.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream). Intermediates live in the caller's workspace and are ordered
 *     by the stream.
 *   - Arguments are validated before anything is launched; a failing call
 *     launches nothing and returns a status; ffn_last_error() then gives a
 *     thread-local message.  Device faults surface at the caller's next
 *     synchronisation.
 *   - bf16 values are passed as raw 16-bit patterns (uint16_t storage).
 *   - M == 0 (or rows == 0) returns FFN_OK and launches nothing.
 *   - Output buffers must not overlap any input or the workspace.
 *   - Results for a fixed variant are run-to-run bitwise deterministic (no
 *     floating-point atomics); different variants may differ by rounding.
 */
#ifndef FFN_H
#define FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums below cross the ABI as plain ints: a caller may pass any value
 * (the library rejects unknown ones).  C++ gives them a fixed int
 * representation so that such a value is well defined there too. */
#ifdef __cplusplus
#define FFN_ENUM_BASE : int
#else
#define FFN_ENUM_BASE
#endif

typedef enum FFN_ENUM_BASE {
  FFN_OK = 0,
  FFN_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, bad enum, overlap */
  FFN_ERR_UNSUPPORTED = 2,      /* shape/alignment outside what the kernels take   */
  FFN_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required      */
  FFN_ERR_LAUNCH = 4            /* a kernel launch was rejected by the runtime     */
} ffn_status;

typedef enum FFN_ENUM_BASE { FFN_F32 = 0, FFN_BF16 = 1 } ffn_dtype;

/* Schedule of the block.  FUSED computes both gate/up projections in one
 * kernel whose epilogue applies silu(G)*U; SPLIT runs the gate GEMM, the up
 * GEMM and a separate activation pass ("Unfusing a Kernel Made It 1.63x
 * Faster", Finding 1).  PERSISTENT (bf16, 1 <= M <= 16 only) runs the whole
 * block as one dispatch whose work items wait on device-scope completion
 * counters instead of kernel boundaries ("Megakernels on Mac", the
 * persistent-kernel experiment); a second, tiny launch before it clears the
 * counters.  AUTO takes, for bf16, the weight-streaming decode kernels up
 * to 64 tokens (the norm folded into the gate/up kernel, FUSED's
 * schedule) and FUSED beyond (measured faster than SPLIT at the prefill
 * shapes on this device); for fp32 it is FUSED.  FUSED_NORM (bf16) also
 * folds the RMSNorm into the fused gate/up GEMM of the prefill regime
 * (more than 64 tokens): the GEMM reads x, multiplies it by g on its way
 * into shared memory, sums x^2 over the K loop and scales both projections
 * by r_m in the epilogue, so no norm launch and no n round trip
 * ("Megakernels on Mac", "Dependencies and synchronization": the scale is
 * applied only after the whole row's sum); up to 64 tokens it is AUTO
 * (whose decode kernels fold the norm already). */
typedef enum FFN_ENUM_BASE {
  FFN_VARIANT_AUTO = 0,
  FFN_VARIANT_FUSED = 1,
  FFN_VARIANT_SPLIT = 2,
  FFN_VARIANT_PERSISTENT = 3,
  FFN_VARIANT_FUSED_NORM = 4
} ffn_variant;

/* One Q8_0 weight matrix [N, K] in split (structure-of-arrays) form:
 *   qs     : int8  [N, K]      quants, 32 consecutive along K form a block
 *   scales : fp16  [N, K/32]   IEEE binary16 bit patterns, one per block
 * weight[j,k] = qs[j,k] * scales[j, k/32].  Subnormal scales are honoured.
 * Both pointers are device pointers; qs 16-byte aligned, scales 2-byte. */
typedef struct {
  const int8_t *qs;
  const uint16_t *scales;
} ffn_q8_matrix;

/* One Q4_0 weight matrix [N, K] in split (repacked) form:
 *   qs     : uint8 [N, K/2]    16 bytes per 32-weight block; byte i of block
 *                              b holds weight 32b + i in its low nibble and
 *                              weight 32b + i + 16 in its high nibble
 *   scales : fp16  [N, K/32]   IEEE binary16 bit patterns, one per block
 * weight[j,k] = (nibble[j,k] - 8) * scales[j, k/32].  The 18-byte interleaved
 * blocks of the format are this layout's rows of (scale, 16 bytes); keeping
 * a row's nibble bytes contiguous lets every byte be fetched once.
 * Both pointers are device pointers; qs 16-byte aligned, scales 2-byte. */
typedef struct {
  const uint8_t *qs;
  const uint16_t *scales;
} ffn_q4_matrix;

/* RMSNorm of `rows` rows of length d:
 *   y[m,k] = x[m,k] * r_m * g[k],  r_m = 1/sqrt(sum_k x[m,k]^2 / d + eps)
 * ("When to hand-write a GPU kernel on Apple Silicon", Rung 2; the 16-byte
 * vector loads and the wavefront reduction follow Rung 4's lesson).
 *   dt    : FFN_F32 or FFN_BF16; x, g, y all have this dtype; the sum of
 *           squares and the scaling are computed in fp32, y rounded once.
 *   x [rows, d], g [d], y [rows, d]: device pointers, 16-byte aligned.
 *   d     : > 0; multiple of 8 (bf16) or 4 (fp32).
 *   eps   : >= 0.
 * Returns FFN_OK, INVALID_ARGUMENT (null, rows < 0, d <= 0, eps < 0 or NaN,
 * y overlapping x or g), UNSUPPORTED (d multiple / alignment), LAUNCH. */
ffn_status ffn_rmsnorm(ffn_dtype dt, const void *x, const void *g, void *y,
                       int64_t rows, int64_t d, float eps, void *stream);

/* Workspace bytes ffn_swiglu_block needs for this shape and variant (0 on a
 * shape it would reject).  It holds n [M,d] and h [M,f] (plus G, U [M,f]
 * for SPLIT; for PERSISTENT, fp32 partial sums [S, M, d] and
 * 4 * (2 + S + ceil(d/16)) bytes of counters, S = the schedule's number of
 * K ranges of the down projection, 1 to 8), each 256-byte aligned.  For
 * bf16 with AUTO, FUSED or FUSED_NORM and M <= 64 (the decode kernels) h
 * takes ceil(M/16) * 16 rows of ceil(f/128) * 128 elements: it is kept in
 * the down projection's operand order, not row-major.  For bf16 with more
 * than 64 tokens, GEMMs whose tiles (256 tokens x 256 weight rows; 128
 * tokens up to 128 tokens) number fewer than the device's compute units
 * are split over K: the workspace then also holds their fp32 partial sums,
 * one region sized for the larger of the fused gate/up GEMM's (2 Z_gu
 * [M, f] planes; not for SPLIT) and the down GEMM's (Z_dn [M, d] planes),
 * Z = floor(compute units / tiles), at most 16, at least one 64-deep K tile
 * per range (at d = 4096, f = 11008 on 256 CUs: Z_gu = 2 up to 256 tokens;
 * Z_dn = 16 / 8 / 4 / 2 up to 256 / 512 / 1024 / 2048 tokens).  A GEMM of
 * whole tiles needing more than one round of resident tiles, whose last
 * round holds at most half a round, splits only its last output columns
 * (those beyond the ones filling the earlier rounds): its planes are then
 * [M, columns split] (at 768 tokens and f = 11008, 16 planes of the last
 * 128 gate and up columns).  The size therefore depends on the current
 * device's compute-unit count and occupancy (256 CUs, one tile each, are
 * assumed where no device can be queried).  The workspace's contents are
 * the library's own between calls; the sizes are what a caller relies on. */
size_t ffn_swiglu_block_workspace_size(ffn_dtype dt, int64_t M, int64_t d, int64_t f,
                                       ffn_variant variant);

/* The full block y = x + W_down (silu(W_gate n) * (W_up n)), n = rmsnorm(x) g.
 *   dt        : FFN_BF16 (bf16 storage, fp32 accumulation; n and h are
 *               rounded to bf16 where they are a matrix-core operand) or
 *               FFN_F32 (all fp32).
 *   x [M,d], g [d], w_gate [f,d], w_up [f,d], w_down [d,f], y [M,d]: device
 *               pointers of dtype dt, 16-byte aligned.
 *   d, f      : > 0; multiples of 8 (bf16) or 4 (fp32); each weight matrix
 *               smaller than 2 GiB (32-bit buffer offsets).
 *   variant   : gate/up schedule (see ffn_variant).
 *   workspace : device buffer of at least
 *               ffn_swiglu_block_workspace_size(dt, M, d, f, variant) bytes,
 *               256-byte aligned; its contents are scratch.
 * Returns FFN_OK, INVALID_ARGUMENT, UNSUPPORTED, WORKSPACE or LAUNCH. */
/* PERSISTENT's bounded waits: a work item that gives up waiting for the
 * items it depends on (which only a fault elsewhere on the device could
 * cause) sets a 32-bit error word in the workspace and the call's result is
 * then wrong.  After the call has completed, the uint32 at byte offset
 * ffn_swiglu_block_persistent_status_offset(M, d, f) of the workspace is 0
 * on success and nonzero otherwise.  Its counter words must not be shared
 * with a call that overlaps on the device. */
ffn_status ffn_swiglu_block(ffn_dtype dt, const void *x, const void *g,
                            const void *w_gate, const void *w_up, const void *w_down,
                            void *y, int64_t M, int64_t d, int64_t f, float eps,
                            ffn_variant variant, void *workspace, size_t workspace_bytes,
                            void *stream);

/* Size of the library's own scratch array, per GPU (see below). */
#define FFN_NOALLOC_SCRATCH_BYTES (16u << 20)

/* ffn_swiglu_block for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, kernels and results as ffn_swiglu_block
 * minus the workspace: the intermediates live in a device array the
 * library itself holds, FFN_NOALLOC_SCRATCH_BYTES on every GPU it runs on,
 * from the library's load until the process ends.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); the
 * caller still passes every input and the output, on the current device.
 *   - A shape whose ffn_swiglu_block_workspace_size exceeds the array
 *     returns FFN_ERR_UNSUPPORTED (e.g. M = 64 fits for d + f up to 131072
 *     with FUSED; the 8192-token prefill shapes do not).
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents: calls that overlap on one GPU (two streams, two
 *     threads) race and give wrong results; serialise them.  Nothing in
 *     the array has to start at zero (PERSISTENT clears its counters with
 *     a kernel of its own).  PERSISTENT's error word is at
 *     ffn_swiglu_block_persistent_status_offset in that array, which the
 *     caller cannot read: use ffn_swiglu_block to check it.
 * Returns what ffn_swiglu_block returns, plus UNSUPPORTED as above and
 * LAUNCH if the array's device address cannot be found. */
ffn_status ffn_swiglu_block_noalloc(ffn_dtype dt, const void *x, const void *g,
                                    const void *w_gate, const void *w_up, const void *w_down,
                                    void *y, int64_t M, int64_t d, int64_t f, float eps,
                                    ffn_variant variant, void *stream);

/* Byte offset, inside a PERSISTENT call's workspace, of its uint32 error
 * word (see above); 0 for a shape PERSISTENT rejects (bf16, 1 <= M <= 16). */
size_t ffn_swiglu_block_persistent_status_offset(int64_t M, int64_t d, int64_t f);

/* Workspace bytes ffn_swiglu_block_q8 needs: n [M,d] (not when the norm is
 * folded into the gate/up kernel: M <= 8) and h [M,f] in bf16,
 * then the fp32 partial sums of the split-K down projection,
 * [splits, min(M, 32), d] (splits, 1..8, is fixed by d and f); 0 on a shape
 * the entry point would reject for its sizes (M > 64 included). */
size_t ffn_swiglu_block_q8_workspace_size(int64_t M, int64_t d, int64_t f);

/* The block with Q8_0 weights, bf16 activations:
 *   x [M,d], g [d], y [M,d]: bf16 device pointers, 16-byte aligned.
 *   w_gate, w_up : Q8_0 [f, d]; w_down : Q8_0 [d, f] (host structs holding
 *                  device pointers).
 *   M    : 0..64.  The weights stream from memory once per launch of at most
 *          32 tokens, so this is a weight-streaming (decode) entry point;
 *          M > 64 returns UNSUPPORTED.
 *   d, f : multiples of 32 (so no block straddles a row); f*d < 2^31.
 * Weights are dequantised in registers (q * s, exact in fp32) and never
 * written back; accumulation is fp32.
 * Returns FFN_OK, INVALID_ARGUMENT, UNSUPPORTED, WORKSPACE or LAUNCH. */
/* With the norm folded (see the workspace size) the gate/up kernel stages
 * bf16(x * g) and applies r_m to the fp32 sums, as the bf16 decode path
 * does; otherwise n is materialised in bf16 first.  h is rounded to bf16. */
ffn_status ffn_swiglu_block_q8(const void *x, const void *g, const ffn_q8_matrix *w_gate,
                               const ffn_q8_matrix *w_up, const ffn_q8_matrix *w_down,
                               void *y, int64_t M, int64_t d, int64_t f, float eps,
                               void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes ffn_swiglu_block_q4 needs: n [M,d] (not when the norm is
 * folded into the gate/up kernel: M <= 8 and (f/16) * (d/256) <= 10240,
 * both rounded up) and h [M,f] in bf16,
 * then the fp32 partial sums of the split-K down projection,
 * [splits, min(M, 32), d] (splits, 1..8, is fixed by d and f); 0 on a shape
 * the entry point would reject for its sizes (M > 64 included). */
size_t ffn_swiglu_block_q4_workspace_size(int64_t M, int64_t d, int64_t f);

/* The block with Q4_0 weights, bf16 activations ("Unfusing a Kernel Made It
 * 1.63x Faster", "The finding that keeps us honest about microbenchmarks"):
 *   x [M,d], g [d], y [M,d]: bf16 device pointers, 16-byte aligned.
 *   w_gate, w_up : Q4_0 [f, d]; w_down : Q4_0 [d, f] (host structs holding
 *                  device pointers).
 *   M    : 0..64 (weight-streaming regime, as for Q8_0; M > 64 returns
 *          UNSUPPORTED).
 *   d, f : multiples of 32 (so no block straddles a row); f*d/2 < 2^31 bytes
 *          of nibbles per matrix.
 * Weights are dequantised in registers ((nibble - 8) * s, exact in fp32) and
 * never written back; accumulation is fp32.  n (or, with the norm folded,
 * x * g) and h are rounded to bf16.
 * Returns FFN_OK, INVALID_ARGUMENT (null pointer, bad sizes or eps, y
 * overlapping an input or the workspace), UNSUPPORTED (multiples, alignment,
 * size limit), WORKSPACE or LAUNCH. */
ffn_status ffn_swiglu_block_q4(const void *x, const void *g, const ffn_q4_matrix *w_gate,
                               const ffn_q4_matrix *w_up, const ffn_q4_matrix *w_down,
                               void *y, int64_t M, int64_t d, int64_t f, float eps,
                               void *workspace, size_t workspace_bytes, void *stream);

/* Human-readable name of a status. Never NULL. */
const char *ffn_status_string(ffn_status s);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char *ffn_last_error(void);

/* ---- measurement helpers -------------------------------------------------
 * The pages separate a read-only streaming ceiling from a read+write one
 * and warn that the wrong one understates weight streaming
 * ("Unfusing a Kernel Made It 1.63x Faster", "Two published claims we got
 * wrong", claim 1).  These two kernels measure both on this device. */

/* Streams `bytes` (multiple of 16, >= 16) from src and writes one 16-byte
 * value per workgroup into sink (>= 16 * ffn_probe_read_groups() bytes) so
 * the loads cannot be removed. `waves_per_cu` (1..32) sets the grid. */
ffn_status ffn_probe_read(const void *src, size_t bytes, void *sink, int waves_per_cu,
                          void *stream);
int ffn_probe_read_groups(int waves_per_cu);

/* Copies `bytes` (multiple of 16) from src to dst with 16-byte streaming
 * loads and 16-byte stores (streaming stores if `nontemporal`).
 * groups_per_cu 1..64: a grid-stride loop over that many 256-thread
 * workgroups per CU; 0: one workgroup per contiguous 16 KiB chunk (the
 * pattern of a row-per-wave elementwise kernel).  Sweep both: the best is
 * the read+write ceiling. */
ffn_status ffn_probe_copy(const void *src, void *dst, size_t bytes, int groups_per_cu,
                          int nontemporal, void *stream);

/* The dense bf16 matrix-core ceiling at the clock the chip holds under that
 * load: ffn_probe_mfma_groups(waves_per_cu) workgroups of 4 waves, each wave
 * issuing 8 * iters independent v_mfma_f32_16x16x32_bf16 (16384 flop each)
 * from registers.  sink: >= 4 * 256 * groups bytes, written only in the
 * practically impossible case that the result equals a fixed value.
 * Returns INVALID_ARGUMENT for iters < 1 or waves_per_cu outside 1..32. */
ffn_status ffn_probe_mfma(int iters, int waves_per_cu, void *sink, void *stream);
int ffn_probe_mfma_groups(int waves_per_cu);

/* ---- per-kernel timing ----------------------------------------------------
 * When enabled, every kernel the library enqueues FROM THE CALLING THREAD
 * gets a pair of HIP events bound to the dispatch itself
 * (hipExtLaunchKernel), so a duration is the kernel's own begin-to-end
 * time, as a profiler's kernel trace reports it; ffn_timing_collect()
 * waits for them and accumulates per-kernel totals under the launch site's
 * name ("decode_gateup", "q8_down", ...; a site's second and later kernels
 * are "<name>/2", "<name>/3").  The state (switch, events, totals) is the
 * calling thread's own: timing enabled on one thread neither records nor
 * changes anything on another, so the library stays reentrant.  Off by
 * default.  Events are created at a thread's first timed dispatch and
 * destroyed when that thread disables timing.  At most max_launches
 * dispatches are timed between two collects; later ones run untimed. */
ffn_status ffn_timing_enable(int on, int max_launches);
int ffn_timing_enabled(void);            /* 1 if on for the calling thread  */
ffn_status ffn_timing_collect(void);     /* synchronises the recorded events */
int ffn_timing_count(void);              /* number of distinct kernel names   */
ffn_status ffn_timing_get(int index, const char **name, int64_t *launches, double *total_ms);
void ffn_timing_reset(void);

#ifdef __cplusplus
}
#endif
#endif /* FFN_H */
