"""fp64 CPU oracle for the pre-norm SwiGLU FFN block.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the tests, the smoke
check and the benchmark's CPU-baseline leg may import this module.  It
shares no code with the HIP path and imports nothing from it: it receives
plain numpy arrays (bf16 as uint16 bit patterns, fp16 scales as uint16 bit
patterns, fp32 as float32, Q8 quants as int8) and decodes them itself.

Every function is the plain definition, evaluated in float64, written so
that it can be checked against the pages by eye:

  n = rmsnorm(x) * g                 per row: r = 1 / sqrt(mean(x^2) + eps)
  G = n W_gate^T,  U = n W_up^T      the gate and up projections
  h = silu(G) * U                    silu(v) = v / (1 + exp(-v))
  y = x + h W_down^T                 down projection plus residual

Library primitives used as single steps: numpy matmul (fp64), numpy exp,
numpy's fp16 decoder.  There is no blocking, fusion or reordering beyond
what the definitions state.

Readings taken where the pages leave a step open:
  * eps sits inside the root, added to the mean of squares (as the
    RMSNorm reduction on "When to hand-write a GPU kernel on Apple Silicon",
    Rung 2, computes it);
  * the gain multiplies (n = x * r * g), it is not (1 + g);
  * weights are row-major [out, in], so each projection is act @ W^T;
  * the residual adds the un-normalised input x (pre-norm placement; the
    pages never state where the norm sits);
  * Q8_0 blocks run along the reduction axis of each matrix; the 32 quants
    of a block share the block's fp16 scale;
  * Q4_0 blocks likewise; inside a block byte i holds weight i (low nibble)
    and weight i + 16 (high nibble), and a weight is (nibble - 8) * scale;
  * the oracle keeps every intermediate in fp64 (it does not mimic the
    GPU's bf16 roundings of n and h).

Parity status: every function here is pinned by the CPU tests (closed
forms, invariants, hand-derived fixtures, special cases), the stored-format
wrappers at the end included (hand-worked fixtures encoded as bf16 and fp32
bit patterns, known-bit fp32 values); planted mistakes in each of them make
the pins fail.
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------
# exact decoders (the oracle's own, independent of any other module)
# ----------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64.  Exact: bf16 is the top half of
    an IEEE binary32, so widening by a 16-bit shift and converting is exact."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> float64, exact, subnormals kept."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Decode a stored tensor ('bf16' bit patterns or 'f32') to float64."""
    if dtype == "bf16":
        return bf16_to_f64(a)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(a, dtype=np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# the method
# ----------------------------------------------------------------------------
def silu(v: np.ndarray) -> np.ndarray:
    """silu(v) = v / (1 + exp(-v)), the gate activation of SwiGLU
    ("When to hand-write a GPU kernel on Apple Silicon", Rung 1).

    Evaluated in the algebraically equal form v * e^v / (1 + e^v) for v < 0
    so that exp never overflows."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    pos = v >= 0
    out[pos] = v[pos] / (1.0 + np.exp(-v[pos]))
    e = np.exp(v[~pos])
    out[~pos] = v[~pos] * e / (1.0 + e)
    return out


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of each row of x (fp64 in, fp64 out)
    ("When to hand-write a GPU kernel on Apple Silicon", Rung 2):
      r_m = 1 / sqrt( (1/d) * sum_k x[m,k]^2 + eps ),   n[m,k] = x[m,k] * r_m * g[k].
    The sum of squares runs sequentially along the row."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    d = x.shape[-1]
    ms = np.zeros(x.shape[:-1], dtype=np.float64)
    for k in range(d):
        ms += x[..., k] * x[..., k]
    ms /= d
    r = 1.0 / np.sqrt(ms + eps)
    return x * r[..., None] * g


def swiglu_block(x, g, w_gate, w_up, w_down, eps: float) -> np.ndarray:
    """The pre-norm SwiGLU feed-forward block on fp64 arrays:
      n = rmsnorm(x) * g                                     (Rung 2, first page)
      G = n W_gate^T, U = n W_up^T     gate and up projections of the SwiGLU MLP
                                       ("Unfusing a Kernel Made It 1.63x Faster", Finding 1)
      h = silu(G) * U                                        (Rung 1, first page)
      y = x + h W_down^T               FFN-down projection ("Megakernels on Mac",
                                       "Projection shape changes the achieved rate"),
                                       plus the residual x.
    Shapes: x [M,d], g [d], w_gate/w_up [f,d], w_down [d,f] -> y [M,d]."""
    x = np.asarray(x, dtype=np.float64)
    n = rmsnorm(x, g, eps)
    G = n @ np.asarray(w_gate, dtype=np.float64).T
    U = n @ np.asarray(w_up, dtype=np.float64).T
    h = silu(G) * U
    return x + h @ np.asarray(w_down, dtype=np.float64).T


def swiglu_block_intermediates(x, g, w_gate, w_up, w_down, eps: float):
    """Same as swiglu_block, also returning (n, G, U, h) for diagnostics."""
    x = np.asarray(x, dtype=np.float64)
    n = rmsnorm(x, g, eps)
    G = n @ np.asarray(w_gate, dtype=np.float64).T
    U = n @ np.asarray(w_up, dtype=np.float64).T
    h = silu(G) * U
    y = x + h @ np.asarray(w_down, dtype=np.float64).T
    return y, n, G, U, h


def q8_dequant(qs: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """Q8_0 matrix [N, K] -> fp64 weights: w[j,k] = q[j,k] * s[j, k // 32].
    The Q8_0 format (named on "Unfusing a Kernel Made It 1.63x Faster",
    Finding 2) holds 32 int8 quants and one fp16 scale per block; blocks run
    along K, the reduction axis."""
    q = np.asarray(qs, dtype=np.int8).astype(np.float64)
    s = f16_to_f64(scale_bits)
    N, K = q.shape
    if s.shape != (N, K // 32) or K % 32:
        raise ValueError("scales must be [N, K/32] with K % 32 == 0")
    return q * np.repeat(s, 32, axis=1)


def swiglu_block_q8(x_bits, g_bits, wg, wu, wd, eps: float) -> np.ndarray:
    """The block with Q8_0 weights (each weight matrix given as a pair
    (qs, scale_bits)) and bf16 activations; weights are dequantised exactly
    and the block is evaluated by swiglu_block in fp64."""
    x = bf16_to_f64(x_bits)
    g = bf16_to_f64(g_bits)
    return swiglu_block(x, g, q8_dequant(*wg), q8_dequant(*wu), q8_dequant(*wd), eps)


def q4_dequant(qs: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """Q4_0 matrix -> fp64 weights [N, K].  The format (the 18-byte blocks of
    "Unfusing a Kernel Made It 1.63x Faster", "The finding that keeps us
    honest about microbenchmarks": one fp16 scale and 16 bytes whose low and
    high nibbles hold different weights) is taken here as: per block of 32
    weights along K, byte i of the block's 16 holds weight i in its low four
    bits and weight i + 16 in its high four bits, and w = (nibble - 8) * s.
    qs [N, K/2] bytes, scale_bits [N, K/32] fp16 bits."""
    b = np.asarray(qs, dtype=np.uint8)
    N, H = b.shape
    K = 2 * H
    s = f16_to_f64(scale_bits)
    if K % 32 or s.shape != (N, K // 32):
        raise ValueError("qs must be [N, K/2] and scales [N, K/32] with K % 32 == 0")
    w = np.empty((N, K), dtype=np.float64)
    for blk in range(K // 32):
        byte = b[:, 16 * blk:16 * blk + 16].astype(np.int64)
        low = (byte & 0x0F) - 8                      # weights 32*blk + 0 .. 15
        high = (byte >> 4) - 8                       # weights 32*blk + 16 .. 31
        w[:, 32 * blk:32 * blk + 16] = low * s[:, blk:blk + 1]
        w[:, 32 * blk + 16:32 * blk + 32] = high * s[:, blk:blk + 1]
    return w


def swiglu_block_q4(x_bits, g_bits, wg, wu, wd, eps: float) -> np.ndarray:
    """The block with Q4_0 weights (each matrix a pair (qs, scale_bits)) and
    bf16 activations; weights are dequantised exactly (4-bit integer times an
    fp16 scale) and the block is evaluated by swiglu_block in fp64."""
    x = bf16_to_f64(x_bits)
    g = bf16_to_f64(g_bits)
    return swiglu_block(x, g, q4_dequant(*wg), q4_dequant(*wu), q4_dequant(*wd), eps)


# ----------------------------------------------------------------------------
# convenience wrappers taking stored-format inputs
# ----------------------------------------------------------------------------
def block_from_stored(dtype: str, x, g, w_gate, w_up, w_down, eps: float) -> np.ndarray:
    """swiglu_block on stored-format inputs ('bf16' bit patterns or 'f32'):
    each tensor is decoded exactly to fp64 by as_f64, then the block's
    definition is evaluated with the operands in their own roles."""
    return swiglu_block(as_f64(x, dtype), as_f64(g, dtype), as_f64(w_gate, dtype),
                        as_f64(w_up, dtype), as_f64(w_down, dtype), eps)


def rmsnorm_from_stored(dtype: str, x, g, eps: float) -> np.ndarray:
    """rmsnorm on stored-format inputs ('bf16' bit patterns or 'f32')."""
    return rmsnorm(as_f64(x, dtype), as_f64(g, dtype), eps)
