"""Seeded synthetic inputs for the pre-norm SwiGLU FFN block.

This module only draws and encodes numbers; it holds none of the block's
arithmetic (no norm, no activation, no projection).  Both the GPU path (via
the tests and the benchmark) and the fp64 oracle receive the exact same
host arrays produced here, so the two sides compare on identical bits.

Recipe (one generator per workload, numpy PCG64 seeded per workload):
  draw order is x, g, W_gate, W_up, W_down; every tensor is drawn in fp32,
  scaled/shifted in fp32, then rounded ONCE to the storage dtype
  (round-to-nearest-even for bf16).
  * x      ~ N(0, 1)
  * g      ~ 1 + N(0, 0.1)
  * W_*    ~ N(0, 0.02), row-major, W_gate/W_up [f, d], W_down [d, f]
  * the large RMSNorm workload scales a seeded 1% subset of rows by 100
    (before the single rounding) to create outlier rows;
  * Q8_0 weights: integers uniform in [-127, 127] and one fp16 scale per
    32 consecutive weights along the reduction axis, drawn as
    fp16(|N(0, 0.02)| / 127 * 4).

Storage formats handed out:
  * bf16 tensors as uint16 bit patterns (numpy has no bfloat16),
  * fp32 tensors as float32,
  * Q8_0 matrices as (qs int8 [N, K], scales uint16 fp16-bits [N, K/32]).
"""
from __future__ import annotations

import dataclasses

import numpy as np

EPS = float(np.float32(1e-6))


# ----------------------------------------------------------------------------
# encoders (storage formats only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even), return the uint16 bit patterns.

    Inputs here are finite by construction, so no NaN handling is needed."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact). Used by test helpers only."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to IEEE fp16 (numpy's round-to-nearest-even), keep subnormals."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class BlockInputs:
    """One block's inputs.  dtype 'bf16' -> uint16 bit arrays; 'f32' -> float32."""
    dtype: str
    x: np.ndarray        # [M, d]
    g: np.ndarray        # [d]
    w_gate: np.ndarray   # [f, d]
    w_up: np.ndarray     # [f, d]
    w_down: np.ndarray   # [d, f]
    eps: float = EPS

    @property
    def M(self) -> int:
        return self.x.shape[0]

    @property
    def d(self) -> int:
        return self.x.shape[1]

    @property
    def f(self) -> int:
        return self.w_gate.shape[0]


@dataclasses.dataclass
class Q8Matrix:
    qs: np.ndarray       # int8 [N, K]
    scales: np.ndarray   # uint16 (fp16 bits) [N, K // 32]


@dataclasses.dataclass
class Q8BlockInputs:
    x: np.ndarray        # bf16 bits [M, d]
    g: np.ndarray        # bf16 bits [d]
    w_gate: Q8Matrix     # [f, d]
    w_up: Q8Matrix       # [f, d]
    w_down: Q8Matrix     # [d, f]
    eps: float = EPS

    @property
    def M(self) -> int:
        return self.x.shape[0]

    @property
    def d(self) -> int:
        return self.x.shape[1]

    @property
    def f(self) -> int:
        return self.w_gate.qs.shape[0]


def _normal(rng: np.random.Generator, shape, std: float, mean: float = 0.0) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return a


def _encode(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(a)
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    raise ValueError(dtype)


def make_block(seed: int, M: int, d: int, f: int, dtype: str = "bf16",
               x_std: float = 1.0, w_std: float = 0.02, g_std: float = 0.1,
               eps: float = EPS) -> BlockInputs:
    """Seeded block inputs, draw order x, g, W_gate, W_up, W_down."""
    rng = np.random.default_rng(seed)
    x = _normal(rng, (M, d), x_std)
    g = _normal(rng, (d,), g_std, 1.0)
    wg = _normal(rng, (f, d), w_std)
    wu = _normal(rng, (f, d), w_std)
    wd = _normal(rng, (d, f), w_std)
    return BlockInputs(dtype, _encode(x, dtype), _encode(g, dtype), _encode(wg, dtype),
                       _encode(wu, dtype), _encode(wd, dtype), eps)


def make_rmsnorm(seed: int, rows: int, d: int, dtype: str = "bf16",
                 outlier_frac: float = 0.01, outlier_scale: float = 100.0,
                 eps: float = EPS):
    """Seeded RMSNorm inputs: x ~ N(0,1) with round(outlier_frac*rows) rows
    (chosen by a seeded permutation, without replacement) scaled by
    outlier_scale before the single rounding; g ~ 1 + N(0, 0.1).

    Returns (x, g, eps, outlier_rows)."""
    rng = np.random.default_rng(seed)
    x = _normal(rng, (rows, d), 1.0)
    g = _normal(rng, (d,), 0.1, 1.0)
    n_out = int(round(outlier_frac * rows))
    out_rows = np.sort(rng.permutation(rows)[:n_out]) if n_out else np.zeros(0, np.int64)
    if n_out:
        x[out_rows] *= np.float32(outlier_scale)
    return _encode(x, dtype), _encode(g, dtype), eps, out_rows


def make_q8_matrix(rng: np.random.Generator, N: int, K: int,
                   s_std: float = 0.02) -> Q8Matrix:
    """Q8_0 matrix [N, K]: int8 uniform in [-127, 127]; one fp16 scale per 32
    consecutive weights of a row, fp16(|N(0, s_std)| / 127 * 4)."""
    if K % 32:
        raise ValueError("Q8_0 needs K % 32 == 0")
    qs = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    z = np.abs(rng.standard_normal(size=(N, K // 32), dtype=np.float32))
    z *= np.float32(s_std)
    s = (z / np.float32(127.0)) * np.float32(4.0)
    return Q8Matrix(qs, f32_to_f16_bits(s))


def make_q8_block(seed: int, M: int, d: int, f: int, eps: float = EPS) -> Q8BlockInputs:
    """Seeded Q8_0 block inputs, draw order x, g, W_gate, W_up, W_down."""
    rng = np.random.default_rng(seed)
    x = f32_to_bf16_bits(_normal(rng, (M, d), 1.0))
    g = f32_to_bf16_bits(_normal(rng, (d,), 0.1, 1.0))
    wg = make_q8_matrix(rng, f, d)
    wu = make_q8_matrix(rng, f, d)
    wd = make_q8_matrix(rng, d, f)
    return Q8BlockInputs(x, g, wg, wu, wd, eps)


def q8_aos_to_soa(blocks: np.ndarray, N: int, K: int) -> Q8Matrix:
    """Convert the interleaved 34-byte block form (2-byte fp16 scale, then 32
    int8) of an [N, K] matrix, as a uint8 array of N*K/32*34 bytes, into the
    split form the library takes (qs [N, K] + scales [N, K/32])."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(N, K // 32, 34)
    scales = b[:, :, 0:2].copy().view(np.uint16).reshape(N, K // 32)
    qs = b[:, :, 2:34].copy().view(np.int8).reshape(N, K)
    return Q8Matrix(qs, scales)


def q8_soa_to_aos(m: Q8Matrix) -> np.ndarray:
    """Inverse of q8_aos_to_soa."""
    N, K = m.qs.shape
    out = np.empty((N, K // 32, 34), dtype=np.uint8)
    out[:, :, 0:2] = m.scales.reshape(N, K // 32, 1).view(np.uint8).reshape(N, K // 32, 2)
    out[:, :, 2:34] = m.qs.reshape(N, K // 32, 32).view(np.uint8)
    return out.reshape(-1)


@dataclasses.dataclass
class Q4Matrix:
    qs: np.ndarray       # uint8 [N, K // 2]: per block of 32 weights along K, byte i
                         # holds weight i (low four bits) and weight i + 16 (high four bits)
    scales: np.ndarray   # uint16 (fp16 bits) [N, K // 32]


@dataclasses.dataclass
class Q4BlockInputs:
    x: np.ndarray        # bf16 bits [M, d]
    g: np.ndarray        # bf16 bits [d]
    w_gate: Q4Matrix     # [f, d]
    w_up: Q4Matrix       # [f, d]
    w_down: Q4Matrix     # [d, f]
    eps: float = EPS

    @property
    def M(self) -> int:
        return self.x.shape[0]

    @property
    def d(self) -> int:
        return self.x.shape[1]

    @property
    def f(self) -> int:
        return self.w_gate.qs.shape[0]


def pack_q4_nibbles(n: np.ndarray) -> np.ndarray:
    """[N, K] nibbles (uint8 in [0, 15]) -> [N, K // 2] bytes, block layout
    of Q4Matrix.qs (storage format only)."""
    N, K = n.shape
    b = n.reshape(N, K // 32, 2, 16)
    return (b[:, :, 0, :] | (b[:, :, 1, :] << 4)).astype(np.uint8).reshape(N, K // 2)


def make_q4_matrix(rng: np.random.Generator, N: int, K: int,
                   s_std: float = 0.02) -> Q4Matrix:
    """Q4_0 matrix [N, K]: nibbles uniform in [0, 15] (weight = nibble - 8);
    one fp16 scale per 32 consecutive weights of a row, fp16(|N(0, s_std)| / 8 * 4)."""
    if K % 32:
        raise ValueError("Q4_0 needs K % 32 == 0")
    n = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    z = np.abs(rng.standard_normal(size=(N, K // 32), dtype=np.float32))
    z *= np.float32(s_std)
    s = (z / np.float32(8.0)) * np.float32(4.0)
    return Q4Matrix(pack_q4_nibbles(n), f32_to_f16_bits(s))


def make_q4_block(seed: int, M: int, d: int, f: int, eps: float = EPS) -> Q4BlockInputs:
    """Seeded Q4_0 block inputs, draw order x, g, W_gate, W_up, W_down."""
    rng = np.random.default_rng(seed)
    x = f32_to_bf16_bits(_normal(rng, (M, d), 1.0))
    g = f32_to_bf16_bits(_normal(rng, (d,), 0.1, 1.0))
    wg = make_q4_matrix(rng, f, d)
    wu = make_q4_matrix(rng, f, d)
    wd = make_q4_matrix(rng, d, f)
    return Q4BlockInputs(x, g, wg, wu, wd, eps)


def q4_aos_to_soa(blocks: np.ndarray, N: int, K: int) -> Q4Matrix:
    """Convert the interleaved 18-byte block form (2-byte fp16 scale, then 16
    bytes of nibbles) of an [N, K] matrix into the split form the library
    takes (qs [N, K/2] + scales [N, K/32])."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(N, K // 32, 18)
    scales = b[:, :, 0:2].copy().view(np.uint16).reshape(N, K // 32)
    qs = b[:, :, 2:18].copy().reshape(N, K // 2)
    return Q4Matrix(qs, scales)


def q4_soa_to_aos(m: Q4Matrix) -> np.ndarray:
    """Inverse of q4_aos_to_soa."""
    N, H = m.qs.shape
    nb = H // 16
    out = np.empty((N, nb, 18), dtype=np.uint8)
    out[:, :, 0:2] = m.scales.reshape(N, nb, 1).view(np.uint8).reshape(N, nb, 2)
    out[:, :, 2:18] = m.qs.reshape(N, nb, 16)
    return out.reshape(-1)


# Named workloads (sizes of the pages' two regimes plus the tiny, norm and Q8 cases).
WORKLOADS = {
    "tiny_f32":   dict(seed=1, M=8, d=256, f=704, dtype="f32"),
    "rmsnorm":    dict(seed=2, rows=16384, d=4096, dtype="bf16"),
    "decode":     dict(seed=3, M=16, d=4096, f=11008, dtype="bf16"),
    "prefill":    dict(seed=4, M=8192, d=4096, f=14336, dtype="bf16"),
    "q8_decode":  dict(seed=5, M=8, d=5120, f=17408),
    "q4_decode":  dict(seed=6, M=8, d=5120, f=17408),
    # one GPU's share of a block tensor-parallel over f on 8 GPUs: W_gate and
    # W_up keep f/8 rows, W_down f/8 columns (f/8 stays a multiple of 32)
    "decode_tp8_shard":  dict(seed=7, M=16, d=4096, f=11008 // 8, dtype="bf16"),
    "prefill_tp8_shard": dict(seed=8, M=8192, d=4096, f=14336 // 8, dtype="bf16"),
    "q8_tp8_shard":      dict(seed=9, M=8, d=5120, f=17408 // 8),
    "q4_tp8_shard":      dict(seed=10, M=8, d=5120, f=17408 // 8),
    # between decode and prefill: the decode block's weights at batch sizes
    # whose GEMM tiles do not fill the chip (the first M rows of x)
    "mid_batch":         dict(seed=11, M=(128, 512, 768, 2048), d=4096, f=11008, dtype="bf16"),
}
