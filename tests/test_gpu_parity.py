"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerances (per output tensor):
  * RMSNorm, strict per element |a - r| / |r|: 1e-2 for bf16 output (its own
    rounding alone is up to 2^-8), 1e-5 for fp32;
  * the block, max_i |a_i - r_i| / max_i |r_i|: 1e-2 for bf16, 2e-2 for Q8_0
    and Q4_0 (their dequantisation is exact on both sides; the bf16 roundings
    of n and h are the error, as in the bf16 block, with more cancellation in
    the down projection's sums), 1e-4 for the all-fp32 path (fp32 dot products of length K <= 1e3 carry at
    most ~K * 2^-24 relative error).
Every case is seeded; full-size cases use the sizes and launch configuration
the benchmark times.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import ffn_oracle as O
from transformer_ffn_block_amd import inputs as I
from helpers import dev, host_f64, host_bits, max_norm_err, elementwise_rel_err, rel_l2, record

pytestmark = pytest.mark.gpu

TOL_BF16 = 1e-2
TOL_Q8 = 2e-2
TOL_Q4 = 2e-2
TOL_F32_BLOCK = 1e-4
TOL_F32_NORM = 1e-5


def _say(*a):
    print(*a, flush=True)


def _block_dev(b: I.BlockInputs):
    dt = b.dtype
    return [dev(a, dt) for a in (b.x, b.g, b.w_gate, b.w_up, b.w_down)]


def _run_block(ffn, b: I.BlockInputs, variant: str):
    import torch
    x, g, wg, wu, wd = _block_dev(b)
    y = ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant=variant)
    torch.cuda.synchronize()
    return y


# ----------------------------------------------------------------------------
# RMSNorm
# ----------------------------------------------------------------------------
def test_rmsnorm_full_size_with_outlier_rows(gpu_lib):
    from transformer_ffn_block_amd import ffn
    import torch
    wl = I.WORKLOADS["rmsnorm"]
    _say("rmsnorm", wl)
    x, g, eps, out_rows = I.make_rmsnorm(wl["seed"], wl["rows"], wl["d"], "bf16")
    y = ffn.rmsnorm(dev(x), dev(g), eps)
    torch.cuda.synchronize()
    a = host_f64(y)
    r = O.rmsnorm_from_stored("bf16", x, g, eps)
    err = elementwise_rel_err(a, r)
    _say("outlier rows", len(out_rows))
    assert len(out_rows) == 164
    assert record("C2 rmsnorm 16384x4096 bf16", err, TOL_BF16, "elementwise_rel") <= TOL_BF16
    record("C2 rmsnorm 16384x4096 bf16", rel_l2(a, r), TOL_BF16, "rel_l2")
    # outlier rows (x100) are normalised like any other row
    assert elementwise_rel_err(a[out_rows], r[out_rows]) <= TOL_BF16


@pytest.mark.parametrize("rows,d", [(1, 8), (37, 264), (5, 4096), (3, 8200), (64, 520), (7, 16384)])
def test_rmsnorm_bf16_shapes(gpu_lib, rows, d):
    from transformer_ffn_block_amd import ffn
    import torch
    _say("rmsnorm bf16", rows, d)
    x, g, eps, _ = I.make_rmsnorm(100 + rows, rows, d, "bf16", outlier_frac=0.0)
    y = ffn.rmsnorm(dev(x), dev(g), eps)
    torch.cuda.synchronize()
    err = elementwise_rel_err(host_f64(y), O.rmsnorm_from_stored("bf16", x, g, eps))
    assert record(f"rmsnorm bf16 {rows}x{d}", err, TOL_BF16, "elementwise_rel") <= TOL_BF16


@pytest.mark.parametrize("rows,d", [(8, 256), (37, 260), (3, 4100), (2, 20000)])
def test_rmsnorm_f32_shapes(gpu_lib, rows, d):
    from transformer_ffn_block_amd import ffn
    import torch
    _say("rmsnorm f32", rows, d)
    x, g, eps, _ = I.make_rmsnorm(200 + rows, rows, d, "f32", outlier_frac=0.0)
    y = ffn.rmsnorm(dev(x, "f32"), dev(g, "f32"), eps)
    torch.cuda.synchronize()
    err = elementwise_rel_err(host_f64(y), O.rmsnorm_from_stored("f32", x, g, eps))
    assert record(f"rmsnorm f32 {rows}x{d}", err, TOL_F32_NORM, "elementwise_rel") <= TOL_F32_NORM


def test_rmsnorm_zero_row_and_scale(gpu_lib):
    from transformer_ffn_block_amd import ffn
    import torch
    x, g, eps, _ = I.make_rmsnorm(7, 4, 512, "f32", outlier_frac=0.0)
    x = x.copy()
    x[1] = 0.0
    x[2] = x[3] * np.float32(64.0)  # exact power-of-two scaling of row 3
    y = host_f64(ffn.rmsnorm(dev(x, "f32"), dev(g, "f32"), eps))
    torch.cuda.synchronize()
    assert np.array_equal(y[1], np.zeros(512))
    # with eps tiny relative to the mean square, rows 2 and 3 normalise alike
    assert np.max(np.abs(y[2] - y[3])) <= 1e-5 * np.max(np.abs(y[3]))


# ----------------------------------------------------------------------------
# the block: tiny fp32 workload
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("variant", ["fused", "split", "auto"])
def test_block_tiny_f32(gpu_lib, variant):
    from transformer_ffn_block_amd import ffn
    wl = I.WORKLOADS["tiny_f32"]
    _say("block tiny f32", wl, variant)
    b = I.make_block(wl["seed"], wl["M"], wl["d"], wl["f"], "f32")
    y = host_f64(_run_block(ffn, b, variant))
    r = O.block_from_stored("f32", b.x, b.g, b.w_gate, b.w_up, b.w_down, b.eps)
    err = max_norm_err(y, r)
    record(f"C1 tiny f32 {variant}", rel_l2(y, r), TOL_F32_BLOCK, "rel_l2")
    assert record(f"C1 tiny f32 {variant}", err, TOL_F32_BLOCK) <= TOL_F32_BLOCK


@pytest.mark.parametrize("M,d,f", [(1, 4, 4), (3, 36, 44), (70, 260, 300)])
def test_block_f32_ragged(gpu_lib, M, d, f):
    from transformer_ffn_block_amd import ffn
    _say("block f32 ragged", M, d, f)
    b = I.make_block(300 + M, M, d, f, "f32")
    r = O.block_from_stored("f32", b.x, b.g, b.w_gate, b.w_up, b.w_down, b.eps)
    for variant in ("fused", "split"):
        err = max_norm_err(host_f64(_run_block(ffn, b, variant)), r)
        assert record(f"f32 block {M}x{d}x{f} {variant}", err, TOL_F32_BLOCK) <= TOL_F32_BLOCK


# ----------------------------------------------------------------------------
# decode regime (weight streaming)
# ----------------------------------------------------------------------------
@pytest.fixture(scope="module")
def decode_inputs():
    wl = I.WORKLOADS["decode"]
    return I.make_block(wl["seed"], wl["M"], wl["d"], wl["f"], "bf16")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_block_decode_full_size(gpu_lib, decode_inputs, M):
    from transformer_ffn_block_amd import ffn
    import torch
    b16 = decode_inputs
    _say("block decode", M, b16.d, b16.f)
    x = b16.x[:M]  # first M rows of the 16-token draw, same weights
    xd, gd, wg, wu, wd = _block_dev(b16)
    xd = xd[:M].contiguous()
    y = ffn.swiglu_block(xd, gd, wg, wu, wd, b16.eps, variant="auto")
    torch.cuda.synchronize()
    a = host_f64(y)
    r = O.block_from_stored("bf16", x, b16.g, b16.w_gate, b16.w_up, b16.w_down, b16.eps)
    err = max_norm_err(a, r)
    record(f"C3 decode M={M}", rel_l2(a, r), TOL_BF16, "rel_l2")
    assert record(f"C3 decode M={M}", err, TOL_BF16) <= TOL_BF16


@pytest.mark.parametrize("M,d,f", [(2, 512, 704), (3, 520, 712), (5, 64, 8), (9, 520, 712),
                                   (12, 1032, 136), (17, 256, 384), (24, 520, 712), (33, 1032, 520),
                                   (40, 1032, 200), (63, 512, 1024), (64, 264, 136)])
def test_block_decode_ragged(gpu_lib, M, d, f):
    """Decode kernels (norm folded, h kept in the down projection's operand
    order) at token counts across the one- and two-tile kernels and chunked
    launches, with d and f off the 128-k stage (partial last stages)."""
    from transformer_ffn_block_amd import ffn
    _say("block decode ragged", M, d, f)
    b = I.make_block(400 + M, M, d, f, "bf16")
    r = O.block_from_stored("bf16", b.x, b.g, b.w_gate, b.w_up, b.w_down, b.eps)
    err = max_norm_err(host_f64(_run_block(ffn, b, "auto")), r)
    assert record(f"decode ragged {M}x{d}x{f}", err, TOL_BF16) <= TOL_BF16


@pytest.mark.parametrize("M,d,f", [(33, 520, 4104), (64, 1032, 4200), (36, 264, 10248),
                                   (57, 520, 10312), (48, 136, 16400)])
def test_block_decode_wide_gateup(gpu_lib, M, d, f):
    """33..64 tokens with enough 16-row tiles for one gate/up launch over
    every token tile: on a 256-CU device f = 4104 and 4200 take two-wave
    workgroups, f >= 10248 one wave per workgroup (the narrower f of the
    ragged cases take two 32-token launches).  d and f are off the 128-k
    stage."""
    from transformer_ffn_block_amd import ffn
    _say("block decode wide gate/up", M, d, f)
    b = I.make_block(500 + M, M, d, f, "bf16")
    r = O.block_from_stored("bf16", b.x, b.g, b.w_gate, b.w_up, b.w_down, b.eps)
    err = max_norm_err(host_f64(_run_block(ffn, b, "auto")), r)
    assert record(f"decode wide gate/up {M}x{d}x{f}", err, TOL_BF16) <= TOL_BF16


# ----------------------------------------------------------------------------
# bf16 SPLIT with few tokens: norm kernel, the prefill GEMMs on partial
# token tiles, the activation pass, then the decode down projection
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("M,d,f", [(1, 264, 136), (7, 520, 712), (16, 512, 704), (33, 1032, 520),
                                   (64, 264, 136)])
def test_block_split_few_tokens(gpu_lib, M, d, f):
    from transformer_ffn_block_amd import ffn
    _say("block split few tokens", M, d, f)
    b = I.make_block(3000 + M, M, d, f, "bf16")
    r = O.block_from_stored("bf16", b.x, b.g, b.w_gate, b.w_up, b.w_down, b.eps)
    err = max_norm_err(host_f64(_run_block(ffn, b, "split")), r)
    assert record(f"split few tokens {M}x{d}x{f}", err, TOL_BF16) <= TOL_BF16


def test_block_split_64_and_65_tokens_agree(gpu_lib):
    """At 64 tokens SPLIT ends with the decode down kernel, at 65 with the
    prefill down GEMM; the gate/up GEMMs and the activation pass are the
    same kernels on the same rows.  Shared rows agree to the bf16 tolerance
    (the two down kernels sum K in different orders), and both meet the
    oracle."""
    from transformer_ffn_block_amd import ffn
    import torch
    b = I.make_block(3100, 65, 520, 712, "bf16")
    x, g, wg, wu, wd = _block_dev(b)
    y64 = ffn.swiglu_block(x[:64].contiguous(), g, wg, wu, wd, b.eps, variant="split")
    y65 = ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant="split")
    torch.cuda.synchronize()
    r = O.block_from_stored("bf16", b.x, b.g, b.w_gate, b.w_up, b.w_down, b.eps)
    a64, a65 = host_f64(y64), host_f64(y65)
    assert record("split 64 tokens vs oracle", max_norm_err(a64, r[:64]), TOL_BF16) <= TOL_BF16
    assert record("split 65 tokens vs oracle", max_norm_err(a65, r), TOL_BF16) <= TOL_BF16
    assert max_norm_err(a64, a65[:64]) <= TOL_BF16


# ----------------------------------------------------------------------------
# single-dispatch (persistent) decode schedule
# ----------------------------------------------------------------------------
def _r256(n):
    return (n + 255) // 256 * 256


def _run_persistent(ffn, xd, gd, wg, wu, wd, eps):
    """The persistent schedule with an explicit workspace; returns y and the
    kernel's error word (nonzero if a work item gave up waiting), read at
    the offset the library names."""
    import torch
    M, d = xd.shape
    f = wg.shape[0]
    need = ffn.workspace_size(ffn.FFN_BF16, M, d, f, "persistent")
    ws = ffn.alloc_workspace(need)
    y = ffn.swiglu_block(xd, gd, wg, wu, wd, eps, variant="persistent", workspace=ws,
                         check_status=False)
    torch.cuda.synchronize()
    return y, ffn.persistent_status(ws, M, d, f)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_block_persistent_full_size(gpu_lib, decode_inputs, M):
    from transformer_ffn_block_amd import ffn
    b16 = decode_inputs
    _say("block persistent", M, b16.d, b16.f)
    xd, gd, wg, wu, wd = _block_dev(b16)
    y, err_word = _run_persistent(ffn, xd[:M].contiguous(), gd, wg, wu, wd, b16.eps)
    r = O.block_from_stored("bf16", b16.x[:M], b16.g, b16.w_gate, b16.w_up, b16.w_down, b16.eps)
    err = max_norm_err(host_f64(y), r)
    assert err_word == 0
    assert record(f"C3 decode M={M} persistent", err, TOL_BF16) <= TOL_BF16


# d, f not multiples of 16 (partial tiles) or of 128 (partial stages); f <= 384
# gives fewer than four K ranges
@pytest.mark.parametrize("M,d,f", [(1, 8, 8), (3, 520, 712), (11, 264, 136), (16, 1032, 384),
                                   (7, 64, 2056)])
def test_block_persistent_ragged(gpu_lib, M, d, f):
    from transformer_ffn_block_amd import ffn
    _say("block persistent ragged", M, d, f)
    b = I.make_block(1400 + M, M, d, f, "bf16")
    y, err_word = _run_persistent(ffn, *_block_dev(b), b.eps)
    r = O.block_from_stored("bf16", b.x, b.g, b.w_gate, b.w_up, b.w_down, b.eps)
    err = max_norm_err(host_f64(y), r)
    assert err_word == 0
    assert record(f"persistent ragged {M}x{d}x{f}", err, TOL_BF16) <= TOL_BF16


def test_block_persistent_deterministic_and_close_to_two_launch_path(gpu_lib):
    from transformer_ffn_block_amd import ffn
    import torch
    b = I.make_block(1500, 16, 1024, 2816, "bf16")
    dev = _block_dev(b)
    y1, e1 = _run_persistent(ffn, *dev, b.eps)
    y2, e2 = _run_persistent(ffn, *dev, b.eps)
    y_ref = ffn.swiglu_block(*dev, b.eps, variant="fused")
    torch.cuda.synchronize()
    assert e1 == 0 and e2 == 0
    assert np.array_equal(host_bits(y1), host_bits(y2))
    # different summation order of the down projection: equal within rounding
    assert max_norm_err(host_f64(y1), host_f64(y_ref)) <= TOL_BF16


# ----------------------------------------------------------------------------
# prefill regime (MFMA GEMMs), fused and split gate/up
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("M,d,f", [(65, 512, 704), (300, 520, 712), (513, 1024, 2048), (1000, 256, 136)])
@pytest.mark.parametrize("variant", ["fused", "split", "fused_norm"])
def test_block_prefill_ragged(gpu_lib, M, d, f, variant):
    from transformer_ffn_block_amd import ffn
    _say("block prefill ragged", M, d, f, variant)
    b = I.make_block(500 + M, M, d, f, "bf16")
    r = O.block_from_stored("bf16", b.x, b.g, b.w_gate, b.w_up, b.w_down, b.eps)
    err = max_norm_err(host_f64(_run_block(ffn, b, variant)), r)
    assert record(f"prefill ragged {M}x{d}x{f} {variant}", err, TOL_BF16) <= TOL_BF16


@pytest.mark.parametrize("M,d,f", [(256, 256, 128), (512, 512, 768), (768, 1024, 1280)])
@pytest.mark.parametrize("variant", ["fused", "split", "fused_norm"])
def test_block_prefill_whole_tiles(gpu_lib, M, d, f, variant):
    """Shapes made of whole 256-token tiles with an even number of 64-deep K
    tiles, the ones the two-group (ping-pong) GEMM schedule takes; K = 128
    is its shortest loop."""
    from transformer_ffn_block_amd import ffn
    _say("block prefill whole tiles", M, d, f, variant)
    b = I.make_block(700 + M, M, d, f, "bf16")
    r = O.block_from_stored("bf16", b.x, b.g, b.w_gate, b.w_up, b.w_down, b.eps)
    err = max_norm_err(host_f64(_run_block(ffn, b, variant)), r)
    assert record(f"prefill whole tiles {M}x{d}x{f} {variant}", err, TOL_BF16) <= TOL_BF16


@pytest.mark.parametrize("M,d,f", [(512, 256, 16640), (4352, 4096, 128)])
def test_block_prefill_persistent_tile_walk(gpu_lib, M, d, f):
    """More whole tiles than resident workgroups: the ping-pong GEMM walks
    them persistently (one workgroup per slot, tiles b, b + grid, ...), so
    some workgroups take one tile more than others.  (512, 256, 16640): 260
    fused gate/up tiles; (4352, 4096, 128): 272 down tiles with the
    shortest K loop.  Every output against the oracle."""
    from transformer_ffn_block_amd import ffn
    _say("block prefill persistent walk", M, d, f)
    b = I.make_block(900 + M, M, d, f, "bf16")
    r = O.block_from_stored("bf16", b.x, b.g, b.w_gate, b.w_up, b.w_down, b.eps)
    a = host_f64(_run_block(ffn, b, "fused"))
    assert record(f"prefill persistent walk {M}x{d}x{f}", max_norm_err(a, r), TOL_BF16) <= TOL_BF16
    per_row = max(max_norm_err(a[i], r[i]) for i in range(M))
    assert record(f"prefill persistent walk {M}x{d}x{f} worst row", per_row, TOL_BF16,
                  "max_norm_per_row") <= TOL_BF16


@pytest.fixture(scope="module")
def prefill_inputs():
    wl = I.WORKLOADS["prefill"]
    return I.make_block(wl["seed"], wl["M"], wl["d"], wl["f"], "bf16")


def test_block_prefill_full_size_sampled_rows(gpu_lib, prefill_inputs):
    """M=8192, d=4096, f=14336: both variants vs the oracle on 256 seeded rows
    (rows 0 and 8191, both sides of a token-tile boundary, and random rows;
    rows are independent, so the oracle computes just these), and fused vs
    split on every row."""
    from transformer_ffn_block_amd import ffn
    import torch
    b = prefill_inputs
    _say("block prefill full", b.M, b.d, b.f)
    x, g, wg, wu, wd = _block_dev(b)
    y_f = ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant="fused")
    y_s = ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant="split")
    y_n = ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant="fused_norm")
    torch.cuda.synchronize()
    fixed = np.array([0, 1, 255, 256, 4095, 4096, b.M - 256, b.M - 1])
    rest = np.setdiff1d(np.arange(b.M), fixed)
    rows = np.sort(np.concatenate([fixed, np.random.default_rng(44).choice(rest, 256 - fixed.size,
                                                                           replace=False)]))
    assert rows.size == 256 and rows[0] == 0 and rows[-1] == b.M - 1
    r = O.block_from_stored("bf16", b.x[rows], b.g, b.w_gate, b.w_up, b.w_down, b.eps)
    af = host_f64(y_f)
    as_ = host_f64(y_s)
    ef, es = max_norm_err(af[rows], r), max_norm_err(as_[rows], r)
    record("C4 prefill fused (256 rows)", rel_l2(af[rows], r), TOL_BF16, "rel_l2")
    record("C4 prefill split (256 rows)", rel_l2(as_[rows], r), TOL_BF16, "rel_l2")
    assert record("C4 prefill fused (256 rows)", ef, TOL_BF16) <= TOL_BF16
    assert record("C4 prefill split (256 rows)", es, TOL_BF16) <= TOL_BF16
    an = host_f64(y_n)
    assert record("C4 prefill fused_norm (256 rows)", max_norm_err(an[rows], r), TOL_BF16) <= TOL_BF16
    # per row too: no row's error hides under another row's larger outputs
    per_row = max(max_norm_err(a[rows][i], r[i]) for a in (af, as_) for i in range(rows.size))
    assert record("C4 prefill worst row (row-normalised)", per_row, TOL_BF16, "max_norm_per_row") <= TOL_BF16
    assert max_norm_err(af, as_) <= TOL_BF16


# ----------------------------------------------------------------------------
# prefill GEMMs split over K (fewer tiles than compute units): fp32 partials
# plus a second pass (SwiGLU for the fused gate/up GEMM, residual for the
# down GEMM).  On a 256-CU device: (256, 1024, 2048) takes the two-group
# schedule with 8 / 16 ranges; (65, 512, 704) and (300, 4096, 1024) the
# one-group schedule (ragged token tiles; f = 704 also a ragged weight tile,
# and 11 K tiles, an odd count, for the down GEMM) with 4 / 11 and 16 / 8
# ranges; d = 1032 is off the K tile, so its gate/up GEMM stays unsplit
# (register-staged) while its down GEMM (K = 576) splits 9 ways.
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("variant", ["fused", "split", "fused_norm"])
@pytest.mark.parametrize("M,d,f", [(256, 1024, 2048), (65, 512, 704), (300, 4096, 1024),
                                   (100, 1032, 576)])
def test_block_prefill_split_k(gpu_lib, M, d, f, variant):
    from transformer_ffn_block_amd import ffn
    _say("block prefill split-K", M, d, f, variant)
    b = I.make_block(5600 + M, M, d, f, "bf16")
    r = O.block_from_stored("bf16", b.x, b.g, b.w_gate, b.w_up, b.w_down, b.eps)
    a = host_f64(_run_block(ffn, b, variant))
    assert record(f"prefill split-K {M}x{d}x{f} {variant}", max_norm_err(a, r), TOL_BF16) <= TOL_BF16
    per_row = max(max_norm_err(a[i], r[i]) for i in range(M))
    assert record(f"prefill split-K {M}x{d}x{f} {variant} worst row", per_row, TOL_BF16,
                  "max_norm_per_row") <= TOL_BF16


def test_block_prefill_split_k_decode_shape_sampled_rows(gpu_lib):
    """128 tokens at the decode shape d = 4096, f = 11008 (86 gate/up and 16
    down tiles: 2 and 16 K ranges on 256 CUs) against the oracle on 24 rows
    (rows are independent, so the oracle computes just these), and the same
    bits on a second call."""
    from transformer_ffn_block_amd import ffn
    import torch
    M, d, f = 128, 4096, 11008
    _say("block prefill split-K decode shape", M, d, f)
    b = I.make_block(5700, M, d, f, "bf16")
    x, g, wg, wu, wd = _block_dev(b)
    y1 = ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant="auto")
    y2 = ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant="auto")
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y1), host_bits(y2))
    rows = np.sort(np.concatenate([[0, 1, 63, 64, 126, 127],
                                   np.random.default_rng(45).choice(np.arange(2, 126), 18, replace=False)]))
    r = O.block_from_stored("bf16", b.x[rows], b.g, b.w_gate, b.w_up, b.w_down, b.eps)
    a = host_f64(y1)[rows]
    assert record("prefill split-K 128x4096x11008 (24 rows)", max_norm_err(a, r), TOL_BF16) <= TOL_BF16


# Tile counts just past a whole round: the columns filling the earlier rounds
# run unsplit (row stride of the full output) and the last columns split over
# K.  On a 256-CU device, one 256 x 256 tile resident per CU: (2304, 512,
# 3712) has 9 x 29 = 261 gate/up tiles -> 28 column tiles unsplit, the last
# one's 9 tiles over 4 K ranges (its down GEMM splits whole, 14 ways);
# (4352, 4096, 256) has 17 x 16 = 272 down tiles -> 15 columns unsplit, the
# last one's 17 over 2 ranges (K = 256).  The workspace size shows the plan.
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("M,d,f,part_bytes", [(2304, 512, 3712, max(2 * 4 * 2304 * 128 * 4, 14 * 2304 * 512 * 4)),
                                              (4352, 4096, 256, max(2 * 7 * 4352 * 256 * 4, 2 * 4352 * 256 * 4))])
def test_block_prefill_split_tail(gpu_lib, M, d, f, part_bytes):
    from transformer_ffn_block_amd import ffn
    import torch
    _say("block prefill split tail", M, d, f)
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("plan sizes stated for 256 compute units")
    r256 = lambda n: (n + 255) // 256 * 256
    assert ffn.workspace_size(ffn.FFN_BF16, M, d, f) == r256(M * d * 2) + r256(M * f * 2) + r256(part_bytes)
    b = I.make_block(5800 + M, M, d, f, "bf16")
    r = O.block_from_stored("bf16", b.x, b.g, b.w_gate, b.w_up, b.w_down, b.eps)
    a = host_f64(_run_block(ffn, b, "fused"))
    assert record(f"prefill split tail {M}x{d}x{f}", max_norm_err(a, r), TOL_BF16) <= TOL_BF16
    per_row = max(max_norm_err(a[i], r[i]) for i in range(M))
    assert record(f"prefill split tail {M}x{d}x{f} worst row", per_row, TOL_BF16,
                  "max_norm_per_row") <= TOL_BF16


def test_block_prefill_split_tail_mid_batch_sampled_rows(gpu_lib):
    """768 tokens at d = 4096, f = 11008 (258 gate/up tiles: 85 column tiles
    unsplit, the last 3 tiles over 16 K ranges; 48 down tiles split whole)
    against the oracle on 24 rows, spanning the unsplit and the split columns
    of every row, and the same bits on a second call."""
    from transformer_ffn_block_amd import ffn
    import torch
    M, d, f = 768, 4096, 11008
    _say("block prefill split tail mid batch", M, d, f)
    b = I.make_block(5900, M, d, f, "bf16")
    x, g, wg, wu, wd = _block_dev(b)
    y1 = ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant="auto")
    y2 = ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant="auto")
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y1), host_bits(y2))
    rows = np.sort(np.concatenate([[0, 255, 256, 511, 512, 767],
                                   np.random.default_rng(46).choice(np.arange(1, 767), 18, replace=False)]))
    rows = np.unique(rows)
    r = O.block_from_stored("bf16", b.x[rows], b.g, b.w_gate, b.w_up, b.w_down, b.eps)
    a = host_f64(y1)[rows]
    assert record("prefill split tail 768x4096x11008 (24 rows)", max_norm_err(a, r), TOL_BF16) <= TOL_BF16


# Up to 128 tokens the prefill GEMMs take 128-token tiles.  On a 256-CU
# device: (128, 1024, 32768) has 256 fused gate/up tiles (one round,
# unsplit) and a down GEMM of 4 tiles over 16 K ranges; (128, 512, 76800)
# has 600 gate/up tiles -> 512 walked persistently and the last 88 over 2 K
# ranges; (96, 512, 704) ragged tokens on the one-group schedule.
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("M,d,f", [(128, 1024, 32768), (128, 512, 76800), (96, 512, 704)])
def test_block_prefill_128_token_tiles(gpu_lib, M, d, f):
    from transformer_ffn_block_amd import ffn
    _say("block prefill 128-token tiles", M, d, f)
    b = I.make_block(6000 + M + f, M, d, f, "bf16")
    r = O.block_from_stored("bf16", b.x, b.g, b.w_gate, b.w_up, b.w_down, b.eps)
    for variant in ("fused", "split"):
        a = host_f64(_run_block(ffn, b, variant))
        assert record(f"prefill 128-token tiles {M}x{d}x{f} {variant}", max_norm_err(a, r), TOL_BF16) <= TOL_BF16
        per_row = max(max_norm_err(a[i], r[i]) for i in range(M))
        assert record(f"prefill 128-token tiles {M}x{d}x{f} {variant} worst row", per_row, TOL_BF16,
                      "max_norm_per_row") <= TOL_BF16


# ----------------------------------------------------------------------------
# properties
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("M", [16, 300])
def test_block_deterministic_and_row_permutation(gpu_lib, M):
    from transformer_ffn_block_amd import ffn
    import torch
    _say("determinism/permutation", M)
    b = I.make_block(600 + M, M, 512, 704, "bf16")
    x, g, wg, wu, wd = _block_dev(b)
    y1 = host_bits(ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant="fused"))
    y2 = host_bits(ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant="fused"))
    p = np.random.default_rng(0).permutation(M)
    yp = host_bits(ffn.swiglu_block(x[torch.from_numpy(p).cuda()].contiguous(), g, wg, wu, wd, b.eps,
                                    variant="fused"))
    torch.cuda.synchronize()
    assert np.array_equal(y1, y2)
    assert np.array_equal(yp, y1[p])


def test_calls_on_a_side_stream_match_the_default_stream(gpu_lib):
    """Every entry point enqueues on the stream it is given: results computed
    on a side stream (inputs made on that stream, no device-wide sync before
    the call) equal the default-stream ones bit for bit."""
    from transformer_ffn_block_amd import ffn
    import torch
    b = I.make_block(1600, 12, 512, 704, "bf16")
    q = I.make_q8_block(1601, 5, 256, 512)
    q4 = I.make_q4_block(1602, 5, 256, 512)
    bp = I.make_block(1603, 130, 256, 384, "bf16")

    def run_all(stream):
        out = []
        x, g, wg, wu, wd = [t.clone() for t in _block_dev(b)]
        out.append(ffn.swiglu_block(x, g, wg, wu, wd, b.eps, stream=stream))
        out.append(ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant="persistent", stream=stream))
        xp, gp, pg, pu, pd = [t.clone() for t in _block_dev(bp)]
        out.append(ffn.swiglu_block(xp, gp, pg, pu, pd, bp.eps, stream=stream))
        out.append(ffn.swiglu_block_q8(dev(q.x), dev(q.g), _q8_dev(q.w_gate), _q8_dev(q.w_up),
                                       _q8_dev(q.w_down), q.eps, stream=stream))
        out.append(ffn.swiglu_block_q4(dev(q4.x), dev(q4.g), _q4_dev(q4.w_gate), _q4_dev(q4.w_up),
                                       _q4_dev(q4.w_down), q4.eps, stream=stream))
        n = torch.empty_like(x)
        ffn.rmsnorm(x, g, b.eps, out=n, stream=stream)
        out.append(n)
        return out

    ref = [host_bits(t) for t in run_all(None)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        got = run_all(side)
    side.synchronize()
    for a, r in zip(got, ref):
        assert np.array_equal(host_bits(a), r)


@pytest.mark.parametrize("M", [4, 200])
def test_block_zero_down_projection_returns_x_bitwise(gpu_lib, M):
    from transformer_ffn_block_amd import ffn
    import torch
    b = I.make_block(700 + M, M, 256, 512, "bf16")
    x, g, wg, wu, _ = _block_dev(b)
    wd = torch.zeros((256, 512), dtype=torch.bfloat16, device="cuda")
    for variant in ("fused", "split"):
        y = ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant=variant)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(y), b.x)


# ----------------------------------------------------------------------------
# M-tail consistency: the first a rows of an M=b call, run as an M=a call
# ----------------------------------------------------------------------------
def _tail_pair(kind, a, b, d, f):
    """(y of rows 0..a-1 from an M=a call, the same rows from an M=b call), bf16 bits."""
    from transformer_ffn_block_amd import ffn
    import torch
    if kind == "bf16":
        blk = I.make_block(2000 + a + b, b, d, f, "bf16")
        x, g, wg, wu, wd = _block_dev(blk)
        ya = ffn.swiglu_block(x[:a].contiguous(), g, wg, wu, wd, blk.eps, variant="auto")
        yb = ffn.swiglu_block(x, g, wg, wu, wd, blk.eps, variant="auto")
    elif kind == "q8":
        q = I.make_q8_block(2100 + a + b, b, d, f)
        mats = [_q8_dev(m) for m in (q.w_gate, q.w_up, q.w_down)]
        x = dev(q.x)
        ya = ffn.swiglu_block_q8(x[:a].contiguous(), dev(q.g), *mats, q.eps)
        yb = ffn.swiglu_block_q8(x, dev(q.g), *mats, q.eps)
    else:
        q = I.make_q4_block(2200 + a + b, b, d, f)
        mats = [_q4_dev(m) for m in (q.w_gate, q.w_up, q.w_down)]
        x = dev(q.x)
        ya = ffn.swiglu_block_q4(x[:a].contiguous(), dev(q.g), *mats, q.eps)
        yb = ffn.swiglu_block_q4(x, dev(q.g), *mats, q.eps)
    torch.cuda.synchronize()
    return host_bits(ya), host_bits(yb)[:a]


# Rows are independent and each kernel's summation order depends on M only
# through the kernel choice and, for prefill GEMMs split over K, the number of
# token tiles (which sets the K ranges), so rows shared by two calls that take
# the same kernels are bitwise equal: decode 17 vs 32 tokens (the two-tile
# kernels), prefill 300 vs 512 tokens (two token tiles each: ragged tiles in
# the one-group schedule vs whole tiles in the two-group one, both split over
# K at the same places), Q8/Q4 5 vs 8 and 17 vs 32 tokens.
@pytest.mark.parametrize("kind,a,b,d,f", [("bf16", 17, 32, 1024, 2816), ("bf16", 300, 512, 512, 768),
                                          ("q8", 5, 8, 512, 1024), ("q8", 17, 32, 512, 704),
                                          ("q4", 5, 8, 512, 1024), ("q4", 17, 32, 512, 704)])
def test_m_tail_rows_bitwise_equal(gpu_lib, kind, a, b, d, f):
    _say("m-tail", kind, a, b, d, f)
    ya, yb = _tail_pair(kind, a, b, d, f)
    assert np.array_equal(ya, yb)


# ----------------------------------------------------------------------------
# one GPU's share of the tensor-parallel block (f/8), at its real shapes
# ----------------------------------------------------------------------------
def test_tp8_shard_decode(gpu_lib):
    from transformer_ffn_block_amd import ffn
    wl = I.WORKLOADS["decode_tp8_shard"]
    _say("tp8 shard decode", wl)
    blk = I.make_block(wl["seed"], wl["M"], wl["d"], wl["f"], "bf16")
    r = O.block_from_stored("bf16", blk.x, blk.g, blk.w_gate, blk.w_up, blk.w_down, blk.eps)
    err = max_norm_err(host_f64(_run_block(ffn, blk, "auto")), r)
    assert record("tp8 shard decode", err, TOL_BF16) <= TOL_BF16


def test_tp8_shard_prefill_sampled_rows(gpu_lib):
    from transformer_ffn_block_amd import ffn
    wl = I.WORKLOADS["prefill_tp8_shard"]
    _say("tp8 shard prefill", wl)
    blk = I.make_block(wl["seed"], wl["M"], wl["d"], wl["f"], "bf16")
    rows = np.unique(np.concatenate([[0, 255, 256, blk.M - 1],
                                     np.random.default_rng(45).choice(blk.M, 28, replace=False)]))
    r = O.block_from_stored("bf16", blk.x[rows], blk.g, blk.w_gate, blk.w_up, blk.w_down, blk.eps)
    for variant in ("fused", "split"):
        err = max_norm_err(host_f64(_run_block(ffn, blk, variant))[rows], r)
        assert record(f"tp8 shard prefill {variant}", err, TOL_BF16) <= TOL_BF16


@pytest.mark.parametrize("kind", ["q8", "q4"])
def test_tp8_shard_quantised(gpu_lib, kind):
    from transformer_ffn_block_amd import ffn
    wl = I.WORKLOADS[f"{kind}_tp8_shard"]
    _say("tp8 shard", kind, wl)
    if kind == "q8":
        q = I.make_q8_block(wl["seed"], wl["M"], wl["d"], wl["f"])
        err = max_norm_err(_run_q8(ffn, q), _q8_ref(q))
        tol = TOL_Q8
    else:
        q = I.make_q4_block(wl["seed"], wl["M"], wl["d"], wl["f"])
        err = max_norm_err(_run_q4(ffn, q), _q4_ref(q))
        tol = TOL_Q4
    assert record(f"tp8 shard {kind}", err, tol) <= tol


# ----------------------------------------------------------------------------
# Q8_0
# ----------------------------------------------------------------------------
def _q8_dev(m: I.Q8Matrix):
    return dev(m.qs, "i8"), dev(m.scales, "u16")


def _q8_ref(q: I.Q8BlockInputs, x=None):
    return O.swiglu_block_q8(q.x if x is None else x, q.g, (q.w_gate.qs, q.w_gate.scales),
                             (q.w_up.qs, q.w_up.scales), (q.w_down.qs, q.w_down.scales), q.eps)


def _run_q8(ffn, q: I.Q8BlockInputs):
    import torch
    y = ffn.swiglu_block_q8(dev(q.x), dev(q.g), _q8_dev(q.w_gate), _q8_dev(q.w_up), _q8_dev(q.w_down), q.eps)
    torch.cuda.synchronize()
    return host_f64(y)


def test_q8_full_size(gpu_lib):
    from transformer_ffn_block_amd import ffn
    wl = I.WORKLOADS["q8_decode"]
    _say("q8 full", wl)
    q = I.make_q8_block(wl["seed"], wl["M"], wl["d"], wl["f"])
    sub = np.count_nonzero((q.w_gate.scales & 0x7C00) == 0)
    a = _run_q8(ffn, q)
    r = _q8_ref(q)
    err = max_norm_err(a, r)
    _say("subnormal-or-zero gate scales", sub)
    assert sub > 0
    record("C5 q8 decode M=8", rel_l2(a, r), TOL_Q8, "rel_l2")
    assert record("C5 q8 decode M=8", err, TOL_Q8) <= TOL_Q8


# d, f not multiples of 256 leave a partial last stage in the 8-token (1, 3,
# 5), 16-token (12) and 32-row staged (17, 24, 32, 33, 48) kernels and in the
# split-K down pass; d = 544 and 800 also take the scale loads of unaligned
# rows in the 32-row gate/up kernel
@pytest.mark.parametrize("M,d,f", [(1, 64, 32), (3, 160, 96), (12, 288, 352), (17, 512, 704),
                                   (33, 256, 800), (64, 256, 256), (5, 128, 4224), (24, 544, 416),
                                   (32, 1024, 2048), (48, 800, 288)])
def test_q8_ragged_tokens(gpu_lib, M, d, f):
    from transformer_ffn_block_amd import ffn
    _say("q8 ragged", M, d, f)
    q = I.make_q8_block(800 + M, M, d, f)
    err = max_norm_err(_run_q8(ffn, q), _q8_ref(q))
    assert record(f"q8 ragged {M}x{d}x{f}", err, TOL_Q8) <= TOL_Q8


# d = 4096: the down projection's 256 row tiles fill a round of 256 CUs, so
# up to 16 tokens it runs unsplit in four-wave workgroups (no partials);
# f = 800 leaves a partial last stage, 11008 is the decode shape
@pytest.mark.parametrize("M,f", [(1, 800), (8, 11008), (13, 800), (16, 11008), (17, 800)])
def test_q8_whole_round_down(gpu_lib, M, f):
    from transformer_ffn_block_amd import ffn
    d = 4096
    _say("q8 whole-round down", M, d, f)
    q = I.make_q8_block(900 + M, M, d, f)
    err = max_norm_err(_run_q8(ffn, q), _q8_ref(q))
    assert record(f"q8 whole-round down {M}x{d}x{f}", err, TOL_Q8) <= TOL_Q8


@pytest.mark.parametrize("M", [8, 12, 33])
def test_q8_quant_minus_128(gpu_lib, M):
    """The int8 range's extra value -128 (never drawn by the generator, but a
    valid quant): about 1 in 8 quants of every matrix set to -128, plus one
    whole block per row, through the folded (8 tokens), staged (12) and
    chunked (33) kernels."""
    from transformer_ffn_block_amd import ffn
    _say("q8 -128", M)
    q = I.make_q8_block(2700 + M, M, 512, 1024)
    rng = np.random.default_rng(2800 + M)
    for m in (q.w_gate, q.w_up, q.w_down):
        m.qs[rng.random(m.qs.shape) < 0.125] = -128
        blk = rng.integers(0, m.qs.shape[1] // 32, size=m.qs.shape[0])
        for row, b0 in enumerate(blk):
            m.qs[row, 32 * b0:32 * b0 + 32] = -128
    assert np.count_nonzero(q.w_down.qs == -128) > q.w_down.qs.size // 10
    err = max_norm_err(_run_q8(ffn, q), _q8_ref(q))
    assert record(f"q8 quants -128 M={M}", err, TOL_Q8) <= TOL_Q8


def test_q8_folded_and_materialised_norm_agree(gpu_lib):
    """Up to 8 tokens the norm is folded into the gate/up kernel; from 9 on n
    is materialised first: the rows shared by an 8- and a 9-token call agree
    to the tolerance (different roundings of the normalised activations)."""
    from transformer_ffn_block_amd import ffn
    import torch
    q = I.make_q8_block(2400, 9, 512, 1024)
    mats = [_q8_dev(m) for m in (q.w_gate, q.w_up, q.w_down)]
    x = dev(q.x)
    y8 = ffn.swiglu_block_q8(x[:8].contiguous(), dev(q.g), *mats, q.eps)
    y9 = ffn.swiglu_block_q8(x, dev(q.g), *mats, q.eps)
    torch.cuda.synchronize()
    r = _q8_ref(q)
    a8, a9 = host_f64(y8), host_f64(y9)
    assert record("q8 folded norm (8 tokens)", max_norm_err(a8, r[:8]), TOL_Q8) <= TOL_Q8
    assert record("q8 materialised norm (9 tokens)", max_norm_err(a9, r), TOL_Q8) <= TOL_Q8
    assert max_norm_err(a8, a9[:8]) <= TOL_Q8


def test_q8_subnormal_scales_are_not_flushed(gpu_lib):
    """Every scale subnormal (bits 0x0100..0x03FF).  x is scaled by 2^-20 and
    eps = 0, so n is unchanged while the residual no longer hides the tiny
    delta; a flush-to-zero dequantisation would return y == x."""
    from transformer_ffn_block_amd import ffn
    q = I.make_q8_block(900, 4, 128, 96)
    rng = np.random.default_rng(901)
    for m in (q.w_gate, q.w_up, q.w_down):
        m.scales[:] = rng.integers(0x0100, 0x0400, size=m.scales.shape, dtype=np.uint16)
    q.x = I.f32_to_bf16_bits(I.bf16_bits_to_f32(q.x) * np.float32(2.0 ** -20))
    q.eps = 0.0
    a = _run_q8(ffn, q)
    r = _q8_ref(q)
    assert max_norm_err(O.bf16_to_f64(q.x), r) > 0.5   # flushed scales would fail by far
    assert record("q8 all-subnormal scales", max_norm_err(a, r), TOL_Q8) <= TOL_Q8


# ----------------------------------------------------------------------------
# Q4_0
# ----------------------------------------------------------------------------
def _q4_dev(m: I.Q4Matrix):
    return dev(m.qs, "u8"), dev(m.scales, "u16")


def _q4_ref(q: I.Q4BlockInputs):
    return O.swiglu_block_q4(q.x, q.g, (q.w_gate.qs, q.w_gate.scales),
                             (q.w_up.qs, q.w_up.scales), (q.w_down.qs, q.w_down.scales), q.eps)


def _run_q4(ffn, q: I.Q4BlockInputs, bits=False):
    import torch
    y = ffn.swiglu_block_q4(dev(q.x), dev(q.g), _q4_dev(q.w_gate), _q4_dev(q.w_up), _q4_dev(q.w_down), q.eps)
    torch.cuda.synchronize()
    return host_bits(y) if bits else host_f64(y)


def test_q4_full_size(gpu_lib):
    from transformer_ffn_block_amd import ffn
    wl = I.WORKLOADS["q4_decode"]
    _say("q4 full", wl)
    q = I.make_q4_block(wl["seed"], wl["M"], wl["d"], wl["f"])
    sub = np.count_nonzero((q.w_gate.scales & 0x7C00) == 0)
    a = _run_q4(ffn, q)
    r = _q4_ref(q)
    err = max_norm_err(a, r)
    _say("subnormal-or-zero gate scales", sub)
    assert sub > 0
    record("q4 decode M=8", rel_l2(a, r), TOL_Q4, "rel_l2")
    assert record("q4 decode M=8", err, TOL_Q4) <= TOL_Q4


# M: 1..8 and 9..16 take the staged-activation kernels, 17..32 the 32-row
# staged two-tile kernel, > 32 several launches; d, f not multiples of 256
# leave a partial last stage and use the per-block scale loads; the down
# projections split K over 1..8 ranges (8 for d = 128, f = 4224)
@pytest.mark.parametrize("M,d,f", [(1, 64, 32), (3, 160, 96), (12, 288, 352), (17, 512, 704),
                                   (33, 256, 800), (64, 256, 256), (5, 128, 4224), (24, 544, 416),
                                   (32, 1024, 2048), (48, 800, 288)])
def test_q4_ragged_tokens(gpu_lib, M, d, f):
    from transformer_ffn_block_amd import ffn
    _say("q4 ragged", M, d, f)
    q = I.make_q4_block(1800 + M, M, d, f)
    err = max_norm_err(_run_q4(ffn, q), _q4_ref(q))
    assert record(f"q4 ragged {M}x{d}x{f}", err, TOL_Q4) <= TOL_Q4


# as for Q8_0: d = 4096 runs the down projection unsplit up to 16 tokens
@pytest.mark.parametrize("M,f", [(1, 800), (8, 11008), (13, 800), (16, 11008), (17, 800)])
def test_q4_whole_round_down(gpu_lib, M, f):
    from transformer_ffn_block_amd import ffn
    d = 4096
    _say("q4 whole-round down", M, d, f)
    q = I.make_q4_block(1900 + M, M, d, f)
    err = max_norm_err(_run_q4(ffn, q), _q4_ref(q))
    assert record(f"q4 whole-round down {M}x{d}x{f}", err, TOL_Q4) <= TOL_Q4


def test_q4_folded_and_materialised_norm_agree(gpu_lib):
    """As for Q8_0: an 8-token call folds the norm, a 9-token call
    materialises n; shared rows agree to the tolerance."""
    from transformer_ffn_block_amd import ffn
    import torch
    q = I.make_q4_block(2500, 9, 512, 1024)
    mats = [_q4_dev(m) for m in (q.w_gate, q.w_up, q.w_down)]
    x = dev(q.x)
    y8 = ffn.swiglu_block_q4(x[:8].contiguous(), dev(q.g), *mats, q.eps)
    y9 = ffn.swiglu_block_q4(x, dev(q.g), *mats, q.eps)
    torch.cuda.synchronize()
    r = _q4_ref(q)
    a8, a9 = host_f64(y8), host_f64(y9)
    assert record("q4 folded norm (8 tokens)", max_norm_err(a8, r[:8]), TOL_Q4) <= TOL_Q4
    assert record("q4 materialised norm (9 tokens)", max_norm_err(a9, r), TOL_Q4) <= TOL_Q4
    assert max_norm_err(a8, a9[:8]) <= TOL_Q4


def test_q4_subnormal_scales_are_not_flushed(gpu_lib):
    """Every scale subnormal and eps = 0, as for Q8_0; the weights are ~16x
    smaller than Q8_0's, so x is scaled by 2^-32 (still a normal bf16) for the
    delta to dominate y: a flush-to-zero dequantisation would return y == x."""
    from transformer_ffn_block_amd import ffn
    q = I.make_q4_block(1900, 4, 128, 128)
    rng = np.random.default_rng(1901)
    for m in (q.w_gate, q.w_up, q.w_down):
        m.scales[:] = rng.integers(0x0100, 0x0400, size=m.scales.shape, dtype=np.uint16)
    q.x = I.f32_to_bf16_bits(I.bf16_bits_to_f32(q.x) * np.float32(2.0 ** -32))
    q.eps = 0.0
    a = _run_q4(ffn, q)
    r = _q4_ref(q)
    assert max_norm_err(O.bf16_to_f64(q.x), r) > 0.5
    assert record("q4 all-subnormal scales", max_norm_err(a, r), TOL_Q4) <= TOL_Q4


@pytest.mark.parametrize("M", [5, 40])
def test_q4_zero_point_nibbles_return_x_bitwise(gpu_lib, M):
    """Every down-projection nibble 8 (weight 0 under any scale): y = x + 0
    exactly, whatever the gate/up path computes."""
    from transformer_ffn_block_amd import ffn
    q = I.make_q4_block(1950 + M, M, 384, 384)
    q.w_down.qs[:] = 0x88
    assert np.array_equal(_run_q4(ffn, q, bits=True), q.x)


@pytest.mark.parametrize("kind", ["q8", "q4"])
def test_prepared_quant_call_matches_wrapper(gpu_lib, kind):
    """A call marshalled once (timing loops) gives the wrapper's output bitwise."""
    from transformer_ffn_block_amd import ffn
    import torch
    _say("prepared", kind)
    make = I.make_q8_block if kind == "q8" else I.make_q4_block
    todev = _q8_dev if kind == "q8" else _q4_dev
    q = make(2600, 8, 512, 1024)
    mats = [todev(m) for m in (q.w_gate, q.w_up, q.w_down)]
    x, g = dev(q.x), dev(q.g)
    ref = (ffn.swiglu_block_q8 if kind == "q8" else ffn.swiglu_block_q4)(x, g, *mats, q.eps)
    ws = ffn.alloc_workspace(getattr(ffn.lib(), f"ffn_swiglu_block_{kind}_workspace_size")(8, 512, 1024))
    y = torch.empty_like(x)
    call = ffn.prepare_swiglu_block_quant(kind, x, g, *mats, q.eps, y, ws)
    call()
    call()
    torch.cuda.synchronize()
    assert torch.equal(y, ref)


# ----------------------------------------------------------------------------
# balanced row ranges: gate/up grids that fill one round of resident
# workgroups give each workgroup an equal share (< 16) of the rows, so row
# ranges start at arbitrary rows and the epilogues store element by element
# at unaligned edges.  On MI355X (256 CUs) these shapes take that path: the
# bf16 16-token kernel holds 3 workgroups per CU (768 slots; f = 8192 is 512
# tiles), the Q8_0 / Q4_0 8-token kernels 2 (512 slots; f = 6144 is 384).
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("M,d,f", [(16, 512, 8192), (12, 264, 8200), (3, 520, 12296)])
def test_block_decode_balanced_row_ranges(gpu_lib, M, d, f):
    from transformer_ffn_block_amd import ffn
    _say("decode balanced", M, d, f)
    b = I.make_block(3200 + M, M, d, f, "bf16")
    r = O.block_from_stored("bf16", b.x, b.g, b.w_gate, b.w_up, b.w_down, b.eps)
    err = max_norm_err(host_f64(_run_block(ffn, b, "auto")), r)
    assert record(f"decode balanced rows {M}x{d}x{f}", err, TOL_BF16) <= TOL_BF16


@pytest.mark.parametrize("M,d,f", [(16, 5120, 1032), (1, 5128, 520), (8, 4104, 264),
                                   (24, 3080, 136), (40, 3080, 200)])
def test_block_decode_balanced_down_rows(gpu_lib, M, d, f):
    """Balanced row ranges in the down projection: on a 256-CU device the
    1..16-token down kernel holds two workgroups per CU (512 slots), so d =
    5120 / 5128 / 4104 (320 / 321 / 257 row tiles) spread as 8-10 rows per
    workgroup; the 17..64-token kernels hold one (256 slots), so d = 3080
    (193 tiles) gives 12-13 rows.  Row ranges start at unaligned rows, so
    the residual loads and output stores go element by element at the
    edges; f is off the 128-k stage in all but one case."""
    from transformer_ffn_block_amd import ffn
    _say("decode balanced down", M, d, f)
    b = I.make_block(3250 + M, M, d, f, "bf16")
    r = O.block_from_stored("bf16", b.x, b.g, b.w_gate, b.w_up, b.w_down, b.eps)
    err = max_norm_err(host_f64(_run_block(ffn, b, "auto")), r)
    assert record(f"decode balanced down rows {M}x{d}x{f}", err, TOL_BF16) <= TOL_BF16


@pytest.mark.parametrize("kind", ["q8", "q4"])
@pytest.mark.parametrize("M,d,f", [(8, 512, 6144), (5, 256, 7680), (16, 256, 6144)])
def test_quant_balanced_row_ranges(gpu_lib, kind, M, d, f):
    from transformer_ffn_block_amd import ffn
    _say("quant balanced", kind, M, d, f)
    if kind == "q8":
        q = I.make_q8_block(3300 + M, M, d, f)
        err, tol = max_norm_err(_run_q8(ffn, q), _q8_ref(q)), TOL_Q8
    else:
        q = I.make_q4_block(3400 + M, M, d, f)
        err, tol = max_norm_err(_run_q4(ffn, q), _q4_ref(q)), TOL_Q4
    assert record(f"{kind} balanced rows {M}x{d}x{f}", err, tol) <= tol


def test_fused_norm_at_decode_sizes_is_auto(gpu_lib):
    """Up to 64 tokens FUSED_NORM takes the decode kernels, which fold the
    norm already: the same bits as AUTO."""
    from transformer_ffn_block_amd import ffn
    import torch
    b = I.make_block(3500, 40, 512, 704, "bf16")
    x, g, wg, wu, wd = _block_dev(b)
    ya = ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant="auto")
    yn = ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant="fused_norm")
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(ya), host_bits(yn))


# ----------------------------------------------------------------------------
# maximum sizes: weight matrices just under the 2 GiB the ABI takes (32-bit
# buffer offsets).  The oracle cannot run these whole, so the checks use
# properties that fix the result at any size: W_down = 0 returns x bit for
# bit, and a one-hot W_down picks one column j of h, which the oracle
# computes from two weight rows (y[:, i] = x[:, i] + h[:, j], every other
# column y = x).  Weights are drawn on the device from a seeded generator
# (N(0, 0.02) as elsewhere); the rows the oracle needs are copied back.
# ----------------------------------------------------------------------------
def _big_normal(shape, seed, std=0.02):
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    return (torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32) * std).to(torch.bfloat16)


@pytest.mark.parametrize("M,variant", [(4, "auto"), (300, "fused")])
def test_block_max_size_one_hot_down(gpu_lib, M, variant):
    from transformer_ffn_block_amd import ffn
    import torch
    d, f = 16384, 65528            # f * d * 2 = 2147221504 < 2^31 bytes
    assert f * d * 2 < 2 ** 31 and (f + 8) * d * 2 >= 2 ** 31
    _say("max size", M, d, f, variant)
    b = I.make_block(3600 + M, M, d, 8, "bf16")   # x, g drawn as elsewhere (weights below)
    x, g = dev(b.x), dev(b.g)
    wg = _big_normal((f, d), 3601)
    wu = _big_normal((f, d), 3602)
    wd = torch.zeros((d, f), dtype=torch.bfloat16, device="cuda")
    y0 = ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant=variant)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y0), b.x)          # W_down = 0: y = x exactly
    i, j = 12345, f - 3                                 # output column i reads h column j
    wd[i, j] = 1.0
    y1 = ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant=variant)
    torch.cuda.synchronize()
    a = host_f64(y1)
    others = np.ones(d, bool)
    others[i] = False
    assert np.array_equal(host_bits(y1)[:, others], b.x[:, others])
    rows = [host_bits(t[j:j + 1].contiguous()) for t in (wg, wu)]
    n = O.rmsnorm_from_stored("bf16", b.x, b.g, b.eps)
    G = n @ O.bf16_to_f64(rows[0][0])
    U = n @ O.bf16_to_f64(rows[1][0])
    want = O.bf16_to_f64(b.x[:, i]) + O.silu(G) * U
    err = float(np.max(np.abs(a[:, i] - want)) / np.max(np.abs(want)))
    assert record(f"max size {M}x{d}x{f} {variant} (one-hot down column)", err, TOL_BF16) <= TOL_BF16


def test_q8_max_size_zero_down_and_one_hot(gpu_lib):
    from transformer_ffn_block_amd import ffn
    import torch
    M, d, f = 8, 16384, 131040     # f * d = 2147155968 < 2^31 quant bytes
    assert f * d < 2 ** 31 and (f + 32) * d >= 2 ** 31
    _say("q8 max size", M, d, f)
    q = I.make_q8_block(3700, M, d, 32)             # x, g (small weights unused)
    x, g = dev(q.x), dev(q.g)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3701)

    def qmat(N, K):
        qs = torch.randint(-127, 128, (N, K), generator=gen, device="cuda", dtype=torch.int8)
        sc = (torch.randn((N, K // 32), generator=gen, device="cuda").abs() * (0.02 / 127 * 4)).half()
        return qs, sc.view(torch.int16)
    wg, wu = qmat(f, d), qmat(f, d)
    wd = (torch.zeros((d, f), dtype=torch.int8, device="cuda"),
          torch.zeros((d, f // 32), dtype=torch.int16, device="cuda"))
    y0 = ffn.swiglu_block_q8(x, g, wg, wu, wd, q.eps)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y0), q.x)
    i, j = 777, 100003
    wd[0][i, j] = 1
    wd[1][i, j // 32] = 0x3C00                          # fp16 1.0: weight (i, j) = 1
    y1 = ffn.swiglu_block_q8(x, g, wg, wu, wd, q.eps)
    torch.cuda.synchronize()
    a = host_f64(y1)
    others = np.ones(d, bool)
    others[i] = False
    assert np.array_equal(host_bits(y1)[:, others], q.x[:, others])
    row = lambda m: O.q8_dequant(m[0][j:j + 1].cpu().numpy(), m[1][j:j + 1].cpu().numpy().view(np.uint16))[0]
    n = O.rmsnorm_from_stored("bf16", q.x, q.g, q.eps)
    want = O.bf16_to_f64(q.x[:, i]) + O.silu(n @ row(wg)) * (n @ row(wu))
    err = float(np.max(np.abs(a[:, i] - want)) / np.max(np.abs(want)))
    assert record(f"q8 max size {M}x{d}x{f} (one-hot down column)", err, TOL_Q8) <= TOL_Q8


# ----------------------------------------------------------------------------
# HIP graphs: a block call captured on torch's capture stream and replayed
# gives the eager call's bits on every replay (with eager work and
# synchronisations between replays).  Decode kernels, and 128 tokens on the
# split-K prefill GEMMs (their partial passes included).
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("M,d,f", [(16, 1024, 2816), (128, 1024, 2048)])
def test_block_replayed_from_hip_graph(gpu_lib, M, d, f):
    from transformer_ffn_block_amd import ffn
    import torch
    _say("block hip graph", M, d, f)
    b = I.make_block(5800 + M, M, d, f, "bf16")
    x, g, wg, wu, wd = _block_dev(b)
    ws = ffn.alloc_workspace(ffn.workspace_size(ffn.FFN_BF16, M, d, f, "auto"))
    y = torch.empty_like(x)
    ref = host_bits(ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant="auto"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream, as capture requires
        ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant="auto", out=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant="auto", out=y, workspace=ws)
    for rep in range(4):
        y.fill_(float("nan"))
        ws.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(y), ref), rep
        # an eager call between replays leaves the captured one unaffected
        ffn.swiglu_block(x, g, wg, wu, wd, b.eps, variant="auto", out=y, workspace=ws)
        torch.cuda.synchronize()
    del graph


# ----------------------------------------------------------------------------
# seeded random shapes across every regime (decode kernels, the 33..64-token
# single launches, split-K and whole prefill GEMMs, balanced grids), each
# against the oracle
# ----------------------------------------------------------------------------
def _random_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.choice([rng.integers(1, 17), rng.integers(17, 65), rng.integers(65, 420)]))
        # half the dimensions on the 64-deep K tile (LDS-fed and split-K
        # GEMMs), half anywhere on the 8-element grid (register-staged GEMMs,
        # ragged decode stages)
        d = int(rng.integers(1, 17)) * 64 if rng.random() < 0.5 else int(rng.integers(1, 129)) * 8
        f = int(rng.integers(1, 17)) * 64 if rng.random() < 0.5 else int(rng.integers(1, 129)) * 8
        v = str(rng.choice(["auto", "fused", "split"]))
        out.append((M, d, f, v))
    return out


@pytest.mark.parametrize("M,d,f,variant", _random_shapes(24, 2026))
def test_block_random_shapes(gpu_lib, M, d, f, variant):
    from transformer_ffn_block_amd import ffn
    _say("block random shape", M, d, f, variant)
    b = I.make_block(6000 + M + d + f, M, d, f, "bf16")
    r = O.block_from_stored("bf16", b.x, b.g, b.w_gate, b.w_up, b.w_down, b.eps)
    a = host_f64(_run_block(ffn, b, variant))
    assert record(f"random {M}x{d}x{f} {variant}", max_norm_err(a, r), TOL_BF16) <= TOL_BF16
