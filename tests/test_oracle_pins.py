"""Pins of the fp64 oracle to facts fixed outside the oracle itself.

Each group targets a plausible mistake: a flipped sign or a sigmoid in place
of silu, eps outside the root or added to the sum instead of the mean, the
gain applied per row, gate and up swapped, a transposed weight, the residual
taken from n instead of x, the wrong Q8 block axis, flushed fp16 subnormals.
Sources: hand-worked fixtures under tests/golden/ (each cites its passage),
closed forms of the logistic function, scipy/torch library routines for
special cases, and invariants of the definitions.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import ffn_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


# ----------------------------------------------------------------------------
# decoders
# ----------------------------------------------------------------------------
def test_bf16_decoder_known_bits():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x0001, 0x7F7F, 0x4049], np.uint16)
    want = [1.0, -2.0, 1.0078125, 0.0, -0.0, 2.0 ** -133, 3.3895313892515355e38, 3.140625]
    got = O.bf16_to_f64(bits)
    assert list(got) == want


def test_f16_decoder_known_bits_keeps_subnormals():
    bits = np.array([0x3C00, 0x0001, 0x03FF, 0x0400, 0x7BFF, 0xBC00, 0x3555], np.uint16)
    want = [1.0, 2.0 ** -24, 1023 * 2.0 ** -24, 2.0 ** -14, 65504.0, -1.0, 0.333251953125]
    assert list(O.f16_to_f64(bits)) == want


# ----------------------------------------------------------------------------
# silu
# ----------------------------------------------------------------------------
def test_silu_zero_is_exactly_zero():
    assert O.silu(np.array([0.0]))[0] == 0.0


def test_silu_odd_part_identity():
    # sigma(v) + sigma(-v) = 1  =>  silu(v) - silu(-v) = v
    v = np.linspace(-40, 40, 4001)
    d = O.silu(v) - O.silu(-v)
    assert np.max(np.abs(d - v) / np.maximum(1.0, np.abs(v))) < 1e-15


def test_silu_large_positive_tends_to_identity():
    # 0 <= v - silu(v) = v e^-v / (1 + e^-v) <= v e^-v
    for v in (5.0, 10.0, 20.0, 50.0):
        s = O.silu(np.array([v]))[0]
        # allow a few ulps of v for the rounding of silu(v) itself
        assert 0.0 <= v - s <= v * math.exp(-v) + 4 * np.spacing(v)
    assert abs(O.silu(np.array([20.0]))[0] - 20.0) < 5e-8


def test_silu_large_negative_tends_to_zero_from_below():
    for v in (-20.0, -50.0, -200.0, -800.0):
        s = O.silu(np.array([v]))[0]
        assert s <= 0.0 and abs(s) <= abs(v) * math.exp(v) * (1 + 1e-12)
    assert np.isfinite(O.silu(np.array([-1000.0, 1000.0]))).all()


def test_silu_known_logistic_values():
    # sigma(1) = e/(e+1), sigma(2) = 1/(1+e^-2), sigma(-1) = 1/(1+e)
    v = np.array([1.0, 2.0, -1.0])
    want = np.array([math.e / (math.e + 1), 2.0 / (1 + math.exp(-2)), -1.0 / (1 + math.e)])
    assert np.allclose(O.silu(v), want, rtol=1e-15, atol=0)


def test_silu_matches_scipy_expit():
    from scipy.special import expit
    v = np.linspace(-60, 60, 10001)
    assert np.allclose(O.silu(v), v * expit(v), rtol=1e-14, atol=1e-300)


def test_silu_minimum_lambert_w():
    # silu'(v) = 0 at v* = -1 - W(1/e), where silu(v*) = v* + 1
    from scipy.special import lambertw
    vstar = -1.0 - lambertw(1.0 / math.e).real
    assert abs(O.silu(np.array([vstar]))[0] - (vstar + 1.0)) < 1e-15
    grid = np.linspace(-5, 5, 200001)
    assert abs(grid[np.argmin(O.silu(grid))] - vstar) < 1e-4
    assert abs(vstar - (-1.2784645427610738)) < 1e-15


# ----------------------------------------------------------------------------
# RMSNorm
# ----------------------------------------------------------------------------
def test_rmsnorm_golden_onehot():
    gd = _load("rmsnorm_onehot.json")
    n = O.rmsnorm(np.array(gd["x"]), np.array(gd["g"]), gd["eps"])
    assert np.array_equal(n, np.array(gd["n"]))


def test_rmsnorm_unit_gain_rows_have_unit_rms():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((13, 96)) * rng.uniform(0.01, 100, (13, 1))
    n = O.rmsnorm(x, np.ones(96), 0.0)
    assert np.allclose(np.sqrt(np.mean(n * n, axis=1)), 1.0, rtol=1e-13, atol=0)
    # with eps > 0: RMS = sqrt(ms / (ms + eps))
    eps = 0.5
    n = O.rmsnorm(x, np.ones(96), eps)
    ms = np.mean(x * x, axis=1)
    assert np.allclose(np.sqrt(np.mean(n * n, axis=1)), np.sqrt(ms / (ms + eps)), rtol=1e-13)


def test_rmsnorm_scale_invariance_without_eps():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64))
    g = 1 + 0.1 * rng.standard_normal(64)
    for c in (1e-3, 7.0, 100.0, -3.0):
        a = O.rmsnorm(c * x, g, 0.0)
        b = O.rmsnorm(x, g, 0.0) * np.sign(c)
        assert np.allclose(a, b, rtol=1e-13, atol=1e-15)


def test_rmsnorm_constant_row_and_per_column_gain():
    # row of constant c: n_k = g_k * c / sqrt(c^2 + eps); c=1, eps=3 -> g_k / 2
    g = np.arange(1.0, 9.0)
    n = O.rmsnorm(np.ones((1, 8)), g, 3.0)
    assert np.array_equal(n[0], g / 2)
    # mean, not sum: four ones with eps=0 give exactly 1
    assert np.array_equal(O.rmsnorm(np.ones((2, 4)), np.ones(4), 0.0), np.ones((2, 4)))


def test_rmsnorm_zero_row_is_zero():
    n = O.rmsnorm(np.zeros((3, 16)), np.full(16, 2.0), 1e-6)
    assert np.array_equal(n, np.zeros((3, 16)))


def test_rmsnorm_matches_torch_rms_norm_fp64():
    import torch
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 200))
    g = 1 + 0.1 * rng.standard_normal(200)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (200,), torch.from_numpy(g), eps=1e-6).numpy()
    assert np.allclose(O.rmsnorm(x, g, 1e-6), want, rtol=1e-13, atol=1e-15)


# ----------------------------------------------------------------------------
# the block
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["block_handcalc_gain.json", "block_handcalc_eps.json"])
def test_block_golden(name):
    gd = _load(name)
    args = [np.array(gd[k], dtype=np.float64) for k in ("x", "g", "w_gate", "w_up", "w_down")]
    y, n, G, U, h = O.swiglu_block_intermediates(*args, gd["eps"])
    assert np.allclose(n, gd["n"], rtol=gd["tol"], atol=0)
    assert np.allclose(h, gd["h"], rtol=gd["tol"], atol=0)
    assert np.allclose(y, gd["y"], rtol=gd["tol"], atol=0)
    assert np.array_equal(O.swiglu_block(*args, gd["eps"]), y)


def _rand_block(seed, M=5, d=24, f=40):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, d))
    g = 1 + 0.1 * rng.standard_normal(d)
    wg = 0.3 * rng.standard_normal((f, d))
    wu = 0.3 * rng.standard_normal((f, d))
    wd = 0.3 * rng.standard_normal((d, f))
    return x, g, wg, wu, wd


def test_block_zero_down_or_up_is_identity():
    x, g, wg, wu, wd = _rand_block(3)
    assert np.array_equal(O.swiglu_block(x, g, wg, wu, np.zeros_like(wd), 1e-6), x)
    assert np.array_equal(O.swiglu_block(x, g, wg, np.zeros_like(wu), wd, 1e-6), x)


def test_block_zero_row_stays_zero():
    x, g, wg, wu, wd = _rand_block(4)
    x[2] = 0.0
    y = O.swiglu_block(x, g, wg, wu, wd, 1e-6)
    assert np.array_equal(y[2], np.zeros(x.shape[1]))


def test_block_linear_in_down_and_up():
    x, g, wg, wu, wd = _rand_block(5)
    base = O.swiglu_block(x, g, wg, wu, wd, 1e-6) - x
    for a in (0.5, -2.0, 3.0):
        assert np.allclose(O.swiglu_block(x, g, wg, wu, a * wd, 1e-6) - x, a * base, rtol=1e-12, atol=1e-14)
        assert np.allclose(O.swiglu_block(x, g, wg, a * wu, wd, 1e-6) - x, a * base, rtol=1e-12, atol=1e-14)


def test_block_gate_closed_forms():
    # gate pushed far negative: silu -> 0 whatever U is, so y -> x
    x, g, wg, wu, wd = _rand_block(6, M=3, d=8, f=4)
    # positive inputs and gains make n > 0, so a constant negative W_gate makes
    # every G_j hugely negative
    x2 = np.abs(x) + 0.5
    n2 = O.rmsnorm(x2, np.abs(g), 1e-6)
    wg_neg = np.zeros_like(wg)
    wg_neg[:, :] = -200.0
    assert (n2 @ wg_neg.T < -100).all()
    y = O.swiglu_block(x2, np.abs(g), wg_neg, 50 * wu, wd, 1e-6)
    assert np.allclose(y, x2, rtol=0, atol=1e-30)
    # gate pushed far positive: silu(G) ~ G, so h ~ G*U exactly bilinear
    wg_pos = np.full_like(wg, 200.0)
    y = O.swiglu_block(x2, np.abs(g), wg_pos, wu, wd, 1e-6)
    G = n2 @ wg_pos.T
    U = n2 @ wu.T
    assert np.allclose(y, x2 + (G * U) @ wd.T, rtol=1e-13, atol=1e-13)


def test_block_one_hot_weights_pick_indices():
    # W_down with a single 1 at (i, j) adds h_j to y_i only; W_gate/W_up one-hot
    # at (j, k) make G_j = n_k, U_j = n_k2: checks every projection's orientation.
    M, d, f = 2, 6, 5
    rng = np.random.default_rng(7)
    x = rng.standard_normal((M, d))
    g = 1 + 0.1 * rng.standard_normal(d)
    wg = np.zeros((f, d)); wg[3, 1] = 1.0
    wu = np.zeros((f, d)); wu[3, 4] = 1.0
    wd = np.zeros((d, f)); wd[2, 3] = 1.0
    n = O.rmsnorm(x, g, 1e-6)
    y = O.swiglu_block(x, g, wg, wu, wd, 1e-6)
    expect = x.copy()
    expect[:, 2] += O.silu(n[:, 1]) * n[:, 4]
    assert np.allclose(y, expect, rtol=1e-15, atol=0)


def test_block_row_permutation_equivariance():
    x, g, wg, wu, wd = _rand_block(8, M=9)
    p = np.random.default_rng(0).permutation(9)
    assert np.array_equal(O.swiglu_block(x[p], g, wg, wu, wd, 1e-6),
                          O.swiglu_block(x, g, wg, wu, wd, 1e-6)[p])


def test_block_matches_torch_functional_fp64():
    import torch
    import torch.nn.functional as F
    x, g, wg, wu, wd = _rand_block(9, M=4, d=32, f=48)
    t = [torch.from_numpy(a) for a in (x, g, wg, wu, wd)]
    n = F.rms_norm(t[0], (32,), t[1], eps=1e-6)
    want = t[0] + F.linear(F.silu(F.linear(n, t[2])) * F.linear(n, t[3]), t[4])
    assert np.allclose(O.swiglu_block(x, g, wg, wu, wd, 1e-6), want.numpy(), rtol=1e-12, atol=1e-13)


def test_block_brute_force_loops_tiny():
    # element-by-element loops on tiny shapes (M<=3, d,f<=16)
    for seed, (M, d, f) in enumerate([(1, 2, 3), (3, 16, 5), (2, 7, 16)]):
        x, g, wg, wu, wd = _rand_block(100 + seed, M, d, f)
        eps = 1e-6
        y_ref = np.zeros((M, d))
        for m in range(M):
            ss = 0.0
            for k in range(d):
                ss += x[m, k] ** 2
            r = 1.0 / math.sqrt(ss / d + eps)
            n = [x[m, k] * r * g[k] for k in range(d)]
            h = []
            for j in range(f):
                a = sum(wg[j, k] * n[k] for k in range(d))
                b = sum(wu[j, k] * n[k] for k in range(d))
                h.append(a / (1.0 + math.exp(-a)) * b)
            for i in range(d):
                y_ref[m, i] = x[m, i] + sum(wd[i, j] * h[j] for j in range(f))
        assert np.allclose(O.swiglu_block(x, g, wg, wu, wd, eps), y_ref, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# Q8_0
# ----------------------------------------------------------------------------
def test_q8_dequant_golden_blocks_and_subnormal_scale():
    gd = _load("q8_dequant_blocks.json")
    w = O.q8_dequant(np.array(gd["qs"], dtype=np.int8), np.array(gd["scale_bits"], dtype=np.uint16))
    assert np.array_equal(w[0, :32], np.full(32, gd["block0_weight"]))
    assert np.array_equal(np.abs(w[0, 32:]), np.full(32, gd["block1_weight_abs"]))
    assert np.array_equal(np.sign(w[0, 32:]), np.tile([-1.0, 1.0], 16))


def test_q8_unit_scales_reduce_to_integer_weights():
    rng = np.random.default_rng(11)
    qs = rng.integers(-128, 128, size=(6, 96), dtype=np.int8)
    ones = np.full((6, 3), 0x3C00, np.uint16)
    assert np.array_equal(O.q8_dequant(qs, ones), qs.astype(np.float64))


def test_q8_doubling_one_block_scale_doubles_its_contribution():
    rng = np.random.default_rng(12)
    N, K = 4, 128
    qs = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    s = (np.abs(rng.standard_normal((N, K // 32))) * 0.01).astype(np.float16)
    s2 = s.copy(); s2[1, 2] *= 2  # exact doubling in fp16
    v = rng.standard_normal(K)
    w1 = O.q8_dequant(qs, s.view(np.uint16))
    w2 = O.q8_dequant(qs, s2.view(np.uint16))
    contrib = w1[1, 64:96] @ v[64:96]
    assert np.allclose(w2 @ v - w1 @ v, np.array([0, contrib, 0, 0]), rtol=1e-13, atol=1e-15)


def test_q8_block_equals_dense_block_on_dequantised_weights():
    rng = np.random.default_rng(13)
    M, d, f = 2, 64, 96
    from transformer_ffn_block_amd import inputs as I
    q = I.make_q8_block(13, M, d, f)
    y = O.swiglu_block_q8(q.x, q.g, (q.w_gate.qs, q.w_gate.scales), (q.w_up.qs, q.w_up.scales),
                          (q.w_down.qs, q.w_down.scales), q.eps)
    # same thing via an independently written dequant (scale via np.float16 arithmetic)
    def deq(m):
        s = m.scales.view(np.float16).astype(np.float64)
        return m.qs.astype(np.float64) * np.kron(s, np.ones((1, 32)))
    y2 = O.swiglu_block(O.bf16_to_f64(q.x), O.bf16_to_f64(q.g), deq(q.w_gate), deq(q.w_up), deq(q.w_down), q.eps)
    assert np.array_equal(y, y2)
    del rng


def test_q8_dequant_product_is_exact_in_fp32():
    # int8 (<= 8 significant bits) times fp16 (11 significant bits) fits the
    # 24-bit fp32 significand, so a fp32 dequantisation is exact.
    rng = np.random.default_rng(14)
    q = rng.integers(-128, 128, size=100000).astype(np.int8)
    s = (np.abs(rng.standard_normal(100000)) * 0.02 / 127 * 4).astype(np.float16)
    p32 = q.astype(np.float32) * s.astype(np.float32)
    p64 = q.astype(np.float64) * s.astype(np.float64)
    assert np.array_equal(p32.astype(np.float64), p64)


# ----------------------------------------------------------------------------
# Q4_0
# ----------------------------------------------------------------------------
def test_q4_dequant_golden_blocks():
    gd = _load("q4_dequant_blocks.json")
    w = O.q4_dequant(np.array(gd["qs"], dtype=np.uint8), np.array(gd["scale_bits"], dtype=np.uint16))
    assert np.array_equal(w, np.array(gd["weights"], dtype=np.float64))


def test_q4_nibble_positions_one_hot():
    # every nibble 8 (weight 0) except one set to 9: the weight vector is the
    # unit vector at that position, for each of the 32 positions of a block
    for p in range(32):
        b = np.full((1, 16), 0x88, dtype=np.uint8)
        byte, shift = p % 16, (0 if p < 16 else 4)
        b[0, byte] = (b[0, byte] & ~np.uint8(0xF << shift)) | np.uint8(9 << shift)
        w = O.q4_dequant(b, np.array([[0x3C00]], dtype=np.uint16))
        e = np.zeros((1, 32)); e[0, p] = 1.0
        assert np.array_equal(w, e), p


def test_q4_unit_scales_give_nibble_minus_eight():
    rng = np.random.default_rng(21)
    n = rng.integers(0, 16, size=(5, 128), dtype=np.uint8)
    packed = n.reshape(5, 4, 2, 16)
    qs = (packed[:, :, 0, :] | (packed[:, :, 1, :] << 4)).reshape(5, 64).astype(np.uint8)
    ones = np.full((5, 4), 0x3C00, np.uint16)
    assert np.array_equal(O.q4_dequant(qs, ones), n.astype(np.float64) - 8.0)


def test_q4_block_equals_dense_block_on_dequantised_weights():
    from transformer_ffn_block_amd import inputs as I
    M, d, f = 2, 64, 96
    q = I.make_q4_block(22, M, d, f)
    y = O.swiglu_block_q4(q.x, q.g, (q.w_gate.qs, q.w_gate.scales), (q.w_up.qs, q.w_up.scales),
                          (q.w_down.qs, q.w_down.scales), q.eps)

    # an independently written dequant: split every byte with unpackbits
    def deq(m):
        N, H = m.qs.shape
        bits = np.unpackbits(m.qs[..., None], axis=-1)          # msb first
        hi = bits[..., :4] @ np.array([8, 4, 2, 1]); lo = bits[..., 4:] @ np.array([8, 4, 2, 1])
        blk = np.concatenate([lo.reshape(N, -1, 16), hi.reshape(N, -1, 16)], axis=2).reshape(N, 2 * H)
        s = m.scales.view(np.float16).astype(np.float64)
        return (blk - 8.0) * np.kron(s, np.ones((1, 32)))
    y2 = O.swiglu_block(O.bf16_to_f64(q.x), O.bf16_to_f64(q.g), deq(q.w_gate), deq(q.w_up), deq(q.w_down), q.eps)
    assert np.array_equal(y, y2)


def test_q4_block_form_roundtrip():
    from transformer_ffn_block_amd import inputs as I
    m = I.make_q4_matrix(np.random.default_rng(23), 3, 96)
    m2 = I.q4_aos_to_soa(I.q4_soa_to_aos(m), 3, 96)
    assert np.array_equal(m.qs, m2.qs) and np.array_equal(m.scales, m2.scales)
    blocks = I.q4_soa_to_aos(m).reshape(3, 3, 18)
    assert np.array_equal(blocks[1, 2, 2:], m.qs[1, 32:48])  # the 16 bytes follow the scale


# ----------------------------------------------------------------------------
# stored-format wrappers (what every GPU parity test uses as its reference)
# ----------------------------------------------------------------------------
def _f32_bits(v: float) -> int:
    """IEEE binary32 bit pattern of v, by the standard library's packer."""
    import struct
    return struct.unpack(">I", struct.pack(">f", v))[0]


def _bf16_bits_exact(a) -> np.ndarray:
    """bf16 bit patterns of values that bf16 holds exactly (the top 16 bits of
    their binary32 pattern; the low 16 bits must be zero)."""
    a = np.asarray(a, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    for idx, v in np.ndenumerate(a):
        b = _f32_bits(float(v))
        assert b & 0xFFFF == 0, f"{v} is not a bf16 value"
        out[idx] = b >> 16
    return out


def test_as_f64_f32_known_bits():
    # 1 + 2^-23, -(1/6 rounded to binary32), 2^-149 (smallest subnormal),
    # 3.4028234663852886e38 (largest finite): none of them fits bf16 or fp16
    bits = np.array([0x3F800001, 0xBE2AAAAB, 0x00000001, 0x7F7FFFFF], dtype=np.uint32)
    want = [1.0 + 2.0 ** -23, -0.1666666716337204, 2.0 ** -149, 3.4028234663852886e38]
    got = O.as_f64(bits.view(np.float32), "f32")
    assert got.dtype == np.float64 and list(got) == want
    assert list(O.as_f64(np.array([0x3F80, 0xBF00], np.uint16), "bf16")) == [1.0, -0.5]


@pytest.mark.parametrize("name", ["block_handcalc_gain.json", "block_handcalc_eps.json"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_block_from_stored_on_golden_fixtures(name, dtype):
    """The hand-worked blocks, handed over as stored bit patterns, reproduce
    the hand-worked outputs: each operand reaches its own role."""
    gd = _load(name)
    keys = ("x", "g", "w_gate", "w_up", "w_down")
    if dtype == "bf16":
        stored = [_bf16_bits_exact(gd[k]) for k in keys]
    else:
        stored = [np.array(gd[k], dtype=np.float32) for k in keys]
    y = O.block_from_stored(dtype, *stored, gd["eps"])
    assert y.dtype == np.float64
    assert np.allclose(y, gd["y"], rtol=gd["tol"], atol=0)


def test_block_from_stored_f32_values_outside_bf16():
    """fp32 inputs that bf16 cannot hold: the wrapper equals the block on the
    same values decoded by the standard library's unpacker."""
    import struct
    rng = np.random.default_rng(31)
    M, d, f = 2, 8, 6
    raw = [rng.integers(0, 1 << 16, size=s, dtype=np.uint32) for s in ((M, d), (d,), (f, d), (f, d), (d, f))]
    # exponent fields of 1/64 .. 2, random low mantissa bits, random signs
    stored = []
    for r in raw:
        e = rng.integers(121, 128, size=r.shape, dtype=np.uint32)
        sgn = rng.integers(0, 2, size=r.shape, dtype=np.uint32)
        stored.append(((sgn << 31) | (e << 23) | (r * 127 % (1 << 23))).astype(np.uint32).view(np.float32))
    assert all(np.any(s.view(np.uint32) & 0xFFFF) for s in stored)
    dec = [np.vectorize(lambda b: struct.unpack(">f", struct.pack(">I", int(b)))[0])(s.view(np.uint32))
           for s in stored]
    want = O.swiglu_block(*dec, 1e-6)
    assert np.array_equal(O.block_from_stored("f32", *stored, 1e-6), want)


def test_block_from_stored_gate_and_up_roles():
    """One-hot weights as bf16 bits: gate reads n_1, up reads n_4, down adds
    to y_2; swapping any two weight roles changes the result."""
    M, d, f = 2, 6, 5
    x = np.array([[1.0, -2.0, 0.5, 4.0, 1.5, -1.0], [0.25, 1.0, -3.0, 2.0, -0.5, 1.0]])
    g = np.array([1.0, 2.0, 0.5, 1.0, 4.0, 1.0])
    wg = np.zeros((f, d)); wg[3, 1] = 1.0
    wu = np.zeros((f, d)); wu[3, 4] = 1.0
    wd = np.zeros((d, f)); wd[2, 3] = 1.0
    n = O.rmsnorm(x, g, 0.0)
    expect = x.copy()
    expect[:, 2] += O.silu(n[:, 1]) * n[:, 4]
    bits = [_bf16_bits_exact(a) for a in (x, g, wg, wu, wd)]
    assert np.allclose(O.block_from_stored("bf16", *bits, 0.0), expect, rtol=1e-15, atol=0)
    swapped = O.block_from_stored("bf16", bits[0], bits[1], bits[3], bits[2], bits[4], 0.0)
    assert not np.allclose(swapped, expect, rtol=1e-6, atol=0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rmsnorm_from_stored_on_golden_onehot(dtype):
    gd = _load("rmsnorm_onehot.json")
    if dtype == "bf16":
        x, g = _bf16_bits_exact(gd["x"]), _bf16_bits_exact(gd["g"])
    else:
        x, g = np.array(gd["x"], np.float32), np.array(gd["g"], np.float32)
    n = O.rmsnorm_from_stored(dtype, x, g, gd["eps"])
    assert n.dtype == np.float64 and np.array_equal(n, np.array(gd["n"]))


def test_rmsnorm_from_stored_bf16_gain_per_column():
    # constant row 1, eps = 3: n_k = g_k / 2 exactly; g as bf16 bits
    g = np.arange(1.0, 9.0)
    n = O.rmsnorm_from_stored("bf16", _bf16_bits_exact(np.ones((1, 8))), _bf16_bits_exact(g), 3.0)
    assert np.array_equal(n[0], g / 2)
