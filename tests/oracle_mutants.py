"""Planted mistakes for the fp64 oracle (CPU only, test infrastructure).

Each mutant is one plausible slip in oracle/ffn_oracle.py, written as a
textual substitution of the source.  `python tests/oracle_mutants.py NAME`
loads the mutated oracle in place of the real one and runs the oracle pins
(tests/test_oracle_pins.py) against it; the exit status is pytest's, so a
mutant that the pins catch exits non-zero.  Not collected by pytest itself
(the file name does not start with test_); test_oracle_mutants.py drives it.
"""
import os
import sys
import types

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "ffn_oracle.py")

# name -> (text in the oracle source, replacement)
MUTANTS = {
    "eps_outside_root": ("r = 1.0 / np.sqrt(ms + eps)", "r = 1.0 / (np.sqrt(ms) + eps)"),
    "eps_added_to_sum_not_mean": ("    ms /= d\n    r = 1.0 / np.sqrt(ms + eps)",
                                  "    r = 1.0 / np.sqrt((ms + eps) / d)"),
    "sum_of_squares_not_mean": ("    ms /= d\n", ""),
    "abs_instead_of_square": ("ms += x[..., k] * x[..., k]", "ms += np.abs(x[..., k])"),
    "gain_dropped": ("return x * r[..., None] * g", "return x * r[..., None]"),
    "gain_one_plus_g": ("return x * r[..., None] * g", "return x * r[..., None] * (1.0 + g)"),
    "gain_per_row": ("return x * r[..., None] * g", "return x * (r * g[: r.shape[-1]] if r.ndim else r)[..., None]"),
    "silu_sign_flip": ("out[pos] = v[pos] / (1.0 + np.exp(-v[pos]))", "out[pos] = v[pos] / (1.0 + np.exp(v[pos]))"),
    "sigmoid_for_negative_v": ("out[~pos] = v[~pos] * e / (1.0 + e)", "out[~pos] = e / (1.0 + e)"),
    "sigmoid_instead_of_silu": ("out[pos] = v[pos] / (1.0 + np.exp(-v[pos]))", "out[pos] = 1.0 / (1.0 + np.exp(-v[pos]))"),
    "gate_and_up_swapped": ("    h = silu(G) * U\n    return x + h", "    h = G * silu(U)\n    return x + h"),
    "up_uses_gate_weights": ("    U = n @ np.asarray(w_up, dtype=np.float64).T\n    h = silu(G) * U\n    return",
                             "    U = n @ np.asarray(w_gate, dtype=np.float64).T\n    h = silu(G) * U\n    return"),
    "residual_dropped": ("    return x + h @ np.asarray(w_down, dtype=np.float64).T\n\n\ndef swiglu_block_intermediates",
                         "    return h @ np.asarray(w_down, dtype=np.float64).T\n\n\ndef swiglu_block_intermediates"),
    "residual_from_n": ("    return x + h @ np.asarray(w_down, dtype=np.float64).T\n\n\ndef swiglu_block_intermediates",
                        "    return n + h @ np.asarray(w_down, dtype=np.float64).T\n\n\ndef swiglu_block_intermediates"),
    "down_weight_transposed": ("    return x + h @ np.asarray(w_down, dtype=np.float64).T\n\n\ndef swiglu_block_intermediates",
                               "    return x + h @ np.asarray(w_down, dtype=np.float64).reshape(w_down.shape[::-1])\n\n\ndef swiglu_block_intermediates"),
    "q8_blocks_interleaved": ("return q * np.repeat(s, 32, axis=1)", "return q * np.tile(s, (1, 32))"),
    "q8_quants_unsigned": ("q = np.asarray(qs, dtype=np.int8).astype(np.float64)",
                           "q = np.asarray(qs, dtype=np.int8).view(np.uint8).astype(np.float64)"),
    "f16_subnormals_flushed": ("return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)",
                               "v = np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)\n"
                               "    return np.where(np.abs(v) < 2.0 ** -14, 0.0, v)"),
    "q4_nibble_halves_swapped": ("        low = (byte & 0x0F) - 8                      # weights 32*blk + 0 .. 15\n        high = (byte >> 4) - 8 ",
                                 "        high = (byte & 0x0F) - 8\n        low = (byte >> 4) - 8 "),
    "q4_offset_seven": ("        low = (byte & 0x0F) - 8 ", "        low = (byte & 0x0F) - 7 "),
    "q4_scale_of_next_block": ("        w[:, 32 * blk:32 * blk + 16] = low * s[:, blk:blk + 1]",
                               "        w[:, 32 * blk:32 * blk + 16] = low * s[:, (blk + 1) % s.shape[1]:(blk + 1) % s.shape[1] + 1]"),
    "bf16_low_half": ("return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)",
                      "return (b.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)"),
    "wrapper_gate_up_swapped": ("as_f64(w_gate, dtype),\n                        as_f64(w_up, dtype)",
                                "as_f64(w_up, dtype),\n                        as_f64(w_gate, dtype)"),
    "wrapper_down_from_up": ("as_f64(w_up, dtype), as_f64(w_down, dtype), eps)",
                             "as_f64(w_up, dtype), as_f64(w_up, dtype).T, eps)"),
    "wrapper_f32_through_f16": ("return np.asarray(a, dtype=np.float32).astype(np.float64)",
                                "return np.asarray(a, dtype=np.float16).astype(np.float64)"),
    "wrapper_f32_truncated_to_bf16": ("return np.asarray(a, dtype=np.float32).astype(np.float64)",
                                      "return bf16_to_f64(np.asarray(a, dtype=np.float32).view(np.uint32) >> 16)"),
    "rmsnorm_wrapper_gain_decoded_as_f32": ("return rmsnorm(as_f64(x, dtype), as_f64(g, dtype), eps)",
                                            "return rmsnorm(as_f64(x, dtype), as_f64(g, \"f32\"), eps)"),
    "rmsnorm_wrapper_gain_dropped": ("return rmsnorm(as_f64(x, dtype), as_f64(g, dtype), eps)",
                                     "return rmsnorm(as_f64(x, dtype), np.ones(np.shape(g)), eps)"),
}


def mutated_source(name: str) -> str:
    src = open(SRC).read()
    if name == "none":  # control: the real oracle through the same harness
        return src
    old, new = MUTANTS[name]
    if src.count(old) != 1:
        raise SystemExit(f"mutant {name}: the text to replace occurs {src.count(old)} times")
    return src.replace(old, new)


def main(argv):
    name = argv[1]
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import oracle  # the package; its ffn_oracle module is replaced below
    mod = types.ModuleType("oracle.ffn_oracle")
    mod.__file__ = SRC
    try:
        exec(compile(mutated_source(name), SRC + f" [{name}]", "exec"), mod.__dict__)
    except BaseException as e:  # a mutant that does not even load proves nothing
        print(f"mutant {name} failed to load: {e!r}")
        return 3
    sys.modules["oracle.ffn_oracle"] = mod
    oracle.ffn_oracle = mod
    import pytest
    return pytest.main(["-x", "-q", "-p", "no:cacheprovider", os.path.join(HERE, "test_oracle_pins.py")])


if __name__ == "__main__":
    sys.exit(main(sys.argv))
