"""bench.py's CPU leg without a GPU: it times the oracle on each kept
workload and reports the error of the "GPU" output handed to it.  Here the
outputs are made on the host: the oracle's own result rounded to bf16 (error
at most 2^-8 of the largest output, the unit roundoff of bf16) and the same with one entry
moved by a known amount (the reported error must see it)."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import ffn_oracle as O  # noqa: E402
from transformer_ffn_block_amd import inputs as I  # noqa: E402


def test_cpu_leg_reports_errors_and_rates():
    b = I.make_block(3, 4, 64, 96, "bf16")
    r = O.block_from_stored("bf16", b.x, b.g, b.w_gate, b.w_up, b.w_down, b.eps)
    good = I.f32_to_bf16_bits(r.astype(np.float32))
    bad = good.copy()
    # one entry off by 1/16 of the largest output
    k = np.unravel_index(np.argmax(np.abs(r)), r.shape)
    bad[k] = I.f32_to_bf16_bits(np.array([r[k] - np.max(np.abs(r)) / 16], np.float32))[0]
    xr, gr, eps, _ = I.make_rmsnorm(2, 8, 64, "bf16", outlier_frac=0.25)
    rn = O.rmsnorm_from_stored("bf16", xr, gr, eps)
    keep = {
        "good": dict(kind="block", inputs=(b, 4), gpu=good, work=bench.decode_bytes(4, 64, 96), unit="GB/s"),
        "bad": dict(kind="block", inputs=(b, 4), gpu=bad, work=bench.decode_bytes(4, 64, 96), unit="GB/s"),
        "norm": dict(kind="rmsnorm", inputs=(xr, gr, eps), gpu=I.f32_to_bf16_bits(rn.astype(np.float32)),
                     work=2 * 8 * 64 * 2, unit="GB/s"),
    }
    timings, errors = bench.cpu_oracle_leg(keep, budget_s=60)
    assert errors["good"]["max_norm"] <= 2.0 ** -8
    assert abs(errors["bad"]["max_norm"] - 1 / 16) < 2e-3
    assert errors["norm"]["elementwise_rel"] <= 2.0 ** -8
    for name in ("good", "bad"):
        assert timings[name]["1_thread"]["threads"] == 1
        assert timings[name]["1_thread"]["value"] > 0
        assert "all_threads" in timings[name]
    assert list(timings["norm"]) == ["1_thread", "note"]


def test_cpu_leg_extrapolates_the_prefill_from_sampled_rows():
    b = I.make_block(4, 300, 64, 96, "bf16")
    r = O.block_from_stored("bf16", b.x, b.g, b.w_gate, b.w_up, b.w_down, b.eps)
    keep = {"prefill": dict(kind="prefill", inputs=b, gpu=I.f32_to_bf16_bits(r.astype(np.float32)),
                            work=6.0 * 300 * 64 * 96, unit="TFLOP/s")}
    timings, errors = bench.cpu_oracle_leg(keep, budget_s=60)
    row = timings["prefill"]["1_thread"]
    assert "32 and 64 sampled rows" in row["sample"] and "extrapolated" in row["sample"]
    assert errors["prefill"]["max_norm"] <= 2.0 ** -8
