"""Calls from several host threads at once, each thread on its own stream
with its own workspace and outputs, give the bits the same calls give one at
a time: the library keeps no mutable state shared between calls (its
one-time device queries aside), so it can be entered from any thread.  The
cases cover the decode kernels (bf16, Q8_0), the split-K prefill GEMMs with
their reductions, SPLIT and the fp32 path.
"""
from __future__ import annotations

import threading

import numpy as np
import pytest

from transformer_ffn_block_amd import inputs as I
from helpers import dev, host_bits

pytestmark = pytest.mark.gpu

REPS = 8
# (M, d, f, dtype, variant); the last two threads repeat the first two cases
CASES = [(16, 1024, 2816, "bf16", "auto"), (300, 512, 1408, "bf16", "auto"),
         (96, 512, 1024, "bf16", "split"), (8, 256, 704, "f32", "fused"),
         (8, 512, 1024, "q8", None), (16, 1024, 2816, "bf16", "auto"),
         (300, 512, 1408, "bf16", "auto")]
SEEDS = [7000, 7001, 7002, 7003, 7004, 7000, 7001]


def test_threads_on_their_own_streams_match_one_at_a_time(gpu_lib):
    from transformer_ffn_block_amd import ffn
    import torch
    print("threads on their own streams", len(CASES), "x", REPS, flush=True)
    blocks, ops = [], []
    for seed, (M, d, f, dt, v) in zip(SEEDS, CASES):
        if dt == "q8":
            q = I.make_q8_block(seed, M, d, f)
            mats = [(dev(m.qs, "i8"), dev(m.scales, "u16")) for m in (q.w_gate, q.w_up, q.w_down)]
            blocks.append(q)
            ops.append([dev(q.x), dev(q.g), *mats])
        else:
            b = I.make_block(seed, M, d, f, dt)
            blocks.append(b)
            ops.append([dev(a, b.dtype) for a in (b.x, b.g, b.w_gate, b.w_up, b.w_down)])

    def call(i, **kw):
        (M, d, f, dt, v), b, t = CASES[i], blocks[i], ops[i]
        if dt == "q8":
            return ffn.swiglu_block_q8(*t, b.eps, **kw)
        return ffn.swiglu_block(*t, b.eps, variant=v, **kw)

    want = []
    for i in range(len(CASES)):
        y = call(i)
        torch.cuda.synchronize()
        want.append(host_bits(y))
    # streams, workspaces and outputs made up front on this thread
    streams = [torch.cuda.Stream() for _ in CASES]

    def ws_bytes(M, d, f, dt, v):
        if dt == "q8":
            return gpu_lib.ffn_swiglu_block_q8_workspace_size(M, d, f)
        return ffn.workspace_size(ffn.FFN_BF16 if dt == "bf16" else ffn.FFN_F32, M, d, f, v)
    wss = [ffn.alloc_workspace(ws_bytes(*c)) for c in CASES]
    outs = [[torch.empty_like(t[0]) for _ in range(REPS)] for t in ops]
    torch.cuda.synchronize()
    errors = []
    start = threading.Barrier(len(CASES))

    def run(i):
        try:
            start.wait()
            with torch.cuda.stream(streams[i]):
                for r in range(REPS):
                    call(i, out=outs[i][r], workspace=wss[i], stream=streams[i])
        except Exception as e:  # reported on the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(CASES))]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a calling thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(len(CASES)):
        for r in range(REPS):
            assert np.array_equal(host_bits(outs[i][r]), want[i]), (CASES[i], r)
