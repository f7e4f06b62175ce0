#!/usr/bin/env python3
"""Benchmark of the pre-norm SwiGLU FFN block on one MI355X.

Headline (`value`): the decode-shape block, M=16 tokens, d=4096, f=11008,
bf16, one whole C-ABI call per step, reported as algorithmic GB/s (weights
+ x + g + y bytes per call / time per call).  Weight sets are rotated over
4 copies (1.08 GB) so the 256 MB last-level cache cannot serve repeats.

The same JSON line also carries:
  roofline      - the dominant kernel (decode gate/up projection) against the
                  8 TB/s HBM peak; its average duration comes from HIP events
                  that the library records around each of its launches, on the
                  call's stream, during a second pass over the same timed
                  steps (the first pass, which gives `value`, is left
                  uninstrumented); `traffic` is the counter-measured HBM bytes
                  of that kernel from the committed profile, when the kernel
                  source is unchanged since the counters were taken;
  cpu_baseline  - the fp64 oracle on the host (1 BLAS thread) on the same
                  decode workload (extra also has an all-cores run);
  extra         - the other workloads: prefill block (M=8192, d=4096,
                  f=14336) fused and split gate/up, interleaved call by call,
                  in TFLOP/s; the standalone RMSNorm (16384 x 4096 bf16);
                  the Q8_0 and Q4_0 decode blocks (M=8, d=5120, f=17408);
                  decode at M=1 and 4; measured HBM read-only and copy
                  ceilings; torch matmul at the prefill shapes as
                  vendor-library context; one GPU's f/8 share of an 8-way
                  tensor-parallel block (decode, prefill, Q8, Q4); per-call
                  p10/median/p90 of the decode call and the GFX clock
                  sampled during decode and prefill calls (separate passes,
                  outside the timed region of `value`).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]
                       [--extras decode_m,persistent,ceilings,rmsnorm,q8,q4,prefill,tp8]
       (W untimed calls, continued until at least --min-warmup-s seconds, default 1,
        have passed; then K timed)
       python bench.py --profile-run   (decode steps plus one 512 MiB copy, for
                                        counter runs; prints nothing)
Progress goes to stderr; stdout gets exactly one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
DECODE = dict(seed=3, M=16, d=4096, f=11008)
PREFILL = dict(seed=4, M=8192, d=4096, f=14336)
RMS = dict(seed=2, rows=16384, d=4096)
Q8 = dict(seed=5, M=8, d=5120, f=17408)
Q4 = dict(seed=6, M=8, d=5120, f=17408)
ROTATE = 4
COPY_BYTES = 512 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_gateup_M16_hbm_traffic.txt")
KERNEL_SOURCE = os.path.join(ROOT, "transformer_ffn_block_amd", "csrc", "decode_stream.hip")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def to_dev(a, torch):
    import numpy as np
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(a).to("cuda")


def decode_bytes(M, d, f):
    """Algorithmic bytes of one decode block call: 3 weight matrices, x, y, g."""
    return 3 * f * d * 2 + 2 * M * d * 2 + d * 2


def gateup_bytes(M, d, f):
    """Algorithmic bytes of the fused norm + gate/up kernel: W_gate, W_up, x, g read; h written."""
    return 2 * f * d * 2 + M * d * 2 + d * 2 + M * f * 2


def time_calls(torch, fn, n):
    """Average ms per call of fn(i) over n calls, HIP events on torch's current stream."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for i in range(n):
        fn(i)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / n


MIN_WARMUP_S = 1.0  # --min-warmup-s


def warm_up(fn, n=20):
    """At least n calls of fn(i), continued until --min-warmup-s seconds have passed (clocks settle)."""
    t0 = time.perf_counter()
    i = 0
    while i < n or time.perf_counter() - t0 < MIN_WARMUP_S:
        fn(i)
        i += 1


def ratio(a, b):
    """a / b rounded, or None when the denominator was not measured."""
    return round(a / b, 4) if b else None


EXTRAS = ("decode_m", "persistent", "ceilings", "rmsnorm", "q8", "q4", "prefill", "tp8")


def per_call_us(torch, fn, n):
    """p10 / median / p90 of single-call durations (us), one event pair per call."""
    import numpy as np
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for i, (s, e) in enumerate(evs):
        s.record()
        fn(i)
        e.record()
    torch.cuda.synchronize()
    t = np.array([s.elapsed_time(e) * 1e3 for s, e in evs])
    return {"p10": round(float(np.percentile(t, 10)), 2), "p50": round(float(np.median(t)), 2),
            "p90": round(float(np.percentile(t, 90)), 2), "calls": n}


class ClockSampler:
    """Samples the GPU's current GFX clock (MHz) from a background thread while
    work runs; None when the system management library is unavailable.  Used
    outside the timed region of `value` (the sampler competes for the
    interpreter lock with the launching thread)."""

    def __init__(self, torch):
        self.h, self.samples, self._stop, self._thr = None, [], False, None
        try:
            import amdsmi
            self.smi = amdsmi
            amdsmi.amdsmi_init()
            pr = torch.cuda.get_device_properties(0)
            bdf = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}.0"
            hs = amdsmi.amdsmi_get_processor_handles()
            match = [h for h in hs if str(amdsmi.amdsmi_get_gpu_device_bdf(h)).lower() == bdf]
            self.h = match[0] if match else (hs[0] if len(hs) == 1 else None)
        except Exception as ex:  # no library, no permission, no match: report nothing
            log("clock sampling unavailable:", repr(ex))
            self.h = None

    def _read(self):
        return float(self.smi.amdsmi_get_clock_info(self.h, self.smi.AmdSmiClkType.GFX)["clk"])

    def __enter__(self):
        import threading
        self.samples, self._stop = [], False
        if self.h is None:
            return self

        def run():
            while not self._stop:
                try:
                    self.samples.append(self._read())
                except Exception:
                    return
                time.sleep(0.002)
        self._thr = threading.Thread(target=run, daemon=True)
        self._thr.start()
        return self

    def __exit__(self, *a):
        self._stop = True
        if self._thr is not None:
            self._thr.join()
        return False

    def summary(self):
        import numpy as np
        if not self.samples:
            return None
        t = np.array(self.samples)
        return {"gfx_mhz_median": round(float(np.median(t)), 0), "gfx_mhz_min": round(float(t.min()), 0),
                "gfx_mhz_max": round(float(t.max()), 0), "samples": int(t.size)}


def sha256(path):
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def read_traffic():
    """HBM bytes per launch of the decode gate/up kernel from the committed
    counter profile, or None when absent or taken on a different source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != sha256(KERNEL_SOURCE):
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(b, target_s=10.0, threads=1):
    """The oracle as it stands on the decode workload with `threads` BLAS
    threads (None: the library's default, all host cores), repeated until
    ~target_s of wall time has been spent (at least once)."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import ffn_oracle as O
    reps, t0 = 0, time.perf_counter()
    with threadpool_limits(limits=threads):
        used = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
        while True:
            O.block_from_stored("bf16", b.x, b.g, b.w_gate, b.w_up, b.w_down, b.eps)
            reps += 1
            if time.perf_counter() - t0 >= target_s:
                break
    dt = (time.perf_counter() - t0) / reps
    gbs = decode_bytes(b.M, b.d, b.f) / dt / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(used), "kind": "oracle",
            "sample": f"whole decode block M={b.M} d={b.d} f={b.f} (bf16 inputs decoded to fp64), "
                      f"{reps} call(s), {dt:.2f} s per call"}


def extras(torch, np, ffn, I, sets, x, g, b, ws, extra, clocks, want):
    best = copy_gbs = None  # ceilings (GB/s), measured when "ceilings" is selected
    M, d, f = b.M, b.d, b.f
    if "decode_m" in want:
        # decode at M = 1 and 4 (first rows of the same draw)
        for m in (1, 4):
            xm = x[:m].contiguous()
            ym = torch.empty_like(xm)

            def stepm(i, xm=xm, ym=ym):
                wg, wu, wd = sets[i % ROTATE]
                ffn.swiglu_block(xm, g, wg, wu, wd, b.eps, "auto", out=ym, workspace=ws)
            for i in range(20):
                stepm(i)
            msm = time_calls(torch, stepm, 200)
            extra[f"decode_M{m}"] = {"us": round(msm * 1e3, 2),
                                     "GBps": round(decode_bytes(m, d, f) / (msm * 1e-3) / 1e9, 1)}
            log(f"decode M={m}: {msm * 1e3:.2f} us/call")
    if "persistent" in want:
        # the single-dispatch (persistent) schedule at M = 16, interleaved with the
        # default two-launch schedule
        wsp = ffn.alloc_workspace(ffn.workspace_size(ffn.FFN_BF16, M, d, f, "persistent"))
        yp = torch.empty_like(x)

        def stepv(i, v):
            wg, wu, wd = sets[i % ROTATE]
            ffn.swiglu_block(x, g, wg, wu, wd, b.eps, v, out=yp, workspace=wsp if v == "persistent" else ws,
                             check_status=False)
        tv = {"auto": [], "persistent": []}
        for v in tv:
            for i in range(10):
                stepv(i, v)
        for _ in range(3):
            for v in tv:
                tv[v].append(time_calls(torch, lambda i, v=v: stepv(i, v), 50))
        torch.cuda.synchronize()
        if ffn.persistent_status(wsp, M, d, f) != 0:
            raise RuntimeError("persistent schedule: a work item gave up waiting")
        tp, ta = sorted(tv["persistent"])[1], sorted(tv["auto"])[1]
        extra["decode_M16_persistent"] = {"us": round(tp * 1e3, 2), "two_launch_us": round(ta * 1e3, 2),
                                          "persistent_over_two_launch": round(tp / ta, 3)}
        log("persistent schedule", extra["decode_M16_persistent"])
        del wsp, yp
        sets.clear()
        torch.cuda.empty_cache()

    if "ceilings" in want:
        # ------------------------------------------------------------ HBM ceilings
        nbytes = 4 << 30
        buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        buf.fill_(1)
        sink = torch.empty(16 * ffn.lib().ffn_probe_read_groups(32), dtype=torch.uint8, device="cuda")
        best, sweep = 0.0, {}
        for wpc in (4, 8, 12, 16, 32):
            for _ in range(2):
                ffn.probe_read(buf, sink, wpc)
            t = time_calls(torch, lambda i: ffn.probe_read(buf, sink, wpc), 5)
            sweep[wpc] = round(nbytes / (t * 1e-3) / 1e9, 1)
            best = max(best, sweep[wpc])
        half = nbytes // 2
        src, dst = buf[:half], buf[half:]
        ffn.probe_copy(src, dst)
        tc = time_calls(torch, lambda i: ffn.probe_copy(src, dst), 5)
        copy_gbs = 2 * half / (tc * 1e-3) / 1e9
        extra["hbm_read_ceiling_GBps"] = best
        extra["hbm_read_sweep_waves_per_cu"] = sweep
        extra["hbm_copy_ceiling_GBps"] = round(copy_gbs, 1)
        extra["decode_M16_frac_of_read_ceiling"] = ratio(extra["decode_M16_GBps"], best)
        log(f"HBM read ceiling {best:.0f} GB/s {sweep}, copy {copy_gbs:.0f} GB/s")
        del buf, sink, src, dst
        torch.cuda.empty_cache()

    if "rmsnorm" in want:
        # ---------------------------------------------------------------- RMSNorm
        log("generating rmsnorm inputs", RMS)
        xr, gr, eps, _ = I.make_rmsnorm(RMS["seed"], RMS["rows"], RMS["d"], "bf16")
        xs = [to_dev(xr, torch)]
        xs += [xs[0].clone() for _ in range(ROTATE - 1)]
        ys = [torch.empty_like(xs[0]) for _ in range(ROTATE)]
        gd = to_dev(gr, torch)
        for i in range(8):
            ffn.rmsnorm(xs[i % ROTATE], gd, eps, out=ys[i % ROTATE])
        tr = time_calls(torch, lambda i: ffn.rmsnorm(xs[i % ROTATE], gd, eps, out=ys[i % ROTATE]), 40)
        rbytes = 2 * RMS["rows"] * RMS["d"] * 2 + RMS["d"] * 2
        rgbs = rbytes / (tr * 1e-3) / 1e9
        extra["rmsnorm"] = {"us": round(tr * 1e3, 2), "GBps": round(rgbs, 1),
                            "frac_of_hbm_peak": round(rgbs / HBM_PEAK_GBS, 4),
                            "frac_of_read_ceiling": ratio(rgbs, best),
                            "frac_of_copy_ceiling": ratio(rgbs, copy_gbs)}
        log("rmsnorm", extra["rmsnorm"])
        del xs, ys
        torch.cuda.empty_cache()

    if "q8" in want:
        # ------------------------------------------------------------------- Q8_0
        log("generating q8 inputs", Q8)
        q = I.make_q8_block(Q8["seed"], Q8["M"], Q8["d"], Q8["f"])
        qx, qg = to_dev(q.x, torch), to_dev(q.g, torch)

        def qdev(m):
            return (torch.from_numpy(m.qs).to("cuda"), torch.from_numpy(m.scales.view(np.int16)).to("cuda"))
        q0 = [qdev(m) for m in (q.w_gate, q.w_up, q.w_down)]
        qsets = [q0] + [[(a.clone(), s.clone()) for a, s in q0] for _ in range(ROTATE - 1)]
        qws = ffn.alloc_workspace(ffn.lib().ffn_swiglu_block_q8_workspace_size(Q8["M"], Q8["d"], Q8["f"]))
        qy = torch.empty_like(qx)

        # calls marshalled once per weight set: the per-call Python work of
        # building the weight structs is comparable to the block's GPU time
        qcalls = [ffn.prepare_swiglu_block_quant("q8", qx, qg, *st, q.eps, qy, qws) for st in qsets]

        def qstep(i):
            qcalls[i % ROTATE]()
        warm_up(qstep)
        tq = time_calls(torch, qstep, 200)
        qbytes = 3 * (Q8["f"] * Q8["d"] + Q8["f"] * Q8["d"] // 32 * 2) + 2 * Q8["M"] * Q8["d"] * 2 + Q8["d"] * 2
        qgbs = qbytes / (tq * 1e-3) / 1e9
        extra["q8_decode"] = {"us": round(tq * 1e3, 2), "GBps": round(qgbs, 1),
                              "frac_of_read_ceiling": ratio(qgbs, best)}
        log("q8", extra["q8_decode"])
        del qcalls, qsets, q0
        torch.cuda.empty_cache()

    if "q4" in want:
        # ------------------------------------------------------------------- Q4_0
        log("generating q4 inputs", Q4)
        q4 = I.make_q4_block(Q4["seed"], Q4["M"], Q4["d"], Q4["f"])
        q4x, q4g = to_dev(q4.x, torch), to_dev(q4.g, torch)
        q40 = [qdev(m) for m in (q4.w_gate, q4.w_up, q4.w_down)]
        q4sets = [q40] + [[(a.clone(), s.clone()) for a, s in q40] for _ in range(ROTATE - 1)]
        q4ws = ffn.alloc_workspace(ffn.lib().ffn_swiglu_block_q4_workspace_size(Q4["M"], Q4["d"], Q4["f"]))
        q4y = torch.empty_like(q4x)

        q4calls = [ffn.prepare_swiglu_block_quant("q4", q4x, q4g, *st, q4.eps, q4y, q4ws) for st in q4sets]

        def q4step(i):
            q4calls[i % ROTATE]()
        warm_up(q4step)
        t4 = time_calls(torch, q4step, 200)
        ffn.timing_reset()
        ffn.timing_enable(True, 256)
        for i in range(40):
            q4step(i)
        k4 = ffn.timing_collect()
        ffn.timing_enable(False)
        fd = Q4["f"] * Q4["d"]
        q4_mat = fd // 2 + fd // 32 * 2          # nibbles + fp16 scales of one matrix
        q4bytes = 3 * q4_mat + 2 * Q4["M"] * Q4["d"] * 2 + Q4["d"] * 2
        q4gbs = q4bytes / (t4 * 1e-3) / 1e9
        gu4 = k4["q4_gateup"][1] / k4["q4_gateup"][0] * 1e3     # us per launch
        dn4 = k4["q4_down"][1] / k4["q4_down"][0] * 1e3
        gu4_bytes = 2 * q4_mat + Q4["M"] * Q4["d"] * 2 + Q4["M"] * Q4["f"] * 2
        dn4_bytes = q4_mat + Q4["M"] * Q4["f"] * 2 + 2 * Q4["M"] * Q4["d"] * 2
        extra["q4_decode"] = {"us": round(t4 * 1e3, 2), "GBps": round(q4gbs, 1),
                              "frac_of_read_ceiling": ratio(q4gbs, best),
                              "gateup_kernel_us": round(gu4, 2),
                              "gateup_kernel_GBps": round(gu4_bytes / (gu4 * 1e-6) / 1e9, 1),
                              "down_kernel_us": round(dn4, 2),
                              "down_kernel_GBps": round(dn4_bytes / (dn4 * 1e-6) / 1e9, 1)}
        log("q4", extra["q4_decode"])
        del q4calls, q4sets, q40
        torch.cuda.empty_cache()

    if "prefill" in want:
        # ---------------------------------------------------------------- prefill
        Mp, dp, fp = PREFILL["M"], PREFILL["d"], PREFILL["f"]
        log("generating prefill inputs", PREFILL)
        bp = I.make_block(PREFILL["seed"], Mp, dp, fp, "bf16")
        px, pg = to_dev(bp.x, torch), to_dev(bp.g, torch)
        pw = [[to_dev(a, torch) for a in (bp.w_gate, bp.w_up, bp.w_down)]]
        pw.append([t.clone() for t in pw[0]])
        pws = ffn.alloc_workspace(ffn.workspace_size(ffn.FFN_BF16, Mp, dp, fp, "split"))
        py = torch.empty_like(px)
        flops = 6.0 * Mp * dp * fp

        def pstep(i, variant):
            wg, wu, wd = pw[i % 2]
            ffn.swiglu_block(px, pg, wg, wu, wd, bp.eps, variant, out=py, workspace=pws)
        for i in range(4):
            pstep(i, "fused")
            pstep(i, "split")
        tf, ts = [], []
        for i in range(10):  # interleaved call by call
            tf.append(time_calls(torch, lambda j: pstep(i, "fused"), 1))
            ts.append(time_calls(torch, lambda j: pstep(i, "split"), 1))
        mf = float(np.median(tf))
        with clocks:  # the clock under MFMA load, in a separate ~0.3 s pass of the same calls
            for i in range(max(1, int(0.3 / (mf * 1e-3)))):
                pstep(i, "fused")
            torch.cuda.synchronize()
        extra["gpu_clock_during_prefill_calls"] = clocks.summary()
        ffn.timing_reset()
        ffn.timing_enable(True, 256)
        for i in range(4):
            pstep(i, "fused")
            pstep(i, "split")
        kp = ffn.timing_collect()
        ffn.timing_enable(False)
        mf, msp = float(np.median(tf)), float(np.median(ts))
        extra["prefill"] = {
            "fused_ms": round(mf, 3), "split_ms": round(msp, 3),
            "fused_TFLOPs": round(flops / (mf * 1e-3) / 1e12, 1),
            "split_TFLOPs": round(flops / (msp * 1e-3) / 1e12, 1),
            "fused_frac_of_bf16_peak": round(flops / (mf * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "split_over_fused_time": round(msp / mf, 3),
            "kernels_avg_ms_event_timed": {k: round(t / n, 4) for k, (n, t) in kp.items()}}
        gu_ms = kp["gemm_gateup_fused"][1] / kp["gemm_gateup_fused"][0]
        extra["prefill"]["gateup_fused_kernel_TFLOPs"] = round(4.0 * Mp * dp * fp / (gu_ms * 1e-3) / 1e12, 1)
        log("prefill", extra["prefill"])

        # vendor-library context at the same shapes (torch matmul -> hipBLASLt)
        wgu = torch.cat([pw[0][0], pw[0][1]], 0)
        hx = torch.empty((Mp, fp), dtype=torch.bfloat16, device="cuda").normal_()
        for _ in range(2):
            torch.nn.functional.linear(px, wgu)
            torch.nn.functional.linear(hx, pw[0][2])
        tgu = time_calls(torch, lambda i: torch.nn.functional.linear(px, wgu), 5)
        tdn = time_calls(torch, lambda i: torch.nn.functional.linear(hx, pw[0][2]), 5)
        extra["prefill_torch_matmul_context"] = {
            "gate_up_concat_ms": round(tgu, 3), "down_ms": round(tdn, 3),
            "gate_up_TFLOPs": round(4.0 * Mp * dp * fp / (tgu * 1e-3) / 1e12, 1),
            "down_TFLOPs": round(2.0 * Mp * dp * fp / (tdn * 1e-3) / 1e12, 1)}
        log("torch matmul context", extra["prefill_torch_matmul_context"])
        del pw, hx, wgu
        torch.cuda.empty_cache()

    if "tp8" in want:
        # ------------------------------------- one GPU's share at tensor parallel 8
        tp8_shards(torch, np, ffn, I, extra, best)


def tp8_shards(torch, np, ffn, I, extra, read_ceiling):
    """The block on one GPU's f/8 slice (the kernels a rank of an 8-way
    tensor-parallel split runs; the all-reduce of the partial sums is not
    built).  Decode and Q8 rotate enough weight copies to exceed the 256 MB
    last-level cache."""
    out = {}
    wl = I.WORKLOADS["decode_tp8_shard"]
    M, d, f = wl["M"], wl["d"], wl["f"]
    bb = I.make_block(wl["seed"], M, d, f, "bf16")
    x, g = to_dev(bb.x, torch), to_dev(bb.g, torch)
    w0 = [to_dev(a, torch) for a in (bb.w_gate, bb.w_up, bb.w_down)]
    nrot = 10
    sets = [w0] + [[t.clone() for t in w0] for _ in range(nrot - 1)]
    ws = ffn.alloc_workspace(ffn.workspace_size(ffn.FFN_BF16, M, d, f, "auto"))
    y = torch.empty_like(x)

    def dstep(i):
        wg, wu, wd = sets[i % nrot]
        ffn.swiglu_block(x, g, wg, wu, wd, bb.eps, "auto", out=y, workspace=ws)
    for i in range(50):
        dstep(i)
    t = time_calls(torch, dstep, 500)
    gbs = decode_bytes(M, d, f) / (t * 1e-3) / 1e9
    out["decode_M16_f1376"] = {"us": round(t * 1e3, 2), "GBps": round(gbs, 1),
                               "frac_of_read_ceiling": ratio(gbs, read_ceiling)}
    del sets, w0
    torch.cuda.empty_cache()

    wl = I.WORKLOADS["prefill_tp8_shard"]
    M, d, f = wl["M"], wl["d"], wl["f"]
    bb = I.make_block(wl["seed"], M, d, f, "bf16")
    x, g = to_dev(bb.x, torch), to_dev(bb.g, torch)
    w = [to_dev(a, torch) for a in (bb.w_gate, bb.w_up, bb.w_down)]
    ws = ffn.alloc_workspace(ffn.workspace_size(ffn.FFN_BF16, M, d, f, "fused"))
    y = torch.empty_like(x)
    for _ in range(3):
        ffn.swiglu_block(x, g, *w, bb.eps, "fused", out=y, workspace=ws)
    tp = time_calls(torch, lambda i: ffn.swiglu_block(x, g, *w, bb.eps, "fused", out=y, workspace=ws), 10)
    tf = 6.0 * M * d * f / (tp * 1e-3) / 1e12
    out["prefill_M8192_f1792_fused"] = {"ms": round(tp, 3), "TFLOPs": round(tf, 1),
                                        "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)}
    del w, x, y, ws
    torch.cuda.empty_cache()

    wl = I.WORKLOADS["q8_tp8_shard"]
    M, d, f = wl["M"], wl["d"], wl["f"]
    q = I.make_q8_block(wl["seed"], M, d, f)
    qx, qg = to_dev(q.x, torch), to_dev(q.g, torch)
    q0 = [(torch.from_numpy(m.qs).to("cuda"), torch.from_numpy(m.scales.view(np.int16)).to("cuda"))
          for m in (q.w_gate, q.w_up, q.w_down)]
    qsets = [q0] + [[(a.clone(), s.clone()) for a, s in q0] for _ in range(nrot - 1)]
    qws = ffn.alloc_workspace(ffn.lib().ffn_swiglu_block_q8_workspace_size(M, d, f))
    qy = torch.empty_like(qx)

    qcalls = [ffn.prepare_swiglu_block_quant("q8", qx, qg, *st, q.eps, qy, qws) for st in qsets]

    def qstep(i):
        qcalls[i % nrot]()
    warm_up(qstep, 50)
    tq = time_calls(torch, qstep, 500)
    qbytes = 3 * (f * d + f * d // 32 * 2) + 2 * M * d * 2 + d * 2
    qgbs = qbytes / (tq * 1e-3) / 1e9
    out["q8_M8_f2176"] = {"us": round(tq * 1e3, 2), "GBps": round(qgbs, 1),
                          "frac_of_read_ceiling": ratio(qgbs, read_ceiling)}
    del qcalls, qsets, q0
    torch.cuda.empty_cache()

    wl = I.WORKLOADS["q4_tp8_shard"]
    M, d, f = wl["M"], wl["d"], wl["f"]
    q4 = I.make_q4_block(wl["seed"], M, d, f)
    qx, qg = to_dev(q4.x, torch), to_dev(q4.g, torch)
    q0 = [(torch.from_numpy(m.qs).to("cuda"), torch.from_numpy(m.scales.view(np.int16)).to("cuda"))
          for m in (q4.w_gate, q4.w_up, q4.w_down)]
    qsets = [q0] + [[(a.clone(), s.clone()) for a, s in q0] for _ in range(2 * nrot - 1)]
    qws = ffn.alloc_workspace(ffn.lib().ffn_swiglu_block_q4_workspace_size(M, d, f))
    qy = torch.empty_like(qx)

    q4calls = [ffn.prepare_swiglu_block_quant("q4", qx, qg, *st, q4.eps, qy, qws) for st in qsets]

    def q4step(i):
        q4calls[i % (2 * nrot)]()
    warm_up(q4step, 50)
    tq = time_calls(torch, q4step, 500)
    qbytes = 3 * (f * d // 2 + f * d // 32 * 2) + 2 * M * d * 2 + d * 2
    qgbs = qbytes / (tq * 1e-3) / 1e9
    out["q4_M8_f2176"] = {"us": round(tq * 1e3, 2), "GBps": round(qgbs, 1),
                          "frac_of_read_ceiling": ratio(qgbs, read_ceiling)}
    del q4calls, qsets, q0
    torch.cuda.empty_cache()
    extra["tp8_shard"] = out
    log("tp8 shard", out)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-extra", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--extras", default="all",
                    help="comma-separated subset of the secondary workloads: " + ",".join(EXTRAS))
    ap.add_argument("--min-warmup-s", type=float, default=1.0,
                    help="continue the warm-up until this many seconds have passed (0: W calls only)")
    ap.add_argument("--profile-run", action="store_true",
                    help="decode steps plus one 512 MiB copy (counter calibration); no output")
    args = ap.parse_args()
    global MIN_WARMUP_S
    MIN_WARMUP_S = args.min_warmup_s
    want = set(EXTRAS) if args.extras == "all" else set(args.extras.split(","))
    if not want <= set(EXTRAS):
        print(f"unknown --extras {sorted(want - set(EXTRAS))}; choose from {','.join(EXTRAS)}", file=sys.stderr)
        return 2
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the FFN block here is a single-GPU library "
              "(multi-GPU sharding is a design note, not built); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from transformer_ffn_block_amd import ffn, inputs as I

    ffn.lib()
    torch.cuda.init()
    dev_name = torch.cuda.get_device_properties(0).name
    log("device", dev_name)

    # ------------------------------------------------------------------ decode
    M, d, f = DECODE["M"], DECODE["d"], DECODE["f"]
    log("generating decode inputs", DECODE)
    b = I.make_block(DECODE["seed"], M, d, f, "bf16")
    x, g = to_dev(b.x, torch), to_dev(b.g, torch)
    w0 = [to_dev(a, torch) for a in (b.w_gate, b.w_up, b.w_down)]
    sets = [w0] + [[t.clone() for t in w0] for _ in range(ROTATE - 1)]
    ws = ffn.alloc_workspace(ffn.workspace_size(ffn.FFN_BF16, M, d, f, "auto"))
    y = torch.empty_like(x)

    def step(i):
        wg, wu, wd = sets[i % ROTATE]
        ffn.swiglu_block(x, g, wg, wu, wd, b.eps, "auto", out=y, workspace=ws)

    # warm-up: W calls, continued until at least one second has passed
    t0 = time.perf_counter()
    i = 0
    while i < args.warmup or time.perf_counter() - t0 < args.min_warmup_s:
        step(i)
        i += 1
        if i % 256 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    log(f"warm-up: {i} calls in {time.perf_counter() - t0:.2f} s")
    ms = time_calls(torch, step, args.steps)              # the timed region
    value = decode_bytes(M, d, f) / (ms * 1e-3) / 1e9
    log(f"decode M={M}: {ms * 1e3:.2f} us/call, {value:.1f} GB/s")

    if args.profile_run:
        half = COPY_BYTES
        buf = torch.empty(2 * half, dtype=torch.uint8, device="cuda")
        buf.fill_(1)
        ffn.probe_copy(buf[:half], buf[half:])
        torch.cuda.synchronize()
        return 0

    # per-kernel durations: the same steps again, each launch bracketed by events
    ffn.timing_reset()
    ffn.timing_enable(True, max_launches=4 * args.steps + 16)
    ms_instr = time_calls(torch, step, args.steps)
    kt = ffn.timing_collect()
    ffn.timing_enable(False)
    n_gu, t_gu = kt["decode_gateup"]
    gu_us = t_gu / n_gu * 1e3
    gu_gbs = gateup_bytes(M, d, f) / (gu_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": "decode_gateup (fused RMSNorm + gate/up + SwiGLU)",
                "achieved": round(gu_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gu_gbs / HBM_PEAK_GBS, 4), "traffic": read_traffic(),
                "avg_launch_us": round(gu_us, 2), "bytes_per_launch": gateup_bytes(M, d, f)}
    kernels = {k: {"launches": n, "avg_us": round(t / n * 1e3, 2)} for k, (n, t) in kt.items()}
    log(f"kernels {kernels}; instrumented pass {ms_instr * 1e3:.2f} us/call")

    pct = per_call_us(torch, step, args.steps)
    # the clock under this load, over ~0.3 s of the same calls (the driver's
    # clock readout refreshes every few ms; a shorter window reads idle)
    clocks = ClockSampler(torch)
    with clocks:
        for i in range(max(1, int(0.3 / (ms * 1e-3)))):
            step(i)
        torch.cuda.synchronize()
    log(f"decode per-call us {pct}; clock {clocks.summary()}")

    extra = {"decode_M16_GBps": round(value, 1), "decode_M16_us": round(ms * 1e3, 2),
             "decode_kernels_event_timed": kernels,
             "decode_M16_instrumented_us": round(ms_instr * 1e3, 2),
             "decode_M16_call_us_percentiles": pct,
             "gpu_clock_during_decode_calls": clocks.summary()}
    if not args.no_extra:
        extras(torch, np, ffn, I, sets, x, g, b, ws, extra, clocks, want)

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle on the decode workload")
        cpu = cpu_baseline(b)
        log("cpu", cpu)
        extra["cpu_oracle_all_cores"] = cpu_baseline(b, target_s=5.0, threads=None)
        log("cpu (all cores)", extra["cpu_oracle_all_cores"])

    line = {
        "metric": "FFN block: decode GB/s & prefill TFLOP/s on 1 GPU, % of HBM/MFMA peak",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights)",
        "config": {"workload": "decode block M=16 d=4096 f=11008 bf16", "M": M, "d": d, "f": f,
                   "rotated_weight_sets": ROTATE, "device": dev_name},
        "roofline": roofline, "cpu_baseline": cpu, "extra": extra,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
