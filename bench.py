#!/usr/bin/env python3
"""Benchmark of the pre-norm SwiGLU FFN block on one MI355X.

Headline (`value`): the decode-shape block, M=16 tokens, d=4096, f=11008,
bf16, one whole C-ABI call per step, reported as algorithmic GB/s (weights
+ x + g + y bytes per call / time per call).  Weight sets are rotated over
4 copies (1.08 GB) so the 256 MB last-level cache cannot serve repeats.

The same JSON line also carries:
  roofline      - the dominant kernel (decode gate/up projection) against the
                  8 TB/s HBM peak; its average duration comes from HIP events
                  the library binds to each of its kernel dispatches
                  (hipExtLaunchKernel: the kernel's own begin/end, as a
                  profiler's kernel trace reports it), recorded on the call's
                  stream during a second pass over the same timed steps (the
                  first pass, which gives `value`, is left uninstrumented);
                  `traffic` is the counter-measured HBM bytes of that kernel
                  from the committed profile, when the kernel source is
                  unchanged since the counters were taken;
  cpu_baseline  - the fp64 oracle on the host (1 thread) on the same decode
                  workload;
  extra         - the other workloads: prefill block (M=8192, d=4096,
                  f=14336) fused and split gate/up, interleaved call by call,
                  in TFLOP/s against both the 2.5 PFLOP/s spec and an
                  MFMA-loop peak measured in this run; the standalone RMSNorm
                  (16384 x 4096 bf16); the Q8_0 and Q4_0 decode blocks (M=8,
                  d=5120, f=17408); decode at M=1 and 4; measured HBM
                  read-only and read+write ceilings (swept probes); torch
                  matmul at the prefill shapes as vendor-library context; one
                  GPU's f/8 share of an 8-way tensor-parallel block; per-call
                  p10/median/p90 of the decode call; clocks; and the CPU leg:
                  the oracle timed on every workload (1 thread and all host
                  threads; the prefill from sampled rows, extrapolated) with
                  each workload's error of this run's GPU output against it.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]
                       [--extras decode_m,persistent,ceilings,rmsnorm,q8,q4,prefill,mid,tiny,tp8]
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
FLOP_PER_CU_CLK = 4096          # dense bf16 MFMA flop per compute unit per clock
DECODE = dict(seed=3, M=16, d=4096, f=11008)
PREFILL = dict(seed=4, M=8192, d=4096, f=14336)
RMS = dict(seed=2, rows=16384, d=4096)
Q8 = dict(seed=5, M=8, d=5120, f=17408)
Q4 = dict(seed=6, M=8, d=5120, f=17408)
TINY = dict(seed=1, M=8, d=256, f=704)
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


def to_host(t):
    """Device tensor -> stored-format numpy array (bf16 as uint16 bits)."""
    import numpy as np
    import torch
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def decode_bytes(M, d, f):
    """Algorithmic bytes of one decode block call: 3 weight matrices, x, y, g."""
    return 3 * f * d * 2 + 2 * M * d * 2 + d * 2


def gateup_bytes(M, d, f):
    """Algorithmic bytes of the fused norm + gate/up kernel: W_gate, W_up, x, g read; h written."""
    return 2 * f * d * 2 + M * d * 2 + d * 2 + M * f * 2


def down_bytes(M, d, f):
    """Algorithmic bytes of the decode down kernel: W_down, h, x read; y written."""
    return d * f * 2 + M * f * 2 + 2 * M * d * 2


def q8_matrix_bytes(N, K):
    return N * K + N * K // 32 * 2


def q4_matrix_bytes(N, K):
    return N * K // 2 + N * K // 32 * 2


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


def kernel_times(ffn, fn, n):
    """{kernel: avg us per launch} over n calls of fn(i), from the events the
    library binds to each dispatch (a separate, instrumented pass)."""
    ffn.timing_reset()
    ffn.timing_enable(True, max_launches=8 * n + 16)
    for i in range(n):
        fn(i)
    kt = ffn.timing_collect()
    ffn.timing_enable(False)
    return {k: round(t / c * 1e3, 2) for k, (c, t) in kt.items()}


EXTRAS = ("decode_m", "persistent", "ceilings", "rmsnorm", "q8", "q4", "prefill", "mid", "tiny", "tp8")


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
    """Samples the GFX clock (MHz) that the system management library reports,
    from a background thread while work runs; None when the library is
    unavailable.  Used outside the timed region of `value` (the sampler
    competes for the interpreter lock with the launching thread).  The
    library's figure is the firmware's current setting; the clock the
    matrix cores actually hold is reported separately, from the MFMA-loop
    probe's rate."""

    def __init__(self, torch):
        self.h, self.samples, self._stop, self._thr, self.smi = None, [], False, None, None
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

    def average_gfxclk(self):
        """The firmware's running average GFX clock (MHz) from the GPU metrics table, or None."""
        if self.h is None:
            return None
        try:
            m = self.smi.amdsmi_get_gpu_metrics_info(self.h)
            v = m.get("average_gfxclk_frequency")
            return None if v in (None, "N/A", 0xFFFF) else float(v)
        except Exception:
            return None

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
                "gfx_mhz_max": round(float(t.max()), 0), "samples": int(t.size),
                "firmware_average_gfxclk_mhz": self.average_gfxclk(),
                "source": "system management library (firmware setting)"}

    def close(self):
        if self.smi is not None:
            try:
                self.smi.amdsmi_shut_down()
            except Exception:
                pass
            self.smi, self.h = None, None


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


def software_versions(torch):
    v = {"torch": torch.__version__, "torch_hip": getattr(torch.version, "hip", None)}
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        try:
            with open(path) as fh:
                v["rocm"] = fh.read().strip()
            break
        except OSError:
            continue
    return v


# ----------------------------------------------------------------------------
# GPU measurements
# ----------------------------------------------------------------------------
def ceilings(torch, ffn, extra, clocks):
    """Read-only and read+write HBM ceilings (swept probes) and the MFMA-loop
    peak at the clock the chip holds under that load."""
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
    copy_best, csweep = 0.0, {}
    for gpc in (0, 2, 4, 8, 16):
        for nt in (False, True):
            ffn.probe_copy(src, dst, gpc, nt)
            tc = time_calls(torch, lambda i: ffn.probe_copy(src, dst, gpc, nt), 5)
            gbs = 2 * half / (tc * 1e-3) / 1e9
            key = ("chunked_16KiB" if gpc == 0 else f"stride_{gpc}_per_cu") + ("_nt_stores" if nt else "")
            csweep[key] = round(gbs, 1)
            copy_best = max(copy_best, gbs)
    extra["hbm_read_ceiling_GBps"] = best
    extra["hbm_read_sweep_waves_per_cu"] = sweep
    extra["hbm_copy_ceiling_GBps"] = round(copy_best, 1)
    extra["hbm_copy_sweep"] = csweep
    log(f"HBM read ceiling {best:.0f} GB/s {sweep}, copy {copy_best:.0f} GB/s {csweep}")
    del buf, sink, src, dst
    torch.cuda.empty_cache()

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    msink = torch.empty(4 * 256 * ffn.lib().ffn_probe_mfma_groups(32), dtype=torch.uint8, device="cuda")
    iters = 20000
    msweep, mbest = {}, 0.0
    with clocks:
        for wpc in (8, 16):
            flop = ffn.probe_mfma(iters, wpc, msink)
            ffn.probe_mfma(iters, wpc, msink)
            t = time_calls(torch, lambda i: ffn.probe_mfma(iters, wpc, msink), 5)
            tf = flop / (t * 1e-3) / 1e12
            msweep[wpc] = round(tf, 1)
            mbest = max(mbest, tf)
    extra["mfma_loop_peak"] = {
        "TFLOPs": round(mbest, 1), "sweep_waves_per_cu": msweep,
        "frac_of_spec_peak": round(mbest / BF16_PEAK_TFLOPS, 4),
        "implied_clock_GHz": round(mbest * 1e12 / (cus * FLOP_PER_CU_CLK) / 1e9, 3),
        "what": "v_mfma_f32_16x16x32_bf16 chains from registers; clock = rate / (CUs x 4096 flop/clk)",
        "smi_clock_during": clocks.summary()}
    log("mfma loop", extra["mfma_loop_peak"])
    del msink
    return best, copy_best, mbest


def same_size_reads(torch, ffn, sizes):
    """The read probe over exactly as many bytes as a kernel streams, kernel
    duration from the dispatch events (as for the decode kernels), best over
    waves per CU; four rotated buffers, so the memory-side cache cannot serve
    them.  A launch this short pays its start-up and drain, which the 4 GiB
    read ceiling amortises: this is what one launch reading that many bytes
    achieves, the context for a kernel's fraction of the ceiling."""
    out = {}
    sink = torch.empty(16 * ffn.lib().ffn_probe_read_groups(32), dtype=torch.uint8, device="cuda")
    for name, n in sizes.items():
        n16 = n // 16 * 16
        bufs = [torch.empty(n16, dtype=torch.uint8, device="cuda") for _ in range(ROTATE)]
        for bb in bufs:
            bb.fill_(1)
        best = None
        for wpc in (4, 8, 12, 16, 32):
            def fn(i, wpc=wpc):
                ffn.probe_read(bufs[i % ROTATE], sink, wpc)
            for i in range(8):
                fn(i)
            us = kernel_times(ffn, fn, 40)["probe_read"]
            if best is None or us < best[0]:
                best = (us, wpc)
        out[name] = {"bytes": n16, "us": best[0], "GBps": round(n16 / (best[0] * 1e-6) / 1e9, 1),
                     "waves_per_cu": best[1]}
        del bufs
    del sink
    torch.cuda.empty_cache()
    return out


def extras(torch, np, ffn, I, sets, x, g, b, ws, extra, clocks, want, keep):
    best = copy_gbs = mfma_peak = None  # ceilings, measured when "ceilings" is selected
    M, d, f = b.M, b.d, b.f
    if "decode_m" in want:
        # decode at M = 1 and 4 (first rows of the same draw)
        for m in (1, 4):
            xm = x[:m].contiguous()
            ym = torch.empty_like(xm)

            def stepm(i, xm=xm, ym=ym):
                wg, wu, wd = sets[i % ROTATE]
                ffn.swiglu_block(xm, g, wg, wu, wd, b.eps, "auto", out=ym, workspace=ws)
            warm_up(stepm)
            msm = time_calls(torch, stepm, 200)
            extra[f"decode_M{m}"] = {"us": round(msm * 1e3, 2),
                                     "GBps": round(decode_bytes(m, d, f) / (msm * 1e-3) / 1e9, 1)}
            keep[f"C3 decode M={m}"] = dict(kind="block", inputs=(b, m), gpu=to_host(ym),
                                            work=decode_bytes(m, d, f), unit="GB/s")
            log(f"decode M={m}: {msm * 1e3:.2f} us/call")
        # M = 16 calls replayed from a HIP graph (40 captured calls over the
        # rotated weight sets): the same kernels without per-call host work
        yg = torch.empty_like(x)

        def stepg(i):
            wg, wu, wd = sets[i % ROTATE]
            ffn.swiglu_block(x, g, wg, wu, wd, b.eps, "auto", out=yg, workspace=ws)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(ROTATE):
                stepg(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        ncap = 40
        with torch.cuda.graph(graph):
            for i in range(ncap):
                stepg(i)
        for _ in range(5):
            graph.replay()
        tg = time_calls(torch, lambda i: graph.replay(), 10) / ncap
        extra["decode_M16_hip_graph"] = {"us": round(tg * 1e3, 2),
                                         "GBps": round(decode_bytes(M, d, f) / (tg * 1e-3) / 1e9, 1),
                                         "calls_per_graph": ncap}
        log(f"decode M=16 from a HIP graph: {tg * 1e3:.2f} us/call")
        del graph
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
        best, copy_gbs, mfma_peak = ceilings(torch, ffn, extra, clocks)
        extra["decode_M16_frac_of_read_ceiling"] = ratio(extra["decode_M16_GBps"], best)
        for m in (1, 4):
            if f"decode_M{m}" in extra:
                extra[f"decode_M{m}"]["frac_of_read_ceiling"] = ratio(extra[f"decode_M{m}"]["GBps"], best)
        kt = extra["decode_kernels_event_timed"]
        sizes = {"decode_gateup": gateup_bytes(M, d, f), "decode_down": down_bytes(M, d, f)}
        same = same_size_reads(torch, ffn, sizes)
        extra["hbm_read_same_size_as_decode_kernels"] = same
        log("read probe at the decode kernels' sizes", same)
        for name, nbytes in sizes.items():
            if name in kt:
                gbs = nbytes / (kt[name]["avg_us"] * 1e-6) / 1e9
                kt[name].update(GBps=round(gbs, 1), frac_of_read_ceiling=ratio(gbs, best),
                                frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4),
                                frac_of_same_size_read=round(same[name]["us"] / kt[name]["avg_us"], 4))

    if "rmsnorm" in want:
        # ---------------------------------------------------------------- RMSNorm
        log("generating rmsnorm inputs", RMS)
        xr, gr, eps, _ = I.make_rmsnorm(RMS["seed"], RMS["rows"], RMS["d"], "bf16")
        xs = [to_dev(xr, torch)]
        xs += [xs[0].clone() for _ in range(ROTATE - 1)]
        ys = [torch.empty_like(xs[0]) for _ in range(ROTATE)]
        gd = to_dev(gr, torch)

        def rstep(i):
            ffn.rmsnorm(xs[i % ROTATE], gd, eps, out=ys[i % ROTATE])
        warm_up(rstep)
        tr = time_calls(torch, rstep, 40)
        rbytes = 2 * RMS["rows"] * RMS["d"] * 2 + RMS["d"] * 2
        rgbs = rbytes / (tr * 1e-3) / 1e9
        extra["rmsnorm"] = {"us": round(tr * 1e3, 2), "GBps": round(rgbs, 1),
                            "frac_of_hbm_peak": round(rgbs / HBM_PEAK_GBS, 4),
                            "frac_of_read_ceiling": ratio(rgbs, best),
                            "frac_of_copy_ceiling": ratio(rgbs, copy_gbs)}
        keep["C2 rmsnorm 16384x4096"] = dict(kind="rmsnorm", inputs=(xr, gr, eps), gpu=to_host(ys[0]),
                                             work=rbytes, unit="GB/s")
        log("rmsnorm", extra["rmsnorm"])
        del xs, ys
        torch.cuda.empty_cache()

    def qdev(m):
        return (torch.from_numpy(m.qs).to("cuda"), torch.from_numpy(m.scales.view(np.int16)).to("cuda"))

    for kind, cfg, make, mbytes in (("q8", Q8, I.make_q8_block, q8_matrix_bytes),
                                    ("q4", Q4, I.make_q4_block, q4_matrix_bytes)):
        if kind not in want:
            continue
        log(f"generating {kind} inputs", cfg)
        Mq, dq, fq = cfg["M"], cfg["d"], cfg["f"]
        q = make(cfg["seed"], Mq, dq, fq)
        qx, qg = to_dev(q.x, torch), to_dev(q.g, torch)
        q0 = [qdev(m) for m in (q.w_gate, q.w_up, q.w_down)]
        qsets = [q0] + [[(a.clone(), s.clone()) for a, s in q0] for _ in range(ROTATE - 1)]
        qws = ffn.alloc_workspace(getattr(ffn.lib(), f"ffn_swiglu_block_{kind}_workspace_size")(Mq, dq, fq))
        qy = torch.empty_like(qx)
        # calls marshalled once per weight set: the per-call Python work of
        # building the weight structs is comparable to the block's GPU time
        qcalls = [ffn.prepare_swiglu_block_quant(kind, qx, qg, *st, q.eps, qy, qws) for st in qsets]

        def qstep(i, qcalls=qcalls):
            qcalls[i % ROTATE]()
        warm_up(qstep)
        tq = time_calls(torch, qstep, 200)
        kq = kernel_times(ffn, qstep, 40)
        mat = mbytes(fq, dq)
        qbytes = 3 * mat + 2 * Mq * dq * 2 + dq * 2
        qgbs = qbytes / (tq * 1e-3) / 1e9
        res = {"us": round(tq * 1e3, 2), "GBps": round(qgbs, 1), "frac_of_read_ceiling": ratio(qgbs, best),
               "kernels_us_event_timed": kq}
        gu, dn = kq.get(f"{kind}_gateup"), kq.get(f"{kind}_down")
        gub = 2 * mat + Mq * dq * 2 + Mq * fq * 2
        dnb = mat + Mq * fq * 2 + 2 * Mq * dq * 2
        if gu:
            res["gateup_kernel_GBps"] = round(gub / (gu * 1e-6) / 1e9, 1)
        if dn:
            res["down_kernel_GBps"] = round(dnb / (dn * 1e-6) / 1e9, 1)
        extra[f"{kind}_decode"] = res
        del qcalls, qsets, q0
        torch.cuda.empty_cache()
        if best and gu and dn:
            # the read probe over each kernel's byte count, as for bf16 decode
            same = same_size_reads(torch, ffn, {"gateup": gub, "down": dnb})
            res["read_probe_same_size_us"] = {k: v["us"] for k, v in same.items()}
            res["gateup_frac_of_same_size_read"] = round(same["gateup"]["us"] / gu, 4)
            res["down_frac_of_same_size_read"] = round(same["down"]["us"] / dn, 4)
        keep[f"{'C5 ' if kind == 'q8' else ''}{kind} decode M={Mq}"] = dict(
            kind=kind, inputs=q, gpu=to_host(qy), work=qbytes, unit="GB/s")
        log(kind, res)

    if "mid" in want:
        # ------------------------------------------ batches between decode and prefill
        wl = I.WORKLOADS["mid_batch"]
        Ms, dm, fm = wl["M"], wl["d"], wl["f"]
        log("generating mid-batch inputs", wl)
        bm = I.make_block(wl["seed"], max(Ms), dm, fm, "bf16")
        mx_all, mg = to_dev(bm.x, torch), to_dev(bm.g, torch)
        mw = [[to_dev(a, torch) for a in (bm.w_gate, bm.w_up, bm.w_down)]]
        nrot_m = max(2, int(600e6 // (3 * fm * dm * 2)) + 1)  # past the memory-side cache
        mw += [[t.clone() for t in mw[0]] for _ in range(nrot_m - 1)]
        res = {}
        for Mm in Ms:
            mx = mx_all[:Mm].contiguous()
            my = torch.empty_like(mx)
            mws = ffn.alloc_workspace(ffn.workspace_size(ffn.FFN_BF16, Mm, dm, fm, "auto"))

            def mstep(i, mx=mx, my=my, mws=mws):
                wg, wu, wd = mw[i % nrot_m]
                ffn.swiglu_block(mx, mg, wg, wu, wd, bm.eps, "auto", out=my, workspace=mws)
            warm_up(mstep)
            t = time_calls(torch, mstep, 40)
            km = kernel_times(ffn, mstep, 8)
            res[f"M={Mm}"] = {"us": round(t * 1e3, 2),
                              "weights_GBps": round(3 * fm * dm * 2 / (t * 1e-3) / 1e9, 1),
                              "TFLOPs": round(6.0 * Mm * dm * fm / (t * 1e-3) / 1e12, 1),
                              "kernels_us_event_timed": km}
            del mws
        res["note"] = ("AUTO at d=4096, f=11008 (the decode block's weights); GEMMs whose tiles "
                       "number fewer than the CUs are split over K (128-token tiles up to 128 "
                       "tokens), and past a whole round of tiles only the last columns split "
                       "(768 tokens: 258 gate/up tiles)")
        extra["mid_batch"] = res
        log("mid batch", res)
        del mw, mx_all
        torch.cuda.empty_cache()

    if "tiny" in want:
        # ------------------------------------------------------- tiny fp32 block
        tb = I.make_block(TINY["seed"], TINY["M"], TINY["d"], TINY["f"], "f32")
        tdev = [to_dev(a, torch) for a in (tb.x, tb.g, tb.w_gate, tb.w_up, tb.w_down)]
        ty = torch.empty_like(tdev[0])
        tws = ffn.alloc_workspace(ffn.workspace_size(ffn.FFN_F32, TINY["M"], TINY["d"], TINY["f"], "auto"))
        for i in range(20):
            ffn.swiglu_block(*tdev, tb.eps, "auto", out=ty, workspace=tws)
        tt = time_calls(torch, lambda i: ffn.swiglu_block(*tdev, tb.eps, "auto", out=ty, workspace=tws), 200)
        tflop = 6 * TINY["M"] * TINY["d"] * TINY["f"]
        extra["tiny_f32"] = {"us": round(tt * 1e3, 2), "GFLOPs": round(tflop / (tt * 1e-3) / 1e9, 2),
                             "note": "launch-bound; parity case, no roofline bar"}
        keep["C1 tiny f32 M=8"] = dict(kind="block", inputs=(tb, TINY["M"]), gpu=to_host(ty), work=tflop,
                                       unit="GFLOP/s")

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
        with clocks:  # the firmware clock under MFMA load, in a separate ~0.3 s pass of the same calls
            for i in range(max(1, int(0.3 / (mf * 1e-3)))):
                pstep(i, "fused")
            torch.cuda.synchronize()
        extra["gpu_clock_during_prefill_calls"] = clocks.summary()
        kp_f = kernel_times(ffn, lambda i: pstep(i, "fused"), 4)
        kp_s = kernel_times(ffn, lambda i: pstep(i, "split"), 4)
        mf, msp = float(np.median(tf)), float(np.median(ts))
        tff = flops / (mf * 1e-3) / 1e12
        extra["prefill"] = {
            "fused_ms": round(mf, 3), "split_ms": round(msp, 3),
            "fused_p10_p90_ms": [round(float(np.percentile(tf, 10)), 3), round(float(np.percentile(tf, 90)), 3)],
            "fused_TFLOPs": round(tff, 1),
            "split_TFLOPs": round(flops / (msp * 1e-3) / 1e12, 1),
            "fused_frac_of_bf16_peak": round(tff / BF16_PEAK_TFLOPS, 4),
            "fused_frac_of_mfma_loop_peak": ratio(tff, mfma_peak),
            "split_over_fused_time": round(msp / mf, 3),
            "fused_kernels_us_event_timed": kp_f, "split_kernels_us_event_timed": kp_s}
        gu_us = kp_f.get("gemm_gateup_fused")
        dn_us = kp_f.get("gemm_down_residual")
        if gu_us:
            t = 4.0 * Mp * dp * fp / (gu_us * 1e-6) / 1e12
            extra["prefill"]["gateup_fused_kernel_TFLOPs"] = round(t, 1)
            extra["prefill"]["gateup_fused_kernel_frac_of_mfma_loop_peak"] = ratio(t, mfma_peak)
        if dn_us:
            t = 2.0 * Mp * dp * fp / (dn_us * 1e-6) / 1e12
            extra["prefill"]["down_kernel_TFLOPs"] = round(t, 1)
            extra["prefill"]["down_kernel_frac_of_mfma_loop_peak"] = ratio(t, mfma_peak)
        log("prefill", extra["prefill"])
        pstep(0, "fused")
        yf = to_host(py)
        pstep(0, "split")
        ysp = to_host(py)
        keep["C4 prefill fused"] = dict(kind="prefill", inputs=bp, gpu=yf, work=flops, unit="TFLOP/s")
        keep["C4 prefill split"] = dict(kind="prefill", inputs=bp, gpu=ysp, work=flops, unit="TFLOP/s")

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
    warm_up(dstep, 50)
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

    for kind, mbytes in (("q8", q8_matrix_bytes), ("q4", q4_matrix_bytes)):
        wl = I.WORKLOADS[f"{kind}_tp8_shard"]
        M, d, f = wl["M"], wl["d"], wl["f"]
        q = (I.make_q8_block if kind == "q8" else I.make_q4_block)(wl["seed"], M, d, f)
        qx, qg = to_dev(q.x, torch), to_dev(q.g, torch)
        q0 = [(torch.from_numpy(m.qs).to("cuda"), torch.from_numpy(m.scales.view(np.int16)).to("cuda"))
              for m in (q.w_gate, q.w_up, q.w_down)]
        n = nrot if kind == "q8" else 2 * nrot
        qsets = [q0] + [[(a.clone(), s.clone()) for a, s in q0] for _ in range(n - 1)]
        qws = ffn.alloc_workspace(getattr(ffn.lib(), f"ffn_swiglu_block_{kind}_workspace_size")(M, d, f))
        qy = torch.empty_like(qx)
        qcalls = [ffn.prepare_swiglu_block_quant(kind, qx, qg, *st, q.eps, qy, qws) for st in qsets]

        def qstep(i, qcalls=qcalls, n=n):
            qcalls[i % n]()
        warm_up(qstep, 50)
        tq = time_calls(torch, qstep, 500)
        qbytes = 3 * mbytes(f, d) + 2 * M * d * 2 + d * 2
        qgbs = qbytes / (tq * 1e-3) / 1e9
        out[f"{kind}_M8_f2176"] = {"us": round(tq * 1e3, 2), "GBps": round(qgbs, 1),
                                   "frac_of_read_ceiling": ratio(qgbs, read_ceiling)}
        del qcalls, qsets, q0
        torch.cuda.empty_cache()
    extra["tp8_shard"] = out
    log("tp8 shard", out)


# ----------------------------------------------------------------------------
# CPU leg: the oracle as it stands, timed, and each workload's error
# ----------------------------------------------------------------------------
def cpu_oracle_leg(keep, budget_s=60.0):
    """Time the fp64 oracle on every kept workload, with 1 thread and with the
    BLAS library's default (all host threads), and compare this run's GPU
    output with the oracle's.  The prefill block is timed on two sampled row
    counts (rows are independent) and extrapolated linearly to all rows; its
    error is taken over the larger sample.  Returns (per-workload timings,
    per-workload errors)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import ffn_oracle as O

    def blas_threads():
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])

    def run(entry, rows=None):
        k, inp = entry["kind"], entry["inputs"]
        if k == "block":
            blk, m = inp
            return O.block_from_stored(blk.dtype, blk.x[:m], blk.g, blk.w_gate, blk.w_up, blk.w_down, blk.eps)
        if k == "rmsnorm":
            xr, gr, eps = inp
            return O.rmsnorm_from_stored("bf16", xr, gr, eps)
        if k == "prefill":
            return O.block_from_stored("bf16", inp.x[rows], inp.g, inp.w_gate, inp.w_up, inp.w_down, inp.eps)
        fn = O.swiglu_block_q8 if k == "q8" else O.swiglu_block_q4
        return fn(inp.x, inp.g, (inp.w_gate.qs, inp.w_gate.scales), (inp.w_up.qs, inp.w_up.scales),
                  (inp.w_down.qs, inp.w_down.scales), inp.eps)

    def timed(entry, threads, rows=None, min_s=0.5):
        with threadpool_limits(limits=threads):
            used = blas_threads()
            reps, t0 = 0, time.perf_counter()
            while True:
                r = run(entry, rows)
                reps += 1
                if time.perf_counter() - t0 >= min_s:
                    break
        return (time.perf_counter() - t0) / reps, used, r, reps

    def decode(a):
        return O.as_f64(a, "bf16" if a.dtype == np.uint16 else "f32")

    t_start = time.perf_counter()
    timings, errors = {}, {}
    prefill_rows = None
    for name, e in keep.items():
        if time.perf_counter() - t_start > budget_s:
            timings[name] = {"skipped": f"CPU leg budget of {budget_s:.0f} s spent"}
            continue
        if e["kind"] == "prefill":
            bp = e["inputs"]
            if prefill_rows is None:
                rng = np.random.default_rng(44)
                prefill_rows = np.sort(np.concatenate(
                    [[0, bp.M - 1], rng.choice(np.arange(1, bp.M - 1), 62, replace=False)]))
            small = prefill_rows[::2]
            row = {}
            ref = None
            for label, thr in (("1_thread", 1), ("all_threads", None)):
                ts, used, _, _ = timed(e, thr, small, min_s=0.0)
                tl, used, r, _ = timed(e, thr, prefill_rows, min_s=0.0)
                ref = r
                per_row = max((tl - ts) / (prefill_rows.size - small.size), 1e-9)
                full = ts + per_row * (bp.M - small.size)
                row[label] = {"value": round(e["work"] / full / 1e12, 6), "unit": e["unit"], "threads": used,
                              "sample": f"{small.size} and {prefill_rows.size} sampled rows "
                                        f"({ts:.2f} / {tl:.2f} s), extrapolated linearly to {bp.M} rows "
                                        f"({full:.1f} s)"}
            timings[name] = row
            a = decode(e["gpu"])[prefill_rows]
        else:
            row = {}
            ref = None
            threads = (("1_thread", 1),) if e["kind"] == "rmsnorm" else (("1_thread", 1), ("all_threads", None))
            for label, thr in threads:
                t, used, r, reps = timed(e, thr)
                ref = r
                scale = 1e12 if e["unit"] == "TFLOP/s" else 1e9
                row[label] = {"value": round(e["work"] / t / scale, 4), "unit": e["unit"], "threads": used,
                              "sample": f"whole workload, {reps} call(s), {t:.3f} s per call"}
            if e["kind"] == "rmsnorm":
                row["note"] = "the oracle's norm is numpy elementwise work: one thread whatever BLAS has"
            timings[name] = row
            a = decode(e["gpu"])
        dlt = np.abs(a - ref)
        den = float(np.max(np.abs(ref))) or 1.0
        err = {"max_norm": float(dlt.max()) / den,
               "rel_l2": float(np.linalg.norm(a - ref) / max(np.linalg.norm(ref), 1e-300))}
        if e["kind"] == "rmsnorm":
            nz = ref != 0
            err["elementwise_rel"] = float(np.max(dlt[nz] / np.abs(ref[nz])))
        errors[name] = {k: float(f"{v:.4g}") for k, v in err.items()}
        log("oracle", name, timings[name], errors[name])
    return timings, errors


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-extra", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
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
        ffn.probe_copy(buf[:half], buf[half:], 8, False)
        torch.cuda.synchronize()
        return 0

    keep = {"C3 decode M=16": dict(kind="block", inputs=(b, M), gpu=to_host(y), work=decode_bytes(M, d, f),
                                   unit="GB/s")}
    # per-kernel durations: the same steps again, each dispatch carrying its own event pair
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
                "avg_launch_us": round(gu_us, 2), "launches": n_gu, "bytes_per_launch": gateup_bytes(M, d, f),
                "duration_source": "HIP events bound to each dispatch (hipExtLaunchKernel), "
                                   "second pass over the timed steps"}
    kernels = {k: {"launches": n, "avg_us": round(t / n * 1e3, 2)} for k, (n, t) in kt.items()}
    log(f"kernels {kernels}; instrumented pass {ms_instr * 1e3:.2f} us/call")

    pct = per_call_us(torch, step, args.steps)
    # the firmware clock under this load, over ~0.3 s of the same calls (the
    # management library's readout refreshes every few ms; a shorter window reads idle)
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
             "gpu_clock_during_decode_calls": clocks.summary(),
             "software": software_versions(torch)}
    if not args.no_extra:
        extras(torch, np, ffn, I, sets, x, g, b, ws, extra, clocks, want, keep)
    clocks.close()

    cpu = None
    if not args.no_cpu:
        log("CPU leg: the oracle on every workload")
        timings, errors = cpu_oracle_leg(keep)
        extra["cpu_oracle"] = timings
        extra["parity_vs_oracle_this_run"] = errors
        c3 = timings.get("C3 decode M=16", {}).get("1_thread")
        if c3:
            cpu = {"value": c3["value"], "unit": "GB/s", "cores": c3["threads"], "kind": "oracle",
                   "sample": f"decode block M={M} d={d} f={f} (bf16 inputs decoded to fp64): {c3['sample']}"}

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
