#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

Every figure is timed on inputs resident in HBM with preallocated outputs;
each launch is bracketed by HIP events recorded on the stream it runs on (the
current stream, which the binding passes to the library).  Each timed loop
follows a warm-up of at least --warmup launches and 0.25 s of back-to-back
launches, so the device clock has settled under the load.

Headline (``value``, ``roofline``): fa_fwd on the largest prefill workload,
MQA B=4, H=64, H_kv=1, N=4096, d=128, non-causal, bf16 -- one step is one
launch, launched back to back (nothing else on the device between launches).
Attention TFLOP/s = 4*B*H*N_q*N_k*d (halved for causal) / launch time.

Beside it, each timed the same way (back to back, its own roofline):
  * ``prefill``: the GQA (B=1, H=32, H_kv=8, N=8192, causal, K x 2) and MHA
    (B=8, H=32, N=2048, causal) workloads, and the headline again;
  * ``decode``: fa_decode on B=32, H=32, H_kv=8, d=128, lengths uniform in
    [8192, 32768], 16 splits (KV-read GB/s against the HBM peak);
  * ``interleaved_step`` (secondary): each MHA prefill launch alternating with
    a decode step, the step of the earlier benchmark;
  * ``next``: sliding-window and chunked prefill, windowed, paged and FP8 decode.

Clock: after a prefill row is timed, the same launches run again, back to back,
through the library's test hook fa_testing_fwd_capped with a clock record: the
kernel's first workgroup on each XCD reads the shader-cycle counter
(s_memtime) and the 100 MHz real-time counter (s_memrealtime) as it starts and
as it finishes.  Each row reports that clock (the one the kernel ran at) and
its fraction of the matrix-core peak at that clock beside the 2.4 GHz one, with
the stamped launches' own times.

CPU baseline: the fp64 oracle on one of the headline's four sequences, timed
on the host cores and compared element by element with the GPU output.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s (% bf16 MFMA peak); decode KV GB/s (% HBM peak)"
PEAK_CLOCK_GHZ = 2.4


def log(msg):
    """Progress on stderr (the JSON line is the only stdout output)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mqa", choices=["mha", "gqa", "mqa"],
                    help="the prefill workload of --only prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the sliding-window, chunked, paged and FP8 measurements (the 'next' object)")
    ap.add_argument("--only", choices=["prefill", "decode", "step", "next", "copy"], default=None,
                    help="time one part only (for profiling runs): one prefill workload back to back, the "
                         "decode step, the interleaved MHA prefill + decode step, the 'next' workloads, or "
                         "'copy', a plain 1 GiB device-to-device copy (the reference for scaling HBM byte "
                         "counters)")
    return ap.parse_args()


def kernel_source_hash(files):
    """Hash of the kernel sources' code: comments and whitespace are dropped,
    so that editing a comment does not disown the committed counter figures."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "transformer_attention_fa_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def counter_record(kernel_key, src_files):
    """The committed rocprofv3 --pmc figures for a kernel and workload, or None
    when the kernel source changed since they were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel_key)
    except (ValueError, OSError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash(src_files):
        return None
    return rec


def traffic_for(kernel_key, src_files):
    """HBM traffic per launch (FETCH_SIZE + WRITE_SIZE, calibrated), or None."""
    rec = counter_record(kernel_key, src_files)
    return rec.get("bytes_per_launch") if rec else None


def counters_for(kernel_key, src_files):
    """Matrix-core busy fraction and LDS bank-conflict fraction from the
    committed counter runs, or None."""
    rec = counter_record(kernel_key, src_files)
    if not rec:
        return None
    out = {k: round(v, 4) for k, v in rec.items()
           if k.startswith("mfma_busy") or k.startswith("lds_bank_conflict") or k == "counter_clock_ghz"}
    return out or None


def cpu_baseline(spec, n_batches, o_gpu=None, lse_gpu=None):
    """The fp64 oracle on a bounded sample (the first n_batches sequences) of the
    prefill workload, timed on the host cores; when the GPU output of the same
    workload is given, its first n_batches sequences are compared with the
    oracle's element by element (max |dO| and the lse error of the parity bar)."""
    import numpy as np
    import oracle
    from transformer_attention_fa_amd import inputs, roofline
    import dataclasses
    log(f"cpu baseline: the oracle on {n_batches} of {spec.B} sequences of {spec.name}")
    sub = dataclasses.replace(spec, B=n_batches)      # blocks are seeded per (tensor, batch, head)
    data = inputs.prefill_inputs(sub)
    t0 = time.perf_counter()
    o_ref, lse_ref = oracle.attention(data.q, data.k, data.v, sub.scale, sub.causal)
    dt = time.perf_counter() - t0
    flops = roofline.attention_flops(sub.B, sub.H, sub.N_q, sub.N_k, sub.d, sub.causal)
    rec = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
           "sample": (f"the whole {spec.name} workload" if n_batches == spec.B else
                      f"{n_batches} of {spec.B} sequences ({n_batches * spec.H} heads x {spec.N_q} rows) of "
                      f"{spec.name}") + f", fp64, {dt:.2f} s wall",
           "cpu_count": os.cpu_count(), "cpu_model": cpu_model()}
    if o_gpu is not None:
        import torch
        o = o_gpu[:n_batches].to(torch.float64).cpu().numpy()
        lse = lse_gpu[:n_batches].to(torch.float64).cpu().numpy()
        rec["parity"] = {"max_abs_dO": float(np.max(np.abs(o - o_ref))),
                         "max_lse_err_rel_floor1": float(np.max(np.abs(lse - lse_ref) / np.maximum(np.abs(lse_ref), 1.0))),
                         "tolerance": {"O": 2e-2, "lse": 1e-3}, "elements": int(o.size)}
    return rec


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo when there is one."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


class ClockRecord:
    """Clock records of prefill launches through the test hook
    fa_testing_fwd_capped (csrc/fa_testing.h): per launch, 8 workgroups (one
    per XCD) x {cycles at start, ticks at start, XCC id, cycles at end, ticks
    at end} of the shader-cycle and 100 MHz counters."""

    def __init__(self, device, capacity):
        import torch
        from transformer_attention_fa_amd import api
        self.lib = api.load()
        fn = self.lib.fa_testing_fwd_capped
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        fn.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, vp, vp]
        fn.restype = i
        self.buf = torch.zeros((capacity, 64), dtype=torch.int64, device=device)
        self.device = device

    def launch(self, run, slot):
        """One launch of run's problem with its clock record in buf[slot]."""
        import torch
        from transformer_attention_fa_amd import api
        s = run.spec
        B, H, N_q, d = run.q.shape
        api.check(self.lib.fa_testing_fwd_capped(
            run.q.data_ptr(), run.k.data_ptr(), run.v.data_ptr(), run.o.data_ptr(), run.lse.data_ptr(), B, H,
            run.k.shape[1], N_q, run.k.shape[2], d, float(s.scale), int(bool(s.causal)), int(s.window or 0), 0,
            self.buf[slot].data_ptr(), torch.cuda.current_stream(self.device).cuda_stream))

    def summary(self, n):
        """Clock over the first n records (after a synchronize)."""
        import numpy as np
        rec = self.buf[:n].cpu().numpy().reshape(n, 8, 8)
        cyc = (rec[..., 3] - rec[..., 0]).astype(np.float64)
        ticks = (rec[..., 4] - rec[..., 1]).astype(np.float64)
        xcc = rec[..., 2]
        ghz = cyc / np.maximum(ticks, 1) * 0.1                      # per launch and workgroup
        per_launch = np.median(ghz, axis=1)
        per_xcd = {str(int(x)): round(float(np.median(ghz[xcc == x])), 4) for x in sorted(set(xcc.ravel().tolist()))}
        return {"ghz_median": round(float(np.median(per_launch)), 4), "ghz_min": round(float(per_launch.min()), 4),
                "ghz_max": round(float(per_launch.max()), 4), "ghz_median_per_xcd": per_xcd, "launches": n,
                "workgroup_span_us_median": round(float(np.median(ticks)) / 100.0, 2),
                "method": "inside the kernel: s_memtime (shader cycles) over s_memrealtime (100 MHz) from the "
                          "start to the end of the first workgroup on each XCD, through fa_testing_fwd_capped"}


WARMUP_SECONDS = 0.25


def time_launches(fn, steps, warmup):
    """Per-launch times (ms) of `steps` launches back to back, each bracketed by
    HIP events on the current stream; fn(i) makes launch i (i < 0: warm-up).
    Warm-up: `warmup` launches, continued until WARMUP_SECONDS of back-to-back
    launches have run -- after the host-side input drawing the device idles
    for seconds, and its clock takes tens of milliseconds of load to settle
    (ten launches of a 0.3 ms kernel measured 10 % slower than the same
    launches right after).  Returns (times, wall seconds of the timed loop)."""
    import numpy as np
    import torch
    t_start = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t_start < WARMUP_SECONDS:
        fn(-1 - i)
        i += 1
        if i % max(warmup, 1) == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i, (a, b) in enumerate(ev):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return t, wall


def stats(t):
    import numpy as np
    return {"ms_avg": float(np.mean(t)), "ms_median": float(np.median(t)), "ms_min": float(np.min(t))}


def mfma_roofline(tflops, key, clock):
    """Roofline object of a prefill row: the matrix-core bound, with the committed
    counter figures while the kernel source matches them."""
    from transformer_attention_fa_amd import roofline
    r = {"bound": "mfma", "achieved": tflops, "peak": roofline.PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
         "frac": tflops / roofline.PEAK_BF16_TFLOPS, "traffic": traffic_for(f"fwd_bf16:{key}", ["fwd_bf16.hip"]),
         "kernel": "fwd_bf16_kernel", "counters": counters_for(f"fwd_bf16:{key}", ["fwd_bf16.hip"])}
    if clock:
        peak_at = roofline.PEAK_BF16_TFLOPS * clock["ghz_median"] / PEAK_CLOCK_GHZ
        r["clock"] = clock
        r["peak_at_observed_clock"] = peak_at
        r["frac_at_observed_clock"] = tflops / peak_at
    return r


def hbm_roofline(gbps, key):
    from transformer_attention_fa_amd import roofline
    return {"bound": "hbm", "achieved": gbps, "peak": roofline.PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": gbps / roofline.PEAK_HBM_GBPS, "traffic": traffic_for(f"decode:{key}", ["decode.hip"]),
            "kernel": "decode_split_kernel + decode_combine_kernel",
            "counters": counters_for(f"decode:{key}", ["decode.hip"])}


def dev_bf16(bits, dev):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


class PrefillRun:
    """A prefill workload on the device: inputs, preallocated outputs, one launch."""

    def __init__(self, spec, dev):
        import torch
        from transformer_attention_fa_amd import inputs
        self.spec = spec
        data = inputs.prefill_inputs(spec)
        self.q, self.k, self.v = (dev_bf16(x, dev) for x in (data.q, data.k, data.v))
        del data
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((spec.B, spec.H, spec.N_q), dtype=torch.float32, device=dev)

    def __call__(self):
        from transformer_attention_fa_amd import api
        s = self.spec
        api.fwd(self.q, self.k, self.v, causal=s.causal, scale=s.scale, out=self.o, lse=self.lse,
                window=s.window or None)

    def free_inputs(self):
        del self.q, self.k, self.v


def prefill_row(run, steps, warmup, clock):
    """One prefill workload timed back to back through fa_fwd: TFLOP/s and its
    roofline; then the same launches with a clock record (the clock the kernel
    ran at, beside those launches' own times)."""
    spec = run.spec
    log(f"timing {spec.name}")
    t, wall = time_launches(lambda i: run(), steps, warmup)
    st = stats(t)
    flops = spec.flops()
    tflops = flops / (st["ms_avg"] * 1e-3) / 1e12
    row = {"entry": "fa_fwd_window" if spec.window else "fa_fwd", "value": tflops, "unit": "TFLOP/s",
           "timing": "back to back", **st, "wall_ms_per_launch": wall / steps * 1e3, "flop_per_launch": flops,
           # exponentials per launch (one per visible score): the VALU /
           # transcendental budget beside the matrix-core work
           "exp_per_launch": flops / (4 * spec.d),
           "shape": {"B": spec.B, "H": spec.H, "H_kv": spec.H_kv, "N_q": spec.N_q, "N_k": spec.N_k, "d": spec.d,
                     "causal": spec.causal, "window": spec.window, "k_scale": spec.k_scale, "seed": spec.seed}}
    summary = None
    if clock is not None and spec.d == 128:
        n = min(steps, clock.buf.shape[0])
        ts, _ = time_launches(lambda i: clock.launch(run, max(i, 0)), n, warmup)
        summary = clock.summary(n)
        summary["stamped_launch_ms_avg"] = float(ts.mean())
        summary["stamped_tflops"] = flops / (ts.mean() * 1e-3) / 1e12
    row["roofline"] = mfma_roofline(tflops, spec.name, summary)
    return row


class DecodeRun:
    """The decode workload on the device (caches, lengths, outputs, workspace)."""

    def __init__(self, spec, dev):
        import torch
        from transformer_attention_fa_amd import api, inputs
        self.spec = spec
        log(f"drawing {spec.name}")
        data = inputs.decode_inputs(spec)
        self.q = dev_bf16(data.q, dev)
        self.kc, self.vc = dev_bf16(data.k_cache, dev), dev_bf16(data.v_cache, dev)
        self.lens = torch.from_numpy(data.seq_lens).to(dev)
        self.seq_lens = data.seq_lens.copy()
        del data
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((spec.B, spec.H), dtype=torch.float32, device=dev)
        self.ws = torch.empty(api.decode_workspace_bytes(spec.B, spec.H, spec.d, spec.num_splits),
                              dtype=torch.uint8, device=dev)

    def __call__(self):
        from transformer_attention_fa_amd import api
        s = self.spec
        api.decode(self.q, self.kc, self.vc, self.lens, num_splits=s.num_splits, scale=s.scale, out=self.o,
                   lse=self.lse, workspace=self.ws)


def decode_row(run, steps, warmup):
    from transformer_attention_fa_amd import roofline
    spec = run.spec
    log(f"timing {spec.name}")
    t, wall = time_launches(lambda i: run(), steps, warmup)
    st = stats(t)
    kv = roofline.decode_kv_bytes(spec.H_kv, spec.d, run.seq_lens)
    gbps = kv / (st["ms_avg"] * 1e-3) / 1e9
    return {"entry": "fa_decode", "value": gbps, "unit": "GB/s", "timing": "back to back", **st,
            "wall_ms_per_launch": wall / steps * 1e3, "kv_bytes": kv,
            "shape": {"B": spec.B, "H": spec.H, "H_kv": spec.H_kv, "d": spec.d,
                      "seq_len_range": [spec.len_lo, spec.len_hi], "num_splits": spec.num_splits, "seed": spec.seed},
            "roofline": hbm_roofline(gbps, spec.name)}


def interleaved_step(prun, drun, steps, warmup, clock):
    """Secondary figure: each MHA prefill launch alternates with a decode step
    (each timed by its own events); then the same with the prefill launches
    carrying a clock record."""
    import numpy as np
    import torch
    from transformer_attention_fa_amd import roofline
    log("timing the interleaved prefill + decode step")

    def loop(launch, n):
        t_start = time.perf_counter()
        i = 0
        while i < warmup or time.perf_counter() - t_start < WARMUP_SECONDS:
            launch(-1 - i)
            drun()
            i += 1
            if i % max(warmup, 1) == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
        for i, e in enumerate(ev):
            e[0].record()
            launch(i)
            e[1].record()
            e[2].record()
            drun()
            e[3].record()
        torch.cuda.synchronize()
        return (np.array([e[0].elapsed_time(e[1]) for e in ev]), np.array([e[2].elapsed_time(e[3]) for e in ev]))

    tp, td = loop(lambda i: prun(), steps)
    n = min(steps, clock.buf.shape[0])
    tps, _ = loop(lambda i: clock.launch(prun, max(i, 0)), n)
    summary = clock.summary(n)
    summary["stamped_launch_ms_avg"] = float(tps.mean())
    tf = prun.spec.flops() / (tp.mean() * 1e-3) / 1e12
    kv = roofline.decode_kv_bytes(drun.spec.H_kv, drun.spec.d, drun.seq_lens)
    return {"note": "secondary: each prefill launch alternates with a decode step; the memory-bound decode lets "
                    "the clock recover between prefill launches",
            "prefill": {"workload": prun.spec.name, "value": tf, "unit": "TFLOP/s", **stats(tp),
                        "frac": tf / roofline.PEAK_BF16_TFLOPS, "clock": summary},
            "decode": {"workload": drun.spec.name, "value": kv / (td.mean() * 1e-3) / 1e9, "unit": "GB/s",
                       **stats(td)}}


def measure_next(dev, steps, warmup, clock, drun=None):
    """The sliding-window, chunked-prefill, windowed, paged and FP8 decode rows,
    each on its own workload, back to back."""
    import numpy as np
    import torch
    from transformer_attention_fa_amd import api, inputs, roofline
    out = {}
    for spec in (inputs.SWA_PREFILL, inputs.CHUNKED_PREFILL):
        run = PrefillRun(spec, dev)
        out[spec.name] = prefill_row(run, steps, warmup, clock)
        del run
    if drun is None:
        return out
    base = drun.spec
    dq, kc, vc, lens, seq_lens = drun.q, drun.kc, drun.vc, drun.lens, drun.seq_lens
    d_o, d_lse = drun.o, drun.lse

    def dec_row(entry, fn, kv, spec, **extra):
        log(f"timing {spec.name}")
        t, wall = time_launches(lambda i: fn(), steps, warmup)
        st = stats(t)
        gbps = kv / (st["ms_avg"] * 1e-3) / 1e9
        return {"entry": entry, "value": gbps, "unit": "GB/s", "timing": "back to back", **st, "kv_bytes": kv,
                "num_splits": spec.num_splits, **extra, "roofline": hbm_roofline(gbps, spec.name)}

    spec = inputs.SWA_DECODE
    assert (spec.B, spec.H, spec.H_kv, spec.d, spec.seed) == (base.B, base.H, base.H_kv, base.d, base.seed)
    ws = torch.empty(api.decode_workspace_bytes(spec.B, spec.H, spec.d, spec.num_splits), dtype=torch.uint8,
                     device=dev)
    out[spec.name] = dec_row(
        "fa_decode_window",
        lambda: api.decode(dq, kc, vc, lens, num_splits=spec.num_splits, scale=spec.scale, out=d_o, lse=d_lse,
                           workspace=ws, window=spec.window),
        roofline.decode_kv_bytes(spec.H_kv, spec.d, [min(int(n), spec.window) for n in seq_lens]), spec,
        window=spec.window)
    # paged cache: the same rows dealt onto shuffled 16-row pages of a pool
    spec = inputs.PAGED_DECODE
    assert (spec.B, spec.H, spec.H_kv, spec.d, spec.seed) == (base.B, base.H, base.H_kv, base.d, base.seed)
    table, num_pages = inputs.page_table(seq_lens, spec.page_size, spec.seed)
    ps = spec.page_size
    b_idx = np.concatenate([np.full(int(n), b) for b, n in enumerate(seq_lens)])
    r_idx = np.concatenate([np.arange(int(n)) for n in seq_lens])
    page_idx = torch.from_numpy(table[b_idx, r_idx // ps].astype(np.int64)).to(dev)
    slot_idx = torch.from_numpy(r_idx % ps).to(dev)
    bi, ri = torch.from_numpy(b_idx).to(dev), torch.from_numpy(r_idx).to(dev)
    pools = []
    for cache in (kc, vc):
        pool = torch.zeros((num_pages, spec.H_kv, ps, spec.d), dtype=cache.dtype, device=dev)
        pool[page_idx, :, slot_idx] = cache[bi, :, ri]
        pools.append(pool)
    del page_idx, slot_idx, bi, ri
    bt = torch.from_numpy(np.maximum(table, 0)).to(dev)
    ws = torch.empty(api.decode_workspace_bytes(spec.B, spec.H, spec.d, spec.num_splits), dtype=torch.uint8,
                     device=dev)
    out[spec.name] = dec_row(
        "fa_decode_paged",
        lambda: api.decode_paged(dq, pools[0], pools[1], bt, lens, num_splits=spec.num_splits, scale=spec.scale,
                                 out=d_o, lse=d_lse, workspace=ws),
        roofline.decode_kv_bytes(spec.H_kv, spec.d, seq_lens), spec, page_size=ps, num_pages=num_pages)
    del pools
    # FP8 E4M3 cache: the same rows quantised per tensor on the device
    spec = inputs.FP8_DECODE
    assert (spec.B, spec.H, spec.H_kv, spec.d, spec.seed) == (base.B, base.H, base.H_kv, base.d, base.seed)
    codes = []
    for cache, sc in ((kc, spec.k_scale), (vc, spec.v_scale)):
        x = (cache.float() * (1.0 / sc)).clamp_(-448.0, 448.0)
        codes.append(x.to(torch.float8_e4m3fn).view(torch.uint8))
        del x
    ws = torch.empty(api.decode_workspace_bytes(spec.B, spec.H, spec.d, spec.num_splits), dtype=torch.uint8,
                     device=dev)
    r = dec_row(
        "fa_decode_fp8",
        lambda: api.decode_fp8(dq, codes[0], codes[1], spec.k_scale, spec.v_scale, lens, num_splits=spec.num_splits,
                               scale=spec.scale, out=d_o, lse=d_lse, workspace=ws),
        roofline.decode_kv_bytes(spec.H_kv, spec.d, seq_lens, elem=1), spec, kv_format="e4m3, per-tensor scales")
    r["bf16_equivalent_GBps"] = 2 * r["value"]
    out[spec.name] = r
    del codes
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(each GPU would run its own shard of heads or sequences).", file=sys.stderr)
        sys.exit(2)

    import torch
    from transformer_attention_fa_amd import api, inputs, roofline

    api.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only == "copy":
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": args.warmup + args.steps}))
        return
    clock = ClockRecord(dev, args.steps)
    base = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1), bf16)"}
    props = torch.cuda.get_device_properties(dev)
    device = {"name": props.name, "cus": props.multi_processor_count, "gcn_arch": getattr(props, "gcnArchName", "")}

    if args.only == "prefill":
        spec = {"mha": inputs.MHA_PREFILL, "gqa": inputs.GQA_PREFILL, "mqa": inputs.MQA_PREFILL}[args.workload]
        row = prefill_row(PrefillRun(spec, dev), args.steps, args.warmup, clock)
        print(json.dumps({**base, "value": row["value"], "unit": "TFLOP/s", "ms_per_step": row["wall_ms_per_launch"],
                          "config": {"workload": spec.name, **row["shape"], "timing": "back to back"},
                          "roofline": row["roofline"], "prefill": {spec.name: row}, "device": device}), flush=True)
        return
    if args.only == "decode":
        row = decode_row(DecodeRun(inputs.GQA_DECODE, dev), args.steps, args.warmup)
        print(json.dumps({**base, "value": row["value"], "unit": "GB/s", "ms_per_step": row["wall_ms_per_launch"],
                          "config": {"workload": inputs.GQA_DECODE.name, **row["shape"]}, "roofline": row["roofline"],
                          "decode": row, "device": device}), flush=True)
        return
    if args.only == "step":
        rec = interleaved_step(PrefillRun(inputs.MHA_PREFILL, dev), DecodeRun(inputs.GQA_DECODE, dev), args.steps,
                               args.warmup, clock)
        print(json.dumps({**base, "value": rec["prefill"]["value"], "unit": "TFLOP/s",
                          "config": {"workload": inputs.MHA_PREFILL.name + " + " + inputs.GQA_DECODE.name},
                          "interleaved_step": rec, "device": device}), flush=True)
        return
    if args.only == "next":
        nxt = measure_next(dev, args.steps, args.warmup, clock, DecodeRun(inputs.GQA_DECODE, dev))
        print(json.dumps({**base, "next": nxt, "device": device}), flush=True)
        return

    # ---- the default run
    head_spec = inputs.MQA_PREFILL
    head = PrefillRun(head_spec, dev)
    head_row = prefill_row(head, args.steps, args.warmup, clock)
    head.free_inputs()
    rows = {head_spec.name: head_row}
    for spec in (inputs.GQA_PREFILL, inputs.MHA_PREFILL):
        run = PrefillRun(spec, dev)
        rows[spec.name] = prefill_row(run, args.steps, args.warmup, clock)
        if spec is inputs.MHA_PREFILL:
            mha = run
        else:
            del run
    drun = DecodeRun(inputs.GQA_DECODE, dev)
    drow = decode_row(drun, args.steps, args.warmup)
    rec = {**base, "value": head_row["value"], "unit": "TFLOP/s", "ms_per_step": head_row["wall_ms_per_launch"],
           "config": {"workload": head_spec.name, **head_row["shape"], "timing": "back to back"},
           "roofline": {**head_row["roofline"], "launch_ms_avg": head_row["ms_avg"],
                        "launch_ms_median": head_row["ms_median"], "launch_ms_min": head_row["ms_min"],
                        "flop_per_launch": head_row["flop_per_launch"], "exp_per_launch": head_row["exp_per_launch"]},
           "prefill": rows, "decode": drow,
           "interleaved_step": interleaved_step(mha, drun, args.steps, args.warmup, clock)}
    del mha
    if not args.no_next:
        rec["next"] = measure_next(dev, args.steps, args.warmup, clock, drun)
    del drun
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(head_spec, 1, head.o, head.lse)
    rec["device"] = device
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
