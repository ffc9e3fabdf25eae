#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  * prefill: fa_fwd on the MHA workload B=8, H=H_kv=32, N=2048, d=128, causal,
    bf16 (the headline: attention TFLOP/s, FLOPs = 4*B*H*N_q*N_k*d halved for
    causal);
  * decode: fa_decode on the GQA decode workload B=32, H=32, H_kv=8, d=128,
    seq lens uniform in [8192, 32768], 16 splits (KV-read GB/s).
Inputs are resident in HBM before the timed region; outputs are preallocated.
Each launch is bracketed by HIP events recorded on the stream it runs on.

Prints ONE JSON line.  ``--workload`` swaps the prefill workload for another
named one (for exploration; the headline is the default).
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s (% bf16 MFMA peak); decode KV GB/s (% HBM peak)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mha", choices=["mha", "gqa", "mqa"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the sliding-window and chunked-prefill measurements (the 'next' object)")
    ap.add_argument("--only", choices=["prefill", "decode", "next", "copy"], default=None,
                    help="time one part only (for profiling runs): one half of the step, the 'next' "
                         "workloads, or 'copy', a plain 1 GiB device-to-device copy (the reference for "
                         "scaling HBM byte counters)")
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


def cpu_baseline(spec, n_batches):
    """The fp64 oracle on a bounded sample (the first n_batches sequences) of the
    prefill workload, timed on the host cores."""
    import oracle
    from transformer_attention_fa_amd import inputs, roofline
    import dataclasses
    sub = dataclasses.replace(spec, B=n_batches)
    data = inputs.prefill_inputs(sub)
    t0 = time.perf_counter()
    oracle.attention(data.q, data.k, data.v, sub.scale, sub.causal)
    dt = time.perf_counter() - t0
    flops = roofline.attention_flops(sub.B, sub.H, sub.N_q, sub.N_k, sub.d, sub.causal)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": (f"the whole {spec.name} workload" if n_batches == spec.B else
                       f"{n_batches} of {spec.B} sequences ({n_batches * spec.H} heads) of {spec.name}")
                      + f", fp64, {dt:.2f} s wall",
            "cpu_count": os.cpu_count(), "cpu_model": cpu_model()}


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


def time_launches(fn, steps, warmup):
    """Average / median / min of `steps` launches (HIP events on the current stream), in ms."""
    import numpy as np
    import torch
    for _ in range(warmup):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return float(t.mean()), float(np.median(t)), float(t.min())


def measure_next(dev_bf16, steps, warmup, decode_state=None):
    """The sliding-window, chunked-prefill and paged-cache rows, each on its own workload."""
    import numpy as np
    import torch
    from transformer_attention_fa_amd import api, inputs, roofline
    out = {}
    for spec in (inputs.SWA_PREFILL, inputs.CHUNKED_PREFILL):
        data = inputs.prefill_inputs(spec)
        q, k, v = (dev_bf16(x) for x in (data.q, data.k, data.v))
        del data
        o = torch.empty_like(q)
        lse = torch.empty((spec.B, spec.H, spec.N_q), dtype=torch.float32, device=q.device)
        win = spec.window or None
        avg, med, mn = time_launches(lambda: api.fwd(q, k, v, causal=spec.causal, scale=spec.scale, out=o, lse=lse,
                                                     window=win), steps, warmup)
        flops = spec.flops()
        tf = flops / (avg * 1e-3) / 1e12
        out[spec.name] = {"entry": "fa_fwd_window" if win else "fa_fwd", "value": tf, "unit": "TFLOP/s",
                          "frac_mfma_peak": tf / roofline.PEAK_BF16_TFLOPS, "ms_avg": avg, "ms_median": med,
                          "ms_min": mn, "flop_per_launch": flops, "exp_per_launch": flops / (4 * spec.d),
                          "window": spec.window,
                          "shape": {"B": spec.B, "H": spec.H, "H_kv": spec.H_kv, "N_q": spec.N_q, "N_k": spec.N_k,
                                    "d": spec.d, "causal": spec.causal}}
        del q, k, v, o, lse
    if decode_state is not None:
        spec = inputs.SWA_DECODE
        dq, kc, vc, lens, seq_lens, base = decode_state
        assert (spec.B, spec.H, spec.H_kv, spec.d, spec.seed) == (base.B, base.H, base.H_kv, base.d, base.seed)
        ws = torch.empty(api.decode_workspace_bytes(spec.B, spec.H, spec.d, spec.num_splits), dtype=torch.uint8,
                         device=dq.device)
        d_o = torch.empty_like(dq)
        d_lse = torch.empty((spec.B, spec.H), dtype=torch.float32, device=dq.device)
        avg, med, mn = time_launches(lambda: api.decode(dq, kc, vc, lens, num_splits=spec.num_splits,
                                                        scale=spec.scale, out=d_o, lse=d_lse, workspace=ws,
                                                        window=spec.window), steps, warmup)
        kv = roofline.decode_kv_bytes(spec.H_kv, spec.d, [min(int(n), spec.window) for n in seq_lens])
        gbps = kv / (avg * 1e-3) / 1e9
        out[spec.name] = {"entry": "fa_decode_window", "value": gbps, "unit": "GB/s",
                          "frac_hbm_peak": gbps / roofline.PEAK_HBM_GBPS, "ms_avg": avg, "ms_median": med,
                          "ms_min": mn, "kv_bytes": kv, "window": spec.window, "num_splits": spec.num_splits}
        # paged cache: the same rows dealt onto shuffled 16-row pages of a pool
        spec = inputs.PAGED_DECODE
        assert (spec.B, spec.H, spec.H_kv, spec.d, spec.seed) == (base.B, base.H, base.H_kv, base.d, base.seed)
        table, num_pages = inputs.page_table(seq_lens, spec.page_size, spec.seed)
        ps = spec.page_size
        b_idx = np.concatenate([np.full(int(n), b) for b, n in enumerate(seq_lens)])
        r_idx = np.concatenate([np.arange(int(n)) for n in seq_lens])
        page_idx = torch.from_numpy(table[b_idx, r_idx // ps].astype(np.int64)).to(dq.device)
        slot_idx = torch.from_numpy(r_idx % ps).to(dq.device)
        bi, ri = torch.from_numpy(b_idx).to(dq.device), torch.from_numpy(r_idx).to(dq.device)
        pools = []
        for cache in (kc, vc):
            pool = torch.zeros((num_pages, spec.H_kv, ps, spec.d), dtype=cache.dtype, device=dq.device)
            pool[page_idx, :, slot_idx] = cache[bi, :, ri]
            pools.append(pool)
        del page_idx, slot_idx, bi, ri
        bt = torch.from_numpy(np.maximum(table, 0)).to(dq.device)
        ws = torch.empty(api.decode_workspace_bytes(spec.B, spec.H, spec.d, spec.num_splits), dtype=torch.uint8,
                         device=dq.device)
        avg, med, mn = time_launches(lambda: api.decode_paged(dq, pools[0], pools[1], bt, lens,
                                                              num_splits=spec.num_splits, scale=spec.scale, out=d_o,
                                                              lse=d_lse, workspace=ws), steps, warmup)
        kv = roofline.decode_kv_bytes(spec.H_kv, spec.d, seq_lens)
        gbps = kv / (avg * 1e-3) / 1e9
        out[spec.name] = {"entry": "fa_decode_paged", "value": gbps, "unit": "GB/s",
                          "frac_hbm_peak": gbps / roofline.PEAK_HBM_GBPS, "ms_avg": avg, "ms_median": med,
                          "ms_min": mn, "kv_bytes": kv, "page_size": ps, "num_pages": num_pages,
                          "num_splits": spec.num_splits}
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
                         device=dq.device)
        avg, med, mn = time_launches(lambda: api.decode_fp8(dq, codes[0], codes[1], spec.k_scale, spec.v_scale, lens,
                                                            num_splits=spec.num_splits, scale=spec.scale, out=d_o,
                                                            lse=d_lse, workspace=ws), steps, warmup)
        kv = roofline.decode_kv_bytes(spec.H_kv, spec.d, seq_lens, elem=1)
        gbps = kv / (avg * 1e-3) / 1e9
        out[spec.name] = {"entry": "fa_decode_fp8", "value": gbps, "unit": "GB/s",
                          "frac_hbm_peak": gbps / roofline.PEAK_HBM_GBPS, "ms_avg": avg, "ms_median": med,
                          "ms_min": mn, "kv_bytes": kv, "kv_format": "e4m3, per-tensor scales",
                          "bf16_equivalent_GBps": 2 * gbps, "num_splits": spec.num_splits}
        del codes
    return out


def add_rooflines(nxt):
    """Roofline objects for the 'next' entries (traffic from the committed counters when current)."""
    from transformer_attention_fa_amd import roofline
    for name, r in nxt.items():
        if r["unit"] == "TFLOP/s":
            r["roofline"] = {"bound": "mfma", "achieved": r["value"], "peak": roofline.PEAK_BF16_TFLOPS,
                             "unit": "TFLOP/s", "frac": r["value"] / roofline.PEAK_BF16_TFLOPS,
                             "traffic": traffic_for(f"fwd_bf16:{name}", ["fwd_bf16.hip"]), "kernel": "fwd_bf16_kernel",
                             "counters": counters_for(f"fwd_bf16:{name}", ["fwd_bf16.hip"])}
        else:
            r["roofline"] = {"bound": "hbm", "achieved": r["value"], "peak": roofline.PEAK_HBM_GBPS, "unit": "GB/s",
                             "frac": r["value"] / roofline.PEAK_HBM_GBPS,
                             "traffic": traffic_for(f"decode:{name}", ["decode.hip"]),
                             "kernel": "decode_split_kernel + decode_combine_kernel",
                             "counters": counters_for(f"decode:{name}", ["decode.hip"])}
    return nxt


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(each GPU would run its own shard of heads or sequences).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
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
    pspec = {"mha": inputs.MHA_PREFILL, "gqa": inputs.GQA_PREFILL, "mqa": inputs.MQA_PREFILL}[args.workload]
    dspec = inputs.GQA_DECODE
    do_prefill = args.only in (None, "prefill")
    do_decode = args.only in (None, "decode", "next")     # 'next' reuses the decode caches

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    if do_prefill:
        pdata = inputs.prefill_inputs(pspec)
        q, k, v = (dev_bf16(x) for x in (pdata.q, pdata.k, pdata.v))
        del pdata
        o = torch.empty_like(q)
        lse = torch.empty((pspec.B, pspec.H, pspec.N_q), dtype=torch.float32, device=dev)
    if do_decode:
        ddata = inputs.decode_inputs(dspec)
        dq = dev_bf16(ddata.q)
        kc, vc = dev_bf16(ddata.k_cache), dev_bf16(ddata.v_cache)
        lens = torch.from_numpy(ddata.seq_lens).to(dev)
        seq_lens = ddata.seq_lens.copy()
        del ddata
        d_o = torch.empty_like(dq)
        d_lse = torch.empty((dspec.B, dspec.H), dtype=torch.float32, device=dev)
        ws = torch.empty(api.decode_workspace_bytes(dspec.B, dspec.H, dspec.d, dspec.num_splits),
                         dtype=torch.uint8, device=dev)

    def step(ev=None):
        if do_prefill:
            if ev is not None:
                ev[0].record()
            api.fwd(q, k, v, causal=pspec.causal, scale=pspec.scale, out=o, lse=lse)
            if ev is not None:
                ev[1].record()
        if do_decode:
            if ev is not None:
                ev[2].record()
            api.decode(dq, kc, vc, lens, num_splits=dspec.num_splits, scale=dspec.scale,
                       out=d_o, lse=d_lse, workspace=ws)
            if ev is not None:
                ev[3].record()

    if args.only == "next":
        rec = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
               "next": add_rooflines(measure_next(dev_bf16, args.steps, args.warmup,
                                                  (dq, kc, vc, lens, seq_lens, dspec)))}
        print(json.dumps(rec), flush=True)
        return
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    rec = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1), bf16)"}
    config = {"workload": "", "prefill": None, "decode": None}
    if do_prefill:
        t_pf = [e[0].elapsed_time(e[1]) for e in events]        # ms
        t_avg = float(np.mean(t_pf))
        flops = pspec.flops()
        tflops = flops / (t_avg * 1e-3) / 1e12
        traffic = traffic_for(f"fwd_bf16:{pspec.name}", ["fwd_bf16.hip"])
        rec.update({"value": tflops, "unit": "TFLOP/s"})
        rec["roofline"] = {"bound": "mfma", "achieved": tflops, "peak": roofline.PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": tflops / roofline.PEAK_BF16_TFLOPS, "traffic": traffic,
                           "kernel": "fwd_bf16_kernel", "launch_ms_avg": t_avg,
                           "launch_ms_median": float(np.median(t_pf)), "launch_ms_min": float(np.min(t_pf)),
                           "flop_per_launch": flops,
                           # exponentials per launch (one per visible score): the VALU /
                           # transcendental budget beside the MFMA work
                           "exp_per_launch": flops / (4 * pspec.d),
                           "counters": counters_for(f"fwd_bf16:{pspec.name}", ["fwd_bf16.hip"])}
        config["workload"] = pspec.name
        config["prefill"] = {"B": pspec.B, "H": pspec.H, "H_kv": pspec.H_kv, "N_q": pspec.N_q, "N_k": pspec.N_k,
                             "d": pspec.d, "causal": pspec.causal, "seed": pspec.seed}
    if do_decode:
        t_dc = [e[2].elapsed_time(e[3]) for e in events]
        t_avg_d = float(np.mean(t_dc))
        kv_bytes = roofline.decode_kv_bytes(dspec.H_kv, dspec.d, seq_lens)
        gbps = kv_bytes / (t_avg_d * 1e-3) / 1e9
        rec["decode"] = {"value": gbps, "unit": "GB/s", "frac_hbm_peak": gbps / roofline.PEAK_HBM_GBPS,
                         "ms_avg": t_avg_d, "ms_median": float(np.median(t_dc)), "ms_min": float(np.min(t_dc)),
                         "kv_bytes": kv_bytes,
                         "roofline": {"bound": "hbm", "achieved": gbps, "peak": roofline.PEAK_HBM_GBPS,
                                      "unit": "GB/s", "frac": gbps / roofline.PEAK_HBM_GBPS,
                                      "traffic": traffic_for(f"decode:{dspec.name}", ["decode.hip"]),
                                      "kernel": "decode_split_kernel + decode_combine_kernel",
                                      "counters": counters_for(f"decode:{dspec.name}", ["decode.hip"])}}
        config["workload"] = (config["workload"] + " + " if config["workload"] else "") + dspec.name
        config["decode"] = {"B": dspec.B, "H": dspec.H, "H_kv": dspec.H_kv, "d": dspec.d,
                            "seq_len_range": [dspec.len_lo, dspec.len_hi], "num_splits": dspec.num_splits,
                            "seed": dspec.seed}
        if not do_prefill:
            rec.update({"value": gbps, "unit": "GB/s"})
    rec["config"] = config
    if args.only is None and not args.no_next:
        rec["next"] = add_rooflines(measure_next(dev_bf16, args.steps, args.warmup,
                                                 (dq, kc, vc, lens, seq_lens, dspec) if do_decode else None))
    if do_prefill and not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(pspec, n_batches=pspec.B)
    props = torch.cuda.get_device_properties(dev)
    rec["device"] = {"name": props.name, "cus": props.multi_processor_count,
                     "gcn_arch": getattr(props, "gcnArchName", "")}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
