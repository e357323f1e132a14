"""Benchmark of the shared-KV cross-attention hot path on one MI355X.

One step = one pass of the whole path over seeded synthetic input resident in HBM:
  * prefill: 16 Cross-Decoder layers, each a causal prefill of its own queries
    [32768, 16 heads, 128] against one shared K^,V^ [32768, 4 KV heads, 128] (bf16);
  * decode: one appended K^,V^ row per sequence, then 16 layer queries against the
    shared cache of 8 sequences x 131072 rows, 2 KV heads, 16 query heads (bf16).
`value` is the prefill rate (algorithmic causal flops 4*d*Hq*N(N+1)/2 per layer
over the measured time); the decode rate (K^ and V^ bytes read once per call plus
Q and O, over the measured call time) is reported beside it in `decode`.
The default run also times, each with its own roofline block:
  * `decode_1m`: the long-context decode, 1 x 1048576 rows, 64 steps of one
    append and 16 layer calls;
  * `ragged`: 16 prompts of log-uniform lengths in [4096, 65536) (Hq=32,
    Hkv=8): their causal prefill, then 32 decode steps;
and reports a streaming-read probe of the device (`device.read_probe_GBps`)
and the pages' own model-level claims as context (`context`).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --workload decode_1m     (long-context decode, 64 steps x 16 layers)
       python bench.py --workload swa           (Self-Decoder sliding window, C = 1024: 32K prefill,
                                                  token decode over ring window caches)
       python bench.py --workload producer      (RMSNorm + [W_K|W_V] projection into the shared cache,
                                                  d_model 3072, 8 KV heads: a 32K prompt, then decode rows)
       python bench.py --workload gret          (gated retention: chunkwise prefill of 32K rows x 16 heads,
                                                  recurrent decode steps for 8 sequences)
       python bench.py --copy-probe             (plain copy kernel of known size, for counter scaling)
       python bench.py --skip decode_1m,ragged  (leave legs out: prefill, decode, decode_1m, ragged)
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
CALL_REPS = 32               # back-to-back calls for the per-call median / min / p90
BF16_DENSE_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = "decode HBM GB/s (% peak) @128K-1M; prefill TFLOP/s (% MFMA peak) @32K"
PROBE_LIB = os.path.join(ROOT, "decoder_shared_kv_amd", "lib", "libyoco_probe.so")

# The pages' end-to-end claims for whole YOCO models, restated (page "YOCO 深度技术分析",
# liuhc.cn, section 3.4 inference-efficiency table). The pages state no hardware,
# precision or kernel for any of them: context beside the kernel figures, not targets.
PUBLISHED_CONTEXT = {
    "note": "model-level claims of the pages for whole YOCO models against a Transformer; hardware, precision "
            "and kernels not stated; context only, not comparable with the kernel rates above",
    "source": "YOCO 深度技术分析 (liuhc.cn), section 3.4",
    "claims": [
        {"what": "KV cache memory per token", "factor": "about 80x smaller", "workload": "65B model",
         "hardware": "not stated"},
        {"what": "prefill latency", "factor": "2.87x faster", "workload": "32K context", "hardware": "not stated"},
        {"what": "prefill latency", "factor": "71.8x faster (Transformer about 300 s)", "workload": "1M context",
         "hardware": "not stated"},
        {"what": "decode throughput", "factor": "9.6x higher (4.5 to 43.1 tokens/s)", "workload": "512K context",
         "hardware": "not stated"},
    ],
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gret_traffic_fields(call_s):
    """Measured HBM bytes of one chunkwise gRet prefill call: the three kernels'
    counter traffic summed, as a rate over the call time, or null when any is
    absent or was taken on a different version of the kernels."""
    from bench_counters import traffic_for
    parts = [traffic_for(k) for k in ("gret_segstate_kernel<128>", "gret_segscan_kernel<128>", "gret_out_kernel<128>")]
    if any(b is None for b in parts):
        return {"traffic": None}
    b = sum(parts)
    return {"traffic": b / call_s / 1e9, "traffic_unit": "GB/s", "traffic_bytes_per_launch": b}


def traffic_fields(kernel, launch_s):
    """Measured HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated
    against a plain copy; see bench_counters.py) as a rate over the measured launch
    time, or null when absent or taken on a different version of the kernel."""
    from bench_counters import traffic_for
    b = traffic_for(kernel)
    if b is None:
        return {"traffic": None}
    return {"traffic": b / launch_s / 1e9, "traffic_unit": "GB/s", "traffic_bytes_per_launch": b}


def prefill_flops(lens, hq, d):
    return sum(4.0 * d * hq * n * (n + 1) / 2.0 for n in lens)


def decode_bytes(lens, hkv, hq, d, elem=2):
    return sum(n * hkv * d * elem * 2 for n in lens) + len(lens) * hq * d * elem * 2


def make_prefill(dk, synth, dev, w):
    c = synth.make_prefill_case(list(w.seq_lens), w.q_heads, w.kv_heads, w.head_dim, w.layers, w.dtype, w.seed,
                                w.value_std)
    cache = dk.SharedKV(c.k_pool.to(dev), c.v_pool.to(dev), c.seq_start.to(dev), c.seq_len.to(dev), c.seq_cap.to(dev))
    qs = [q.to(dev) for q in c.q]
    return c, cache, qs


def make_decode(dk, synth, dev, w, extra_steps):
    steps = max(w.decode_steps, 1)
    c = synth.make_decode_case(list(w.seq_lens), w.q_heads, w.kv_heads, w.head_dim, w.layers, steps, w.dtype,
                               w.seed, w.value_std, cap_extra=extra_steps)
    cache = dk.SharedKV(c.k_pool.to(dev), c.v_pool.to(dev), c.seq_start.to(dev), c.seq_len.to(dev).clone(),
                        c.seq_cap.to(dev))
    return c, cache


def cpu_baseline(synth, oracle, w, budget_s=12.0):
    """The oracle as it stands, on the host cores, over a bounded sample of the
    prefill workload: blocks of the last query rows of layer 0, all heads."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    c = synth.make_prefill_case(list(w.seq_lens), w.q_heads, w.kv_heads, w.head_dim, 1, w.dtype, w.seed,
                                w.value_std)
    q = synth.to_f64(c.q[0])
    k = synth.to_f32(c.k_pool)
    v = synth.to_f32(c.v_pool)
    n = int(w.seq_lens[0])
    done_rows = []
    flops = 0.0
    t0 = time.perf_counter()
    hi = n
    while time.perf_counter() - t0 < budget_s and hi > 0:
        lo = max(0, hi - 128)
        rows = list(range(lo, hi))
        oracle.prefill_ref(q, k, v, c.seq_start.numpy(), c.seq_len.numpy(), c.cu_seqlens.numpy(), c.scale,
                           rows={0: rows})
        flops += sum(4.0 * w.head_dim * w.q_heads * (r + 1) for r in rows)
        done_rows.append((lo, hi))
        hi = lo
    dt = time.perf_counter() - t0
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            model = next(line.split(":", 1)[1].strip() for line in f if line.startswith("model name"))
    except Exception:  # noqa: BLE001
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu": model,
            "sample": f"fp64 NumPy oracle, prefill layer 0 of the 32K workload, query rows "
                      f"{done_rows[-1][0]}..{n - 1} (all {w.q_heads} heads), {dt:.1f} s; "
                      f"rate = causal flops of those rows / time"}


def copy_probe(torch, dev):
    """A plain device copy of known size: its FETCH_SIZE/WRITE_SIZE calibrate the counters."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_per_launch": n, "launches": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="default", choices=["default", "decode_1m", "ragged", "swa", "producer", "gret"])
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--skip", default="", help="comma list of modes to leave out: prefill,decode (profiling only)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import decoder_shared_kv_amd as dk
    import synth

    dev = torch.device("cuda:0")
    dk.load_library()
    if args.copy_probe:
        copy_probe(torch, dev)
        return
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} CUs={props.multi_processor_count}")

    if args.workload == "decode_1m":
        return bench_decode_1m(args, torch, dk, synth, dev)
    if args.workload == "ragged":
        return bench_ragged(args, torch, dk, synth, dev)
    if args.workload == "swa":
        return bench_swa(args, torch, dk, synth, dev)
    if args.workload == "producer":
        return bench_producer(args, torch, dk, synth, dev)
    if args.workload == "gret":
        return bench_gret(args, torch, dk, synth, dev)

    skip = set(x for x in args.skip.split(",") if x)
    wp = synth.WORKLOADS["prefill_32k"]
    wd = synth.WORKLOADS["decode_128k"]
    t = time.perf_counter()
    n = int(wp.seq_lens[0])
    if "prefill" not in skip:
        pc, pcache, qs = make_prefill(dk, synth, dev, wp)
        cu = pc.cu_seqlens.to(dev)
        out_p = torch.empty_like(qs[0])
        lse_p = torch.empty(wp.q_heads, n, device=dev, dtype=torch.float32)
        pws = dk.alloc_prefill_workspace(dev)
    if "decode" not in skip:
        dc, dcache = make_decode(dk, synth, dev, wd, args.steps + args.warmup + 1)
        max_dec = int(dc.seq_len.max()) + args.steps + args.warmup + 1
        ws = dk.alloc_workspace(dcache, wd.q_heads, max_dec)
        out_d = torch.empty(wd.batch, wd.q_heads, wd.head_dim, device=dev, dtype=torch.bfloat16)
        lse_d = torch.empty(wd.batch, wd.q_heads, device=dev, dtype=torch.float32)
        qd = dc.q[0].to(dev)               # [layers, B, Hq, d]
        kn = dc.k_new[0].to(dev)
        vn = dc.v_new[0].to(dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    log(f"inputs ready in {time.perf_counter() - t:.1f} s")

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    lens_now = [int(x) for x in dc.seq_len] if "decode" not in skip else []

    def step(record):
        if "prefill" not in skip:
            if record:
                ev[0].record()
            for layer in range(wp.layers):
                dk.xattn_prefill(pcache, qs[layer], cu, n, pc.scale, out=out_p, lse=lse_p, workspace=pws)
            if record:
                ev[1].record()
        if "decode" not in skip:
            dk.kv_append(dcache, kn, vn, flag)
            if record:
                ev[2].record()
            cur = max(lens_now) + 1
            for layer in range(wd.layers):
                dk.xattn_decode(dcache, qd[layer], cur, dc.scale, ws, out=out_d, lse=lse_d)
            if record:
                ev[3].record()
        for b in range(len(lens_now)):
            lens_now[b] += 1 if "decode" not in skip else 0

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    pre_ms, dec_ms = 0.0, 0.0
    pre_steps, dec_steps = [], []
    dec_bytes = 0.0
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
        if "decode" not in skip:
            dec_bytes += wd.layers * decode_bytes(lens_now, wd.kv_heads, wd.q_heads, wd.head_dim)
        ev[3 if "decode" not in skip else 1].synchronize()
        if "prefill" not in skip:
            pre_steps.append(ev[0].elapsed_time(ev[1]))
            pre_ms += pre_steps[-1]
        if "decode" not in skip:
            dec_steps.append(ev[2].elapsed_time(ev[3]))
            dec_ms += dec_steps[-1]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert int(flag.item()) == 0, "append overflowed"

    def spread(t):
        import numpy as np
        t = np.asarray(t, dtype=np.float64)
        return {"n": int(t.size), "median_ms": float(np.median(t)), "min_ms": float(t.min()),
                "p90_ms": float(np.percentile(t, 90))}

    def call_stats(call, reps=CALL_REPS):
        """Per-call spread after the timed region: one event pair around each of
        `reps` back-to-back calls (the timed region itself records none)."""
        import numpy as np
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for layer, (a, b) in enumerate(evs):
            a.record()
            call(layer)
            b.record()
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) for a, b in evs])
        return {"calls": reps, "median_ms": float(np.median(t)), "min_ms": float(t.min()),
                "p90_ms": float(np.percentile(t, 90))}

    flops_layer = prefill_flops(wp.seq_lens, wp.q_heads, wp.head_dim)
    res = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1)/sqrt(128) bf16)",
           "config": {"workload": "prefill: B=1 N=32768 Hq=16 Hkv=4 d=128 causal, 16 layers on one shared K,V; "
                                  "decode: B=8 N=131072 Hq=16 Hkv=2 d=128, append + 16 layers",
                      "global_batch": 1, "seq_len": n, "parallelism": "none (1 GPU)"}}
    if "prefill" not in skip:
        layer_s = pre_ms / 1e3 / (args.steps * wp.layers)
        tflops = flops_layer / layer_s / 1e12
        res.update({"value": tflops, "unit": "TFLOP/s"})
        res["roofline"] = {"bound": "mfma", "achieved": tflops, "peak": BF16_DENSE_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": tflops / BF16_DENSE_PEAK_TFLOPS,
                           **traffic_fields("prefill_bf16_kernel<128>", layer_s),
                           "kernel": "prefill_bf16_kernel<128>", "avg_launch_ms": layer_s * 1e3,
                           "algorithmic_per_launch": flops_layer}
        res["prefill_steps"] = {**spread(pre_steps), "what": f"{wp.layers} layer calls per step"}
        res["prefill_calls"] = call_stats(
            lambda i: dk.xattn_prefill(pcache, qs[i % wp.layers], cu, n, pc.scale, out=out_p, lse=lse_p,
                                       workspace=pws))
    if "decode" not in skip:
        calls = args.steps * wd.layers
        call_s = dec_ms / 1e3 / calls
        gbs = dec_bytes / (dec_ms / 1e3) / 1e9
        res["decode"] = {"value": gbs, "unit": "GB/s", "avg_call_ms": call_s * 1e3,
                         "algorithmic_bytes_per_call": dec_bytes / calls,
                         "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": gbs / HBM_PEAK_GBS, **traffic_fields("decode_split_bf16_kernel<128, 1, 0>",
                                                                                    call_s),
                                      "kernel": "decode_split_bf16_kernel<128, 1, 0> + decode_merge_kernel "
                                                "(one call: both launches, timed together)"},
                         "steps": {**spread(dec_steps), "what": f"one append and {wd.layers} layer calls per step"},
                         "calls": call_stats(
                             lambda i: dk.xattn_decode(dcache, qd[i % wd.layers], max(lens_now), dc.scale, ws,
                                                       out=out_d, lse=lse_d))}
        if "prefill" in skip:
            res.update({"value": gbs, "unit": "GB/s"})
    # the other legs run on their own inputs: free these first (the closures
    # above hold these names, so they are rebound rather than deleted)
    pc = pcache = qs = out_p = lse_p = dc = dcache = ws = qd = None  # noqa: F841
    torch.cuda.empty_cache()
    if "decode_1m" not in skip:
        res["decode_1m"] = leg_decode_1m(args, torch, dk, synth, dev)
        torch.cuda.empty_cache()
    if "ragged" not in skip:
        res["ragged"] = leg_ragged(args, torch, dk, synth, dev)
        torch.cuda.empty_cache()
    res["device"] = device_info(torch, dev)
    res["context"] = PUBLISHED_CONTEXT
    if not args.no_cpu_baseline:
        import oracle
        log("timing the oracle on the host")
        res["cpu_baseline"] = cpu_baseline(synth, oracle, wp)
    print(json.dumps(res), flush=True)


def read_probe(torch, dev):
    """Streaming-read rate of the device: the probe kernel (lib/libyoco_probe.so)
    reads a 2 GiB buffer (8x the Infinity Cache) with 16-byte nontemporal loads,
    5 passes per grid size; the best grid's rate is reported."""
    import ctypes
    lib = ctypes.CDLL(PROBE_LIB)
    lib.yoco_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_void_p]
    lib.yoco_probe_read.restype = ctypes.c_int
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    grids = (1024, 2048, 4096, 8192)
    sink = torch.zeros(max(grids), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    rates = {}
    for grid in grids:
        assert lib.yoco_probe_read(buf.data_ptr(), nbytes, sink.data_ptr(), grid, stream) == 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            lib.yoco_probe_read(buf.data_ptr(), nbytes, sink.data_ptr(), grid, stream)
        e1.record()
        torch.cuda.synchronize()
        rates[grid] = 5 * nbytes / (e0.elapsed_time(e1) / 1e3) / 1e9
    del buf, sink
    best = max(rates, key=rates.get)
    return {"read_probe_GBps": rates[best],
            "read_probe": f"read_probe_kernel: 2 GiB, 16-byte nontemporal loads, 256 threads x {best} workgroups "
                          f"(best of grids {list(grids)}: " + ", ".join(f"{g}: {r:.0f}" for g, r in rates.items())
                          + " GB/s)"}


def device_info(torch, dev):
    """CU count, a streaming-read probe, and a copy probe: torch's device copy of
    1 GiB (bytes read plus bytes written per second), for context beside the
    8 TB/s published figure."""
    props = torch.cuda.get_device_properties(dev)
    probe = read_probe(torch, dev)
    a = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    gbs = 5 * 2 * a.numel() / (e0.elapsed_time(e1) / 1e3) / 1e9
    del a, b
    return {"name": props.name, "compute_units": props.multi_processor_count, **probe,
            "copy_probe_GBps": gbs, "copy_probe": "torch device copy of 1 GiB, 5 passes, read + write bytes"}


def call_spread(torch, call, reps=CALL_REPS):
    """Per-call spread: one event pair around each of `reps` back-to-back calls."""
    import numpy as np
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        call(i)
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    return {"calls": reps, "median_ms": float(np.median(t)), "min_ms": float(t.min()),
            "p90_ms": float(np.percentile(t, 90))}


def leg_decode_1m(args, torch, dk, synth, dev):
    """The long-context decode: 1 x 1048576 rows, 64 steps of one append and 16
    layer calls (the cache grows to 1048640 rows), timed as one region."""
    w = synth.WORKLOADS["decode_1m"]
    t = time.perf_counter()
    c, cache = make_decode(dk, synth, dev, w, 0)
    log(f"decode 1m inputs ready in {time.perf_counter() - t:.1f} s")
    q = c.q.to(dev)
    kn, vn = c.k_new.to(dev), c.v_new.to(dev)
    max_len = int(c.seq_len.max()) + w.decode_steps
    ws = dk.alloc_workspace(cache, w.q_heads, max_len)
    out = torch.empty(w.batch, w.q_heads, w.head_dim, device=dev, dtype=torch.bfloat16)
    lse = torch.empty(w.batch, w.q_heads, device=dev, dtype=torch.float32)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    # warm-up on a copy of the metadata so that the timed run starts from the initial cache
    saved = cache.seq_len.clone()
    for _ in range(max(1, min(args.warmup, 2))):
        dk.kv_append(cache, kn[0], vn[0], flag)
        dk.xattn_decode(cache, q[0, 0], max_len, c.scale, ws, out=out, lse=lse)
    torch.cuda.synchronize()
    cache.seq_len.copy_(saved)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    lens = [int(x) for x in c.seq_len]
    nbytes = 0.0
    t0 = time.perf_counter()
    e0.record()
    for s in range(w.decode_steps):
        dk.kv_append(cache, kn[s], vn[s], flag)
        lens = [x + 1 for x in lens]
        for layer in range(w.layers):
            dk.xattn_decode(cache, q[s, layer], max_len, c.scale, ws, out=out, lse=lse)
            nbytes += decode_bytes(lens, w.kv_heads, w.q_heads, w.head_dim)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1)
    assert int(flag.item()) == 0
    gbs = nbytes / (ms / 1e3) / 1e9
    calls = w.decode_steps * w.layers
    spread = call_spread(torch, lambda i: dk.xattn_decode(cache, q[-1, i % w.layers], max_len, c.scale, ws,
                                                          out=out, lse=lse))
    last_bytes = decode_bytes(lens, w.kv_heads, w.q_heads, w.head_dim)
    spread["median_GBps"] = last_bytes / (spread["median_ms"] / 1e3) / 1e9
    res = {"value": gbs, "unit": "GB/s", "total_ms": ms, "wall_ms": wall * 1e3, "steps": w.decode_steps,
           "layers": w.layers, "avg_call_ms": ms / calls, "algorithmic_bytes_per_call": nbytes / calls,
           "workload": "decode: B=1 N=1048576 (+64 appends) Hq=16 Hkv=2 d=128, 64 steps x (append + 16 layers)",
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                        "kernel": "decode_split_bf16_kernel<128, 1, 0> + decode_merge_kernel (+ the step's "
                                  "kv_append_kernel inside the timed region)"},
           "calls": {**spread, "what": f"{CALL_REPS} back-to-back decode calls at {lens[0]} rows"}}
    del c, cache, q, kn, vn, ws
    return res


def bench_decode_1m(args, torch, dk, synth, dev):
    leg = leg_decode_1m(args, torch, dk, synth, dev)
    print(json.dumps({
        "metric": METRIC, "value": leg["value"], "unit": "GB/s", "n_gpus": 1, "steps": leg["steps"], "warmup": 2,
        "ms_per_step": leg["wall_ms"] / leg["steps"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1)/sqrt(128) bf16)",
        "config": {"workload": leg["workload"], "global_batch": 1, "seq_len": 1048576, "parallelism": "none (1 GPU)"},
        "roofline": leg["roofline"], "calls": leg["calls"], "total_ms": leg["total_ms"]}), flush=True)


SWA_WINDOW = 1024   # YOCO's Self-Decoder window C


def swa_flops(n, window, hq, d):
    """4 d Hq per (query, visible key) pair; position p sees min(p + 1, C) keys."""
    c = min(window, n)
    return 4.0 * d * hq * (c * (c + 1) / 2.0 + (n - c) * c)


def bench_swa(args, torch, dk, synth, dev):
    """Sliding-window attention with C = 1024 at the prefill workload's shape
    (16 layer calls of a 32K prompt, Hq=16, Hkv=4), then token decode at the
    decode workload's heads (B=8, Hq=16, Hkv=2): per layer one ring append and
    one decode over that layer's full ring of C rows (16 rings)."""
    wp = synth.WORKLOADS["prefill_32k"]
    wd = synth.WORKLOADS["decode_128k"]
    C = SWA_WINDOW
    n = int(wp.seq_lens[0])
    t = time.perf_counter()
    pc, pcache, qs = make_prefill(dk, synth, dev, wp)
    cu = pc.cu_seqlens.to(dev)
    out_p = torch.empty_like(qs[0])
    lse_p = torch.empty(wp.q_heads, n, device=dev, dtype=torch.float32)
    pws = dk.alloc_prefill_workspace(dev)
    g = torch.Generator(device=dev).manual_seed(5)
    B, L = wd.batch, wd.layers
    rings = []
    for _ in range(L):
        kr = (torch.randn(B * C, wd.kv_heads, wd.head_dim, device=dev, generator=g) * wd.value_std).to(torch.bfloat16)
        vr = (torch.randn(B * C, wd.kv_heads, wd.head_dim, device=dev, generator=g) * wd.value_std).to(torch.bfloat16)
        rings.append(dk.SharedKV(kr, vr, torch.arange(B, device=dev, dtype=torch.int64) * C,
                                 torch.full((B,), 131071, device=dev, dtype=torch.int32),
                                 torch.full((B,), C, device=dev, dtype=torch.int32)))
    qd = (torch.randn(L, B, wd.q_heads, wd.head_dim, device=dev, generator=g) * wd.value_std).to(torch.bfloat16)
    kn = (torch.randn(B, wd.kv_heads, wd.head_dim, device=dev, generator=g) * wd.value_std).to(torch.bfloat16)
    ws = dk.alloc_workspace(rings[0], wd.q_heads, C)
    out_d = torch.empty(B, wd.q_heads, wd.head_dim, device=dev, dtype=torch.bfloat16)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    log(f"inputs ready in {time.perf_counter() - t:.1f} s")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def prefill():
        for layer in range(wp.layers):
            dk.xattn_prefill_window(pcache, qs[layer], cu, n, C, pc.scale, out=out_p, lse=lse_p, workspace=pws)

    def decode_step():
        for layer in range(L):
            dk.kv_append_ring(rings[layer], kn, kn, flag)
            dk.xattn_decode(rings[layer], qd[layer], C, wd.scale, ws, out=out_d)

    for _ in range(args.warmup):
        prefill()
        decode_step()
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(args.steps):
        prefill()
    ev[1].record()
    ev[2].record()
    for _ in range(args.steps):
        decode_step()
    ev[3].record()
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    layer_s = ev[0].elapsed_time(ev[1]) / 1e3 / (args.steps * wp.layers)
    flops = swa_flops(n, C, wp.q_heads, wp.head_dim)
    tfl = flops / layer_s / 1e12
    dec_layer_us = ev[2].elapsed_time(ev[3]) * 1e3 / (args.steps * L)
    print(json.dumps({
        "metric": "sliding-window prefill TFLOP/s (% MFMA peak) @32K, C=1024; window decode us per layer",
        "value": tfl, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": layer_s * 1e3 * wp.layers, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1)/sqrt(128) bf16)",
        "config": {"workload": "sliding window C=1024: prefill B=1 N=32768 Hq=16 Hkv=4 d=128, 16 layers; "
                               "decode B=8 Hq=16 Hkv=2 d=128, ring append + decode per layer, 16 layers",
                   "global_batch": 1, "seq_len": n, "window": C, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": tfl, "peak": BF16_DENSE_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tfl / BF16_DENSE_PEAK_TFLOPS, "traffic": None, "kernel": "prefill_bf16_kernel<128>",
                     "avg_launch_ms": layer_s * 1e3, "algorithmic_per_launch": flops},
        "decode": {"us_per_layer": dec_layer_us, "bytes_per_call": B * C * wd.kv_heads * wd.head_dim * 4,
                   "note": "ring append + decode of C rows per layer; 16 rings of 8 MiB fit the 256 MB "
                           "Infinity Cache, so this is a latency figure, not an HBM rate"}}), flush=True)


def bench_producer(args, torch, dk, synth, dev):
    """The shared cache's producer at the YOCO-3B geometry (d_model 3072, 8 KV
    heads of 128): RMSNorm(X) [W_K | W_V] for a 32K-row prompt appended to an
    empty cache (one GEMM of 2 * 32768 * 3072 * 2048 flop), then one row per
    sequence for 8 sequences (the decode-time append)."""
    T, dm, hkv, d, B = 32768, 3072, 8, 128, 8
    g = torch.Generator(device=dev).manual_seed(9)
    x = torch.randn(T, dm, device=dev, generator=g).to(torch.bfloat16)
    gain = (1.0 + 0.1 * torch.randn(dm, device=dev, generator=g)).to(torch.bfloat16)
    wk = (torch.randn(dm, hkv * d, device=dev, generator=g) / dm ** 0.5).to(torch.bfloat16)
    wv = (torch.randn(dm, hkv * d, device=dev, generator=g) / dm ** 0.5).to(torch.bfloat16)
    wp = dk.kv_project_pack(gain, wk, wv, hkv, d)
    kp = torch.empty(T, hkv, d, device=dev, dtype=torch.bfloat16)
    vp = torch.empty_like(kp)
    one = torch.tensor([0], dtype=torch.int64, device=dev)
    cap = torch.tensor([T], dtype=torch.int32, device=dev)
    cache = dk.SharedKV(kp, vp, one, torch.zeros(1, dtype=torch.int32, device=dev), cap)
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    # decode rows: 8 sequences, one row each, into caches with room
    dkp = torch.empty(B * 1024, hkv, d, device=dev, dtype=torch.bfloat16)
    dcache = dk.SharedKV(dkp, torch.empty_like(dkp), torch.arange(B, device=dev, dtype=torch.int64) * 1024,
                         torch.zeros(B, dtype=torch.int32, device=dev), torch.full((B,), 1024, dtype=torch.int32,
                                                                                 device=dev))
    xd = x[:B].contiguous()
    cud = torch.arange(B + 1, dtype=torch.int32, device=dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def prompt():
        cache.seq_len.zero_()
        dk.kv_project_append(cache, x, cu, wp, 1e-6, None, flag)

    def rows():
        dcache.seq_len.zero_()
        for _ in range(16):
            dk.kv_project_append(dcache, xd, cud, wp, 1e-6, None, flag)

    for _ in range(args.warmup):
        prompt()
        rows()
    torch.cuda.synchronize()
    # one event pair per append call: the cache length reset between calls
    # (a fill kernel of torch's) stays outside the timed launches
    pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    ev[0].record()
    for a, b in pev:
        cache.seq_len.zero_()
        a.record()
        dk.kv_project_append(cache, x, cu, wp, 1e-6, None, flag)
        b.record()
    ev[1].record()
    ev[2].record()
    for _ in range(args.steps):
        rows()
    ev[3].record()
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    call_s = sum(a.elapsed_time(b) for a, b in pev) / 1e3 / args.steps
    flops = 2.0 * T * dm * 2 * hkv * d
    tfl = flops / call_s / 1e12
    row_us = ev[2].elapsed_time(ev[3]) * 1e3 / (args.steps * 16)
    wbytes = 2 * hkv * d * dm * 2
    print(json.dumps({
        "metric": "producer TFLOP/s (% MFMA peak) for a 32K prompt; us per decode-time append of 8 rows",
        "value": tfl, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": call_s * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) rows, N(0,1)/sqrt(d_model) weights, bf16)",
        "config": {"workload": "RMSNorm(X) [W_K|W_V] appended to the shared cache: T=32768 d_model=3072 Hkv=8 d=128",
                   "global_batch": 1, "seq_len": T, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": tfl, "peak": BF16_DENSE_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tfl / BF16_DENSE_PEAK_TFLOPS, "traffic": None,
                     "kernel": "kv_project_wide_kernel + kv_commit_kernel (one call, timed together)",
                     "avg_launch_ms": call_s * 1e3, "algorithmic_per_launch": flops},
        "decode_rows": {"us_per_call": row_us, "rows": B, "weight_bytes": wbytes,
                        "weight_read_GBps": wbytes / (row_us / 1e6) / 1e9,
                        "note": "the 12.6 MB of packed weights stay in the Infinity Cache between calls"}}),
        flush=True)


GRET_CHUNK = 256


def gret_chunk_flops(n, d):
    """MFMA work of the chunkwise form per head: per chunk of c rows, the causal
    Q K^T and P V products (2 d c(c+1)/2 each), the carried state Q S and the
    chunk's contribution K^T V (2 c d^2 each)."""
    total, r = 0.0, 0
    while r < n:
        c = min(GRET_CHUNK, n - r)
        total += 2.0 * d * c * (c + 1) + 4.0 * c * d * d
        r += c
    return total


def bench_gret(args, torch, dk, synth, dev):
    """Gated retention at the prefill workload's length: one chunkwise prefill of
    32768 rows x 16 heads (d = 128) per layer call, 16 calls; then recurrent
    decode steps for 8 sequences x 16 heads."""
    N, H, d, B = 32768, 16, 128, 8
    g = torch.Generator(device=dev).manual_seed(13)
    std = d ** -0.25
    q = (torch.randn(N, H, d, device=dev, generator=g) * std).to(torch.bfloat16)
    k = (torch.randn(N, H, d, device=dev, generator=g) * std).to(torch.bfloat16)
    v = torch.randn(N, H, d, device=dev, generator=g).to(torch.bfloat16)
    gam = 0.9 + 0.1 * torch.rand(N, H, device=dev, generator=g)
    cu = torch.tensor([0, N], dtype=torch.int32, device=dev)
    ws = torch.empty(dk.gret_workspace_size(1, H, d, N), dtype=torch.uint8, device=dev)   # N rows in all
    st = torch.empty(1, H, d, d, device=dev)
    out = torch.empty_like(v)
    qd = (torch.randn(B, H, d, device=dev, generator=g) * std).to(torch.bfloat16)
    kd = (torch.randn(B, H, d, device=dev, generator=g) * std).to(torch.bfloat16)
    vd = torch.randn(B, H, d, device=dev, generator=g).to(torch.bfloat16)
    gd = 0.9 + 0.1 * torch.rand(B, H, device=dev, generator=g)
    state = torch.zeros(B, H, d, d, device=dev)
    outd = torch.empty_like(vd)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    L = 16
    for _ in range(args.warmup):
        dk.gret_prefill(q, k, v, gam, cu, ws, state_out=st, out=out)
        dk.gret_decode(qd, kd, vd, gd, state, out=outd)
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(args.steps * L):
        dk.gret_prefill(q, k, v, gam, cu, ws, state_out=st, out=out)
    ev[1].record()
    ev[2].record()
    for _ in range(args.steps * L):
        dk.gret_decode(qd, kd, vd, gd, state, out=outd)
    ev[3].record()
    torch.cuda.synchronize()
    call_s = ev[0].elapsed_time(ev[1]) / 1e3 / (args.steps * L)
    flops = H * gret_chunk_flops(N, d)
    tfl = flops / call_s / 1e12
    # 128 flop per byte of input and output, below the ridge point (2.5 PFLOP/s / 8 TB/s):
    # the bound is HBM; algorithmic bytes = Q, K, V and the gates read once, O and the
    # final state written once
    alg_bytes = 4 * N * H * d * 2 + N * H * 4 + H * d * d * 4
    gbs = alg_bytes / call_s / 1e9
    dec_us = ev[2].elapsed_time(ev[3]) * 1e3 / (args.steps * L)
    state_bytes = B * H * d * d * 4 * 2
    print(json.dumps({
        "metric": "gRet chunkwise prefill GB/s (% HBM peak) @32K x 16 heads; recurrent decode us per step",
        "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": call_s * 1e3 * L, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded q, k ~ N(0, d^-1/2), v ~ N(0,1), gates U[0.9, 1), bf16)",
        "config": {"workload": "gated retention: prefill N=32768 H=16 d=128 (chunk 256), 16 layer calls; "
                               "decode B=8 H=16 d=128, 16 layer steps", "global_batch": 1, "seq_len": N,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, **gret_traffic_fields(call_s),
                     "kernel": "gret_segstate_kernel + gret_segscan_kernel + gret_out_kernel (one call, timed together)",
                     "avg_launch_ms": call_s * 1e3, "algorithmic_per_launch": alg_bytes,
                     "mfma_tflops": tfl, "mfma_flops_per_launch": flops},
        "decode": {"us_per_step": dec_us, "state_bytes_per_step": state_bytes,
                   "GBps": state_bytes / (dec_us / 1e6) / 1e9,
                   "note": "8 MiB of fp32 state read and written per step; it stays in the Infinity Cache"}}),
        flush=True)


def leg_ragged(args, torch, dk, synth, dev):
    """16 prompts of log-uniform lengths (Hq=32, Hkv=8): their causal prefill
    (timed over `steps` calls), then 32 decode steps of one append and one
    layer call, each decode call timed on its own."""
    w = synth.WORKLOADS["ragged"]
    t = time.perf_counter()
    pc = synth.make_prefill_case(list(w.seq_lens), w.q_heads, w.kv_heads, w.head_dim, 1, w.dtype, w.seed,
                                 w.value_std, cap_extra=w.decode_steps)
    dc = synth.make_decode_case([1] * w.batch, w.q_heads, w.kv_heads, w.head_dim, 1, w.decode_steps, w.dtype,
                                w.seed, w.value_std)
    cache = dk.SharedKV(pc.k_pool.to(dev), pc.v_pool.to(dev), pc.seq_start.to(dev), pc.seq_len.to(dev).clone(),
                        pc.seq_cap.to(dev))
    log(f"ragged inputs ready in {time.perf_counter() - t:.1f} s")
    q = pc.q[0].to(dev)
    del pc.q
    cu = pc.cu_seqlens.to(dev)
    maxq = max(w.seq_lens)
    out = torch.empty_like(q)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    steps = max(args.steps, 1)
    pws = dk.alloc_prefill_workspace(dev)
    for _ in range(args.warmup):
        dk.xattn_prefill(cache, q, cu, maxq, pc.scale, out=out, workspace=pws)
    torch.cuda.synchronize()
    e[0].record()
    for _ in range(steps):
        dk.xattn_prefill(cache, q, cu, maxq, pc.scale, out=out, workspace=pws)
    e[1].record()
    torch.cuda.synchronize()
    pre_ms = e[0].elapsed_time(e[1]) / steps
    flops = prefill_flops(w.seq_lens, w.q_heads, w.head_dim)
    qd = dc.q.to(dev)
    kn, vn = dc.k_new.to(dev), dc.v_new.to(dev)
    ws = dk.alloc_workspace(cache, w.q_heads, maxq + w.decode_steps)
    outd = torch.empty(w.batch, w.q_heads, w.head_dim, device=dev, dtype=torch.bfloat16)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    lens = list(w.seq_lens)
    # untimed decode calls first (decode leaves the cache as it is): the first
    # launch of a kernel pays for loading its code object
    for _ in range(max(args.warmup, 1)):
        dk.xattn_decode(cache, qd[0, 0], maxq + w.decode_steps, pc.scale, ws, out=outd, total_kv_len=sum(lens))
    torch.cuda.synchronize()
    nbytes = 0.0
    # one event before each decode call and one after it: the call (split +
    # merge) is timed apart from the step's append, which is its own entry point
    ec = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(w.decode_steps)]
    e[2].record()
    for s in range(w.decode_steps):
        dk.kv_append(cache, kn[s], vn[s], flag)
        lens = [x + 1 for x in lens]
        ec[s][0].record()
        dk.xattn_decode(cache, qd[s, 0], maxq + w.decode_steps, pc.scale, ws, out=outd, total_kv_len=sum(lens))
        ec[s][1].record()
        nbytes += decode_bytes(lens, w.kv_heads, w.q_heads, w.head_dim)
    e[3].record()
    torch.cuda.synchronize()
    dms = e[2].elapsed_time(e[3])
    call_ms = [a.elapsed_time(b) for a, b in ec]
    cms = sum(call_ms)
    assert int(flag.item()) == 0
    tfl = flops / (pre_ms / 1e3) / 1e12
    gbs = nbytes / (cms / 1e3) / 1e9
    gbs_step = nbytes / (dms / 1e3) / 1e9
    res = {"workload": f"ragged: 16 seqs L={list(w.seq_lens)} Hq=32 Hkv=8 d=128; prefill + 32 decode steps",
           "prefill": {"value": tfl, "unit": "TFLOP/s", "avg_call_ms": pre_ms, "calls": steps,
                       "algorithmic_flops_per_call": flops,
                       "roofline": {"bound": "mfma", "achieved": tfl, "peak": BF16_DENSE_PEAK_TFLOPS,
                                    "unit": "TFLOP/s", "frac": tfl / BF16_DENSE_PEAK_TFLOPS, "traffic": None,
                                    "kernel": "prefill_bf16_kernel<128>"}},
           "decode": {"value": gbs, "unit": "GB/s", "avg_call_ms": cms / w.decode_steps,
                      "algorithmic_bytes_per_call": nbytes / w.decode_steps,
                      "what": "per decode call (split + merge launches), bytes of the call over its time",
                      "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                                   "kernel": "decode_split_bf16_kernel<128, 1, 1> + decode_merge_kernel"},
                      "call_median_ms": float(sorted(call_ms)[len(call_ms) // 2]), "call_min_ms": min(call_ms),
                      "steps": {"GB/s": gbs_step, "frac": gbs_step / HBM_PEAK_GBS,
                                "avg_step_ms": dms / w.decode_steps,
                                "what": "append + decode call per step, bytes of the call over the step"}},
           "ms_per_step": pre_ms + dms / w.decode_steps}
    del cache, q, out, qd, kn, vn, ws
    return res


def bench_ragged(args, torch, dk, synth, dev):
    leg = leg_ragged(args, torch, dk, synth, dev)
    w = synth.WORKLOADS["ragged"]
    pre = leg["prefill"]
    print(json.dumps({
        "metric": METRIC, "value": pre["value"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": leg["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1)/sqrt(128) bf16)",
        "config": {"workload": leg["workload"], "global_batch": 16, "seq_len": max(w.seq_lens),
                   "parallelism": "none (1 GPU)"},
        "roofline": {**pre["roofline"], "avg_launch_ms": pre["avg_call_ms"]},
        "decode": leg["decode"]}), flush=True)


if __name__ == "__main__":
    main()
