"""HBM traffic of the benchmark's kernels from rocprofv3 counters.

`python bench_counters.py collect <dir>` (on a GPU machine) runs, each in a
process of its own under rocprofv3, with its raw output under <dir>:
  * FETCH_SIZE, then WRITE_SIZE, of `bench.py --skip decode` (the prefill kernel)
    and of `bench.py --skip prefill` (the decode kernels);
  * the same two counters of `bench.py --copy-probe` (a plain 1 GiB device copy),
    which calibrate them: bytes per KiB of counter = copied bytes / counter.
It writes profiles/traffic.json (per kernel: fetch and write bytes per launch,
the calibration factors, and the SHA-256 of the kernel's source files) and a
text summary per kernel. bench.py reports a kernel's traffic only while those
source hashes still match.

`python bench_counters.py summarize <dir>` rebuilds the files from the CSVs of
an earlier collection without running anything.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "decoder_shared_kv_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")

# kernel name prefix -> source files whose hash identifies it
KERNELS = {
    "prefill_bf16_kernel<128>": ["prefill_bf16.hip", "internal.h", "lds_copy.h", "tile_common.h"],
    "decode_split_bf16_kernel<128, 1, 0>": ["decode_bf16.hip", "internal.h", "tile_common.h"],
    "decode_merge_kernel<128, 16, 1, __hip_bfloat16>": ["decode_merge.hip", "internal.h", "tile_common.h"],
}

RUNS = {
    "prefill": ["--skip", "decode,decode_1m,ragged", "--steps", "1", "--warmup", "0", "--no-cpu-baseline"],
    "decode": ["--skip", "prefill,decode_1m,ragged", "--steps", "2", "--warmup", "1", "--no-cpu-baseline"],
    "copy": ["--copy-probe"],
}
COPY_BYTES = 1 << 30


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def command(run, counter, out):
    d = os.path.join(out, f"{run}_{counter}")
    return ["rocprofv3", "--pmc", counter, "--output-format", "csv", "-d", d, "-o", "run", "--",
            sys.executable, os.path.join(ROOT, "bench.py"), *RUNS[run]], d


def collect(out):
    out = os.path.abspath(out)
    os.makedirs(out, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp")
    for run in RUNS:
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            cmd, d = command(run, counter, out)
            print(f"[counters] {run} {counter}", flush=True)
            t = time.time()
            r = subprocess.run(cmd, cwd="/tmp", env=env, capture_output=True, text=True, timeout=240)
            if r.returncode != 0 or not os.path.exists(os.path.join(d, "run_counter_collection.csv")):
                print(r.stdout[-2000:], r.stderr[-2000:], file=sys.stderr)
                raise SystemExit(f"rocprofv3 failed for {run} {counter}")
            print(f"[counters]   done in {time.time() - t:.0f} s", flush=True)
    summarize(out)


def _per_kernel(path, counter):
    agg = {}
    with open(os.path.join(path, "run_counter_collection.csv")) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            agg.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return agg


def _match(name, prefix):
    return prefix in name


def summarize(src_dir):
    cal = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        agg = _per_kernel(os.path.join(src_dir, f"copy_{counter}"), counter)
        copy = [v for k, v in agg.items() if "copyBuffer" in k]
        kib = sum(copy[0]) / len(copy[0])
        cal[counter] = COPY_BYTES / kib      # bytes per KiB of counter
    result = {"calibration_bytes_per_counter_kib": cal, "copy_bytes": COPY_BYTES, "kernels": {}}
    for prefix, files in KERNELS.items():
        run = "prefill" if prefix.startswith("prefill") else "decode"
        entry = {"source_sha256": source_hash(files), "workload": run}
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            agg = _per_kernel(os.path.join(src_dir, f"{run}_{counter}"), counter)
            vals = [v for k, vs in agg.items() if _match(k, prefix) for v in vs]
            if not vals:
                raise SystemExit(f"no {counter} samples for {prefix}")
            entry[counter.lower() + "_kib_per_launch"] = sum(vals) / len(vals)
            entry[counter.lower().replace("_size", "") + "_bytes_per_launch"] = sum(vals) / len(vals) * cal[counter]
            entry["launches"] = len(vals)
        entry["traffic_bytes_per_launch"] = entry["fetch_bytes_per_launch"] + entry["write_bytes_per_launch"]
        result["kernels"][prefix] = entry
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, "traffic.json"), "w") as f:
        json.dump(result, f, indent=1)
    lines = ["HBM traffic per launch from rocprofv3 counters (FETCH_SIZE, WRITE_SIZE; one counter per run)",
             "command: python bench_counters.py collect <dir>   (runs, per counter and workload:",
             "  rocprofv3 --pmc <COUNTER> --output-format csv -d <dir> -o run -- python bench.py <args>)",
             "workload args: " + "; ".join(f"{k}: {' '.join(v)}" for k, v in RUNS.items()),
             f"calibration (plain 1 GiB device copy): FETCH_SIZE x {cal['FETCH_SIZE']:.1f} B/KiB, "
             f"WRITE_SIZE x {cal['WRITE_SIZE']:.1f} B/KiB", ""]
    for prefix, e in result["kernels"].items():
        lines.append(f"{prefix}: FETCH_SIZE {e['fetch_size_kib_per_launch']:.0f} KiB -> {e['fetch_bytes_per_launch'] / 1e9:.4f} GB, "
                     f"WRITE_SIZE {e['write_size_kib_per_launch']:.0f} KiB -> {e['write_bytes_per_launch'] / 1e9:.4f} GB "
                     f"per launch ({e['launches']} launches), source sha256 {e['source_sha256'][:16]}")
    with open(os.path.join(PROFILES, "hbm_traffic_counters.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def traffic_for(prefix):
    """Bytes per launch for a kernel, or None if absent or its source changed."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    e = data.get("kernels", {}).get(prefix)
    if e is None or e.get("source_sha256") != source_hash(KERNELS[prefix]):
        return None
    return e["traffic_bytes_per_launch"]


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "collect":
        collect(sys.argv[2])
    elif len(sys.argv) >= 3 and sys.argv[1] == "summarize":
        summarize(sys.argv[2])
    else:
        print(__doc__)
        sys.exit(2)
