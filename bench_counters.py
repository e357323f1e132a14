"""HBM traffic of the benchmark's kernels from rocprofv3 counters.

`python bench_counters.py collect <dir>` (on a GPU machine) runs, each in a
process of its own under rocprofv3, with its raw output under <dir>:
  * FETCH_SIZE, then WRITE_SIZE, of the prefill run of `bench.py` (the prefill
    kernel), of its decode run (the decode kernels) and of `bench.py --workload
    gret` (the three gated-retention prefill kernels);
  * the same two counters of `bench.py --copy-probe` (a plain 1 GiB device copy),
    which calibrate them: bytes per KiB of counter = copied bytes / counter.
It writes profiles/traffic.json (per kernel: fetch and write bytes per launch,
the calibration factors, and the SHA-256 of the kernel's source files) and a
text summary per kernel. bench.py reports a kernel's traffic only while those
source hashes still match.

`python bench_counters.py summarize <dir>` rebuilds the files from the CSVs of
an earlier collection without running anything.

`python bench_counters.py collect-sq <dir> [prefill|gret]` collects
shader-sequencer counters (MFMA utilisation, VALU busy, instruction mix, wait
shares, clock) of the prefill kernel, or of the gRet prefill's output and
state-contribution kernels, in two passes and writes
profiles/{prefill,gret}_sq_counters.{txt,json}; `summarize-sq <dir> [target]`
rebuilds them.

`python bench_counters.py stats <run_kernel_stats.csv> <out.txt> <title> <command>`
writes the text summary of a rocprofv3 --kernel-trace --stats run.
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
    "gret_segstate_kernel<128>": ["gret.hip", "internal.h", "lds_copy.h", "tile_common.h"],
    "gret_segscan_kernel<128>": ["gret.hip", "internal.h", "lds_copy.h", "tile_common.h"],
    "gret_out_kernel<128>": ["gret.hip", "internal.h", "lds_copy.h", "tile_common.h"],
}
# the run whose counters describe each kernel
KERNEL_RUN = {"prefill_bf16_kernel<128>": "prefill", "gret_segstate_kernel<128>": "gret",
              "gret_segscan_kernel<128>": "gret", "gret_out_kernel<128>": "gret"}

RUNS = {
    "prefill": ["--skip", "decode,decode_1m,ragged", "--steps", "1", "--warmup", "0", "--no-cpu-baseline"],
    "decode": ["--skip", "prefill,decode_1m,ragged", "--steps", "2", "--warmup", "1", "--no-cpu-baseline"],
    "gret": ["--workload", "gret", "--steps", "1", "--warmup", "0"],
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
        run = KERNEL_RUN.get(prefix, "decode")
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


# Shader-sequencer counters of a benchmark run's kernels, in passes small enough
# for one rocprofv3 collection each (6 SQ counters and GRBM_GUI_ACTIVE per pass).
# MfmaUtil, VALUBusy and LDSBankConflict are rocprofv3's derived metrics
# (reduce(SQ_VALU_MFMA_BUSY_CYCLES, sum) / (reduce(GRBM_GUI_ACTIVE, max) *
# SIMD_NUM) * 100, and alike).
SQ_PASSES = {
    "a": ["MfmaUtil", "VALUBusy", "LDSBankConflict", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_TRANS_F32",
          "GRBM_GUI_ACTIVE"],
    "b": ["SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_LDS",
          "GRBM_GUI_ACTIVE"],
}
# target -> the run, its kernels, the file stem under profiles/ and the workload in words
SQ_TARGETS = {
    "prefill": {"run": "prefill", "kernels": ["prefill_bf16_kernel<128>"], "stem": "prefill_sq_counters",
                "what": "32K causal prefill, Hq=16, Hkv=4, d=128"},
    "gret": {"run": "gret", "kernels": ["gret_out_kernel<128>", "gret_segstate_kernel<128>"],
             "stem": "gret_sq_counters", "what": "gRet chunkwise prefill, 32K rows x 16 heads, d=128"},
}


def _sq_dir(src_dir, target, name):
    # the prefill's passes keep their original directory names
    return os.path.join(src_dir, f"sq_{name}" if target == "prefill" else f"sq_{target}_{name}")


def collect_sq(out, target="prefill"):
    out = os.path.abspath(out)
    os.makedirs(out, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp")
    run = SQ_TARGETS[target]["run"]
    for name, counters in SQ_PASSES.items():
        d = _sq_dir(out, target, name)
        cmd = ["rocprofv3", "--pmc", *counters, "--output-format", "csv", "-d", d, "-o", "run", "--",
               sys.executable, os.path.join(ROOT, "bench.py"), *RUNS[run]]
        print(f"[counters] {target} SQ pass {name}: {' '.join(counters)}", flush=True)
        t = time.time()
        r = subprocess.run(cmd, cwd="/tmp", env=env, capture_output=True, text=True, timeout=240)
        if r.returncode != 0 or not os.path.exists(os.path.join(d, "run_counter_collection.csv")):
            print(r.stdout[-2000:], r.stderr[-2000:], file=sys.stderr)
            raise SystemExit(f"rocprofv3 failed for SQ pass {name}")
        print(f"[counters]   done in {time.time() - t:.0f} s", flush=True)
    summarize_sq(out, target)


def _kernel_rows(path, prefix):
    """{counter: [value per dispatch]} and [(start, end) ns per dispatch] of one kernel."""
    vals, spans = {}, {}
    with open(os.path.join(path, "run_counter_collection.csv")) as f:
        for row in csv.DictReader(f):
            if prefix not in row["Kernel_Name"]:
                continue
            vals.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
            if row.get("Start_Timestamp") and row.get("End_Timestamp"):
                spans[row.get("Dispatch_Id", len(spans))] = (float(row["Start_Timestamp"]), float(row["End_Timestamp"]))
    return vals, list(spans.values())


def _sq_kernel(src_dir, target, kernel):
    per = {}
    durations = []
    for name in SQ_PASSES:
        vals, spans = _kernel_rows(_sq_dir(src_dir, target, name), kernel)
        for k, v in vals.items():
            per.setdefault(k, []).extend(v)
        durations += [e - s for s, e in spans if e > s]
    mean = {k: sum(v) / len(v) for k, v in per.items() if v}
    launches = {k: len(v) for k, v in per.items()}
    dur_ns = sum(durations) / len(durations) if durations else None
    xcc = 8
    derived = {}
    if "GRBM_GUI_ACTIVE" in mean and dur_ns:
        derived["clock_MHz (GRBM_GUI_ACTIVE / 8 XCCs / duration)"] = mean["GRBM_GUI_ACTIVE"] / xcc / dur_ns * 1e3
    if "SQ_INSTS_MFMA" in mean and mean["SQ_INSTS_MFMA"] > 0:
        derived["VALU instructions per MFMA"] = mean.get("SQ_INSTS_VALU", 0) / mean["SQ_INSTS_MFMA"]
        derived["fp32 transcendentals per MFMA"] = mean.get("SQ_INSTS_VALU_TRANS_F32", 0) / mean["SQ_INSTS_MFMA"]
        derived["LDS instructions per MFMA"] = mean.get("SQ_INSTS_LDS", 0) / mean["SQ_INSTS_MFMA"]
    if "SQ_WAVE_CYCLES" in mean and mean["SQ_WAVE_CYCLES"] > 0:
        derived["share of wave time waiting (SQ_WAIT_ANY / SQ_WAVE_CYCLES)"] = mean.get("SQ_WAIT_ANY", 0) / mean["SQ_WAVE_CYCLES"]
        derived["share of wave time waiting for an instruction (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES)"] = \
            mean.get("SQ_WAIT_INST_ANY", 0) / mean["SQ_WAVE_CYCLES"]
    return {"kernel": kernel, "source_sha256": source_hash(KERNELS[kernel]), "mean_per_launch": mean,
            "launches": launches, "duration_ns": dur_ns, "derived": derived}


def summarize_sq(src_dir, target="prefill"):
    tg = SQ_TARGETS[target]
    results = [_sq_kernel(src_dir, target, k) for k in tg["kernels"]]
    workload = "bench.py " + " ".join(RUNS[tg["run"]])
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, tg["stem"] + ".json"), "w") as f:
        if len(results) == 1:
            json.dump({**results[0], "workload": workload, "passes": SQ_PASSES}, f, indent=1)
        else:
            json.dump({"workload": workload, "passes": SQ_PASSES, "kernels": results}, f, indent=1)
    cmd = "python bench_counters.py collect-sq <dir>" + ("" if target == "prefill" else f" {target}")
    lines = []
    for res in results:
        mean, launches, dur_ns = res["mean_per_launch"], res["launches"], res["duration_ns"]
        lines += [f"Shader-sequencer counters of {res['kernel']} ({tg['what']}), per launch",
                  f"command: {cmd}   (per pass: rocprofv3 --pmc <counters> --output-format csv -d <dir> -o run "
                  f"-- python {workload})",
                  "passes: " + "; ".join(f"{k}: {' '.join(v)}" for k, v in SQ_PASSES.items()),
                  f"source sha256 {res['source_sha256'][:16]}, mean kernel duration under the counters: "
                  + (f"{dur_ns / 1e3:.1f} us" if dur_ns else "n/a"), ""]
        for k in sorted(mean):
            lines.append(f"{k:32s} {mean[k]:16.6g}   ({launches[k]} dispatches)")
        lines.append("")
        for k, v in res["derived"].items():
            lines.append(f"{k}: {v:.4g}")
        lines.append("")
    with open(os.path.join(PROFILES, tg["stem"] + ".txt"), "w") as f:
        f.write("\n".join(lines).rstrip("\n") + "\n")
    print("\n".join(lines))


def kernel_stats(csv_path, out_path, title, command):
    """Text summary of a rocprofv3 --kernel-trace --stats run (run_kernel_stats.csv)."""
    import re
    rows = []
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            name = row["Name"]
            m = re.search(r"::([A-Za-z_0-9]+<[^()]*>)\(", name) or re.search(r"::([A-Za-z_0-9]+)\(", name)
            short = m.group(1) if m else name[:70]
            rows.append((short, int(row["Calls"]), float(row["AverageNs"]) / 1e3, float(row["MinNs"]) / 1e3,
                         float(row["MaxNs"]) / 1e3))
    lines = [title, f"command: {command}", "",
             f"{'kernel':72s}{'calls':>7s}{'avg us':>11s}{'min us':>11s}{'max us':>11s}"]
    for short, calls, avg, mn, mx in rows:
        lines.append(f"{short[:72]:72s}{calls:7d}{avg:11.1f}{mn:11.1f}{mx:11.1f}")
    with open(out_path, "w") as f:
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
    elif len(sys.argv) >= 6 and sys.argv[1] == "stats":
        kernel_stats(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5])
    elif len(sys.argv) >= 3 and sys.argv[1] == "collect-sq":
        collect_sq(sys.argv[2], *sys.argv[3:4])
    elif len(sys.argv) >= 3 and sys.argv[1] == "summarize-sq":
        summarize_sq(sys.argv[2], *sys.argv[3:4])
    else:
        print(__doc__)
        sys.exit(2)
