"""Build the HIP libraries in-tree (gfx950):

* decoder_shared_kv_amd/lib/libyoco_xattn.so: the attention path, exporting the
  C ABI declared in include/yoco_xattn.h;
* decoder_shared_kv_amd/lib/libyoco_probe.so: the benchmark's streaming-read
  probe (csrc/read_probe.hip), a measuring instrument kept out of the ABI.

Every source is compiled by hipcc for gfx950 only, with packed fp32
instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "lib", "obj")
LIB = os.path.join(HERE, "lib", "libyoco_xattn.so")
PROBE_LIB = os.path.join(HERE, "lib", "libyoco_probe.so")
PROBE_SOURCES = ["read_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "kv_append.hip", "attn_f32.hip", "decode_merge.hip", "decode_bf16.hip", "prefill_bf16.hip",
           "kv_project.hip", "gret.hip", "scratch.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, src.rsplit(".", 1)[0] + ".o")
    cmd = [HIPCC, "-x", "hip", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in ln)  # the host pass does not know the device feature
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    if errs.strip():
        print(errs, file=sys.stderr)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    sources = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(_compile, sources))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
