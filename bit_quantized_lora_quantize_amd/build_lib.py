"""Build libqlora.so in-tree with hipcc for gfx950 (CDNA4).

Also builds two variants from the same sources:
  libqlora_wide.so   a test build identical except that the backward GEMM
                     takes its per-step weight-descriptor path (otherwise used
                     only for packed weights beyond 2^31 bytes) at every size,
                     so that tests can check that path against the oracle at
                     ordinary sizes;
  libqlora_peaks.so  not the library: the benchmark's streaming-read and
                     MFMA-loop microbenchmarks (measured peaks);
  libqlora_timed.so  a benchmark build that also exports
                     qlora_time_next_weight_kernel (include/qlora_timing.h),
                     an event pair around the next weight-kernel launch; the
                     library proper keeps no such state;
  libqlora_san.so    a test build whose host code in api.cpp and noalloc.hip
                     (argument checks, plans, workspace carving) is built with
                     AddressSanitizer and UndefinedBehaviorSanitizer; the GPU
                     code is the same.  Loaded with the clang ASan runtime
                     preloaded (tests/test_sanitized.py).

Usage: python -m bit_quantized_lora_quantize_amd.build_lib [--jobs N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build", "libqlora")
LIB = os.path.join(PKG, "libqlora.so")
LIB_WIDE = os.path.join(PKG, "libqlora_wide.so")
LIB_TIMED = os.path.join(PKG, "libqlora_timed.so")
LIB_PEAKS = os.path.join(PKG, "libqlora_peaks.so")
LIB_SAN = os.path.join(PKG, "libqlora_san.so")
# host code built with sanitizers in libqlora_san.so (each -fsanitize= applies
# to the host pass only)
SAN_SOURCES = ["api.cpp", "noalloc.hip"]
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
# sources that hold the timing hook or launch a weight kernel
TIMED_SOURCES = ["quant.hip", "gemv.hip", "gemm.hip", "api.cpp"]

SOURCES = ["quant.hip", "quant_blocked.hip", "lora.hip", "gemv.hip", "gemm.hip", "merge.hip", "optim.hip", "dropout.hip", "noalloc.hip", "api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # every FP32 product and sum is rounded on its own (restored weights are
    # defined without fused multiply-add); IEEE division; no fast-math
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # packed FP32 VALU instructions stay off
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _compile(src: str, tag: str = "", defines: tuple = ()) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + tag + ".o")
    cmd = [HIPCC, *CFLAGS, *defines, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    # the host pass does not know the packed-fp32 feature: drop that notice
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in res.stderr.splitlines() if noise not in l).strip()
    if msg:
        print(msg, file=sys.stderr)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)


def build(jobs: int = 6) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        # the slowest compile (the GEMM) of each variant first
        wide = ex.submit(_compile, "gemm.hip", "_wide", ("-DQLORA_WIDE_CODE_BYTES=0",))
        timed = {src: ex.submit(_compile, src, "_timed", ("-DQLORA_TIMING_HOOK=1",))
                 for src in TIMED_SOURCES}
        peaks = ex.submit(_compile, "peaks.hip")
        san = {src: ex.submit(_compile, src, "_san", tuple(SAN_FLAGS)) for src in SAN_SOURCES}
        objs = list(ex.map(_compile, SOURCES))
        wide_obj = wide.result()
        timed_objs = {src: f.result() for src, f in timed.items()}
        san_objs = {src: f.result() for src, f in san.items()}
    _link(objs, LIB)
    _link([wide_obj if os.path.basename(o) == "gemm.hip.o" else o for o in objs], LIB_WIDE)
    _link([timed_objs.get(os.path.basename(o)[:-2], o) for o in objs], LIB_TIMED)
    _link([san_objs.get(os.path.basename(o)[:-2], o) for o in objs], LIB_SAN)
    _link([peaks.result()], LIB_PEAKS)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=6)
    print(build(ap.parse_args().jobs))
