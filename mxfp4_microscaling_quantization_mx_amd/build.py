"""Build libmxfp4.so (and the test probe library) in-tree with hipcc for gfx950.

    python -m mxfp4_microscaling_quantization_mx_amd.build

Every HIP translation unit is compiled with packed-FP32 instruction selection
disabled and without floating-point contraction, so the quantizer's float32
operations happen exactly in the order written.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmxfp4.so")
PROBE_SRC = os.path.join(ROOT, "tests", "gpu_probes.hip")
PROBE_LIB = os.path.join(ROOT, "tests", "libmxprobe.so")

ARCH = os.environ.get("MX_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off", "-Wall", "-Wno-unused-function",
]
SOURCES = ["mx_api.cpp", "quantize.hip", "dequantize.hip", "transpose.hip", "gemm.hip", "gemm_splitk.hip", "clip.hip"]


def _run(cmd):
    print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def _compile(src, obj):
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    _run([HIPCC] + CFLAGS + lang + ["-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj])


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(os.path.join(CSRC, s), os.path.join(BUILD, os.path.splitext(s)[0] + ".o")) for s in SOURCES]
    probe = os.path.exists(PROBE_SRC)
    if probe:
        jobs.append((PROBE_SRC, os.path.join(BUILD, "gpu_probes.o")))
    # the translation units are independent: compile them side by side
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(workers) as pool:
        for f in [pool.submit(_compile, src, obj) for src, obj in jobs]:
            f.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp] + [obj for _, obj in jobs[:len(SOURCES)]])
    os.replace(tmp, LIB)
    if probe:
        tmp = PROBE_LIB + ".tmp"
        _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, jobs[-1][1]])
        os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
