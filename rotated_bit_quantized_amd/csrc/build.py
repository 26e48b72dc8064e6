"""Build librbq.so in-tree for gfx950 (host C++ with g++, kernels with hipcc).

Usage: ``python rotated_bit_quantized_amd/csrc/build.py`` (or ``build()`` from
``__graft_entry__``).  Always recompiles.  The shared library lands next to the
Python binding: ``rotated_bit_quantized_amd/librbq.so``.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "librbq.so")
# the streaming-read probe (a measurement helper, not the method) is a library
# of its own
PROBE_SOURCE = "rbq_probe.hip"
PROBE_LIB = os.path.join(PKG, "librbq_probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_SOURCES = ["rbq_append.hip", "rbq_attn_mfma.hip", "rbq_attn_prefill.hip", "rbq_attn_tile.hip"]
HOST_SOURCES = ["rbq_host.cpp"]
# per-file extras: the attention kernels never rely on NaN semantics (masked
# scores are -inf), which lets max reductions compile to single DPP ops
HIP_FILE_FLAGS = {"rbq_attn_mfma.hip": ["-fno-honor-nans"], "rbq_attn_prefill.hip": ["-fno-honor-nans"]}

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-I", INCLUDE, "-I", HERE,
    # no packed fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division and sqrt, fp32 subnormals kept: the quantizer's
    # decisions must match the definition bit for bit
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-ffp-contract=fast",
]
HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-ffp-contract=off",
              "-I", INCLUDE, "-I", HERE, "-I", "/opt/rocm/include"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build step failed: " + " ".join(cmd[:3]) + " ...")
    out = (r.stdout + r.stderr).strip()
    if verbose and out:
        print(out)


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    jobs = []  # (command, object), compiled side by side
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        jobs.append(["g++", *HOST_FLAGS, "-c", os.path.join(HERE, src), "-o", obj])
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, *HIP_FILE_FLAGS.get(src, []), "-c", os.path.join(HERE, src),
                     "-o", obj])
        objs.append(obj)
    pobj = os.path.join(OUT_DIR, PROBE_SOURCE + ".o")
    jobs.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(HERE, PROBE_SOURCE), "-o", pobj])
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as pool:
        for f in [pool.submit(_run, cmd, verbose) for cmd in jobs]:
            f.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    shutil.move(tmp, LIB)
    ptmp = PROBE_LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", ptmp, pobj], verbose)
    shutil.move(ptmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
