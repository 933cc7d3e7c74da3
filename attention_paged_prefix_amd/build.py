"""Build libkvb.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc.

Usage: ``python -m attention_paged_prefix_amd.build`` or ``build()`` from Python.
Every call recompiles.  Objects go to ``attention_paged_prefix_amd/_build/``.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libkvb.so")
BUILD_DIR = os.path.join(PKG, "_build")
SOURCES = ["api.hip", "scatter_gather.hip", "quant.hip", "decode.hip", "decode_stream.hip",
           "prefill.hip"]
# benchmark probes (peak MFMA rate, HBM read stream, cache flush): a library of their own,
# not part of the kvb C ABI
PROBE_SOURCE = "probe.hip"
PROBE_OUT = os.path.join(PKG, "libkvb_probe.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed-fp32 VALU forms are kept out of the generated code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


# Attention kernels never produce NaN scores (masked keys use -inf), so their max
# reductions need no NaN canonicalisation of every operand.  The host-side argument
# checks (api.hip) are compiled without this flag.
KERNEL_FLAGS = {
    "prefill.hip": ["-fno-honor-nans"],
    "decode.hip": ["-fno-honor-nans"],
    "decode_stream.hip": ["-fno-honor-nans"],
}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build(verbose: bool = False, extra_flags=None) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    flags = FLAGS + list(extra_flags or [])
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC] + flags + KERNEL_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj])
    probe_obj = os.path.join(BUILD_DIR, PROBE_SOURCE.replace(".hip", ".o"))
    cmds.append([HIPCC] + flags + ["-c", os.path.join(CSRC, PROBE_SOURCE), "-o", probe_obj])
    with ThreadPoolExecutor(max_workers=min(4, len(cmds))) as ex:
        for cmd, _ in zip(cmds, ex.map(_run, cmds)):
            if verbose:
                print(" ".join(cmd))
    for out, ob in ((OUT, objs), (PROBE_OUT, [probe_obj])):
        tmp = out + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + ob)
        os.replace(tmp, out)
        if verbose:
            print("built", out)
    return OUT


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
