"""Build libfa.so (the HIP library behind include/fa.h) for gfx950 with hipcc.

Every HIP source is compiled with packed-fp32 instruction selection turned
off.  The library lands next to this file, so it travels with the source tree.
Run as ``python -m online_softmax_04_amd.build``.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libfa.so")
SOURCES = ["fa_api.hip", "attn_fwd.hip", "attn_fwd_fp8.hip", "attn_bwd.hip", "attn_decode.hip",
           "softmax.hip", "copy.hip", "mfma_stream.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
                if "packed-fp32-ops" not in ln]  # the host pass does not know the feature
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
        if verbose and msgs:
            print("\n".join(msgs))
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = OUT + ".tmp"
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, OUT)
    return OUT


PROBE_SRC = os.path.join(ROOT, "tests", "probes", "layout_probe.hip")
PROBE_OUT = os.path.join(ROOT, "tests", "probes", "liblayout_probe.so")


def build_probes() -> str:
    """The single-wave instruction probes the GPU tests load (tests/probes)."""
    tmp = PROBE_OUT + ".tmp"
    r = subprocess.run([HIPCC, *FLAGS, "-shared", PROBE_SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on layout_probe.hip:\n" + r.stderr[-3000:])
    os.replace(tmp, PROBE_OUT)
    return PROBE_OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
