"""Build the gfx950 HIP libraries in-tree with hipcc.

Usage: ``python -m head_latent_attention_cache_amd.build`` (or ``build()``).
Every translation unit under ``csrc/`` is compiled for gfx950 only and linked
into ``libmla_amd.so`` (the MLA library); those under ``probe_csrc/`` into
``libmla_probe.so`` (the measurement probes, not on the MLA path).  Both sit
next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmla_amd.so")
PROBE_CSRC = os.path.join(HERE, "probe_csrc")
PROBE_OUT = os.path.join(HERE, "libmla_probe.so")
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

# -Xclang -target-feature -Xclang -packed-fp32-ops: no packed-fp32 VALU forms
# (v_pk_{add,mul,fma}_f32) are generated anywhere in the device code.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the MLA library)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str, verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    probe_srcs = sorted(glob.glob(os.path.join(PROBE_CSRC, "*.hip")))
    jobs = min(len(srcs) + len(probe_srcs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, srcs + probe_srcs))
    _link(objs[:len(srcs)], OUT, verbose)
    _link(objs[len(srcs):], PROBE_OUT, verbose)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
