"""Build the HIP library libfp4kv.so in-tree for gfx950.

    python -m fp4_kv_cache_fp4kv_amd.build

Cross-compiles with hipcc (no GPU needed), one object per source in
parallel, then links them.  Every HIP source is compiled with packed-FP32
instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfp4kv.so")
SOURCES = ["api.cpp", "codec.hip", "rope.hip", "attention.hip"]
ARCH = os.environ.get("FP4KV_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


# Extra flags per source.  The attention kernel never sees a NaN (inputs
# are finite by contract, masked scores are -inf), so NaN-quieting
# canonicalizations before every max are dropped there; the codec keeps
# full IEEE semantics.
EXTRA = {"attention.hip": ["-fno-honor-nans"]}


def _filter(stderr: str) -> str:
    # the host pass warns that it does not know the packed-fp32 feature
    return "\n".join(l for l in stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())


def build(verbose: bool = True) -> str:
    common = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
              "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", f"-I{INCLUDE}", f"-I{CSRC}"]
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(CSRC, src + ".o")
        cmd = [hipcc()] + common + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                            text=True)))
        objs.append(obj)
    failed = []
    for src, pr in procs:
        _, err = pr.communicate()
        err = _filter(err)
        if pr.returncode != 0:
            failed.append(f"{src} ({pr.returncode}):\n{err}")
        elif err and verbose:
            print(err, file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed: " + "\n".join(failed))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc link failed ({res.returncode}):\n{_filter(res.stderr)}")
    for o in objs:
        os.remove(o)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
