"""Build librtp.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m long_context_sparse_head_amd.build [--jobs N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(OUT_DIR, "librtp.so")
SOURCES = ["attn_window.hip", "attn.hip", "indexer.hip", "decode.hip",
           "cluster.hip", "api.hip"]

# Packed-FP32 VALU ops are turned off for all device code.
HIPFLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]

# Per-file backend options. Asking the backend to prefer the VGPR form of
# MFMA results puts the window kernel's score accumulators and the block
# scores of the indexer in VGPRs, where the VALU reads every one of them,
# instead of in AGPRs that need a copy per value (the sparse kernel and the
# decode kernel are no faster with it and keep the default).
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
# The indexer is built without NaN-preserving float semantics: its block
# scores are maxima over MFMA results, and with NaNs honoured every operand of
# a max is first canonicalised (one extra VALU op per value, which made the
# scoring loop VALU-bound). Its selection logic compares integer order keys;
# a NaN score is not a supported input there either way (the max ignores it).
EXTRA_FLAGS = {
    "attn_window.hip": VGPR_FORM,
    "indexer.hip": VGPR_FORM + ["-fno-honor-nans"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build librtp)")


def _compile(src: str, obj: str) -> None:
    cmd = [hipcc(), *HIPFLAGS, *EXTRA_FLAGS.get(src, []),
           "-I", os.path.join(ROOT, "include"), "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def build(jobs: int = 4) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    objs = [os.path.join(OUT_DIR, s.replace(".hip", ".o")) for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda p: _compile(*p), zip(SOURCES, objs)))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
           *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    print(build(ap.parse_args().jobs))
