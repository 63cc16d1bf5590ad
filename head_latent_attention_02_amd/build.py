"""Build libmla.so (HIP, gfx950) in-tree.

    python -m head_latent_attention_02_amd.build [--resource-usage]

Compiles every csrc/*.hip file to an object with hipcc for gfx950 and links
them into head_latent_attention_02_amd/libmla.so.  Objects go to
head_latent_attention_02_amd/_build/.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmla.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-file compiler options.  The split-KV decode kernel keeps its value
# accumulators in AGPRs through inline assembly; selecting the VGPR form for
# the compiler's own MFMAs keeps the score accumulators (read by the softmax)
# out of the AGPR file that those accumulators fill.
FILE_FLAGS = {
    "mfma_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _compile(src: str, resource_usage: bool) -> tuple[str, str]:
    obj = os.path.join(BUILD, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC, *COMMON_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if resource_usage:
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    log = r.stdout + r.stderr
    # the host pass does not know the packed-fp32 feature; that warning is noise
    log = "\n".join(l for l in log.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{log}")
    return obj, log


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda s: _compile(s, resource_usage), srcs))
    for _, log in results:
        if log.strip() and (verbose or resource_usage):
            print(log)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ru = "--resource-usage" in sys.argv
    path = build(resource_usage=ru, verbose="-v" in sys.argv)
    print(path)
