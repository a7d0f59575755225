"""Build libkvscore.so (gfx950) in-tree with hipcc.

    python -m kv_cache_eviction_lse_amd.build [--verbose] [--resource-usage]
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvscore.so")
# measured ceilings for the benchmark (a copy kernel and an MFMA-only kernel);
# not part of the scoring library's ABI
CALIB_LIB = os.path.join(HERE, "libkvscore_calib.so")
CALIB_SOURCES = ["calib.hip"]
SOURCES = ["api.cpp", "lse.hip", "score.hip", "evict.hip", "attn.hip", "vnorm.hip", "decode.hip", "stream.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-fvisibility=hidden",
    # never emit packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Per-file flags. The scoring kernels never see NaN in their reductions (the
# inputs are finite bf16 values and finite normalisers), so NaN-propagating
# max/min semantics are not needed there: without them the compiler drops the
# IEEE canonicalising moves before every v_max and can form v_max3_f32.
# -amdgpu-mfma-vgpr-form keeps MFMA accumulators in VGPRs, where the VALU
# softmax reads them, instead of AGPRs that need a v_accvgpr_read per value.
FILE_FLAGS = {
    "lse.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
    "score.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
    "vnorm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, obj: str, extra: list[str], verbose: bool) -> None:
    cmd = [HIPCC, *COMMON, *FILE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is harmless
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if msgs and (verbose or r.returncode):
        print("\n".join(msgs), file=sys.stderr, flush=True)
    if r.returncode:
        raise RuntimeError(f"hipcc failed for {src}")


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], extra, verbose or resource_usage), zip(SOURCES, objs)))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    cobjs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in CALIB_SOURCES]
    for so, o in zip(CALIB_SOURCES, cobjs):
        _compile(so, o, extra, verbose or resource_usage)
    ctmp = CALIB_LIB + ".tmp"
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", ctmp, *cobjs], check=True)
    os.replace(ctmp, CALIB_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv, resource_usage="--resource-usage" in sys.argv)
    print(LIB)
