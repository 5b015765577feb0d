"""Builds libmoe.so (the HIP kernels + C ABI) for gfx950, in-tree.

Every HIP source is compiled with hipcc for gfx950 only, in parallel, then
linked into combine_router_softmax_top_amd/libmoe.so.  Packed-fp32 VALU
instructions are switched off for all device code.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
_CSRC = os.path.join(_HERE, "csrc")
_BUILD = os.path.join(_ROOT, "_build", "moe")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-I", os.path.join(_ROOT, "include"), "-I", _CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]


# Per-source extra flags.  route.hip: keep MFMA accumulators in VGPRs.  Its
# logits kernel runs one wave per SIMD; with the accumulators in AGPRs the
# compiler copied them between the two register files every k-chunk.
EXTRA_FLAGS = {"route.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def library_path() -> str:
    return os.path.join(_HERE, "libmoe.so")


def sources():
    return sorted(glob.glob(os.path.join(_CSRC, "*.hip"))) + [os.path.join(_CSRC, "moe_api.cpp")]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(_BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, "-x", "hip", *CFLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), "-c", src,
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(_BUILD, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    out = library_path()
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def clean() -> None:
    shutil.rmtree(_BUILD, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose=True))
