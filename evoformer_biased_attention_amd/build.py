"""Build libevoattn.so in-tree with hipcc for gfx950.

Usage: python evoformer_biased_attention_amd/build.py [-v]
(run as a file: importing the package itself requires the built library)
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libevoattn.so")
SOURCES = ["evo_attn_api.cpp", "evo_attn_f32.hip", "evo_attn_bf16.hip", "evo_attn_bwd.hip",
           "evo_attn_bwd_mfma.hip", "evo_attn_bwd_f32.hip", "evo_trimul.hip", "evo_attn_noalloc.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # Keep the compiler from forming packed fp32 instructions (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in arch VGPRs: the softmax reads every score, and AGPR
    # results would cost a v_accvgpr_read per value.
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature and says so; that is harmless
    noise = "not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln and "ignoring feature" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source of the library into libevoattn.so (always recompiles).

    Each source becomes an object of its own, compiled in parallel (at most MAX_JOBS, default the
    CPU count, at most 16), and the objects are linked into the library."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(os.path.dirname(PKG), "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    jobs = max(1, min(16, int(os.environ.get("MAX_JOBS", os.cpu_count() or 1)), len(SOURCES)))
    # the largest sources first, so that they do not start last
    order = sorted(range(len(SOURCES)), key=lambda i: -os.path.getsize(os.path.join(CSRC, SOURCES[i])))
    with ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_run, [hipcc(), *compile_flags, "-c", "-o", objs[i], os.path.join(CSRC, SOURCES[i])],
                          verbose) for i in order]
        for f in futs:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
