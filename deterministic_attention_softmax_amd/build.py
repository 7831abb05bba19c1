"""Build libjas.so (gfx950) in-tree with hipcc.

Flags that are part of the arithmetic contract: -ffp-contract=off (no FMA is
formed from a*b+c), no fast-math, FP32 denormals kept.  Packed FP32 VALU
instructions are switched off (-packed-fp32-ops).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libjas.so")
SOURCES = [os.path.join(CSRC, f) for f in (
    "jas_kernels_f32.hip", "jas_kernels_bf16.hip", "jas_kernels_f16.hip", "jas_launch.hip",
    "jas_attn.hip", "jas_api.cpp")]
OBJ_DIR = os.path.join(HERE, "_build")
# Per-source flags.  The fused attention kernel keeps its MFMA accumulators
# in architectural VGPRs rather than AGPRs: no copy of each score out of the
# accumulators, and 159 registers per lane instead of 224, which lets three
# waves share a SIMD instead of two.
SOURCE_FLAGS = {"jas_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
_NOISE = "is not a recognized feature for this target"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if _NOISE not in l)
    if r.returncode != 0:
        sys.stderr.write(err + "\n")
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd[-3:])}")
    if verbose and err.strip():
        sys.stderr.write(err + "\n")


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source to an object (in parallel, one hipcc per
    translation unit), then link libjas.so."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = [os.path.join(OBJ_DIR, os.path.basename(src) + ".o") for src in SOURCES]
    jobs = [[HIPCC, *FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
            for src, obj in zip(SOURCES, objs)]
    workers = max(1, min(len(jobs), os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for f in [ex.submit(_run, j, verbose) for j in jobs]:
            f.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
