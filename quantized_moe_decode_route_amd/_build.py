"""Build libmoedecode.so in-tree for gfx950 with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoedecode.so")
BUILD_DIR = os.path.join(os.path.dirname(PKG), "_build", "moedecode")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 instruction selection is disabled for every HIP object; fp32
# division and sqrt stay IEEE-correct (the INT4 conversion rounds w/s).
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wno-unused-command-line-argument",
]


# The single-launch layer's few atomics are issued by one lane and their
# results used much later; the atomic optimizer would rewrite them into a
# lane-0 atomic plus readfirstlane, which waits for the result on the spot.
FUSED_FLAGS = ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]


# fused_units.hip holds the layer kernel's instantiations in this many units,
# compiled separately (-DMOE_FUSED_UNIT=i) so they build in parallel.
FUSED_UNITS = 5


def _compile(job: tuple[str, int | None]) -> str:
    src, unit = job
    os.makedirs(BUILD_DIR, exist_ok=True)
    name = os.path.basename(src) + ("" if unit is None else f".{unit}")
    obj = os.path.join(BUILD_DIR, name + ".o")
    extra = FUSED_FLAGS if os.path.basename(src).startswith("fused") else []
    if unit is not None:
        extra = [*extra, f"-DMOE_FUSED_UNIT={unit}"]
    cmd = [HIPCC, *HIP_FLAGS, *extra, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {name}:\n{r.stderr}")
    return obj


def build(jobs: int | None = None) -> str:
    """Compile every source under csrc/ and link libmoedecode.so (always rebuilds)."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    work = []
    for src in srcs:
        if os.path.basename(src) == "fused_units.hip":
            work += [(src, i) for i in range(FUSED_UNITS)]
        else:
            work.append((src, None))
    # the slow units first, so the pool does not end on one of them
    work.sort(key=lambda j: (j[1] is None, j))
    jobs = jobs or min(8, len(work))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, work))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
