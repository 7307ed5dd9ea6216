"""Build of the HIP library ``libbitlinear.so`` for gfx950 (MI355X).

Every ``csrc/*.hip`` file is compiled with hipcc into ``_build/`` and linked
in-tree next to this file, so the library travels with the source tree.
Flags that matter for results:
  -ffp-contract=off                          no FMA contraction of fp32
                                             expressions (explicit fmaf only);
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE division and square root
                                             (the int8 codes depend on them);
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                             no packed-fp32 VALU instructions.
Usage: python -m ternary_bit_linear_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbitlinear.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# Per-source extras.  The batched kernels of these files take the per-problem
# first workgroups as their eight leading int arguments, which gfx950 can
# preload into scalar registers at wave launch (for the other kernels the
# preload only moves their first arguments into registers).
EXTRA = {
    "gemv_shot.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=8"],
    "gemm.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=8"],
    "gemm32.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=8"],
    "act_quant.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=8"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link libbitlinear.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
