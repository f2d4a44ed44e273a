"""Build libfa.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

    python -m exact_io_aware_attention_amd.build [--jobs N] [--verbose]

Each ``csrc/*.hip`` file is compiled to an object under ``_build/`` and the objects
are linked into ``exact_io_aware_attention_amd/libfa.so``. No GPU is needed: hipcc
cross-compiles for gfx950.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
from typing import List

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32.
# -munsafe-fp-atomics: hardware fp32 atomics instead of compare-and-swap loops.
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-file additions. Where a kernel pins its output accumulators in AGPRs by inline asm
# (forward at head_dim 64, dK/dV at head_dim 128), every other MFMA must use the VGPR
# form, so the score accumulators stay where the softmax arithmetic reads them.
FILE_FLAGS = {
    "fa_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "fa_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libfa")
    return path


def sources() -> List[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd: List[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "unknown target feature" not in line and "-packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(jobs: int = 0, verbose: bool = False) -> str:
    """Compile every source and link libfa.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    srcs = sources()
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_run, [cc, *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(s), []), "-c", s, "-o", o],
                          verbose) for s, o in zip(srcs, objs)]
        for f in futs:
            f.result()
    tmp = LIB_PATH + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))
    return 0


if __name__ == "__main__":
    sys.exit(main())
