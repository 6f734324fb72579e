"""Build libfalcon.so (HIP for gfx950) in-tree with hipcc.

Usage: python -m linear_recurrent_weight_amd.build [-v]
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import pathlib
import shutil
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = ROOT / "_build"
LIB = PKG / "libfalcon.so"
ARCH = os.environ.get("FALCON_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# packed fp32 instructions are kept out of every code object; MFMA results
# stay in VGPRs (no copies out of accumulation registers)
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "--amdgpu-mfma-vgpr-form",
          f"-I{ROOT / 'include'}", "-Wall", "-Wno-unused-function"]


def sources():
    return sorted(CSRC.glob("*.hip")) + sorted(CSRC.glob("*.cpp"))


def _compile(src: pathlib.Path, verbose: bool) -> pathlib.Path:
    obj = BUILD / (src.name + ".o")
    cmd = [HIPCC, *COMMON, "-c", str(src), "-o", str(obj)]
    if src.suffix == ".cpp":
        cmd = [HIPCC, *COMMON, "-x", "hip", "-c", str(src), "-o", str(obj)]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src.name}:\n{err}")
    if verbose and err.strip():
        print(err)
    return obj


def build(verbose: bool = False) -> pathlib.Path:
    BUILD.mkdir(exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB



# source file of each kernel name that falcon_kernel_name reports
KERNEL_SOURCES = {"passthrough": "feature.hip", "feature": "feature.hip", "recurrent": "recurrent.hip",
                  "decode": "decode.hip",
                  "chunk_f1_prep": "chunk_f1.hip", "chunk_f1_scan": "chunk_f1.hip",
                  "chunk_f2": "chunk_f2.hip", "chunk_f2a": "chunk_f2a.hip",
                  "f3_prep": "chunk_f3.hip", "f3_scan": "chunk_f3.hip", "f3_xfer": "chunk_f3_xfer.hip",
                  "f1_xfer": "chunk_f1_xfer.hip", "f1_carry": "chunk_f1_xfer.hip",
                  "f1_segmap": "chunk_f1_xfer.hip", "f1_segscan": "chunk_f1_xfer.hip",
                  "bwd_states": "falcon_bwd.hip", "bwd_sweep": "falcon_bwd.hip", "bwd_reduce": "falcon_bwd.hip",
                  "bwd_ops": "bwd_chunk.hip", "bwd_carry_fwd": "bwd_chunk.hip", "bwd_carry_rev": "bwd_chunk.hip",
                  "bwd_grads": "bwd_chunk.hip",
                  "a_segment": "chunk_a.hip", "a_segscan": "chunk_a.hip", "a_output": "chunk_a.hip",
                  "a1_segment": "chunk_a1.hip", "a1_segscan": "chunk_a1.hip", "a1_output": "chunk_a1.hip",
                  "a3_window": "chunk_a1.hip"}


def sources_digest(kernels=None) -> str:
    """sha256 over library sources and the public header, to tell whether a
    stored profile still describes the current kernels.  With `kernels` (names
    as falcon_kernel_name reports them), only their sources, the shared
    headers, the planner and the dispatcher count."""
    import hashlib
    h = hashlib.sha256()
    if kernels is None:
        files = sources()
    else:
        files = sorted({CSRC / KERNEL_SOURCES[k] for k in kernels} |
                       {CSRC / "plan.cpp", CSRC / "falcon_fwd.hip"})
    for p in files + sorted(CSRC.glob("*.h")) + [ROOT / "include" / "falcon.h"]:
        h.update(p.name.encode())
        h.update(p.read_bytes())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
