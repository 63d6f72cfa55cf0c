"""Build libidxcache.so for gfx950 with hipcc (no GPU needed: hipcc cross-compiles)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libidxcache.so")
SOURCES = ["abi.cpp", "indexer.hip", "topk.hip", "sparse_mla.hip", "sparse_mla_wide.hip", "overlap.hip", "paged.hip",
           "calib.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 instructions are disabled for all device code.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]
# Per-source code-generation options.  The sparse MLA kernel keeps its output
# accumulators in architectural VGPRs (MFMA VGPR form) so that the rare
# softmax rescale is a plain VALU multiply instead of AGPR round trips.
SOURCE_FLAGS = {"sparse_mla.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, obj: str, defines=()) -> None:
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []), *[f"-D{d}" for d in defines], "-c", src,
           "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")


def build(verbose: bool = False, out: str = LIB_PATH, defines=()) -> str:
    """Compile every HIP source and link the shared library (in-tree by
    default; ``out`` and ``defines`` serve other builds of the same sources)."""
    obj_dir = os.path.dirname(out) if out == LIB_PATH else out + ".objs"
    os.makedirs(obj_dir, exist_ok=True)
    objs = []
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        for s in SOURCES:
            src = os.path.join(CSRC, s)
            obj = os.path.join(obj_dir, s + ".o")
            objs.append(obj)
            jobs.append(ex.submit(_compile, src, obj, tuple(defines)))
        for j in jobs:
            j.result()
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
