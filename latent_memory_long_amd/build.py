"""Build libmsa.so (HIP, gfx950) in-tree with hipcc.

    python latent_memory_long_amd/build.py [-v]

Each csrc/*.hip is compiled to an object in parallel, then linked into
latent_memory_long_amd/libmsa.so.  Device code is built for gfx950 only.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmsa.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 ops stay disabled in device code: the compiler keeps scalar fp32 math
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


# Per-file flags.  attn_bwd.hip: the MFMA results stay in ordinary vector registers instead
# of accumulation registers, from which the backward's softmax would copy them out first
# (bwd_dkv: 208 vector registers and no accumulation registers, still two waves per SIMD;
# 24 fewer register moves per 32 MFMAs, the backward 0.835 -> 0.80 ms).
FILE_FLAGS = {"attn_bwd.hip": ("-mllvm", "-amdgpu-mfma-vgpr-form=1")}


def _compile(src: str, verbose: bool, obj_dir: str, extra: tuple) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), ()), *extra, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is expected
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False, obj_dir: str = OBJ, lib: str = LIB, extra: tuple = ()) -> str:
    """Compile every csrc/*.hip into obj_dir and link them into lib; extra flags go to every
    compile and to the link."""
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, obj_dir, extra), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
