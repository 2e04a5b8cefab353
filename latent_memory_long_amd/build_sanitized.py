"""Host-sanitizer build of the library: AddressSanitizer and UndefinedBehaviorSanitizer
instrument the host code (argument validation, bank-file I/O, launch set-up); device code is
built as in build.py and is not instrumented.

    python latent_memory_long_amd/build_sanitized.py

writes latent_memory_long_amd/_build_san/libmsa_san.so.  The binding loads it in place of
the default build when MSA_LIBRARY names it; the Python interpreter is not instrumented, so
the sanitizer runtime (runtime()) has to be preloaded with LD_PRELOAD.
"""
from __future__ import annotations

import importlib.util
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
OBJ = os.path.join(PKG, "_build_san")
LIB = os.path.join(OBJ, "libmsa_san.so")
CLANG = os.environ.get("MSA_CLANG", "/opt/rocm/llvm/bin/clang")

# every sanitizer flag applies to the host pass only
HOST_SANITIZE = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                 "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -shared-libasan "
                 "-Xarch_host -fno-omit-frame-pointer -Xarch_host -g").split()


def runtime() -> str:
    """Path of the shared AddressSanitizer runtime (it carries the UBSan handlers too)."""
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True, check=True)
    path = r.stdout.strip()
    if not os.path.isfile(path):
        raise RuntimeError(f"no AddressSanitizer runtime at {path!r}")
    return path


def build(verbose: bool = False) -> str:
    spec = importlib.util.spec_from_file_location("_msa_build", os.path.join(PKG, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.build(verbose, obj_dir=OBJ, lib=LIB, extra=tuple(HOST_SANITIZE))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
