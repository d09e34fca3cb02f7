"""Host-sanitized build of libdmtp.so for the argument-validation tests.

Every source is compiled for gfx950 as in build.py, with AddressSanitizer and
UndefinedBehaviorSanitizer instrumenting the HOST code only (each sanitizer
flag is passed to the host compilation alone); the device code is the normal
build.  The library goes to _build/sanitized/libdmtp.so.  It is loaded into a
Python process that preloads the sanitizer runtime (sanitizer_runtime()),
where the C-ABI validation, the workspace planning and the refusals run
under both sanitizers without a GPU.
"""
from __future__ import annotations

import glob
import importlib.util
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
OUT = os.path.join(ROOT, "_build", "sanitized")

_spec = importlib.util.spec_from_file_location("_dmtp_build", os.path.join(PKG, "build.py"))
_b = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(_b)

HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-shared-libsan", "-g"]


def sanitizer_runtime() -> str:
    """The shared ASan runtime of the compiler hipcc drives (it also carries UBSan)."""
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise FileNotFoundError("no clang ASan runtime under /opt/rocm/lib/llvm")
    return hits[-1]


def _compile(src: str) -> str:
    obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
    cmd = ([_b.HIPCC, "-x", "hip", "-c", os.path.join(_b.CSRC, src), "-o", obj] + _b.FLAGS +
           _b.EXTRA.get(src, []) + HOST_SAN)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build() -> str:
    os.makedirs(OUT, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(_b.SOURCES))) as ex:
        objs = list(ex.map(_compile, _b.SOURCES))
    lib = os.path.join(OUT, "libdmtp.so")
    cmd = [_b.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib] + objs + HOST_SAN
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return lib


if __name__ == "__main__":
    print(build())
    sys.exit(0)
