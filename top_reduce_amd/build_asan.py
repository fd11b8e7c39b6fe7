"""Host-side AddressSanitizer build of libtopreduce, for CPU checks of the
C-ABI layer (argument checks, workspace layout, error messages).

    python -m top_reduce_amd.build_asan

Every source is compiled with AddressSanitizer on the host compilation pass
only (-Xarch_host before each sanitizer flag); the device code is the
ordinary gfx950 code. The result is _build_asan/libtopreduce_asan.so. A
Python process loads it with the sanitizer runtime preloaded
(LD_PRELOAD=asan_runtime()) and TOP_REDUCE_LIB pointing at it; the ABI tests
run that way in tests/test_abi_asan.py. Not for GPU runs.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from top_reduce_amd import build as B

BUILD = os.path.join(B.ROOT, "_build_asan")
LIB = os.path.join(BUILD, "libtopreduce_asan.so")
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime that hipcc links against."""
    r = subprocess.run([B.HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True, check=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"AddressSanitizer runtime not found (hipcc printed {path!r})")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [B.HIPCC, *B.FLAGS, *HOST_ASAN, "-c", os.path.join(B.CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(B.SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, B.SOURCES))
    tmp = LIB + ".tmp"
    subprocess.run([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *objs,
                    "-shared-libasan", *HOST_ASAN, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
    print(asan_runtime(), file=sys.stderr)
