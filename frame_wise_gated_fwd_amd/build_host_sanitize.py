"""The library with its host code under AddressSanitizer and
UndefinedBehaviorSanitizer, for the CPU tests of the C ABI's host paths
(argument checks, workspace layout, dispatch).  Device code is built as in
build.py.

    python -m frame_wise_gated_fwd_amd.build_host_sanitize
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

from .build import BUILD_DIR, SOURCES, _compile

# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the library's
# host code (argument checks, workspace layout, dispatch); device code is
# built as usual.  Each -fsanitize= follows -Xarch_host, so it reaches the
# host compilation only.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
SAN_DIR = os.path.join(BUILD_DIR, "host_sanitize")
SAN_LIB = os.path.join(SAN_DIR, "libgdn.so")
CLANGXX = "/opt/rocm/lib/llvm/bin/clang++"


def build_host_sanitized(verbose: bool = False) -> str:
    """The same library with its host code under AddressSanitizer and
    UndefinedBehaviorSanitizer (_build/host_sanitize/libgdn.so), for the CPU
    tests of the C ABI's host paths.  Linked by the LLVM clang++ with the
    shared sanitizer runtime, which the process must preload
    (sanitizer_runtime())."""
    os.makedirs(SAN_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, SAN_DIR, SANITIZE_HOST), SOURCES))
    tmp = SAN_LIB + ".tmp"
    cmd = [CLANGXX, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libasan", "-o", tmp] + objs + \
        ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print("built", SAN_LIB)
    return SAN_LIB


def sanitizer_runtime() -> str:
    """Path of the shared AddressSanitizer runtime of the LLVM that built it."""
    r = subprocess.run([CLANGXX, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the LLVM AddressSanitizer runtime was not found")
    return path


if __name__ == "__main__":
    build_host_sanitized(verbose=True)
