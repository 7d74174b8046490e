"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds libgdn with its host code instrumented (frame_wise_gated_fwd_amd.
build_host_sanitize; device code unchanged) and runs the C ABI's host-side
tests against it in a child process that preloads the sanitizer runtime:
every argument check, workspace query, path query and refusal of every entry
point, with any memory error or undefined behaviour ending the run.  No GPU
is needed (the paths that reach the device find none and report it)."""
import os
import subprocess
import sys

ROOT = os.path.abspath(os.path.join(os.path.dirname(__file__), ".."))


def test_abi_host_paths_under_asan_and_ubsan():
    from frame_wise_gated_fwd_amd.build_host_sanitize import build_host_sanitized, sanitizer_runtime
    lib = build_host_sanitized()
    env = dict(os.environ, LD_PRELOAD=sanitizer_runtime(), GDN_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # the child really runs the instrumented library with the runtime loaded
    probe = ("import ctypes, os; l = ctypes.CDLL(os.environ['GDN_LIB']); "
             "maps = open('/proc/self/maps').read(); "
             "assert 'libclang_rt.asan' in maps and os.environ['GDN_LIB'] in maps; "
             "ctypes.CDLL(None).__asan_report_load8; print('instrumented')")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "instrumented" in r.stdout, r.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "tests/test_abi_property.py", "-q", "-x",
                        "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, out
