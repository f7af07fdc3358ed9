"""The library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU: a copy of libdflash built with
sanitized host code (build.build_host_sanitized) is loaded in a fresh
process with the sanitizer runtime preloaded, and tests/host_abi_driver.py
drives everything in it that runs without a GPU: version and error
strings, the adaptive block-size policy, phase names, the argument checks
of the entry points and a seeded fuzz of configurations and policy calls.
A sanitizer report (out-of-bounds access, use after free, signed overflow,
misaligned or null dereference, ...) ends that process with a nonzero
status."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "block_diffusion_drafting_amd"))
import build  # noqa: E402


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    try:
        build.hipcc()
        rt = build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = build.build_host_sanitized(str(tmp_path_factory.mktemp("san")))
    return lib, rt


@pytest.mark.timeout(300)
def test_host_code_under_asan_and_ubsan(sanitized_lib):
    lib, rt = sanitized_lib
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    # Python's own allocations are never freed at exit: leak reports are off;
    # every other ASan and UBSan error stops the process
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=24"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "host_abi_driver.py"), lib],
                       env=env, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, f"exit {r.returncode}\n{r.stdout[-2000:]}\n{r.stderr[-6000:]}"
    assert "calls with the expected status" in r.stdout


@pytest.mark.timeout(300)
def test_sanitizers_are_active(sanitized_lib):
    """The preloaded runtime is live in that process: ASan flags a heap
    read past the end of a block in the driver process's own memory
    (made through the runtime's own check, no invalid access is executed)."""
    lib, rt = sanitized_lib
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0")
    code = ("import ctypes as C, sys\n"
            "C.CDLL(sys.argv[1])\n"
            "rt = C.CDLL(None)\n"
            "rt.malloc.restype = C.c_void_p\n"
            "p = rt.malloc(24)\n"
            "f = rt.__asan_address_is_poisoned\n"
            "f.argtypes = [C.c_void_p]\n"
            "print(f(p), f(p + 24))\n")
    r = subprocess.run([sys.executable, "-c", code, lib], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.split() == ["0", "1"], r.stdout
