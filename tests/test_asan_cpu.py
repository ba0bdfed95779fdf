"""The C ABI's host logic (argument validation, workspace layout, path and launch-shape choice,
status strings) under AddressSanitizer: the library's host code is rebuilt with
-fsanitize=address (device code unchanged) and the ABI tests of test_abi_cpu.py run against it in
a Python process that preloads the clang ASan runtime.  Any invalid read or write in the host
paths those tests drive aborts that process with an AddressSanitizer report.  No GPU is used: the
tests call only entry points that need none.
"""
import os
import subprocess
import sys

import pytest

from state_space_sequence_mamba_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _env(lib, runtime):
    env = dict(os.environ)
    env.update(SSD_LIBRARY=lib, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               PYTHONPATH=ROOT + os.pathsep + env.get("PYTHONPATH", ""))
    return env


@pytest.fixture(scope="module")
def asan_lib():
    runtime = B.asan_runtime()
    if runtime is None:
        pytest.skip("clang ASan runtime not installed")
    try:
        lib = B.build_asan()
    except RuntimeError as e:                      # (no hipcc: nothing to sanitize)
        pytest.skip(f"cannot build the sanitized library: {e}")
    return lib, runtime


def test_sanitized_library_is_instrumented_and_loaded(asan_lib):
    lib, runtime = asan_lib
    probe = ("import ctypes; from state_space_sequence_mamba_amd import ssd; ssd.load_library(); "
             "m = open('/proc/self/maps').read(); "
             "assert 'libssd_asan.so' in m and 'libclang_rt.asan' in m, 'not the sanitized build'; print('ok')")
    r = subprocess.run([sys.executable, "-c", probe], env=_env(lib, runtime), capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 0 and "ok" in r.stdout, r.stderr[-2000:]


def test_abi_host_logic_under_address_sanitizer(asan_lib):
    lib, runtime = asan_lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       env=_env(lib, runtime), capture_output=True, text=True, timeout=600, cwd=ROOT)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0 and " passed" in r.stdout, out[-4000:]
