"""Host-code sanitizers (CPU only).

The oracle is rebuilt with AddressSanitizer and UndefinedBehaviorSanitizer
and the oracle's pin tests run against that build; the HIP library is
rebuilt with the same sanitizers on its host code only (device code is
compiled as usual) and the boundary tests, which drive every entry point's
argument validation, run against it.  Each run is a subprocess with the
sanitizer runtime preloaded, halting on the first report; before the tests
it checks that the runtime and the instrumented library are the ones loaded.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}

# loaded as the pytest run's first step: the sanitizer runtime is in the
# process and the library under test is the instrumented build
_PROBE = """
import ctypes, os, sys
ctypes.CDLL(None).__asan_init
lib = os.path.realpath(os.environ[sys.argv[1]])
import {module}
{touch}
assert lib in open('/proc/self/maps').read(), (lib, 'not loaded')
print('sanitized build loaded:', lib)
"""


def _tool(cmd):
    try:
        out = subprocess.run(cmd, capture_output=True, text=True, timeout=60).stdout.strip()
    except (OSError, subprocess.TimeoutExpired):
        return None
    return out if out and os.path.isabs(out) and os.path.exists(out) else None


def _run_under(preload, env_var, lib, module, touch, tests):
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=preload, **{env_var: lib})
    probe = subprocess.run([sys.executable, "-c", _PROBE.format(module=module, touch=touch),
                            env_var], cwd=ROOT, env=env, capture_output=True, text=True,
                           timeout=600)
    assert probe.returncode == 0, probe.stdout + probe.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-m", "not gpu",
                        "-p", "no:cacheprovider", *tests], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan = _tool(["g++", "-print-file-name=libasan.so"])
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_asan.so")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
                    "-fPIC", "-shared", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", lib,
                    os.path.join(ROOT, "oracle", "kvq_oracle.cpp"), "-lpthread"],
                   check=True, timeout=600)
    _run_under(asan, "KVQ_ORACLE_LIB", lib, "oracle", "oracle._load()",
               ["tests/test_oracle_pins.py", "tests/test_oracle_mx_pins.py"])


def test_library_host_validation_under_asan_ubsan(tmp_path):
    rt = _tool(["/opt/rocm/llvm/bin/clang", "-print-file-name=libclang_rt.asan-x86_64.so"])
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    from bit_kv_cache_amd import _build
    lib = str(tmp_path / "libkvq_asan.so")
    flags = [f for f in _build.HIP_FLAGS if f not in ("-O3", "-Wall")]
    # host code only: every sanitizer flag follows -Xarch_host
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    subprocess.run(["/opt/rocm/bin/hipcc", *flags, "-O1", "-g", *san, "-I",
                    os.path.join(ROOT, "include"), "-o", lib, *_build.sources()],
                   check=True, capture_output=True, timeout=900)
    _run_under(rt, "KVQ_LIB", lib, "bit_kv_cache_amd", "", ["tests/test_boundary.py"])
