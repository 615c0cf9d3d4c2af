"""Host code under AddressSanitizer and UBSan (CPU only, no GPU needed).

Two builds of the host code run existing CPU test modules in subprocesses
with the sanitizer runtime preloaded; any sanitizer report fails the run
(UBSan is built not to recover, ASan stops at its first error):

- the C ABI layer (attn_api.cpp: argument validation, declines, the error
  string, the tuning-cache bookkeeping reachable without a device), compiled
  with the sanitizers on its host side only and linked with the regular
  device objects (build.build_host_sanitized), under clang's ASan runtime,
  running test_abi.py and test_binding_checks.py;
- the CPU oracle (attn_oracle.c, built with gcc's sanitizers), under gcc's
  libasan, running the oracle's pin and tile-floor tests.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")

RUNNER = """
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import {module} as m
m.{attr} = {lib!r}
import pytest
rc = pytest.main([{files}, "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu"])
loaded = {check}
assert loaded == {lib!r}, ("the sanitized library was not the one loaded", loaded)
sys.exit(int(rc))
"""


def _runtime(cmd):
    try:
        path = subprocess.run(cmd, capture_output=True, text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run(runtime, module, attr, lib, files, check):
    code = RUNNER.format(root=ROOT, tests=TESTS, module=module, attr=attr, lib=lib,
                         files=", ".join(repr(os.path.join(TESTS, f)) for f in files),
                         check=check)
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "Sanitizer" not in out and "runtime error:" not in out, out[-4000:]


def test_c_abi_layer_under_asan_and_ubsan():
    from gqa_flash_attention_prefill_amd import build
    runtime = _runtime(["/opt/rocm/llvm/bin/clang", "-print-file-name=libclang_rt.asan-x86_64.so"])
    if runtime is None:
        pytest.skip("clang's ASan runtime is not installed")
    try:
        lib = build.build_host_sanitized()
    except RuntimeError as e:
        pytest.skip(str(e))
    _run(runtime, "gqa_flash_attention_prefill_amd.binding", "LIB_PATH", lib,
         ["test_abi.py", "test_binding_checks.py"], "m._lib._name if m._lib else None")


def test_oracle_under_asan_and_ubsan():
    from oracle import build
    runtime = _runtime(["gcc", "-print-file-name=libasan.so"])
    if runtime is None:
        pytest.skip("gcc's libasan is not installed")
    lib = build.build(sanitize=True)
    _run(runtime, "oracle", "_LIB_PATH", lib,
         ["test_oracle_pins.py", "test_oracle_lse_pins.py", "test_oracle_noncausal_pins.py",
          "test_tile_floor.py"], "m._lib._name if m._lib else None")
