"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The oracle, built by gcc with -fsanitize=address,undefined, runs every pin.
* The library, built with its host code (argument checks, the launch table,
  the launch path up to the HIP runtime) instrumented by clang's ASan and
  UBSan, runs the host-only ABI tests (tests/test_abi.py), which exercise
  validation and planning over every documented error and shape rule.

Each runs in a child process that preloads the matching sanitizer runtime,
so any report aborts the child and fails the test with the report."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))


def _env(preload, **extra):
    env = dict(os.environ)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.update(extra)
    return env


def test_oracle_pins_under_asan_ubsan(tmp_path):
    import oracle
    lib = oracle.build(out=str(tmp_path / "liboracle_san.so"), sanitize=True)
    code = ("import functools, sys; sys.path[:0] = [%r, %r]\n"
            "import oracle, oracle_pins\n"
            "upd = functools.partial(oracle.update, lib_path=%r)\n"
            "for pin in oracle_pins.ALL_PINS:\n"
            "    pin(upd)\n"
            "print('pins', len(oracle_pins.ALL_PINS))\n") % (ROOT, HERE, lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600,
                       env=_env(oracle.sanitizer_runtime()))
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-6000:]
    assert "pins" in r.stdout


def test_library_host_code_under_asan_ubsan(tmp_path):
    from linear_attention_recurrent_gating_amd import build
    lib = build.build(out=str(tmp_path / "libgdn_san.so"), sanitize=True)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi.py")], capture_output=True, text=True,
                       timeout=900, cwd=ROOT, env=_env(build.asan_runtime(), GDN_LIBRARY=lib))
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-6000:]
    assert " passed" in r.stdout
