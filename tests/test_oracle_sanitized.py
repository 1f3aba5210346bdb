"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The oracle is rebuilt from the same source with -fsanitize=address,undefined
and the pins of tests/test_oracle_pins.py run against that build in a child
process (the sanitizer runtimes preloaded, leak checks off: the interpreter
itself is not leak-clean).  Any out-of-bounds access, use after free or
undefined behaviour aborts the child, and the test fails with its report.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    sys.path.insert(0, ROOT)
    from oracle import build
    lib = build.build(out=str(tmp_path / "liboracle_san.so"), sanitize=True)
    env = dict(os.environ, KVQ_ORACLE_LIB=lib, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_vgroup_layout.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in out and "runtime error" not in out, out
