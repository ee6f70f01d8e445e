"""The oracle's C under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle (plain C, loaded through ctypes) is built a second time with both
sanitizers and the oracle test files run against that build in a child
process with the sanitizer runtimes preloaded; any out-of-bounds access,
use after free or undefined behaviour aborts the child.  CPU only."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    if shutil.which("gcc") is None:
        return None
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    sys.path.insert(0, ROOT)
    from oracle import build as obuild
    lib = obuild.build(out=str(tmp_path / "libmoe_ref_asan.so"), sanitize=True)
    env = dict(os.environ, MOE_REF_LIB=lib, LD_PRELOAD=f"{asan} {ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_numerics.py"),
                        os.path.join(ROOT, "tests", "test_oracle_ops.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
