"""The oracle's pins again, against a build of the oracle with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc, CPU only).

The pins of test_oracle_pins.py run in a child process whose oracle package loads the
sanitized library (SFI_ORACLE_LIB) with the sanitizer runtimes preloaded, so an out-of-bounds
access, a use after free or undefined behaviour (signed overflow, a misaligned load, a bad
shift) anywhere in the oracle fails the run even where the numbers would still match.  No
test here needs a GPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    try:
        path = subprocess.check_output(["gcc", f"-print-file-name={name}"], text=True).strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    sys.path.insert(0, ROOT)
    import oracle

    lib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    env = dict(os.environ)
    env.update({
        "SFI_ORACLE_LIB": lib,
        "LD_PRELOAD": f"{asan}:{ubsan}",
        # the interpreter's own allocations are not the oracle's: no leak report at exit
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "OMP_NUM_THREADS": "4",
    })
    # -s: a sanitizer report goes to the process's own stderr, not to pytest's capture
    proc = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_oracle_pins.py")],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = proc.stdout + proc.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert "runtime error" not in out, out[-4000:]
    assert proc.returncode == 0, out[-4000:]
    assert " passed" in out, out[-4000:]


def test_sanitized_build_is_what_the_child_loads(tmp_path):
    """The override really selects the library: a missing path fails the child's first call."""
    env = dict(os.environ)
    env["SFI_ORACLE_LIB"] = str(tmp_path / "missing.so")
    proc = subprocess.run(
        [sys.executable, "-c", "import oracle; oracle.lib()"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert proc.returncode != 0
    assert "missing.so" in proc.stderr
