"""The oracle's pins under builds that expose data races and memory errors (CPU).

The committed build is -O2; a loop index shared by OpenMP threads, or a read past a buffer, can stay
hidden there because the compiler keeps the variable in a register.  Here every pin runs again, in a
child process with eight OpenMP threads, against
  * an -O0 build (every variable lives in memory, so threads that share one step on each other), and
  * an AddressSanitizer + UndefinedBehaviorSanitizer build (the runtimes preloaded into the child),
    which aborts on the first out-of-bounds access or undefined operation.
"""
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CHILD = r"""
import sys
sys.path.insert(0, {root!r})
from tests.oracle_pins import ALL_PINS
failed = []
for pin in ALL_PINS:
    try:
        pin({lib!r})
    except Exception as exc:  # report every pin, not only the first
        failed.append(f"{{pin.__name__}}: {{type(exc).__name__}}: {{exc}}")
print("\n".join(failed) if failed else "all pins passed")
sys.exit(1 if failed else 0)
"""


def _run_pins(lib: str, env_extra: dict) -> subprocess.CompletedProcess:
    env = dict(os.environ, OMP_NUM_THREADS="8", OMP_DYNAMIC="false", **env_extra)
    return subprocess.run([sys.executable, "-c", _CHILD.format(root=ROOT, lib=lib)], env=env,
                          capture_output=True, text=True, timeout=900)


def _gcc_runtime(name: str) -> str:
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else ""


def test_pins_unoptimised_eight_threads():
    with tempfile.TemporaryDirectory() as tmp:
        lib = oracle.build(out=os.path.join(tmp, "liboracle_o0.so"), extra_flags=["-O0"])
        r = _run_pins(lib, {})
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]


@pytest.mark.slow
def test_pins_address_and_ub_sanitizers_eight_threads():
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    with tempfile.TemporaryDirectory() as tmp:
        lib = oracle.build(out=os.path.join(tmp, "liboracle_san.so"),
                           extra_flags=["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                                        "-fno-sanitize-recover=undefined"])
        r = _run_pins(lib, {"LD_PRELOAD": f"{asan}:{ubsan}",
                            "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
                            "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
