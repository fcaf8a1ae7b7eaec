"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, OpenMP off) must pass every pin: no out-of-bounds access, no use of
freed memory and no undefined behaviour anywhere on the paths the pins
exercise.  CPU only.

The sanitizer runtime has to be the first library in the process, so the
pins run in a child interpreter started with the runtime preloaded; the
child swaps the sanitized build in for the oracle's own library and calls
every check of ``tests/oracle_pins.py``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
SRC = ROOT / "oracle" / "gdr_oracle.c"

CHILD = r"""
import ctypes, sys
sys.path.insert(0, sys.argv[1])
import oracle
from tests import oracle_pins
oracle._lib = oracle._bind(ctypes.CDLL(sys.argv[2]))
assert oracle.threads_used(8) == 1, "the sanitized build runs without OpenMP"
for check in oracle_pins.ALL_CHECKS:
    check()
    print("ok", check.__name__, flush=True)
print("all pins passed", flush=True)
"""


def _runtime(name: str) -> str:
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and Path(path).exists() else ""


@pytest.mark.timeout(900)
def test_pins_pass_on_sanitized_oracle(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    asan = _runtime("libasan.so")
    if not asan:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    so = tmp_path / "libgdr_oracle_san.so"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", str(SRC), "-o", str(so),
           "-lm"]
    subprocess.run(cmd, check=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    # Python itself keeps allocations alive at exit; leaks are not what is checked here.
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    res = subprocess.run([sys.executable, "-c", CHILD, str(ROOT), str(so)], env=env,
                         capture_output=True, text=True, timeout=850)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "all pins passed" in res.stdout, tail
    assert "runtime error" not in res.stderr, tail
