"""The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc, host code
only) runs every pin it implements and the cross-checks against the numpy oracle in a
child process; any out-of-bounds access, use after free or undefined operation aborts it."""
import os
import subprocess
import sys

import pytest

from oracle import build_ref

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle_pins as P
import test_c_oracle as T
from oracle.c_oracle import COracle
C = COracle({lib!r}, threads=4)
for pin in T.C_PINS:
    P.O = C
    pin()
for i in range(len(T.ROUTES)):
    T.test_route_matches_numpy(i, C)
for i in range(len(T.LAYERS)):
    T.test_layer_matches_numpy(i, C)
T.test_fp8_matches_numpy(C)
T.test_threads_do_not_change_results(C)
T.test_bad_arguments_raise(C)
print("sanitized run complete", len(T.C_PINS))
"""


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_c_oracle_under_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc's sanitizer runtimes are not installed")
    lib = build_ref.build(out=str(tmp_path / "libmoe_ref_san.so"),
                          extra=("-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                                 "-fno-omit-frame-pointer", "-g"))
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    p = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, tests=HERE, lib=lib)],
                       env=env, capture_output=True, text=True, timeout=600)
    assert p.returncode == 0 and "sanitized run complete" in p.stdout, \
        (p.returncode, p.stdout[-2000:], p.stderr[-4000:])
