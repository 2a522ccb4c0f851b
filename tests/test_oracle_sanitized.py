"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host code only):
the oracle source is built again with -fsanitize=address,undefined and
-fno-sanitize-recover=all, and the four pin suites run against that build in a child
process with the sanitizer runtime preloaded.  Any out-of-bounds access, use after free
or undefined behaviour in the oracle ends the child with a report, and the test fails."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_oracle_pins.py", "tests/test_oracle_delta_pins.py", "tests/test_oracle_variant_pins.py",
          "tests/test_oracle_softmax_pins.py"]


def _runtime(name):
    r = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_pin_suites_under_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    lib = oracle.build_oracle_sanitized(str(tmp_path / "liblinattn_oracle_asan.so"))
    env = dict(os.environ)
    env.update({
        "LINATTN_ORACLE_LIB": lib,
        "LD_PRELOAD": asan,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:verify_asan_link_order=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    probe = subprocess.run([sys.executable, "-c", "import oracle, numpy as np; "
                            "oracle.recurrence(np.ones((2, 3)), np.ones((2, 3)), np.ones((2, 1)), None, 1e-6); "
                            "print(oracle.loaded_library())"], cwd=ROOT, env=env, capture_output=True, text=True,
                           timeout=300)
    assert probe.returncode == 0, probe.stderr[-3000:]
    assert probe.stdout.strip().endswith("liblinattn_oracle_asan.so")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *SUITES], cwd=ROOT,
                       env=env, capture_output=True, text=True, timeout=1200)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    assert " passed" in r.stdout, tail


def test_sanitizer_build_catches_a_planted_overrun(tmp_path):
    """Control: the same flags on a three-line C program that reads one element past a
    heap array must stop it with an AddressSanitizer report, so the suite above is checked."""
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    src = tmp_path / "overrun.c"
    src.write_text("#include <stdlib.h>\n#include <stdio.h>\n"
                   "int main(void) { double *a = malloc(4 * sizeof(double)); for (int i = 0; i < 4; ++i) a[i] = i;\n"
                   "volatile int n = 4; printf(\"%f\\n\", a[n]); free(a); return 0; }\n")
    exe = str(tmp_path / "overrun")
    subprocess.run(["gcc", *oracle.SANITIZE_FLAGS, "-o", exe, str(src)], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    # UBSan's object-size check or ASan's heap check, whichever sees it first
    assert r.returncode != 0 and ("heap-buffer-overflow" in r.stderr or "runtime error:" in r.stderr), r.stderr
