"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle.c does raw index arithmetic over caller arrays (hash indices, tile and
pixel lists, per-Gaussian gradient buffers).  Here it is rebuilt with
-fsanitize=address,undefined (host code, gcc) and every oracle pin test
(the Tiny scene, the closed forms, the central-difference gradient pins of
the render, decoder and SH chains, the training and densify steps) runs
against that build in a child process that preloads the sanitizer runtimes;
any out-of-bounds access, use after free or undefined operation aborts it.

A first test plants a heap overflow, a use after free and a signed overflow
in a throwaway C program built with the same flags and checks that each is
reported, so that a green run means the instrumentation was active.
"""
import glob
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

from oracle import build as B  # noqa: E402

PLANTED = r"""
#include <stdio.h>
#include <stdlib.h>
#include <limits.h>
int main(int argc, char** argv) {
    if (argv[1][0] == 'h') {           /* heap overflow: one past the end */
        int* a = malloc(8 * sizeof(int));
        a[argc + 6] = 1;
        printf("%d\n", a[0]);
        free(a);
    } else if (argv[1][0] == 'u') {    /* use after free */
        int* a = malloc(8 * sizeof(int));
        free(a);
        printf("%d\n", a[argc]);
    } else {                           /* signed overflow */
        int x = INT_MAX - 1 + argc;
        printf("%d\n", x + 1);
    }
    return 0;
}
"""


def _san_env():
    env = dict(os.environ)
    env.update(ORACLE_SANITIZED="1", LD_PRELOAD=":".join(B.sanitizer_runtimes()),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               OMP_NUM_THREADS="4", PYTHONPATH=ROOT)
    return env


def test_sanitizers_report_planted_errors(tmp_path):
    src = tmp_path / "planted.c"
    src.write_text(PLANTED)
    exe = tmp_path / "planted"
    subprocess.run(["gcc", *B.SAN_FLAGS, str(src), "-o", str(exe)], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([str(exe), "heap"], capture_output=True, text=True, env=env)
    # UBSan's object-size check or ASan's redzone, whichever sees it first
    assert r.returncode != 0 and ("heap-buffer-overflow" in r.stderr or "insufficient space" in r.stderr)
    r = subprocess.run([str(exe), "use"], capture_output=True, text=True, env=env)
    assert r.returncode != 0 and "heap-use-after-free" in r.stderr
    r = subprocess.run([str(exe), "signed"], capture_output=True, text=True, env=env)
    assert r.returncode != 0 and "signed integer overflow" in r.stderr


@pytest.mark.timeout(900)
def test_oracle_pins_under_sanitizers():
    B.build(sanitize=True)
    env = _san_env()
    # the child really loads the instrumented library
    probe = ("import oracle as O; import os; L = O.lib(); "
             "assert os.path.basename(L._name) == 'liboracle_san.so', L._name; print('loaded', L._name)")
    r = subprocess.run([sys.executable, "-c", probe], capture_output=True, text=True, env=env, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    files = sorted(glob.glob(os.path.join(HERE, "test_oracle_*.py")))
    assert len(files) >= 7
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *files],
                       capture_output=True, text=True, env=env, cwd=ROOT)
    tail = (r.stdout[-3000:] + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "failed" not in r.stdout, tail
