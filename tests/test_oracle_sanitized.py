"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only): oracle.c is built with both, and the oracle's pin and
whole-layer suites run against that build in a child process (the
sanitizer runtime preloaded, any report fatal).  An out-of-bounds access,
use after free, signed overflow or bad shift anywhere on those paths fails
this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_oracle_pins.py", "tests/test_oracle_e2e.py",
          "tests/test_oracle_balance.py", "tests/test_oracle_backward.py",
          "tests/test_oracle_dense.py"]
# cases left out under the sanitizers (each repeats the code paths of a case
# that stays, at several times the cost there)
SKIP = ("not (test_branch_backward_matches_autograd and (chunks or tight))"
        " and not (test_e2e_tiny_matches_brute_force and (dedup_chunks or chunks_tight"
        " or k1_tight))")


def _runtime(name):
    out = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc has no sanitizer runtime")
def test_oracle_suites_clean_under_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-Wall", "-fPIC", "-shared",
                           "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", os.path.join(ROOT, "oracle", "oracle.c"),
                           "-o", lib, "-lm"])
    env = dict(os.environ)
    # the suites run side by side: one BLAS / OpenMP thread each
    env.update(OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    env.update(ORACLE_LIB=lib, LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    from concurrent.futures import ThreadPoolExecutor

    def run(suite):  # one child process per suite, in parallel
        return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p",
                               "no:cacheprovider", "-m", "not gpu", "-k", SKIP, suite],
                              cwd=ROOT, env=env, capture_output=True, text=True, timeout=1500)

    with ThreadPoolExecutor(len(SUITES)) as ex:
        results = list(ex.map(run, SUITES))
    for suite, p in zip(SUITES, results):
        tail = (p.stdout + p.stderr)[-4000:]
        assert p.returncode == 0, suite + "\n" + tail
        assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
