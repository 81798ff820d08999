"""The host C code (the fp64 oracle and the input generator) built with
AddressSanitizer and UndefinedBehaviorSanitizer, and every oracle pin run
against those builds in a child process: an out-of-bounds access, a use after
free or undefined arithmetic anywhere in them fails this test. CPU only; the
sanitized builds go to a temporary directory and the in-tree libraries are
left alone."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fPIC", "-shared", "-pthread"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(_runtime("libasan.so") is None or _runtime("libubsan.so") is None,
                    reason="gcc's sanitizer runtimes are not installed")
def test_oracle_and_generator_pins_under_asan_and_ubsan(tmp_path):
    libs = {}
    for env, src, lib in (("TVO_LIB", "oracle/oracle.c", "liboracle_san.so"),
                          ("TVG_LIB", "tvgen/tvgen.c", "libtvgen_san.so")):
        out = str(tmp_path / lib)
        extra = ["-std=c11"] if "oracle" in src else ["-fopenmp"]
        subprocess.check_call(["gcc", *FLAGS, *extra, "-o", out, os.path.join(ROOT, src), "-lm"])
        libs[env] = out
    env = dict(os.environ, **libs)
    env["LD_PRELOAD"] = ":".join([_runtime("libasan.so"), _runtime("libubsan.so")])
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=87"
    tests = sorted(f for f in os.listdir(os.path.join(ROOT, "tests")) if f.startswith("test_oracle_"))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *[os.path.join(ROOT, "tests", t) for t in tests]],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    log = r.stdout + r.stderr
    assert "AddressSanitizer" not in log and "runtime error" not in log, log[-4000:]
    assert r.returncode == 0, log[-4000:]
    assert " passed" in r.stdout
