"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

``oracle/oracle.c`` is compiled with ``-fsanitize=address,undefined`` (no
recovery: the first report aborts) into pytest's tmp_path, and every pin of
``test_oracle_pins.py`` runs against that copy in a child Python process with
the ASan runtime preloaded (it must come first in the process); the child
finds the copy through the ORACLE_LIB variable the oracle wrapper honours.  The pins must
all pass and the sanitizers must report nothing: no out-of-bounds access, no
use after free, no signed overflow, no misaligned or null access in the
oracle's arithmetic or its thread split.  Host code only; no GPU is involved.
"""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))

def test_pins_pass_under_sanitizers(tmp_path):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc has no AddressSanitizer runtime here")
    so = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", str(so), oracle._SRC,
                    "-lm", "-lpthread"], check=True)
    env = dict(os.environ)
    env["ORACLE_LIB"] = str(so)
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    cmd = [sys.executable, "-m", "pytest", os.path.join(HERE, "test_oracle_pins.py"), "-q", "-x", "-s",
           "-p", "no:cacheprovider", "-m", "not gpu"]
    res = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=900, cwd=os.path.dirname(HERE))
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in res.stdout and "failed" not in res.stdout, res.stdout[-2000:]
