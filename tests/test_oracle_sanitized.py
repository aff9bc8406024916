"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc,
host code only) and driven over ragged shapes by tests/csrc/oracle_sanitize.c,
every buffer allocated at exactly the size its layout needs.  Host logic only:
no GPU."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_sanitize")
    subprocess.run([gcc, "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-Wno-unknown-pragmas",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "csrc", "oracle_sanitize.c"),
                    "-o", exe, "-lm"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "oracle under sanitizers: ok" in res.stdout
