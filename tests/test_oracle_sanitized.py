"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: every
function of oracle/lcd_oracle.c and oracle/lcd_oracle_bench.c runs over seeded
random and edge-case inputs held in exact-size heap buffers
(tests/oracle_sanitize_main.c); the sanitized build must report nothing and
print the same output checksum as a plain build."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(ROOT, "oracle", "lcd_oracle.c"), os.path.join(ROOT, "oracle", "lcd_oracle_bench.c"),
           os.path.join(HERE, "oracle_sanitize_main.c")]


def _build(out, flags):
    cmd = ["gcc", "-std=c11", "-g", "-Wall", "-pthread", *flags, *SOURCES, "-o", out, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    plain, san = str(tmp_path / "plain"), str(tmp_path / "san")
    _build(plain, ["-O1"])
    _build(san, ["-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                 "-fno-omit-frame-pointer"])
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    a = subprocess.run([plain, "300"], capture_output=True, text=True, timeout=300)
    b = subprocess.run([san, "300"], capture_output=True, text=True, timeout=600, env=env)
    assert a.returncode == 0, a.stderr
    assert b.returncode == 0, b.stderr[-4000:]
    assert "runtime error" not in b.stderr and "AddressSanitizer" not in b.stderr, b.stderr[-4000:]
    assert a.stdout.strip() == b.stdout.strip() and len(a.stdout.strip()) == 16
