"""The oracle and the input generators (plain C) built with AddressSanitizer
and UndefinedBehaviorSanitizer and run on small inputs by a C driver
(tests/sanitize_driver.c): any out-of-bounds access, use after free, leak or
undefined behaviour fails the test.  Host code only; no GPU."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_and_generators_under_asan_ubsan(tmp_path):
    exe = tmp_path / "sanitize_driver"
    srcs = [os.path.join(HERE, "sanitize_driver.c"), os.path.join(ROOT, "oracle", "maple_oracle.c"),
            os.path.join(ROOT, "ternary_weight_moe_amd", "synth", "synth.c")]
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", *srcs, "-o",
                    str(exe), "-lm"], check=True, capture_output=True, text=True)
    env = dict(os.environ, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
