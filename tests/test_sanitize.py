"""AddressSanitizer + UndefinedBehaviorSanitizer build of the C oracle and the
C test helpers (host code only, gcc), driven through every mode and option on
small inputs, ordinary and out-of-range values (tests/helpers/
sanitize_driver.c).  Any out-of-bounds access, leak, signed overflow or
invalid shift fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_and_helpers_clean_under_asan_ubsan(tmp_path):
    exe = tmp_path / "sanitize_driver"
    srcs = [os.path.join(ROOT, "tests", "helpers", "sanitize_driver.c"),
            os.path.join(ROOT, "oracle", "lamp_oracle.c"),
            os.path.join(ROOT, "oracle", "lamp_mlp_oracle.c"),
            os.path.join(ROOT, "tests", "helpers", "rn_bits_check.c"),
            os.path.join(ROOT, "tests", "helpers", "fast_ps_emul.c"),
            os.path.join(ROOT, "tests", "helpers", "exp64_emul.c")]
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fno-fast-math", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-o", str(exe), *srcs, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    # verify_asan_link_order=0: the environment may preload other libraries
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "clean" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
