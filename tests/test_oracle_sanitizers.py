"""The oracle under CPU sanitizers: oracle/selftest.c drives every
multi-threaded oracle routine on small seeded inputs (1 and 7 threads, which
must agree), built once with AddressSanitizer + UndefinedBehaviorSanitizer
(any report aborts) and once with ThreadSanitizer. Host code only; no GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")

FLAVOURS = {
    "asan_ubsan": ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                   "-fno-omit-frame-pointer"],
    "tsan": ["-fsanitize=thread"],
}


@pytest.mark.parametrize("flavour", list(FLAVOURS))
def test_oracle_clean_under_sanitizer(tmp_path, flavour):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = tmp_path / f"selftest_{flavour}"
    cmd = [gcc, "-std=c11", "-O1", "-g", "-ffp-contract=off", *FLAVOURS[flavour],
           os.path.join(ORACLE, "oracle.c"), os.path.join(ORACLE, "selftest.c"),
           "-o", str(exe), "-lm", "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    # verify_asan_link_order=0: run whatever the environment preloads
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "selftest ok" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
