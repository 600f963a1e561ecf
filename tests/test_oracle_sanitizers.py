"""The CPU oracle under the host sanitizers: tests/oracle_sanitize_driver.cpp
calls every C entry point of oracle/kvp_oracle.cpp on small and degenerate
shapes, with one and several threads.  Built with AddressSanitizer and
UndefinedBehaviorSanitizer (any report aborts the run), and separately with
ThreadSanitizer for the oracle's worker threads, which write disjoint slices
and are summed in a fixed order."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
DRIVER = os.path.join(HERE, "oracle_sanitize_driver.cpp")
ORACLE = os.path.join(ROOT, "oracle", "kvp_oracle.cpp")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ is not installed")


def build_and_run(tmp_path, sanitizer_flags, env_extra):
    exe = os.path.join(str(tmp_path), "driver")
    # host compiler only: this binary never touches a GPU
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-pthread", *sanitizer_flags, DRIVER, ORACLE, "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, **env_extra)
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)


def test_oracle_asan_ubsan(tmp_path):
    proc = build_and_run(tmp_path, ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
                         {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
                          "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert proc.returncode == 0, proc.stdout + proc.stderr
    assert "oracle sanitizer driver: ok" in proc.stdout
    assert "runtime error" not in proc.stderr


def test_oracle_tsan(tmp_path):
    proc = build_and_run(tmp_path, ["-fsanitize=thread"], {"TSAN_OPTIONS": "halt_on_error=1"})
    if proc.returncode != 0 and "unexpected memory mapping" in proc.stderr:
        pytest.skip("ThreadSanitizer cannot map its shadow memory in this environment")
    assert proc.returncode == 0, proc.stdout + proc.stderr
    assert "oracle sanitizer driver: ok" in proc.stdout
    assert "WARNING: ThreadSanitizer" not in proc.stderr


def test_asan_catches_a_planted_overrun(tmp_path):
    """The harness itself: a copy of the oracle whose LSE row sum reads one
    logit past the row must be reported by AddressSanitizer."""
    src = open(ORACLE).read()
    line = "for (int64_t j = 0; j <= i; ++j) z += std::exp(logit[j] - m);"
    assert src.count(line) == 1
    mutant = os.path.join(str(tmp_path), "kvp_oracle_overrun.cpp")
    with open(mutant, "w") as f:
        f.write(src.replace(line, line.replace("j <= i;", "j <= i + 1;")))
    exe = os.path.join(str(tmp_path), "driver_overrun")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-pthread", "-fsanitize=address",
                    DRIVER, mutant, "-o", exe], check=True, capture_output=True, text=True)
    proc = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                          env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    assert proc.returncode != 0
    assert "heap-buffer-overflow" in proc.stderr
