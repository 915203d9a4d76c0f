"""AddressSanitizer + UndefinedBehaviorSanitizer over the oracle and the
library's host-only code, and ThreadSanitizer over CPU-Adam's worker pool
(CPU only).

Two drivers under tests/sanitize/ call every oracle function, and the
planner, bucket planner and CPU-Adam of the library, on small inputs with
padding, N = 1, odd rank counts, injected overflow, unaligned offsets and the
error paths.  They are built with g++/gcc -fsanitize=address,undefined
(no recovery: the first report fails the run) and must finish cleanly.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-ffp-contract=off"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, exe):
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    out = _run(["gcc", "-std=c99", *SAN, "-I", os.path.join(ROOT, "oracle"), "-o", exe,
                os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                os.path.join(ROOT, "oracle", "zf_oracle.c"), "-lm"], exe)
    assert "oracle driver: ok" in out


def test_host_library_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_driver")
    csrc = os.path.join(ROOT, "fsdp_sharded_mixed_amd", "csrc")
    out = _run(["g++", "-std=c++17", "-pthread", *SAN, "-I", os.path.join(ROOT, "include"),
                "-I", csrc, "-o", exe, os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"),
                os.path.join(csrc, "zf_plan.cpp"), os.path.join(csrc, "zf_cpu_adam.cpp")], exe)
    assert "host driver: ok" in out


def test_cpu_adam_pool_under_thread_sanitizer(tmp_path):
    """Five threads call the multithreaded CPU-Adam at once (the pool grows
    while callers take turns); results equal single-threaded runs bit for
    bit and ThreadSanitizer reports no race."""
    exe = str(tmp_path / "threads_driver")
    csrc = os.path.join(ROOT, "fsdp_sharded_mixed_amd", "csrc")
    cmd = ["g++", "-std=c++17", "-pthread", "-O1", "-g", "-fsanitize=thread",
           "-ffp-contract=off", "-I", os.path.join(ROOT, "include"), "-I", csrc, "-o", exe,
           os.path.join(ROOT, "tests", "sanitize", "threads_driver.cpp"),
           os.path.join(csrc, "zf_plan.cpp"), os.path.join(csrc, "zf_cpu_adam.cpp")]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1:second_deadlock_stack=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "ThreadSanitizer" not in r.stderr, r.stderr[-4000:]
    assert "threads driver: ok" in r.stdout or "nothing to check" in r.stdout
