"""Host-only tests of the proxy thread and its stall watchdog (CPU only).

The proxy class (page "arx.cu", proxy_loop: post the seqs one after another, report
stalls after 2 s) is built with g++ against a fake device thread in ordinary
memory, once plainly, once under ThreadSanitizer and once under
AddressSanitizer with UndefinedBehaviorSanitizer (host code only)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "proxy_harness.cpp")
INC = os.path.join(ROOT, "signal_pad_sync_amd", "csrc")
OUT = os.path.join(ROOT, "tests", "host", "_build")


def build(name, flags):
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, name)
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Werror", "-pthread", *flags, "-I", INC, SRC, "-o", exe],
                   check=True)
    return exe


SCENARIOS = ["lockstep", "runahead", "manual", "no_skip_no_lead", "watchdog", "concurrent_publish", "stress",
             "stress_switch"]


@pytest.mark.parametrize("variant,flags", [("plain", ["-O2"]), ("tsan", ["-O1", "-g", "-fsanitize=thread"]),
                                           ("asan_ubsan", ["-O1", "-g", "-fsanitize=address,undefined",
                                                           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"])])
def test_proxy_scenarios(variant, flags):
    exe = build(f"proxy_{variant}", flags)
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 second_deadlock_stack=1",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    for s in SCENARIOS:
        assert f"ok {s}" in r.stdout, r.stdout
    assert "WARNING: ThreadSanitizer" not in r.stderr, r.stderr
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, r.stderr
