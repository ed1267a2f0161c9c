"""Brute-force check of the host's hazard tracker (csrc/hazard.h), built for
the CPU: random descriptor streams of byte-range accesses (prefixes,
arbitrary sub-ranges, accesses spanning neighbouring tensors, a rotating
arena, hot tensors read by many descriptors) with a completion process that
retires descriptors in a random order their dependencies allow.  Every live
earlier descriptor whose accesses conflict with a new one must be reached
through the dependencies the tracker returns (tests/native/hazard_check.cpp)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "persistent_micro_dispatch_amd", "csrc")


def test_tracker_orders_every_conflict(tmp_path):
    exe = str(tmp_path / "hazard_check")
    subprocess.run(["g++", "-O2", "-std=c++17", f"-I{CSRC}", os.path.join(HERE, "native", "hazard_check.cpp"),
                    "-o", exe], check=True)
    r = subprocess.run([exe, "3000"], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = r.stdout.split()
    assert r.stdout.count("ok") == 18
