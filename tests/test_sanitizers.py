"""Host code under the compilers' sanitizers (CPU only; no GPU code is built
with them): the host library's protocol code driven through the C ABI on a
loopback context (a producer submitting bursts and rebinding op ids, a
second thread polling sync, query and stats, the loopback consumer thread)
under ThreadSanitizer and under AddressSanitizer with UndefinedBehavior-
Sanitizer; the executor protocol model under ThreadSanitizer; the hazard
tracker's brute-force check and the oracle's pins under AddressSanitizer
with UndefinedBehaviorSanitizer.  Any report fails the test."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "persistent_micro_dispatch_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIP_FLAGS = ["-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include", f"-I{CSRC}"]


def _build(out, srcs, san, extra=()):
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-pthread", f"-fsanitize={san}", "-fno-omit-frame-pointer",
           *HIP_FLAGS, *srcs, *extra, "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=env)
    text = r.stdout + r.stderr
    assert r.returncode == 0, text[-4000:]
    for word in ("ThreadSanitizer", "AddressSanitizer", "runtime error:"):
        assert word not in text, text[-4000:]
    return text


@pytest.mark.parametrize("san", ["thread", "address,undefined"])
def test_host_library_loopback(tmp_path, san):
    exe = str(tmp_path / "host_loopback")
    _build(exe, [os.path.join(HERE, "native", "host_loopback.cpp"), os.path.join(CSRC, "gpuos_host.cpp"),
                 os.path.join(CSRC, "gpuos_jit.cpp")], san,
           [f"-L{ROCM}/lib", "-lamdhip64", "-ldl", f"-Wl,-rpath,{ROCM}/lib"])
    env = dict(os.environ, UBSAN_OPTIONS="halt_on_error=1", ASAN_OPTIONS="detect_leaks=0")
    assert "ok 5000 descriptors" in _run([exe, "5000"], env)


def test_executor_model_under_thread_sanitizer(tmp_path):
    exe = str(tmp_path / "executor_model")
    _build(exe, [os.path.join(HERE, "native", "executor_model.cpp")], "thread")
    out = _run([exe, "200"], timeout=900)
    assert out.count("ok") >= 10


def test_hazard_tracker_under_address_sanitizer(tmp_path):
    exe = str(tmp_path / "hazard_check")
    _build(exe, [os.path.join(HERE, "native", "hazard_check.cpp")], "address,undefined")
    env = dict(os.environ, UBSAN_OPTIONS="halt_on_error=1")
    assert _run([exe, "1000"], env).count("ok") == 18


def test_oracle_pins_under_address_sanitizer(tmp_path):
    lib = str(tmp_path / "liboracle_asan.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-o", lib,
                    os.path.join(ROOT, "oracle", "gpuos_oracle.c"), "-lm"], check=True, capture_output=True)
    rt = [subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True, text=True, check=True).stdout.strip()
          for n in ("libasan.so", "libubsan.so")]
    env = dict(os.environ, LD_PRELOAD=":".join(rt), ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1", GPUOS_ORACLE_LIB=lib)
    # the sanitized build is the one loaded, then the pins run against it
    probe = ("import oracle, os; oracle.lib(); "
             "assert any(oracle.LIB in l for l in open(f'/proc/{os.getpid()}/maps')), oracle.LIB")
    _run([sys.executable, "-c", probe], env)
    out = _run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_oracle_pins.py"), "-q", "-x",
                "-p", "no:cacheprovider"], env, timeout=900)
    assert " passed" in out
