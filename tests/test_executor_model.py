"""Host model of the executor's work-distribution protocol (tests/native/
executor_model.cpp): one thread per wave over bounds-checked arrays, with
the executor's own claim-shard, queue-position, queue-entry and capacity
arithmetic (csrc/gpuos_internal.h).  Checks bounds, that every queue entry
read is the one published for the claimed position, exactly-once units,
dependency order, and that every wave leaves after the stop, for 2-24
workgroups, 1-4 waves per workgroup, one or two units per wave, 1-8 claim
shards (also shards served by two or three workgroups), rings of 8-512 entries, small and large unit queues, and stops with
work in flight."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_protocol_model_passes_every_configuration(tmp_path):
    exe = str(tmp_path / "executor_model")
    subprocess.run(["g++", "-O2", "-std=c++17", "-pthread", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    f"-I{ROOT}/include", f"-I{ROOT}/persistent_micro_dispatch_amd/csrc",
                    os.path.join(HERE, "native", "executor_model.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe, "2000"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("ok ") == 36, r.stdout
