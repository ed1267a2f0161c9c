"""Host check of the executor's RoPE angle routines (persistent_micro_dispatch_amd/
csrc/rope_math.h) against the C library in long double: the same source the
device compiles, built for the CPU."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "persistent_micro_dispatch_amd", "csrc")

# a double ulp is 2.2e-16 relative; each routine rounds a few dozen times
LIMITS = {"log2": 1e-15, "exp2": 1e-15, "sin": 1e-15, "cos": 1e-15, "angle": 2e-15}


@pytest.fixture(scope="module")
def results(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("rope_math") / "check")
    subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", f"-I{CSRC}",
                    os.path.join(HERE, "native", "rope_math_check.cpp"), "-o", exe], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    return {ln.split()[0]: float(ln.split()[1]) for ln in out.splitlines()}


@pytest.mark.parametrize("name", sorted(LIMITS))
def test_rope_math_accuracy(results, name):
    assert results[name] <= LIMITS[name], (name, results[name])
