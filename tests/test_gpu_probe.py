"""The HBM probe through the C ABI: a copy reproduces its source byte for
byte and both modes report a positive bandwidth (no executor is resident
while it runs)."""
import numpy as np
import pytest

from gpu_harness import say
from persistent_micro_dispatch_amd import gpuos as G

pytestmark = pytest.mark.gpu


def test_hbm_probe_copy_and_read():
    import torch
    n = 64 << 20
    say(f"hbm probe {n} bytes")
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros(n, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream()
    s.synchronize()
    g_copy = G.gpuos_hbm_probe(src.data_ptr(), dst.data_ptr(), n, 1, 2, s.cuda_stream)
    g_read = G.gpuos_hbm_probe(src.data_ptr(), dst.data_ptr(), n, 0, 2, s.cuda_stream)
    assert torch.equal(src, dst)
    say(f"  copy {g_copy:.0f} GB/s, read {g_read:.0f} GB/s")
    assert g_copy > 0 and g_read > 0


@pytest.mark.parametrize("wg", [1, 8, 64, 300])
def test_hbm_probe_grid_copy_reproduces_its_source(wg):
    import torch
    n = (16 << 20) + 4096 + 16
    say(f"hbm probe grid {wg} workgroups, {n} bytes")
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros(n, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream()
    s.synchronize()
    g = G.gpuos_hbm_probe_grid(src.data_ptr(), dst.data_ptr(), n, 1, 1, wg, s.cuda_stream)
    assert torch.equal(src, dst) and g > 0
    say(f"  copy {g:.0f} GB/s")
