"""CPU check of the verify-mode machinery used by the GPU stream tests: with
the oracle standing in for the device every record passes, and a planted
error in one logged output (a perturbed oracle result) is caught."""
import numpy as np
import pytest

import gpu_harness as H
import workloads as W


class _HostPool:
    """Stands in for the device pool: host arrays."""

    def __init__(self, arrays):
        self.tensors = [np.ascontiguousarray(a).view(np.uint8).reshape(-1).copy() for a in arrays]

    def append_zeros(self, nbytes):
        self.tensors.append(np.zeros(nbytes, np.uint8))

    def download(self, i):
        return self.tensors[i].copy()


def _fake_run_gpu(perturb=None):
    def run(pool, recs, bursts=None, ctx=None, **kw):
        out = H.run_oracle(pool.tensors, recs)
        if perturb is not None:
            perturb(out)
        return out
    return run


@pytest.fixture(autouse=True)
def _host_pool(monkeypatch):
    monkeypatch.setattr(H, "DevicePool", _HostPool)


def test_verify_passes_when_device_equals_oracle(monkeypatch):
    s = W.make_mixed(tokens=1, layers=1, capacity=128, l0_range=(16, 100), n_tok_pool=2)
    monkeypatch.setattr(H, "run_gpu", _fake_run_gpu())
    res = H.verify_stream([b.host_bytes() for b in s.buffers], s.recs)
    assert not res["fails"] and res["kv_ok"] and res["n_logged"] > 10


def test_verify_catches_a_planted_error(monkeypatch):
    s = W.make_elementwise(n_desc=200, n_per_dtype=4, n_elem=4096)
    arrays = [b.host_bytes() for b in s.buffers]
    aug, layout, _ = H.with_log(s.recs, len(arrays))
    k, b, o, n, p = layout[len(layout) // 2]

    def bump(out):
        out[-1][p + 1] ^= 0x40   # flip a bit inside one logged output
    monkeypatch.setattr(H, "run_gpu", _fake_run_gpu(bump))
    res = H.verify_stream(arrays, s.recs)
    assert [f[0] for f in res["fails"]] == [k]
