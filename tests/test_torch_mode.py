"""CPU tests of the PyTorch routing layer (persistent_micro_dispatch_amd/
torch_mode.py): the four-dimensional filter's decisions, the fallback to a
normal launch when the ring is full, and the ordering between routed and
normal ops.  The library calls are replaced by fakes here (no GPU); the GPU
parity of routed sequences is in test_gpu_torch_mode.py."""
import pytest
import torch
import torch.nn.functional as F

from persistent_micro_dispatch_amd import gpuos as G
from persistent_micro_dispatch_amd import torch_mode as TM

aten = torch.ops.aten


def _f(*shape, dtype=torch.float32):
    return torch.randn(*shape).to(dtype)


def test_filter_operation_type_size_and_context():
    flt = TM.RoutingFilter(max_elems=4096, hot_after=2, device_type="cpu")
    a, b = _f(16, 64), _f(16, 64)
    # dimension 3: the first sighting of a key stays on the normal path
    assert flt.decide(aten.add.Tensor, (a, b), {}).reason == "cold"
    d = flt.decide(aten.add.Tensor, (a, b), {})
    assert d.route and d.kind == G.GPUOS_OP_ADD and d.out is None
    # a different shape is a different key
    assert flt.decide(aten.add.Tensor, (_f(8, 64), _f(8, 64)), {}).reason == "cold"
    flt.hot_after = 1
    # dimension 1: operation type and the forms its body takes
    assert flt.decide(aten.mm.default, (a, b.t()), {}).reason == "matmul form"  # fp32: not a bf16 matmul
    assert flt.decide(aten.bmm.default, (a[None], b.t()[None]), {}).reason == "op type"
    assert flt.decide(aten.add.Tensor, (a, b), {"alpha": 2}).reason == "op form"
    assert flt.decide(aten.add.Tensor, (a, _f(1, 64)), {}).reason == "broadcast"
    assert flt.decide(aten.add.Tensor, (a, 2.0), {}).reason == "not a tensor"
    assert flt.decide(aten.mul.Tensor, (a, b.to(torch.bfloat16)), {}).reason == "mixed operands"
    assert flt.decide(aten.relu.default, (torch.ones(4, dtype=torch.int32),), {}).reason == "dtype"
    assert flt.decide(aten.relu.default, (_f(64, 16).t(),), {}).reason == "layout"
    assert flt.decide(aten.gelu.default, (a,), {}).reason == "gelu variant"
    d = flt.decide(aten.gelu.default, (a,), {"approximate": "tanh"})
    assert d.route and d.kind == G.GPUOS_OP_GELU
    d = flt.decide(aten.add_.Tensor, (a, b), {})
    assert d.route and d.out is a
    d = flt.decide(aten.sum.dim_IntList, (a, [-1]), {})
    assert d.route and (d.rows, d.h, d.out_shape) == (16, 64, (16,))
    d = flt.decide(aten.amax.default, (a, [1], True), {})
    assert d.route and d.kind == G.GPUOS_OP_MAX and d.out_shape == (16, 1)
    assert flt.decide(aten.sum.dim_IntList, (a, [0]), {}).reason == "reduction dims"
    assert flt.decide(aten.sum.dim_IntList, (a, [0, 1]), {}).reason == "reduction dims"
    assert flt.decide(aten._softmax.default, (a, 0, False), {}).reason == "softmax dim"
    d = flt.decide(aten._softmax.default, (a, -1, False), {})
    assert d.route and d.kind == G.GPUOS_OP_SOFTMAX and d.rows == 16
    d = flt.decide(aten.copy_.default, (_f(16, 64), a), {})
    assert d.route and d.kind == G.GPUOS_OP_COPY
    # dimension 2: size
    big = _f(128, 64)
    assert flt.decide(aten.relu.default, (big,), {}).reason == "size"
    # only the context's device
    assert TM.RoutingFilter(device_type="cuda").decide(aten.relu.default, (a,), {}).reason == "device"


class _FakeLib:
    """Stands in for the library: records submissions and syncs; routed ops
    complete only when synced."""

    def __init__(self, full=False):
        self.full, self.seq, self.submitted, self.syncs = full, 100, [], 0

    def install(self, mp):
        mp.setattr(G, "gpuos_init", lambda **kw: 1)
        mp.setattr(G, "gpuos_shutdown", lambda ctx: 0)
        mp.setattr(G, "gpuos_submit", self.submit)
        mp.setattr(G, "gpuos_sync", self.sync)
        mp.setattr(G, "gpuos_query", lambda ctx, s: 0)

    def submit(self, ctx, descs, flags):
        assert flags == 0  # never blocks: a full ring means the normal path
        if self.full:
            return G.GPUOS_E_FULL, 0
        self.submitted.append(descs.copy())
        self.seq += 1
        return G.GPUOS_OK, self.seq - 1

    def sync(self, ctx, upto, timeout):
        self.syncs += 1
        return G.GPUOS_OK, 0, 0


def test_full_ring_falls_back_to_a_normal_launch(monkeypatch):
    lib = _FakeLib(full=True)
    lib.install(monkeypatch)
    x, y = _f(32), _f(32)
    with TM.GpuosMode(filter=TM.RoutingFilter(hot_after=1, device_type="cpu")) as m:
        z = x + y
    assert torch.equal(z, x + y)
    assert m.stats.fallback["ring full"] == 1 and not m.stats.routed


def test_routed_and_normal_ops_are_ordered_by_storage(monkeypatch):
    lib = _FakeLib()
    lib.install(monkeypatch)
    x, y = _f(4, 8), _f(4, 8)
    with TM.GpuosMode(filter=TM.RoutingFilter(hot_after=1, device_type="cpu")) as m:
        z = x + y                      # routed: x, y, z in flight
        assert len(lib.submitted) == 1 and lib.syncs == 0
        d = lib.submitted[0][0]
        assert (d["op_id"], d["size"]) == (G.GPUOS_OP_ADD, 32)
        assert (d["input_a"], d["input_b"], d["output"]) == (x.data_ptr(), y.data_ptr(), z.data_ptr())
        w = torch.ones(3) * 2.0        # normal, touches nothing in flight: no sync
        assert lib.syncs == 0
        q = z * 3.0                    # normal (scalar operand) reading z: waits for the executor
        assert lib.syncs == 1
        r = torch.softmax(q, -1)       # routed: q was written on torch's stream (synced first)
        assert len(lib.submitted) == 2 and lib.submitted[1][0]["dim"][0] == 8
        s = F.gelu(r, approximate="tanh").sum(-1)   # two routed ops
        assert len(lib.submitted) == 4 and lib.submitted[3][0]["op_id"] == G.GPUOS_OP_SUM
    assert lib.syncs == 2              # the exit waits for everything in flight
    assert m.stats.routed == {"elementwise": 2, "softmax": 1, "reduction": 1}
    assert w.shape == (3,) and s.shape == (4,)


def test_filter_routes_small_bf16_matmuls_in_linear_layout():
    flt = TM.RoutingFilter(hot_after=1, device_type="cpu")
    x = _f(16, 256, dtype=torch.bfloat16)
    w = _f(512, 256, dtype=torch.bfloat16)          # [out, in]
    d = flt.decide(aten.mm.default, (x, w.t()), {})
    assert d.route and d.kind == G.GPUOS_OP_MATMUL and (d.rows, d.h, d.out_shape) == (16, 256, (16, 512))
    assert flt.decide(aten.mm.default, (x, w.t().contiguous()), {}).reason == "matmul form"
    assert flt.decide(aten.mm.default, (x.float(), w.t().float()), {}).reason == "matmul form"
    assert flt.decide(aten.mm.default, (_f(65, 256, dtype=torch.bfloat16), w.t()), {}).reason == "matmul size"
    assert flt.decide(aten.mm.default, (_f(16, 100, dtype=torch.bfloat16),
                                        _f(512, 100, dtype=torch.bfloat16).t()), {}).reason == "matmul size"
