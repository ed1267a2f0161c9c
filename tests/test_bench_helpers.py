"""Host logic of bench.py: the dependency-DAG depth it reports and the
PyTorch-eager baseline's op mapping (run here on CPU tensors, compared
with the oracle, so that the baseline times the same work)."""
import numpy as np

import bench
import oracle
import workloads as W
from oracle_util import rec


def _ew(op, a, b, o, n=16):
    return rec(op, dtype=W.F32, size=n, a=a, b=b, out=o)


def test_dag_levels_by_hand():
    # t0 = t1 + t2 (1); t3 = relu(t0) (2, RAW); t1 = t2 * t2 (2, WAR on t1
    # after the first op read it); t0 = t1 + t3 (3: RAW on t1 and t3, WAW/WAR on t0)
    recs = np.concatenate([_ew(W.OP_ADD, 1, 2, 0), _ew(W.OP_RELU, 0, -1, 3), _ew(W.OP_MUL, 2, 2, 1),
                           _ew(W.OP_ADD, 1, 3, 0)])
    assert bench.dag_levels(recs) == 3
    # independent ops on disjoint tensors: one level
    recs = np.concatenate([_ew(W.OP_ADD, 3 * i, 3 * i + 1, 3 * i + 2) for i in range(5)])
    assert bench.dag_levels(recs) == 1
    # a chain through one tensor: one level per op
    recs = np.concatenate([_ew(W.OP_ADD, 0, 1, 0) for _ in range(7)])
    assert bench.dag_levels(recs) == 7


class _Pool:
    def __init__(self, arrays):
        import torch
        self.tensors = [torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1).copy()) for a in arrays]


def _compare(stream, n):
    arrays = [b.host_bytes() for b in stream.buffers]
    recs = stream.recs[:n]
    pool = _Pool(arrays)
    for c in bench.torch_eager_calls(recs, pool, n):
        c()
    ref = oracle.Pool([a.copy() for a in arrays])
    ref.run(recs)
    return [t.numpy() for t in pool.tensors], ref.arrays


def test_torch_eager_baseline_matches_the_oracle_on_exact_ops():
    s = W.make_elementwise(n_desc=400, ops=(W.OP_ADD, W.OP_MUL, W.OP_RELU))
    got, ref = _compare(s, 400)
    # equal as values (torch's clamp keeps -0 where the oracle's ReLU gives +0;
    # the baseline only has to do the same work), NaN as a class
    for g, r, b in zip(got, ref, s.buffers):
        if b.dtype == W.F32:
            g, r = g.view(np.float32), r.view(np.float32)
        else:
            g, r = W.bf16_bits_to_f32(g.view(np.uint16)), W.bf16_bits_to_f32(r.view(np.uint16))
        nan = np.isnan(r)
        assert np.array_equal(np.isnan(g), nan)
        assert np.array_equal(g[~nan], r[~nan])


def test_torch_eager_baseline_row_ops_within_tolerance():
    s = W.make_rows(n_desc=60, n_pool=4, arena_bytes=8 << 20)
    got, ref = _compare(s, 60)
    for r in s.recs[:60]:
        for (bi, off, nb) in W.output_ranges(r):
            g = got[bi][off: off + nb].view(np.float32).astype(np.float64)
            x = ref[bi][off: off + nb].view(np.float32).astype(np.float64)
            assert np.allclose(g, x, rtol=1e-4, atol=1e-4 * max(1.0, float(np.abs(x).max()))), W.OP_NAMES[int(r["op"])]
