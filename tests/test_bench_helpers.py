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


def _conflict(recs, i, j):
    """Descriptors i and j touch a common pool tensor and one of them writes
    it (every access of the element-wise stream is a prefix of a tensor)."""
    def acc(k):
        ins = {int(recs["buf"][k, W.A])} | ({int(recs["buf"][k, W.B])} if int(recs["buf"][k, W.B]) >= 0 else set())
        return ins, int(recs["buf"][k, W.OUT])
    ri, wi = acc(i)
    rj, wj = acc(j)
    return wi in rj or wj in ri or wi == wj


def test_critical_path_walks_dependencies(monkeypatch):
    """critical_path on a synthetic trace: every step of the path goes to a
    conflicting earlier descriptor, the one among them that completed last,
    and the phases add up to the hop."""
    from persistent_micro_dispatch_amd import gpuos as G
    s = W.make_elementwise(n_desc=300, n_per_dtype=4)
    recs = s.recs
    n = len(recs)
    rng = np.random.default_rng(7)
    units = rng.integers(1, 4, n)
    seq = np.repeat(np.arange(n), units)
    tr = np.zeros(len(seq), G.TRACE_DTYPE)
    tr["seq"] = 500 + seq
    # completion times rise with sequence (plus jitter); units of one
    # descriptor start 0-3 ticks apart and finish together
    done = 1000 + 100 * np.arange(n) + rng.integers(0, 90, n)
    off = rng.integers(0, 4, len(seq))
    tr["t_done"] = done[seq]
    tr["t_body"] = done[seq] - 5
    tr["t_ready"] = done[seq] - 40 + off
    tr["t_claim"] = done[seq] - 60 + off
    tr = tr[rng.permutation(len(tr))]
    for f, v in (("gpuos_init", lambda **k: 1), ("gpuos_pause", lambda c, t: 0), ("gpuos_resume", lambda c: 0),
                 ("gpuos_submit_bursts", lambda c, d, b, fl: (0, 500, len(d))),
                 ("gpuos_sync", lambda c, u, t: (0, 0, 0)), ("gpuos_trace_read", lambda c, m: tr),
                 ("gpuos_shutdown", lambda c: 0)):
        monkeypatch.setattr(G, f, v)
    out = bench.critical_path(recs, np.zeros(n), np.ones(1, np.uint32), 1, 512, 0, 1)
    assert out["hops"] >= 1 and 0.0 < out["path_share_of_span"] <= 1.0
    # rebuild the path by brute force and compare its length and hop time
    k, path = int(np.argmax(done)), [int(np.argmax(done))]
    while True:
        deps = [j for j in range(k) if _conflict(recs, k, j)]
        if not deps:
            break
        k = max(deps, key=lambda j: done[j])
        path.append(k)
    assert out["hops"] == len(path) - 1
    hops = [(done[a] - done[b]) * 1e-2 for a, b in zip(path[:-1], path[1:])]
    assert abs(out["hop_us_mean"] - np.mean(hops)) < 1e-9
    ph = out["phases_us_mean"]
    assert abs(sum(ph.values()) - out["hop_us_mean"]) < 1e-9  # the four phases partition each hop
    assert abs(ph["tail"] - np.mean([(done[a] - (done[a] - 40 + 3)) * 1e-2 for a in path[:-1]])) < 0.03 + 1e-9
