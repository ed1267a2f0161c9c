"""Seeded input generators: determinism and the shapes of each stream."""
import numpy as np

import workloads as W


def test_splitmix64_reference_values():
    # Published first outputs of SplitMix64 for seed 0 (the reference
    # implementation in Steele et al. / Vigna's splitmix64.c).
    got = W.splitmix64(0, 0, 3).tolist()
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_generators_are_deterministic():
    a, b = W.make_elementwise(n_desc=2000), W.make_elementwise(n_desc=2000)
    assert np.array_equal(a.recs, b.recs) and np.array_equal(a.bursts, b.bursts)
    assert np.array_equal(a.buffers[5].host_bytes(), b.buffers[5].host_bytes())
    c = W.make_elementwise(seed=7, n_desc=2000)
    assert not np.array_equal(a.recs, c.recs)


def test_elementwise_stream_shape():
    s = W.make_elementwise(n_desc=20000)
    r = s.recs
    assert r["size"].min() >= 256 and r["size"].max() <= 65536
    assert abs(np.mean(r["dtype"] == W.BF16) - 0.5) < 0.02
    inplace = r["buf"][:, W.OUT] == r["buf"][:, W.A]
    assert abs(inplace.mean() - 0.1) < 0.01
    # operands never cross dtypes
    same = (r["buf"][:, W.A] >= 32) == (r["dtype"] == W.BF16)
    assert same.all()
    assert s.bursts.sum() == len(r) and s.bursts.max() <= 64 and s.bursts.min() >= 1
    # log-uniform sizes: median near 256 * 16 = 4096
    assert 3000 < np.median(r["size"]) < 5500


def test_pr1_stream_shape():
    s = W.make_pr1()
    assert len(s) == 1000 and set(np.unique(s.recs["op"])) == {W.OP_ADD, W.OP_MUL, W.OP_RELU}
    v = s.buffers[0].host_values()
    assert v.dtype == np.float32 and v.min() >= -1 and v.max() < 1


def test_rows_decode_mixed_shapes():
    s = W.make_rows(n_desc=500, n_pool=4, arena_bytes=8 << 20)
    assert set(np.unique(s.recs["size"])) <= {1, 2, 4, 8, 16, 32, 64}
    assert set(np.unique(s.recs["dim"][:, 0])) <= set(W.ROW_HIDDEN)
    d = W.make_decode(steps=5, layers=2, capacity=256, l_min=16, n_triples=4)
    assert len(d) == 5 * 2 * 3
    assert (d.recs["lens"][:, 0] >= 16).all() and (d.recs["lens"].max() <= 256)
    m = W.make_mixed(tokens=2, layers=2, capacity=128, l0_range=(8, 64))
    assert len(m) == 2 * (1 + 11 * 2)
