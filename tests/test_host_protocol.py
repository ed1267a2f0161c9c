"""Host-side protocol tests that run without a GPU.

The C-ABI library must load and export every entry point of gpuos.h.  The
ring producer, hazard annotation, slot recycling, error statuses and table
flips are exercised with a loopback context: a host thread plays the
consumer, completes committed descriptors in a random order allowed by
their dependency annotations, and computes nothing.  Descriptors point at
host addresses that are never dereferenced.
"""
import re

import numpy as np
import pytest

import workloads as W
from persistent_micro_dispatch_amd import gpuos as G
from workloads.gpu import to_descs

HEADER = "include/gpuos.h"


def test_library_exports_every_declared_entry_point():
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    text = open(os.path.join(root, HEADER)).read()
    declared = set(re.findall(r"^(?:int|uint64_t)\s+(gpuos_\w+)\s*\(", text, re.M))
    assert declared == set(G.EXPORTS)
    L = G.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert G.gpuos_abi_version() == 5


def _ranges(recs):
    """Independent byte ranges per record: (buf, lo, hi, write)."""
    out = []
    for r in recs:
        es = W.DTYPE_BYTES[int(r["dtype"])]
        n = int(r["size"])
        ops = []
        if r["op"] in (W.OP_ADD, W.OP_MUL):
            ops = [(W.A, False), (W.B, False), (W.OUT, True)]
        elif r["op"] in (W.OP_RELU, W.OP_GELU):
            ops = [(W.A, False), (W.OUT, True)]
        rr = []
        for role, w in ops:
            b = int(r["buf"][role])
            lo = int(r["off"][role])
            rr.append((b, lo, lo + n * es, w))
        out.append(rr)
    return out


def _check_order(recs, order, first_seq):
    """Every conflicting earlier record completed before a later one."""
    n = len(recs)
    pos = np.empty(n, np.int64)
    idx = np.asarray(order, np.int64) - first_seq
    assert sorted(idx.tolist()) == list(range(n)), "each descriptor completes exactly once"
    pos[idx] = np.arange(n)
    rng = _ranges(recs)
    violations = 0
    for j in range(n):
        for i in range(max(0, j - 400), j):
            conflict = False
            for (b1, l1, h1, w1) in rng[i]:
                for (b2, l2, h2, w2) in rng[j]:
                    if b1 == b2 and l1 < h2 and l2 < h1 and (w1 or w2):
                        conflict = True
            if conflict and pos[i] > pos[j]:
                violations += 1
    return violations


def _fake_ptrs(nbuf):
    # distinct, widely spaced fake device addresses (never dereferenced)
    return [0x10_0000_0000 + i * 0x100_0000 for i in range(nbuf)]


def _loopback(ring=4096):
    return G.gpuos_init(flags=G.GPUOS_INIT_LOOPBACK, ring_entries=ring)


def _run(ctx, descs, bursts=None, flags=G.GPUOS_SUBMIT_BLOCK):
    first = None
    sl = [slice(0, len(descs))] if bursts is None else \
        [slice(int(a), int(b)) for a, b in zip(np.r_[0, np.cumsum(bursts)[:-1]], np.cumsum(bursts))]
    for s in sl:
        rc, f = G.gpuos_submit(ctx, descs[s], flags)
        assert rc == 0, G.ERR_NAMES.get(rc)
        first = f if first is None else first
    rc, es, st = G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 20_000_000_000)
    assert rc == 0, (rc, es, st)
    return first


@pytest.mark.parametrize("ring", [8, 64, 4096])
def test_loopback_respects_hazards_pr1(ring):
    s = W.make_pr1()
    descs = to_descs(s.recs, _fake_ptrs(len(s.buffers)))
    ctx = _loopback(ring)
    try:
        bursts = np.full(len(descs) // 8, 8) if ring <= 64 else None
        first = _run(ctx, descs, bursts)
        order = G.gpuos_loopback_order(ctx)
    finally:
        assert G.gpuos_shutdown(ctx) == 0
    assert _check_order(s.recs, order, first) == 0
    # concurrency actually happened: the order is not the submission order
    if ring >= 64:
        assert not np.array_equal(order, np.arange(first, first + len(descs)))


def test_loopback_respects_hazards_elementwise_partial_overlaps():
    s = W.make_elementwise(n_desc=3000)
    r = s.recs.copy()
    # add partial overlaps: random byte offsets inside the operand buffers
    rng = np.random.default_rng(3)
    for role in (W.A, W.B, W.OUT):
        r["off"][:, role] = (rng.integers(0, 4096, len(r)) * 4) * (rng.random(len(r)) < 0.5)
    r["size"] = np.minimum(r["size"], 65536 - 4096 * 4)
    descs = to_descs(r, _fake_ptrs(len(s.buffers)))
    ctx = _loopback()
    try:
        first = _run(ctx, descs, s.bursts)
        order = G.gpuos_loopback_order(ctx)
        st = G.gpuos_stats_get(ctx)
    finally:
        G.gpuos_shutdown(ctx)
    assert st["completed"] == len(descs) and st["submitted"] == len(descs)
    assert _check_order(r, order, first) == 0


def test_loopback_respects_hazards_in_a_large_arena():
    """Thousands of small reads and writes scattered over one buffer: the
    tracker splits the buffer's interval list into several clusters and an
    access may straddle two; the order must still respect every conflict."""
    rng = np.random.default_rng(11)
    n = 3000
    r = np.zeros(n, W.REC_DTYPE)
    r["buf"] = -1
    r["dtype"] = r["out_dtype"] = W.F32
    r["op"] = np.where(rng.random(n) < 0.5, W.OP_ADD, W.OP_RELU)
    r["size"] = rng.integers(64, 1024, n)
    cap = 1 << 20
    for role in (W.A, W.B, W.OUT):
        r["buf"][:, role] = 0
        r["off"][:, role] = rng.integers(0, (cap - 1024) // 4, n) * 16
    descs = to_descs(r, _fake_ptrs(1))
    ctx = _loopback()
    try:
        first = _run(ctx, descs, np.full(n // 50, 50))
        order = G.gpuos_loopback_order(ctx)
    finally:
        G.gpuos_shutdown(ctx)
    assert _check_order(r, order, first) == 0


@pytest.mark.parametrize("n_read", [25, 40, 62, 70])
def test_many_readers_give_explicit_dependencies(n_read):
    """A write after n reads of its output waits on exactly those n
    descriptors: explicit dependencies up to the 62 a descriptor carries (six
    in the body, 56 in the side words), beyond that a range from the oldest
    reader."""
    r = np.zeros(n_read + 1, W.REC_DTYPE)
    r["buf"] = -1
    r["dtype"] = r["out_dtype"] = W.F32
    r["op"] = W.OP_RELU
    r["size"] = 256
    r["buf"][:n_read, W.A] = 0                          # all read buffer 0
    r["buf"][:n_read, W.OUT] = np.arange(1, n_read + 1)  # each writes its own buffer
    r["buf"][n_read, W.A] = n_read + 1                  # then buffer 0 is overwritten
    r["buf"][n_read, W.OUT] = 0
    descs = to_descs(r, _fake_ptrs(n_read + 2))
    ctx = _loopback()
    try:
        first = _run(ctx, descs)
        order = G.gpuos_loopback_order(ctx)
        st = G.gpuos_stats_get(ctx)
    finally:
        G.gpuos_shutdown(ctx)
    if n_read <= 62:
        assert st["deps_range"] == 0 and st["deps_explicit"] == n_read
    else:
        assert st["deps_range"] == 1
    assert _check_order(r, order, first) == 0
    assert order[-1] == first + n_read or list(order).index(first + n_read) == len(order) - 1


def test_serial_flag_gives_submission_order():
    s = W.make_elementwise(n_desc=500)
    descs = to_descs(s.recs, _fake_ptrs(len(s.buffers)))
    ctx = _loopback()
    try:
        first = _run(ctx, descs, flags=G.GPUOS_SUBMIT_BLOCK | G.GPUOS_SUBMIT_SERIAL)
        order = G.gpuos_loopback_order(ctx)
    finally:
        G.gpuos_shutdown(ctx)
    assert np.array_equal(order, np.arange(first, first + 500, dtype=np.uint64))


def test_full_ring_returns_e_full_then_block_waits():
    ctx = _loopback(8)
    try:
        d = G.new_descs(9)
        rc, _ = G.gpuos_submit(ctx, d, 0)          # 9 > ring entries: invalid
        assert rc == G.GPUOS_E_INVAL
        rc, f0 = G.gpuos_submit(ctx, d[:8], G.GPUOS_SUBMIT_BLOCK)
        assert rc == 0
        # the loopback consumer frees slots asynchronously; BLOCK waits for them
        rc, f1 = G.gpuos_submit(ctx, d[:8], G.GPUOS_SUBMIT_BLOCK)
        assert rc == 0 and f1 == f0 + 8
        assert G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 5_000_000_000)[0] == 0
        st = G.gpuos_stats_get(ctx)
        assert st["completed"] == 16
    finally:
        G.gpuos_shutdown(ctx)


def test_full_without_block_is_reported():
    # a loopback consumer that cannot run: NOPs whose ring is refilled faster
    # than 1 us is not guaranteed, so check the E_FULL path deterministically
    # by asking for more slots than remain before any completion is observed
    ctx = _loopback(8)
    try:
        d = G.new_descs(8)
        rc, _ = G.gpuos_submit(ctx, d, 0)
        assert rc == 0
        rc2, _ = G.gpuos_submit(ctx, d, 0)
        assert rc2 in (0, G.GPUOS_E_FULL)
        if rc2 == G.GPUOS_E_FULL:
            assert G.gpuos_stats_get(ctx)["full_rejections"] == 1
        assert G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 5_000_000_000)[0] == 0
    finally:
        G.gpuos_shutdown(ctx)


def test_bad_op_id_is_reported_by_sync():
    ctx = _loopback()
    try:
        d = G.new_descs(3)
        d["op_id"] = [G.GPUOS_OP_NOP, 200, G.GPUOS_OP_NOP]   # 200 is unbound
        rc, f = G.gpuos_submit(ctx, d, G.GPUOS_SUBMIT_BLOCK)
        assert rc == 0
        rc, es, st = G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 5_000_000_000)
        assert rc == G.GPUOS_E_DEVICE and es == f + 1 and st == G.GPUOS_ST_BAD_OP
        assert G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 5_000_000_000)[0] == 0  # reported once
    finally:
        G.gpuos_shutdown(ctx)


def test_descriptor_unit_limit_follows_the_unit_queue():
    """A descriptor may take at most half the unit queue: with 2^12 queue
    positions, an fp32 add of 2048 units of 2048 values and a copy of 2048
    units of 32 KiB are accepted, one element more of either is refused
    before submission (the pointers are never used)."""
    ctx = G.gpuos_init(flags=G.GPUOS_INIT_LOOPBACK, ring_entries=64, unit_queue_log2=12)
    try:
        d = G.new_descs(1)
        d["op_id"] = G.GPUOS_OP_ADD
        d["flags"] = G.flags(G.GPUOS_F32)
        d["input_a"], d["input_b"], d["output"] = 1 << 40, 2 << 40, 3 << 40
        d["size"] = 2048 * 2048            # 16 MiB per operand: units of 8 KiB
        assert G.gpuos_submit(ctx, d, G.GPUOS_SUBMIT_BLOCK)[0] == 0
        d["size"] = 2048 * 2048 + 1
        assert G.gpuos_submit(ctx, d, 0)[0] == G.GPUOS_E_INVAL
        c = G.new_descs(1)
        c["op_id"] = G.GPUOS_OP_COPY
        c["input_a"], c["output"] = 1 << 40, 3 << 40
        c["size"] = 2048 * 32768            # units of 32 KiB
        assert G.gpuos_submit(ctx, c, G.GPUOS_SUBMIT_BLOCK)[0] == 0
        c["size"] = 2048 * 32768 + 1
        assert G.gpuos_submit(ctx, c, 0)[0] == G.GPUOS_E_INVAL
        assert G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 5_000_000_000)[0] == 0
        assert G.gpuos_stats_get(ctx)["submitted"] == 2
    finally:
        G.gpuos_shutdown(ctx)


def test_invalid_shapes_rejected_before_submission():
    ctx = _loopback()
    try:
        d = G.new_descs(1)
        d["op_id"] = G.GPUOS_OP_ADD
        d["size"] = 100          # null pointers with n > 0
        assert G.gpuos_submit(ctx, d, 0)[0] == G.GPUOS_E_INVAL
        d = G.new_descs(1)
        d["op_id"] = G.GPUOS_OP_SDPA
        d["flags"] = G.flags(G.GPUOS_BF16, G.GPUOS_F32)
        d["size"] = 9            # B > 8
        d["dim"] = (32, 128, 4096, 0)
        d["input_a"] = d["output"] = 1 << 40
        d["aux"][0, :2] = 1 << 41
        G.set_lens(d, [5] * 8)
        assert G.gpuos_submit(ctx, d, 0)[0] == G.GPUOS_E_INVAL
        d["size"] = 2
        d["dim"] = (32, 96, 4096, 0)   # head_dim 96 not supported
        assert G.gpuos_submit(ctx, d, 0)[0] == G.GPUOS_E_INVAL
        d["dim"] = (32, 128, 4096, 0)
        assert G.gpuos_submit(ctx, d, 0)[0] == 0
        G.set_lens(d, [5000, 5])        # L > C
        assert G.gpuos_submit(ctx, d, 0)[0] == G.GPUOS_E_INVAL
        d["dim"] = (32, 128, 65535, 0)
        G.set_lens(d, [65535, 5])       # the longest row a descriptor can carry: 64 splits of 1024 keys
        assert G.gpuos_submit(ctx, d, 0)[0] == 0
        d["dim"] = (32, 128, 4096, 0)
        assert G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 5_000_000_000)[0] == 0
        assert G.gpuos_stats_get(ctx)["submitted"] == 2
    finally:
        G.gpuos_shutdown(ctx)


def test_register_op_flips_table_for_later_descriptors():
    ctx = _loopback()
    try:
        assert G.gpuos_register_op(ctx, 300, G.GPUOS_OP_ADD) == G.GPUOS_E_NOOP
        assert G.gpuos_register_op(ctx, 70, 99) == G.GPUOS_E_NOOP
        d = G.new_descs(1)
        d["op_id"] = 70
        rc, f = G.gpuos_submit(ctx, d, G.GPUOS_SUBMIT_BLOCK)
        assert rc == 0
        rc, es, st = G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 5_000_000_000)
        assert rc == G.GPUOS_E_DEVICE and st == G.GPUOS_ST_BAD_OP   # unbound before
        assert G.gpuos_register_op(ctx, 70, G.GPUOS_OP_NOP) == 0
        rc, f = G.gpuos_submit(ctx, d, G.GPUOS_SUBMIT_BLOCK)
        assert rc == 0 and G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 5_000_000_000)[0] == 0
        # several flips in a row reuse both slots
        for k in range(5):
            assert G.gpuos_register_op(ctx, 71, G.GPUOS_OP_NOP if k % 2 == 0 else G.GPUOS_KIND_EMPTY) == 0
        d["op_id"] = 71   # last binding: NOP (k = 4)
        rc, f = G.gpuos_submit(ctx, d, G.GPUOS_SUBMIT_BLOCK)
        assert G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 5_000_000_000)[0] == 0
        # unbinding makes it fail again
        assert G.gpuos_register_op(ctx, 71, G.GPUOS_KIND_EMPTY) == 0
        G.gpuos_submit(ctx, d, G.GPUOS_SUBMIT_BLOCK)
        assert G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 5_000_000_000)[0] == G.GPUOS_E_DEVICE
    finally:
        G.gpuos_shutdown(ctx)


def test_bad_init_params():
    with pytest.raises(G.GpuosError):
        G.gpuos_init(flags=G.GPUOS_INIT_LOOPBACK, ring_entries=100)
    with pytest.raises(G.GpuosError):
        G.gpuos_init(flags=G.GPUOS_INIT_LOOPBACK, waves_per_wg=5)


def test_hbm_probe_rejects_bad_arguments():
    # checked before any HIP call
    lib = G.lib()
    g = G.ctypes.c_double(0)
    for src, dst, n, mode, reps in [(0, 64, 4096, 0, 1), (64, 64, 4100, 1, 1), (64, 64, 1024, 0, 1),
                                    (64, 64, (1 << 30) + 16, 1, 1), (64, 64, 4096, 2, 1), (64, 64, 4096, 1, 0)]:
        assert lib.gpuos_hbm_probe(src, dst, n, mode, reps, None, G.ctypes.byref(g)) == G.GPUOS_E_INVAL


def test_loopback_respects_hazards_with_merging_ranges():
    """Random byte ranges in one 1 MiB region, from a few bytes to many KiB,
    so that clusters of the tracker are created, merged, split and recycled
    all the time, with the same start addresses recurring (the lookup cache
    keyed by start address must never return a retired or shrunk cluster)."""
    rng = np.random.default_rng(11)
    n = 4000
    base = 0x20_0000_0000
    starts = rng.integers(0, 1 << 20, 64) // 16 * 16  # recurring start addresses
    d = G.new_descs(n)
    d["op_id"] = G.GPUOS_OP_COPY
    ranges = []
    for i in range(n):
        a = int(starts[rng.integers(64)]) if rng.random() < 0.5 else int(rng.integers(0, 1 << 20))
        o = int(starts[rng.integers(64)]) if rng.random() < 0.5 else int(rng.integers(0, 1 << 20))
        size = int(min(rng.choice([16, 256, 4096, 65536]) * rng.random() + 1, (1 << 20) - max(a, o)))
        d["input_a"][i], d["output"][i], d["size"][i] = base + a, base + o, size
        if a < o + size and o < a + size:  # a copy's input and output must coincide or not overlap
            d["output"][i] = base + a
            o = a
        ranges.append(((a, a + size, False), (o, o + size, True)))
    ctx = _loopback()
    try:
        first = _run(ctx, d, np.full(n // 16, 16))
        order = G.gpuos_loopback_order(ctx)
    finally:
        assert G.gpuos_shutdown(ctx) == 0
    pos = np.empty(n, np.int64)
    idx = np.asarray(order, np.int64) - first
    assert sorted(idx.tolist()) == list(range(n))
    pos[idx] = np.arange(n)
    bad = 0
    for j in range(n):
        for i in range(max(0, j - 300), j):
            if pos[i] < pos[j]:
                continue
            if any(l1 < h2 and l2 < h1 and (w1 or w2) for (l1, h1, w1) in ranges[i] for (l2, h2, w2) in ranges[j]):
                bad += 1
    assert bad == 0


def test_register_expr_validates_programs():
    X, P = W.xins, W.program
    ctx = _loopback()
    try:
        good = P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_ADD, 0, 1, 2)])
        assert G.gpuos_register_expr(ctx, 100, good) == 0
        assert G.gpuos_register_expr(ctx, 256, good) == G.GPUOS_E_NOOP
        assert G.gpuos_register_op(ctx, 100, G.GPUOS_OP_EXPR) == G.GPUOS_E_INVAL
        for bad in [P([X(0, 0)]), P([X(W.X_RELU + 1, 0)]), P([X(W.X_LDA, 4)]), P([X(W.X_MOV, 0, 7)]),
                    P([X(W.X_CONST, 0, 0, 0, 1)], [1.0]), good[:-1], np.array([0], np.uint32),
                    P([X(W.X_LDA, 0)] * 33), P([X(W.X_LDA, 0)], [1.0] * 17),
                    P([X(W.X_LDA, 0) | (1 << 28)])]:
            assert G.gpuos_register_expr(ctx, 100, bad) == G.GPUOS_E_INVAL
        # a program that reads b needs b; one that does not may omit it
        d = G.new_descs(2)
        d["op_id"] = 100
        d["size"] = 64
        d["input_a"], d["output"] = 0x1000, 0x2000
        assert G.gpuos_submit(ctx, d[:1], G.GPUOS_SUBMIT_BLOCK)[0] == G.GPUOS_E_INVAL
        assert G.gpuos_register_expr(ctx, 101, P([X(W.X_LDA, 1), X(W.X_EXP, 0, 1)])) == 0
        d["op_id"] = 101
        assert G.gpuos_submit(ctx, d, G.GPUOS_SUBMIT_BLOCK)[0] == 0
        assert G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 10_000_000_000)[0] == 0
    finally:
        assert G.gpuos_shutdown(ctx) == 0


def test_loopback_orders_expr_ops_like_binary_ops():
    """EXPR descriptors read a (and b) and write out: the tracker orders
    them against the element-wise ops on the same tensors."""
    s = W.make_elementwise(n_desc=2000)
    r = s.recs.copy()
    sel = np.arange(len(r)) % 3 == 0
    r["op"][sel] = W.OP_EXPR
    r["dim"][sel, 3] = 120
    ctx = _loopback()
    try:
        X, P = W.xins, W.program
        assert G.gpuos_register_expr(ctx, 120, P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_SUB, 0, 1, 2)])) == 0
        ptrs = _fake_ptrs(len(s.buffers))
        descs = to_descs(r, ptrs)
        # unary ops have no b: give EXPR descriptors their a as b (the program reads b)
        m = sel & (descs["input_b"] == 0)
        descs["input_b"][m] = descs["input_a"][m]
        first = _run(ctx, descs, s.bursts)
        order = G.gpuos_loopback_order(ctx)
    finally:
        G.gpuos_shutdown(ctx)
    r2 = r.copy()
    r2["op"][sel] = W.OP_ADD  # same operand roles for the order check
    r2["buf"][m, W.B] = r2["buf"][m, W.A]
    assert _check_order(r2, order, first) == 0


def test_latency_bench_submits_and_waits_one_at_a_time():
    s = W.make_elementwise(n_desc=50)
    descs = to_descs(s.recs, _fake_ptrs(len(s.buffers)))
    ctx = _loopback()
    try:
        lat = G.gpuos_latency_bench(ctx, descs)
        order = G.gpuos_loopback_order(ctx)
        st = G.gpuos_stats_get(ctx)
    finally:
        G.gpuos_shutdown(ctx)
    assert lat.shape == (50,) and (lat > 0).all()
    assert len(order) == 50 and np.array_equal(np.sort(order), order)  # one at a time: in order
    assert st["full_rejections"] == 0


def test_six_dependencies_leave_no_stale_side_words():
    """A descriptor with more than six dependencies keeps the extra ones in
    side words of its stage index; a later descriptor at the same stage index
    with exactly six (dep_delta[5] set, so the side words are read) must
    carry none of them: stale words would make it wait on unrelated older
    descriptors."""
    def relu(a, out):
        r = np.zeros(1, W.REC_DTYPE)
        r["buf"] = -1
        r["dtype"] = r["out_dtype"] = W.F32
        r["op"] = W.OP_RELU
        r["size"] = 256
        r["buf"][0, W.A], r["buf"][0, W.OUT] = a, out
        return r

    def nop():
        r = np.zeros(1, W.REC_DTYPE)
        r["buf"] = -1
        return r
    ptrs = _fake_ptrs(32)
    # call 1: ten readers of buffer 0, then a writer of buffer 0 (ten deps) at index 10
    c1 = np.concatenate([relu(0, 1 + i) for i in range(10)] + [relu(30, 0)])
    # call 2: four NOPs, six readers of buffer 0, then a writer (six deps) at index 10
    c2 = np.concatenate([nop() for _ in range(4)] + [relu(0, 11 + i) for i in range(6)] + [relu(31, 0)])
    ctx = _loopback()
    try:
        rc, f1 = G.gpuos_submit(ctx, to_descs(c1, ptrs), G.GPUOS_SUBMIT_BLOCK)
        assert rc == 0
        rc, d1, x1 = G.gpuos_ring_peek(ctx, f1 + 10)
        assert rc == 0
        rc, f2 = G.gpuos_submit(ctx, to_descs(c2, ptrs), G.GPUOS_SUBMIT_BLOCK)
        assert rc == 0
        rc, d2, x2 = G.gpuos_ring_peek(ctx, f2 + 10)
        assert rc == 0
        assert G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 20_000_000_000)[0] == 0
        assert G.gpuos_ring_peek(ctx, f2 + 11)[0] == G.GPUOS_E_STATE  # not submitted
    finally:
        G.gpuos_shutdown(ctx)
    deps1 = sorted(int(v) for v in list(d1["dep_delta"]) + list(x1) if v)
    assert deps1 == list(range(1, 11))          # the ten readers, by delta
    assert sorted(int(v) for v in d2["dep_delta"]) == list(range(1, 7))
    assert not x2.any(), f"stale side words {x2[:8]}"


def test_static_eager_submit_rejects_oversized_split_partials_before_launching():
    """A vector-matrix product whose split partials exceed the static array
    (here 1024 row splits x 65536 columns x 4 B = 256 MiB) is refused with
    E_INVAL before anything is launched (the pointers are never used)."""
    d = G.new_descs(2)
    d["op_id"] = G.GPUOS_OP_GEMV
    d["flags"] = G.flags(G.GPUOS_BF16)
    d["input_a"], d["input_b"], d["output"] = 0x10_0000_0000, 0x20_0000_0000, 0x30_0000_0000
    d["dim"][:, 0], d["dim"][:, 1] = 1024, 64
    d["dim"][1, 0], d["dim"][1, 1] = 131072, 65536
    assert G.gpuos_eager_scratch_bytes(d[1:]) > G.GPUOS_EAGER_STATIC_SCRATCH_BYTES
    assert G.gpuos_eager_submit_static(d, 0) == G.GPUOS_E_INVAL
    bad = G.new_descs(1)
    bad["op_id"] = G.GPUOS_OP_EXPR  # needs a table; the eager path has none
    assert G.gpuos_eager_submit_static(bad, 0) == G.GPUOS_E_INVAL


def _precise_ranges(r):
    """Exact byte ranges a record reads and writes, from the op definitions
    (per-head KV-cache rows, per-row attention keys), independent of the
    library's declared ranges: [(buf, lo, hi, write)]."""
    op = int(r["op"])
    es = W.DTYPE_BYTES[int(r["dtype"])]
    n = int(r["size"])
    d = [int(v) for v in r["dim"]]
    buf, off = r["buf"], r["off"]

    def rng(role, nbytes, rel=0):
        b = int(buf[role])
        return (b, int(off[role]) + rel, int(off[role]) + rel + nbytes)
    reads = []
    if op in (W.OP_ADD, W.OP_MUL):
        reads = [rng(W.A, n * es), rng(W.B, n * es)]
    elif op in (W.OP_RELU, W.OP_GELU):
        reads = [rng(W.A, n * es)]
    elif op in (W.OP_SUM, W.OP_MAX, W.OP_MIN, W.OP_SOFTMAX):
        reads = [rng(W.A, n * d[0] * es)]
    elif op == W.OP_LAYERNORM:
        reads = [rng(W.A, n * d[0] * es), rng(W.AUX0, d[0] * es), rng(W.AUX1, d[0] * es)]
    elif op == W.OP_ROPE:
        reads = [(b, o, o + k) for (b, o, k) in W.output_ranges(r)]
    elif op == W.OP_KV_APPEND:
        reads = [rng(W.A, n * d[0] * d[1] * es), rng(W.B, n * d[0] * d[1] * es)]
    elif op == W.OP_SDPA:
        H, D, C = d[0], d[1], d[2]
        hkv = d[3] or H
        reads = [rng(W.A, n * H * D * es)]
        for bb in range(n):
            L = int(r["lens"][bb])
            for h in range(hkv):
                rel = (bb * hkv + h) * C * D * es
                reads += [rng(W.AUX0, L * D * es, rel), rng(W.AUX1, L * D * es, rel)]
    elif op == W.OP_GEMV:
        reads = [rng(W.A, d[0] * es), rng(W.B, d[0] * d[1] * es)]
    elif op == W.OP_COPY:
        reads = [rng(W.A, n)]
    writes = [(b, o, o + k) for (b, o, k) in W.output_ranges(r)]
    return [(b, lo, hi, False) for (b, lo, hi) in reads] + [(b, lo, hi, True) for (b, lo, hi) in writes]


def _check_order_precise(recs, order, first_seq, window=600):
    """Every pair of records whose exact ranges conflict completed in order."""
    n = len(recs)
    idx = np.asarray(order, np.int64) - first_seq
    assert sorted(idx.tolist()) == list(range(n)), "each descriptor completes exactly once"
    pos = np.empty(n, np.int64)
    pos[idx] = np.arange(n)
    R = [np.array(_precise_ranges(r), np.int64).reshape(-1, 4) for r in recs]
    owner = [np.full(len(x), i) for i, x in enumerate(R)]
    violations = 0
    for j in range(1, n):
        lo_i = max(0, j - window)
        A = np.concatenate(R[lo_i:j])
        own = np.concatenate(owner[lo_i:j])
        Bj = R[j]
        if not len(A) or not len(Bj):
            continue
        c = ((A[:, None, 0] == Bj[None, :, 0]) & (A[:, None, 1] < Bj[None, :, 2]) & (Bj[None, :, 1] < A[:, None, 2])
             & ((A[:, None, 3] | Bj[None, :, 3]) != 0)).any(axis=1)
        earlier = np.unique(own[c])
        violations += int((pos[earlier] > pos[j]).sum())
    return violations


@pytest.mark.parametrize("kind", ["decode", "decode_gqa", "mixed"])
def test_loopback_respects_hazards_attention_streams(kind):
    """Decode and mixed streams: the library declares the KV caches whole;
    every pair of descriptors whose exact accesses (per-head cache rows,
    per-row keys) conflict must still complete in submission order."""
    if kind == "mixed":
        s = W.make_mixed(tokens=4, layers=3, capacity=64, l0_range=(8, 40), n_tok_pool=2)
    else:
        s = W.make_decode(steps=30, layers=3, heads=8, kv_heads=2 if kind == "decode_gqa" else 0,
                          capacity=64, l_min=8, n_triples=4, n_out=8)
    descs = to_descs(s.recs, _fake_ptrs(len(s.buffers)))
    ctx = _loopback(ring=64)
    try:
        first = _run(ctx, descs, np.full(len(descs) // 16 + 1, 16)[: (len(descs) + 15) // 16])
        order = G.gpuos_loopback_order(ctx)
    finally:
        G.gpuos_shutdown(ctx)
    assert _check_order_precise(s.recs, order, first) == 0
    if kind != "mixed":  # the mixed pipeline is one dependency chain per token
        assert not np.array_equal(order, np.arange(first, first + len(descs)))


def test_paged_cache_descriptors_validated_and_ordered():
    """Paged caches: the page size must be a power of two from 64 to 1024,
    the pool and the table must be given, rows may not pass MP pages; an
    append and the attentions around it order through the whole-pool ranges
    (loopback consumer)."""
    ctx = _loopback()
    try:
        B, H, D, PS, MP, NP = 2, 8, 128, 64, 8, 20
        base = 1 << 40
        app = G.new_descs(1)
        app["op_id"] = G.GPUOS_OP_KV_APPEND
        app["flags"] = G.flags(G.GPUOS_BF16) | G.GPUOS_F_KV_PAGED
        app["size"] = B | (NP << 32)
        app["dim"] = (H, D, PS, 0)
        app["input_a"], app["input_b"] = base, base + (1 << 20)
        app["aux"][0] = (base + (1 << 30), base + (2 << 30), base + (3 << 30))
        app["param"][0, 5] = MP
        G.set_lens(app, [300, 512])
        att = G.new_descs(1)
        att["op_id"] = G.GPUOS_OP_SDPA
        att["flags"] = G.flags(G.GPUOS_BF16, G.GPUOS_F32) | G.GPUOS_F_KV_PAGED
        att["size"] = B | (NP << 32)
        att["dim"] = (H, D, PS, 0)
        att["input_a"], att["output"], att["input_b"] = base + (4 << 20), base + (5 << 20), base + (3 << 30)
        att["aux"][0, :2] = (base + (1 << 30), base + (2 << 30))
        att["param"][0, 5] = MP
        G.set_lens(att, [300, 512])
        for d in (app, att):
            for bad in ("ps", "np", "table", "len"):
                x = d.copy()
                if bad == "ps":
                    x["dim"][0, 2] = 96                  # not a power of two
                elif bad == "np":
                    x["size"] = B                         # no pool pages
                elif bad == "table":
                    if d is app:
                        x["aux"][0, 2] = 0
                    else:
                        x["input_b"] = 0
                else:
                    G.set_lens(x, [MP * PS + 1, 5])       # past the table row
                assert G.gpuos_submit(ctx, x, 0)[0] == G.GPUOS_E_INVAL, (int(d["op_id"][0]), bad)
        x = att.copy()
        x["param"][0, 5] = 1024
        G.set_lens(x, [65535, 5])                          # attention units span pages: up to 64 splits of 1024
        assert G.gpuos_submit(ctx, x, 0)[0] == 0
        assert G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 5_000_000_000)[0] == 0
        # append, attention, append: each waits for the one before
        rc, first = G.gpuos_submit(ctx, np.concatenate([app, att, app]), G.GPUOS_SUBMIT_BLOCK)
        assert rc == 0
        assert G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 5_000_000_000)[0] == 0
        order = list(G.gpuos_loopback_order(ctx))
        assert order.index(first) < order.index(first + 1) < order.index(first + 2)
        for i in (1, 2):  # the attention waits on the append, the second append on the attention
            rc, dd, _ = G.gpuos_ring_peek(ctx, first + i)
            assert rc == 0 and 1 in list(dd["dep_delta"])
    finally:
        G.gpuos_shutdown(ctx)
