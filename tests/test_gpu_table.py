"""GPU tests of the operator table and the error paths, through the C ABI.

- Bounds checking (GPUOS digest page, section 3 Q2 "Dynamic Operator
  Table"): descriptors with an unbound or out-of-range op id complete as
  no-ops with status BAD_OP; gpuos_sync reports each one's sequence number
  in order; the descriptors around them still run.
- Live rebinding: gpuos_register_op and gpuos_register_expr flip the table
  many times while a stream is in flight; every descriptor must run the
  operator bound when it was submitted (checked against the oracle, which
  runs each record under that binding).
- Exactly-once execution: with the unit trace on, every unit of every
  descriptor appears once, and the device's unit counter equals the trace.
- Shutdown with work in flight finishes that work first.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_harness import say
from parity import bits_equal
from persistent_micro_dispatch_amd import gpuos as G
from workloads.gpu import DevicePool, to_descs

pytestmark = pytest.mark.gpu
SYNC_NS = 60_000_000_000


def _oracle_final(arrays, recs):
    p = oracle.Pool([np.array(a, copy=True) for a in arrays])
    p.run(recs)
    return p.arrays


def _assert_pool_equal(pool, ref, buffers):
    for i, b in enumerate(buffers):
        eq = bits_equal(pool.download(i).copy(), ref[i].copy(), b.dtype)
        assert eq.all(), f"buffer {i}: {int((~eq).sum())} mismatches"


def _drain_errors(ctx, limit=1000):
    """Call gpuos_sync until it returns OK; the (seq, status) pairs it reports."""
    errs = []
    for _ in range(limit):
        rc, es, st = G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, SYNC_NS)
        if rc == G.GPUOS_OK:
            return errs
        assert rc == G.GPUOS_E_DEVICE, G.ERR_NAMES.get(rc)
        errs.append((es, st))
    raise AssertionError("too many errors")


@pytest.mark.parametrize("ring", [64, 4096])
def test_bad_op_ids_complete_as_noops_with_status(ring):
    s = W.make_pr1(n_desc=400)
    arrays = [b.host_bytes() for b in s.buffers]
    pool = DevicePool(arrays)
    descs = to_descs(s.recs, pool.ptrs)
    bad = {37: 200, 38: 300, 150: G.GPUOS_OP_USER + 5, 151: 0xFFFF, 399: 255}  # index -> op id
    ref_recs = s.recs.copy()
    for i, op in bad.items():
        descs["op_id"][i] = op
        ref_recs["op"][i] = W.OP_NOP
    say(f"bad op ids at {sorted(bad)}, ring {ring}")
    ctx = G.gpuos_init(ring_entries=ring)
    try:
        first = None
        for k in range(0, len(descs), 25):
            rc, f = G.gpuos_submit(ctx, descs[k:k + 25], G.GPUOS_SUBMIT_BLOCK)
            assert rc == 0, G.ERR_NAMES.get(rc)
            first = f if first is None else first
        errs = _drain_errors(ctx)
    finally:
        assert G.gpuos_shutdown(ctx) == 0
    assert errs == [(first + i, G.GPUOS_ST_BAD_OP) for i in sorted(bad)]
    _assert_pool_equal(pool, _oracle_final(arrays, ref_recs), s.buffers)


def test_register_op_rebinds_a_user_id_while_the_stream_runs():
    s = W.make_pr1(n_desc=720)
    arrays = [b.host_bytes() for b in s.buffers]
    pool = DevicePool(arrays)
    descs = to_descs(s.recs, pool.ptrs)
    ref_recs = s.recs.copy()
    rng = np.random.default_rng(11)
    uid = G.GPUOS_OP_USER + 6
    cycle = [G.GPUOS_OP_ADD, G.GPUOS_OP_MUL, G.GPUOS_KIND_EMPTY, G.GPUOS_OP_MUL, G.GPUOS_OP_ADD]
    ctx = G.gpuos_init(ring_entries=64)
    expect_bad = []
    try:
        first = None
        for blk in range(12):
            kind = cycle[blk % len(cycle)]
            assert G.gpuos_register_op(ctx, uid, kind) == 0
            lo, hi = 60 * blk, 60 * blk + 60
            binary = [i for i in range(lo, hi) if int(s.recs["op"][i]) in (W.OP_ADD, W.OP_MUL)]
            sel = [i for i in binary if rng.random() < 0.6]
            for i in sel:
                descs["op_id"][i] = uid
                ref_recs["op"][i] = W.OP_NOP if kind == G.GPUOS_KIND_EMPTY else kind
                if kind == G.GPUOS_KIND_EMPTY:
                    expect_bad.append(i)
            for k in range(lo, hi, 20):   # the stream keeps the ring busy across flips
                rc, f = G.gpuos_submit(ctx, descs[k:k + 20], G.GPUOS_SUBMIT_BLOCK)
                assert rc == 0, G.ERR_NAMES.get(rc)
                first = f if first is None else first
        say(f"12 rebinds of op {uid}; {len(expect_bad)} descriptors submitted while it was unbound")
        errs = _drain_errors(ctx)
    finally:
        assert G.gpuos_shutdown(ctx) == 0
    assert errs == [(first + i, G.GPUOS_ST_BAD_OP) for i in expect_bad]
    _assert_pool_equal(pool, _oracle_final(arrays, ref_recs), s.buffers)


def _exact_programs():
    X, P = W.xins, W.program
    return [
        P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_ADD, 0, 1, 2)]),
        P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_MUL, 0, 1, 2)]),
        P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_NEG, 2, 2), X(W.X_MAX, 0, 1, 2),
           X(W.X_CONST, 3, 0, 0, 0), X(W.X_MUL, 0, 0, 3)], [0.5]),
        P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_SUB, 0, 1, 2), X(W.X_ABS, 3, 2),
           X(W.X_CONST, 2, 0, 0, 0), X(W.X_ADD, 3, 3, 2), X(W.X_DIV, 0, 0, 3)], [1.0]),
        P([X(W.X_LDA, 1), X(W.X_CONST, 2, 0, 0, 0), X(W.X_MIN, 0, 1, 2), X(W.X_MUL, 0, 0, 1)], [2.0]),
        P([X(W.X_LDA, 1), X(W.X_ABS, 1, 1), X(W.X_SQRT, 1, 1), X(W.X_LDB, 2), X(W.X_RELU, 2, 2),
           X(W.X_ADD, 0, 1, 2)]),
    ]


def test_register_expr_flip_storm_while_a_pr1_stream_runs():
    """Twenty program flips of one op id while a PR1 stream is in flight;
    every descriptor of that op id runs the program bound when it was
    submitted, bit for bit (all steps correctly rounded)."""
    s = W.make_pr1(n_desc=1000)
    progs = _exact_programs()
    arrays = [b.host_bytes() for b in s.buffers]
    prog_base = len(arrays)
    arrays += progs
    pool = DevicePool(arrays)
    descs = to_descs(s.recs, pool.ptrs)
    ref_recs = s.recs.copy()
    uid = 90
    rng = np.random.default_rng(5)
    ctx = G.gpuos_init(ring_entries=128)
    try:
        for blk in range(20):
            pk = int(rng.integers(len(progs)))
            assert G.gpuos_register_expr(ctx, uid, progs[pk]) == 0
            lo, hi = 50 * blk, 50 * blk + 50
            for i in range(lo, hi):
                if int(s.recs["op"][i]) in (W.OP_ADD, W.OP_MUL) and rng.random() < 0.5:
                    descs["op_id"][i] = uid
                    ref_recs["op"][i] = W.OP_EXPR
                    ref_recs["dim"][i, 2] = len(progs[pk])
                    ref_recs["dim"][i, 3] = uid
                    ref_recs["buf"][i, W.AUX2] = prog_base + pk
                    ref_recs["off"][i, W.AUX2] = 0
            for k in range(lo, hi, 10):
                rc, _ = G.gpuos_submit(ctx, descs[k:k + 10], G.GPUOS_SUBMIT_BLOCK)
                assert rc == 0, G.ERR_NAMES.get(rc)
        n_expr = int((ref_recs["op"] == W.OP_EXPR).sum())
        say(f"20 program flips; {n_expr} of 1000 descriptors ran a program")
        rc, es, st = G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, SYNC_NS)
        assert rc == 0, (G.ERR_NAMES.get(rc), es, st)
    finally:
        assert G.gpuos_shutdown(ctx) == 0
    ref = _oracle_final(arrays, ref_recs)
    _assert_pool_equal(pool, ref, s.buffers)


@pytest.mark.parametrize("waves,upw", [(1, 1), (4, 2)])
def test_every_unit_runs_exactly_once(waves, upw):
    s = W.make_elementwise(n_desc=3000, ops=(W.OP_ADD, W.OP_MUL, W.OP_RELU))
    arrays = [b.host_bytes() for b in s.buffers]
    pool = DevicePool(arrays)
    descs = to_descs(s.recs, pool.ptrs)
    say(f"unit trace, 3000 descriptors, {waves} waves per workgroup, {upw} units per wave")
    ctx = G.gpuos_init(ring_entries=256, waves_per_wg=waves, units_per_wave=upw, flags=G.GPUOS_INIT_TRACE)
    try:
        rc, first, n = G.gpuos_submit_bursts(ctx, descs, np.asarray(s.bursts, np.uint32), G.GPUOS_SUBMIT_BLOCK)
        assert rc == 0 and n == len(descs)
        assert G.gpuos_pause(ctx, SYNC_NS) == 0
        st = G.gpuos_stats_get(ctx)
        tr = G.gpuos_trace_read(ctx)
    finally:
        assert G.gpuos_shutdown(ctx) == 0
    assert len(tr) == st["units"] > len(descs)
    key = (tr["seq"].astype(np.uint64) << np.uint64(24)) | tr["tile"].astype(np.uint64)
    assert len(np.unique(key)) == len(tr), "a unit ran twice"
    seqs, counts = np.unique(tr["seq"], return_counts=True)
    assert np.array_equal(seqs, np.arange(first, first + len(descs)))
    top = np.zeros(len(seqs), np.int64)
    np.maximum.at(top, np.searchsorted(seqs, tr["seq"]), tr["tile"].astype(np.int64))
    assert np.array_equal(top + 1, counts), "a descriptor's units are not 0..n-1"
    _assert_pool_equal(pool, _oracle_final(arrays, s.recs), s.buffers)


def test_shutdown_with_work_in_flight_finishes_it():
    s = W.make_elementwise(n_desc=5000, ops=(W.OP_ADD, W.OP_MUL, W.OP_RELU))
    arrays = [b.host_bytes() for b in s.buffers]
    pool = DevicePool(arrays)
    descs = to_descs(s.recs, pool.ptrs)
    ctx = G.gpuos_init(ring_entries=512)
    rc, _, n = G.gpuos_submit_bursts(ctx, descs, np.asarray(s.bursts, np.uint32), G.GPUOS_SUBMIT_BLOCK)
    assert rc == 0 and n == len(descs)
    say("shutdown right after the last submit")
    assert G.gpuos_shutdown(ctx) == 0
    _assert_pool_equal(pool, _oracle_final(arrays, s.recs), s.buffers)


def test_second_live_context_on_a_device_is_refused():
    """One live context per device and process: the second gpuos_init gets
    E_STATE (its executor could not be placed beside the first one's), and
    a context can be made again once the first is shut down."""
    say("second context refused")
    c1 = G.gpuos_init()
    try:
        with pytest.raises(G.GpuosError) as e:
            G.gpuos_init()
        assert e.value.rc == G.GPUOS_E_STATE
    finally:
        assert G.gpuos_shutdown(c1) == 0
    c2 = G.gpuos_init(num_wgs=8, waves_per_wg=1)
    assert G.gpuos_shutdown(c2) == 0


def test_idle_exit_and_relaunch():
    """With an idle-exit interval the executor leaves the GPU once nothing is
    committed and no call of the context has come for that long; the next
    call that has work for it launches it again from where its fetcher
    stopped, and the stream's results are unchanged.  Calls keep it
    resident."""
    import time
    s = W.make_elementwise(n_desc=2000, ops=(W.OP_ADD, W.OP_MUL, W.OP_RELU))
    arrays = [b.host_bytes() for b in s.buffers]
    pool = DevicePool(arrays)
    descs = to_descs(s.recs, pool.ptrs)
    say("idle exit and relaunch, 2000 descriptors, 50 ms interval")
    ctx = G.gpuos_init(ring_entries=256, idle_exit_ms=50)
    try:
        for i in range(0, 1000, 250):
            assert G.gpuos_submit(ctx, descs[i:i + 250], G.GPUOS_SUBMIT_BLOCK)[0] == 0
        assert G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, SYNC_NS)[0] == 0
        # calls every 10 ms for 0.3 s: the executor stays
        for _ in range(30):
            assert G.gpuos_query(ctx, 0) >= 0
            time.sleep(0.01)
        assert G.gpuos_stats_get(ctx)["idle_exits"] == 0
        time.sleep(0.5)  # no call: it leaves
        assert G.gpuos_query(ctx, 0) >= 0
        st = G.gpuos_stats_get(ctx)
        assert st["idle_exits"] == 1 and st["launches"] == 1, st
        for i in range(1000, 2000, 250):
            assert G.gpuos_submit(ctx, descs[i:i + 250], G.GPUOS_SUBMIT_BLOCK)[0] == 0
        assert G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, SYNC_NS)[0] == 0
        st = G.gpuos_stats_get(ctx)
        assert st["launches"] == 2 and st["completed"] == 2000, st
    finally:
        assert G.gpuos_shutdown(ctx) == 0
    _assert_pool_equal(pool, _oracle_final(arrays, s.recs), s.buffers)
