"""GPU parity on whole descriptor streams through the C ABI.

PR1 and the element-wise stream restricted to {add, mul, relu} run free
(no intervention) and the final pool must be bit-identical to the oracle's:
this also checks that concurrent claiming keeps sequential semantics under
heavy aliasing."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_harness import run_gpu, say
from parity import bits_equal
from persistent_micro_dispatch_amd import gpuos as G

pytestmark = pytest.mark.gpu


def _final_pools(stream, n, **init):
    arrays = [b.host_bytes() for b in stream.buffers]
    recs = stream.recs[:n]
    gpu = run_gpu(arrays, recs, bursts=stream.bursts, **init)
    p = oracle.Pool([a.copy() for a in arrays])
    p.run(recs)
    return gpu, p.arrays


@pytest.mark.parametrize("n", [1, 100, 1000])
def test_pr1_bit_exact(n):
    s = W.make_pr1()
    say(f"pr1 prefix {n}")
    gpu, orc = _final_pools(s, n)
    for i, b in enumerate(s.buffers):
        eq = bits_equal(gpu[i].copy(), orc[i].copy(), b.dtype)
        assert eq.all(), f"buffer {i}: {int((~eq).sum())} mismatches"
    if n == 1000:  # and byte for byte the recorded final pool (tests/golden)
        import hashlib
        import os
        h = hashlib.sha256()
        for a in gpu:
            h.update(np.ascontiguousarray(a).tobytes())
        rec_file = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pr1_final_pool.sha256")
        assert h.hexdigest() == open(rec_file).read().split()[0]


@pytest.mark.parametrize("ring,waves,upw", [(8, 4, 1), (4096, 1, 1), (8, 4, 2), (64, 1, 2)])
def test_pr1_bit_exact_small_ring_and_one_wave(ring, waves, upw):
    s = W.make_pr1()
    s.bursts = np.full(125, 8)
    say(f"pr1 ring={ring} waves={waves} units_per_wave={upw}")
    gpu, orc = _final_pools(s, 1000, ring_entries=ring, waves_per_wg=waves, units_per_wave=upw)
    for i, b in enumerate(s.buffers):
        assert bits_equal(gpu[i].copy(), orc[i].copy(), b.dtype).all()


# few workgroups: claim shards of one or two workgroups each (with one wave
# per workgroup, workgroup 0 holds only the fetcher)
@pytest.mark.parametrize("num_wgs,waves,upw", [(2, 1, 1), (3, 1, 1), (9, 1, 2), (5, 2, 1), (12, 4, 2)])
def test_pr1_bit_exact_few_workgroups(num_wgs, waves, upw):
    s = W.make_pr1()
    s.bursts = np.full(125, 8)
    say(f"pr1 num_wgs={num_wgs} waves={waves} units_per_wave={upw}")
    gpu, orc = _final_pools(s, 1000, ring_entries=64, num_wgs=num_wgs, waves_per_wg=waves, units_per_wave=upw)
    for i, b in enumerate(s.buffers):
        assert bits_equal(gpu[i].copy(), orc[i].copy(), b.dtype).all()


@pytest.mark.parametrize("upw", [1, 2])
def test_elementwise_exact_ops_bit_exact(upw):
    s = W.make_elementwise(n_desc=5000, ops=(W.OP_ADD, W.OP_MUL, W.OP_RELU))
    say(f"elementwise exact 5000, units_per_wave={upw}")
    gpu, orc = _final_pools(s, len(s), units_per_wave=upw)
    for i, b in enumerate(s.buffers):
        eq = bits_equal(gpu[i].copy(), orc[i].copy(), b.dtype)
        assert eq.all(), f"buffer {i}: {int((~eq).sum())} mismatches"


def test_elementwise_exact_ops_small_unit_queue():
    # A unit queue of 4096 entries: 512 descriptors in flight hold more units
    # than that, so the fetcher keeps waiting for queue capacity (and reads
    # done[] again to see it free up).
    s = W.make_elementwise(n_desc=3000, ops=(W.OP_ADD, W.OP_MUL, W.OP_RELU))
    say("elementwise exact 3000, unit queue of 4096 entries")
    gpu, orc = _final_pools(s, len(s), unit_queue_log2=12, ring_entries=512)
    for i, b in enumerate(s.buffers):
        eq = bits_equal(gpu[i].copy(), orc[i].copy(), b.dtype)
        assert eq.all(), f"buffer {i}: {int((~eq).sum())} mismatches"


# --------------------------------------------------------------------------
# Verify mode (every output logged on the GPU, teacher-forced oracle replay)
# --------------------------------------------------------------------------
from gpu_harness import verify_stream  # noqa: E402


def _report(name, res):
    say(f"{name}: logged {res['n_logged']} outputs; worst error ratio per op {res['worst']}; "
        f"plain relative error per op {res['plain']}")
    assert not res["fails"], res["fails"][:3]
    assert res["kv_ok"]


def test_elementwise_stream_verify():
    # the element-wise stream with GELU, 20,000 descriptors, in the bench's
    # launch configuration (512-entry ring, two waves per workgroup), and with
    # one wave per workgroup
    s = W.make_elementwise(n_desc=20000)
    for waves in (2, 1):
        say(f"elementwise verify, 20000 descriptors with GELU, {waves} waves per workgroup")
        res = verify_stream([b.host_bytes() for b in s.buffers], s.recs, bursts=s.bursts, ring_entries=512,
                            waves_per_wg=waves, units_per_wave=1)
        _report("elementwise", res)


def test_rows_stream_verify():
    s = W.make_rows(n_desc=600, n_pool=8, arena_bytes=32 << 20)
    res = verify_stream([b.host_bytes() for b in s.buffers], s.recs)
    _report("rows", res)


@pytest.mark.parametrize("upw", [1, 2])
def test_decode_stream_verify(upw):
    s = W.make_decode(steps=4, layers=2, heads=8, capacity=512, l_min=100, n_triples=4, n_out=16)
    say(f"decode verify, units_per_wave={upw}")
    res = verify_stream([b.host_bytes() for b in s.buffers], s.recs, units_per_wave=upw)
    _report("decode", res)


@pytest.mark.parametrize("upw", [1, 2])
def test_mixed_stream_verify(upw):
    s = W.make_mixed(tokens=2, layers=2, capacity=256, l0_range=(32, 200))
    say(f"mixed verify, units_per_wave={upw}")
    res = verify_stream([b.host_bytes() for b in s.buffers], s.recs, units_per_wave=upw)
    _report("mixed", res)


def test_mixed_stream_verify_bench_shape():
    """The mixed pipeline at the shape bench.py times: 32 layers, hidden 1024,
    8 heads x 128, KV capacity 4096, L0 in [64, 2048]; two tokens (706
    descriptors, every output logged), with the bench's launch configuration
    (512-entry ring, one wave per workgroup, one unit per wave, 256 MiB of
    scratch).  The 1.1 GiB pool (weights N(0, 0.02), caches N(0, 1)) is drawn
    on the GPU and its initial contents downloaded for the oracle."""
    from workloads.gpu import DevicePool
    s = W.make_mixed(tokens=2)
    say(f"mixed verify at the bench shape: {len(s.recs)} descriptors, 32 layers, C=4096")
    pool = DevicePool.from_stream(s, fill="device")
    res = verify_stream(None, s.recs, bursts=s.bursts, pool=pool, ring_entries=512, waves_per_wg=1,
                        units_per_wave=1)
    _report("mixed (bench shape)", res)


def test_decode_grouped_kv_heads_stream_verify():
    s = W.make_decode(steps=3, layers=2, heads=8, kv_heads=2, capacity=512, l_min=100, n_triples=4, n_out=16)
    say("decode verify, 8 query heads sharing 2 key/value heads")
    res = verify_stream([b.host_bytes() for b in s.buffers], s.recs, units_per_wave=2)
    _report("decode gqa", res)


def test_mixed_stream_verify_small_scratch():
    # 1 MiB of scratch: the split partials of the vector-matrix products and
    # attention ops in flight need more, so the fetcher waits for scratch
    # held by incomplete descriptors to be released.
    s = W.make_mixed(tokens=2, layers=2, capacity=256, l0_range=(32, 200))
    say("mixed verify, 1 MiB of scratch")
    res = verify_stream([b.host_bytes() for b in s.buffers], s.recs, scratch_bytes=1 << 20)
    _report("mixed small scratch", res)


def test_decode_stream_verify_few_waves_two_units():
    # seven worker waves holding two units each: ready RoPE and KV-append
    # units keep running before ready attention units, and every attention
    # unit still runs (a ready long unit is passed over at most four times)
    s = W.make_decode(steps=4, layers=2, heads=8, capacity=512, l_min=100, n_triples=4, n_out=16)
    say("decode verify, 4 workgroups x 2 waves, two units per wave")
    res = verify_stream([b.host_bytes() for b in s.buffers], s.recs, num_wgs=4, waves_per_wg=2, units_per_wave=2)
    _report("decode few waves", res)
