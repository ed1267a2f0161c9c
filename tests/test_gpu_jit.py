"""Compiled operator injection on the GPU, through the C ABI.

Element-wise programs are compiled at run time (gpuos_register_jit), loaded
while the executor is resident, and called by it through a function
pointer.  They are checked against the oracle (which interprets the same
program records), bit for bit against the executor's own interpreter where
every step is correctly rounded, re-bound between descriptors, bound in
the middle of a running stream, and used inside a dependent stream (the
element-wise stream's add and mul descriptors run as injected code,
bit-exact on the final pool)."""
import time

import numpy as np
import pytest

import workloads as W
from expr_programs import programs
from gpu_harness import check_record, run_gpu, run_oracle, say, untouched_equal
from oracle_util import bf16, rec
from parity import bits_equal

pytestmark = pytest.mark.gpu
RNG = np.random.default_rng(77)


@pytest.fixture(scope="module")
def jctx():
    from persistent_micro_dispatch_amd import gpuos as G
    c = G.gpuos_init(flags=G.GPUOS_INIT_JIT)
    yield c
    assert G.gpuos_shutdown(c) == 0


def _special(n, dt):
    x = (RNG.standard_normal(n) * 3).astype(np.float32)
    sp = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-40, 3e38, -3e38, 1.0, -1.0], np.float32)
    x[:min(len(sp), n)] = sp[:min(len(sp), n)]
    return x if dt == W.F32 else bf16(x)


def _program_records(dt, base_op):
    """One record per (program, size): sizes span one element, a partial
    unit, several units with a ragged tail (misaligned by one element) and
    a large descriptor."""
    recs, arrays, outs = [], [], []
    for k, (name, (prog, exact)) in enumerate(programs().items()):
        op_id = base_op + k
        unary = not any((int(w) & 0xFF) == W.X_LDB for w in prog[1:1 + (int(prog[0]) & 0xFF)])
        for n, sh in [(1, 0), (777, 0), (2053, 1), (70001, 0)]:
            if exact:
                a, b = _special(n + sh, dt), _special(n + sh, dt)[::-1].copy()
            else:
                a = RNG.standard_normal(n + sh).astype(np.float32)
                b = RNG.standard_normal(n + sh).astype(np.float32)
                if dt == W.BF16:
                    a, b = bf16(a), bf16(b)
            base = len(arrays)
            arrays += [a, b, np.zeros_like(a), prog]
            roles = dict(a=(base, sh * a.itemsize), out=(base + 2, sh * a.itemsize), aux2=base + 3)
            if not unary:
                roles["b"] = (base + 1, sh * a.itemsize)
            recs.append(rec(W.OP_EXPR, dtype=dt, size=n, dim=(0, 0, len(prog), op_id), **roles))
            outs.append((base + 2, exact))
    return arrays, np.concatenate(recs), outs


@pytest.mark.parametrize("dt", [W.F32, W.BF16])
def test_jit_programs_against_oracle_and_interpreter(jctx, dt):
    from persistent_micro_dispatch_amd import gpuos as G
    say(f"jit programs dt={dt}")
    base_op = 100
    arrays, recs, outs = _program_records(dt, base_op)
    for k, (name, (prog, _)) in enumerate(programs().items()):
        rc, info = G.gpuos_register_jit(jctx, base_op + k, prog)
        assert rc == 0, (name, rc, info)
        assert info["vgprs"] <= G.GPUOS_JIT_MAX_VGPRS and info["stack_bytes"] == 0
        say(f"  {name}: compile {info['compile_ms']:.0f} ms, load {info['load_ms']:.2f} ms, "
            f"flip {info['flip_ms']:.3f} ms, {info['vgprs']} VGPRs, reused {info['reused']}")
    gpu = run_gpu(arrays, recs, ctx=jctx)
    orc, hps = run_oracle(arrays, recs, capture=True)
    inputs = [np.ascontiguousarray(a).view(np.uint8).reshape(-1) for a in arrays]
    res = [check_record(r, inputs, gpu, orc, hp) for r, hp in zip(recs, hps)]
    bad = [x for x in res if not x["ok"]]
    assert not bad, bad[:5]
    assert untouched_equal(recs, gpu, orc)
    say("  worst vs oracle", max(r["worst"] for r in res))
    # the same records with the same op ids bound to the interpreter
    for k, (name, (prog, _)) in enumerate(programs().items()):
        assert G.gpuos_register_expr(jctx, base_op + k, prog) == 0
    interp = run_gpu(arrays, recs, ctx=jctx)
    for i, exact in outs:
        if exact:
            assert np.array_equal(gpu[i], interp[i]), i


def test_jit_rebinding_flips_between_descriptors(jctx):
    """A descriptor submitted before a re-binding runs the old code, one
    submitted after it the new code; the first binding is interpreted, the
    second compiled."""
    from persistent_micro_dispatch_amd import gpuos as G
    from workloads.gpu import DevicePool, to_descs
    X, P = W.xins, W.program
    p1 = P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_ADD, 0, 1, 2)])
    p2 = P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_MUL, 0, 1, 2)])
    p3 = P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_SUB, 0, 1, 2)])
    n = 50000
    a = RNG.standard_normal(n).astype(np.float32)
    b = RNG.standard_normal(n).astype(np.float32)
    arrays = [a, b, np.zeros_like(a), np.zeros_like(a), np.zeros_like(a), p1, p2, p3]
    r = [rec(W.OP_EXPR, size=n, dim=(0, 0, len(p1), 91), a=0, b=1, out=2 + i, aux2=5 + i) for i in range(3)]
    pool = DevicePool(arrays)
    d = to_descs(np.concatenate(r), pool.ptrs)
    say("jit rebinding")
    assert G.gpuos_register_expr(jctx, 91, p1) == 0
    assert G.gpuos_submit(jctx, d[:1], G.GPUOS_SUBMIT_BLOCK)[0] == 0
    assert G.gpuos_register_jit(jctx, 91, p2)[0] == 0  # the first may still be running
    assert G.gpuos_submit(jctx, d[1:2], G.GPUOS_SUBMIT_BLOCK)[0] == 0
    assert G.gpuos_register_jit(jctx, 91, p3)[0] == 0
    assert G.gpuos_submit(jctx, d[2:], G.GPUOS_SUBMIT_BLOCK)[0] == 0
    assert G.gpuos_sync(jctx, G.GPUOS_SEQ_ALL, 30_000_000_000)[0] == 0
    assert np.array_equal(pool.download(2).view(np.float32), a + b)
    assert np.array_equal(pool.download(3).view(np.float32), a * b)
    assert np.array_equal(pool.download(4).view(np.float32), a - b)


def test_jit_bound_during_running_stream_and_used_in_dependent_stream(jctx):
    """6,000 descriptors of the element-wise stream (its exactly rounded
    ops: add, mul, ReLU), the add and mul descriptors after the first 2,000
    bound to compiled a+b and a*b programs registered once those 2,000 were
    submitted (without waiting for them): the final pool must equal the
    oracle's run of the original stream bit for bit."""
    from persistent_micro_dispatch_amd import gpuos as G
    import oracle
    from workloads.gpu import DevicePool, to_descs
    s = W.make_elementwise(n_desc=6000, ops=(W.OP_ADD, W.OP_MUL, W.OP_RELU))
    recs = s.recs
    arrays = [bf.host_bytes() for bf in s.buffers]
    X, P = W.xins, W.program
    p_add = P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_ADD, 0, 1, 2)])
    p_mul = P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_MUL, 0, 1, 2)])
    pool = DevicePool(arrays)
    d = to_descs(recs, pool.ptrs)
    jit_add, jit_mul = 120, 121
    tail = d[2000:]
    tail["op_id"] = np.where(tail["op_id"] == W.OP_ADD, jit_add,
                             np.where(tail["op_id"] == W.OP_MUL, jit_mul, tail["op_id"])).astype(np.uint32)
    say("jit during stream: 2000 built-in descriptors in flight, then binding")
    ring = G.gpuos_stats_get(jctx)["ring_entries"]
    for i in range(0, 2000, ring):
        assert G.gpuos_submit(jctx, d[i:min(2000, i + ring)], G.GPUOS_SUBMIT_BLOCK)[0] == 0
    t0 = time.perf_counter()
    before = G.gpuos_query(jctx, G.gpuos_stats_get(jctx)["next_seq"] - 1)
    rc1, i1 = G.gpuos_register_jit(jctx, jit_add, p_add)
    rc2, i2 = G.gpuos_register_jit(jctx, jit_mul, p_mul)
    assert rc1 == 0 and rc2 == 0
    say(f"  bound in {(time.perf_counter() - t0) * 1e3:.0f} ms (compile {i1['compile_ms']:.0f} + "
        f"{i2['compile_ms']:.0f} ms); last built-in descriptor complete at binding start: {before == 1}")
    for i in range(0, len(tail), ring):
        assert G.gpuos_submit(jctx, tail[i:i + ring], G.GPUOS_SUBMIT_BLOCK)[0] == 0
    assert G.gpuos_sync(jctx, G.GPUOS_SEQ_ALL, 60_000_000_000)[0] == 0
    got = [pool.download(i) for i in range(len(arrays))]
    p = oracle.Pool([a.copy() for a in arrays])
    p.run(recs)
    for i, b in enumerate(s.buffers):
        eq = bits_equal(got[i].copy(), p.arrays[i].copy(), b.dtype)
        assert eq.all(), f"buffer {i}: {int((~eq).sum())} mismatches"
