"""GPU parity at the full sizes of the element-wise, row-op, decode and
small-matmul streams, in the launch configuration bench.py times (512-entry
ring; two waves per workgroup for the element-wise stream, four waves and
two units per wave for the row ops and decode, four waves and one unit per
wave for the small matmuls), through the C ABI.

- Element-wise: all 100,000 descriptors with the op set restricted to the
  exactly rounded ones (add, mul, ReLU), free-running; the final pool must
  equal the oracle's bit for bit (NaN as a class).
- Row ops: all 50,000 descriptors over the 2 GiB input pool (drawn on the
  GPU).  The ops are independent (read-only inputs, outputs in a rotating
  arena), so outputs that no later descriptor overwrites -- those after the
  arena's last wrap -- are checked one by one: each sampled descriptor is
  replayed by the oracle on its own input slice, downloaded from the GPU.
- Small matmuls: all 1,920 projections; sampled outputs of the last pass
  are checked against the oracle on their own x and weights."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_harness import check_record, run_gpu, run_record_oracle, say
from parity import bits_equal
from persistent_micro_dispatch_amd import gpuos as G
from workloads.gpu import DevicePool, to_descs

pytestmark = pytest.mark.gpu


def test_elementwise_full_stream_exact_ops_bit_exact():
    s = W.make_elementwise(ops=(W.OP_ADD, W.OP_MUL, W.OP_RELU))
    say(f"elementwise full stream, {len(s)} descriptors, ring 512, two waves per workgroup")
    arrays = [b.host_bytes() for b in s.buffers]
    gpu = run_gpu(arrays, s.recs, bursts=s.bursts, ring_entries=512, waves_per_wg=2, units_per_wave=1)
    p = oracle.Pool([a.copy() for a in arrays])
    p.run(s.recs)
    for i, b in enumerate(s.buffers):
        eq = bits_equal(gpu[i].copy(), p.arrays[i].copy(), b.dtype)
        assert eq.all(), f"buffer {i}: {int((~eq).sum())} mismatches"


def test_elementwise_full_stream_with_gelu_verify():
    """All 100,000 descriptors of the element-wise stream, GELU included, in
    verify mode (every output logged on the GPU, 3.5 GB of log): add, mul and
    ReLU bit-exact from identical inputs, GELU within its tolerance of the
    oracle's unrounded value."""
    from gpu_harness import verify_stream
    s = W.make_elementwise()
    say(f"elementwise full stream with GELU, verify mode, {len(s)} descriptors, ring 512, two waves per workgroup")
    res = verify_stream([b.host_bytes() for b in s.buffers], s.recs, bursts=s.bursts, ring_entries=512,
                        waves_per_wg=2, units_per_wave=1)
    say(f"  logged {res['n_logged']}; worst error ratio {res['worst']}; plain relative {res['plain']}")
    assert not res["fails"], res["fails"][:3]


def test_rows_full_stream_sampled_outputs():
    import torch
    s = W.make_rows()
    recs = s.recs
    say(f"rows full stream, {len(recs)} descriptors, 2 GiB pool, ring 512, 4 waves, 2 units per wave")
    pool = DevicePool.from_stream(s, fill="device")
    descs = to_descs(recs, pool.ptrs)
    ctx = G.gpuos_init(ring_entries=512, waves_per_wg=4, units_per_wave=2)
    try:
        rc, _, n = G.gpuos_submit_bursts(ctx, descs, np.asarray(s.bursts, np.uint32), G.GPUOS_SUBMIT_BLOCK)
        assert rc == 0 and n == len(descs)
        rc, es, st = G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 120_000_000_000)
        assert rc == 0, (rc, es, st)
    finally:
        assert G.gpuos_shutdown(ctx) == 0
    # descriptors after the last wrap of the output arena
    offs = recs["off"][:, W.OUT].astype(np.int64)
    last_wrap = int(np.nonzero(np.diff(offs) < 0)[0][-1]) + 1
    tail = np.arange(last_wrap, len(recs))
    rng = np.random.default_rng(33)
    pick = []
    for op in (W.OP_SUM, W.OP_MAX, W.OP_MIN, W.OP_SOFTMAX, W.OP_LAYERNORM):
        cand = tail[recs["op"][tail] == op]
        pick += list(rng.choice(cand, size=min(40, len(cand)), replace=False))
    pick = sorted(int(i) for i in pick)
    say(f"  checking {len(pick)} descriptors after the arena's last wrap (index {last_wrap})")
    es = W.DTYPE_BYTES[W.F32]
    arena = pool.tensors[int(recs["buf"][0, W.OUT])]
    torch.cuda.current_stream().synchronize()
    bad = []
    for i in pick:
        r = recs[i:i + 1].copy()
        rows, h = int(r["size"][0]), int(r["dim"][0, 0])
        op = int(r["op"][0])
        a_buf, a_off = int(r["buf"][0, W.A]), int(r["off"][0, W.A])
        x = pool.tensors[a_buf][a_off: a_off + rows * h * es].cpu().numpy()
        arrays = [x]
        r["buf"][0, W.A], r["off"][0, W.A] = 0, 0
        if op == W.OP_LAYERNORM:
            for role in (W.AUX0, W.AUX1):
                bi = int(r["buf"][0, role])
                arrays.append(pool.tensors[bi][: h * es].cpu().numpy())
                r["buf"][0, role], r["off"][0, role] = len(arrays) - 1, 0
        out_n = rows if op in (W.OP_SUM, W.OP_MAX, W.OP_MIN) else rows * h
        o_off = int(r["off"][0, W.OUT])
        g_out = arena[o_off: o_off + out_n * es].cpu().numpy()
        arrays.append(np.zeros(out_n * es, np.uint8))
        r["buf"][0, W.OUT], r["off"][0, W.OUT] = len(arrays) - 1, 0
        p = oracle.Pool([a.copy() for a in arrays])
        hp = run_record_oracle(p, r[0], op in (W.OP_MAX, W.OP_MIN))
        gpu_arrays = [a.copy() for a in arrays[:-1]] + [g_out]
        res = check_record(r[0], arrays, gpu_arrays, p.arrays, hp)
        if not res["ok"]:
            bad.append((i, res))
    assert not bad, bad[:3]


@pytest.mark.parametrize("kv_heads", [None, 8], ids=["mha", "gqa"])
def test_decode_full_stream_last_step_sampled(kv_heads):
    """The decode streams bench.py times (2,000 steps x 32 layers, caches of
    [8, Hkv, 4096, 128] bf16 per layer drawn on the GPU: 32 key/value heads,
    16 GiB, or 8 shared by groups of four query heads on the matrix cores),
    with four waves and two units per wave.  The last step's attention outputs are
    final (their output buffers are not written again), and so are the
    caches and the q/k buffers that step used (rotated in place by its RoPE,
    not used again): for sampled layers the oracle recomputes that step's
    SDPA from them, and the appended cache rows must equal k bit for bit."""
    import torch
    s = W.make_decode(steps=2000) if kv_heads is None else W.make_decode(steps=2000, kv_heads=kv_heads)
    recs = s.recs
    L = s.meta["layers"]
    say(f"decode full stream ({'32' if kv_heads is None else kv_heads} key/value heads), {len(recs)} descriptors, "
        "ring 512, 4 waves, 2 units per wave")
    pool = DevicePool.from_stream(s, fill="device")
    descs = to_descs(recs, pool.ptrs)
    ctx = G.gpuos_init(ring_entries=512, waves_per_wg=4, units_per_wave=2)
    try:
        rc, _, n = G.gpuos_submit_bursts(ctx, descs, np.asarray(s.bursts, np.uint32), G.GPUOS_SUBMIT_BLOCK)
        assert rc == 0 and n == len(descs)
        rc, es, st = G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 120_000_000_000)
        assert rc == 0, (rc, es, st)
    finally:
        assert G.gpuos_shutdown(ctx) == 0
    torch.cuda.current_stream().synchronize()
    last = len(recs) - 3 * L  # first record of the last step
    for layer in (0, L - 1):
        rope, app, sdpa = recs[last + 3 * layer: last + 3 * layer + 3]
        assert (int(rope["op"]), int(app["op"]), int(sdpa["op"])) == (W.OP_ROPE, W.OP_KV_APPEND, W.OP_SDPA)
        B_, (H, D, C, Hkv) = int(sdpa["size"]), [int(v) for v in sdpa["dim"]]
        Hkv = Hkv or H
        assert Hkv == (kv_heads or H)
        say(f"  layer {layer}: batch {B_}, lengths {[int(x) for x in sdpa['lens'][:B_]]}")
        q = pool.tensors[int(sdpa["buf"][W.A])][: B_ * H * D * 2].cpu().numpy()
        kb = pool.tensors[int(app["buf"][W.A])][: B_ * Hkv * D * 2].cpu().numpy()
        Kc = pool.tensors[int(sdpa["buf"][W.AUX0])][: B_ * Hkv * C * D * 2].cpu().numpy()
        Vc = pool.tensors[int(sdpa["buf"][W.AUX1])][: B_ * Hkv * C * D * 2].cpu().numpy()
        o_buf = int(sdpa["buf"][W.OUT])
        es_o = W.DTYPE_BYTES[int(sdpa["out_dtype"])]
        g_out = pool.tensors[o_buf][: B_ * H * D * es_o].cpu().numpy()
        # the appended rows are k, bit for bit
        kc = Kc.view(np.uint16).reshape(B_, Hkv, C, D)
        kk = kb.view(np.uint16).reshape(B_, Hkv, D)
        for b in range(B_):
            assert np.array_equal(kc[b, :, int(sdpa["lens"][b]) - 1, :], kk[b]), (layer, b)
        # attention against the oracle on the final q and caches
        r = sdpa.copy().reshape(1)
        arrays = [q, Kc, Vc, np.zeros(B_ * H * D * es_o, np.uint8)]
        r["buf"][0] = -1
        r["buf"][0, W.A], r["buf"][0, W.AUX0], r["buf"][0, W.AUX1], r["buf"][0, W.OUT] = 0, 1, 2, 3
        r["off"][0] = 0
        p = oracle.Pool([a.copy() for a in arrays])
        hp = run_record_oracle(p, r[0], False)
        res = check_record(r[0], arrays, arrays[:3] + [g_out], p.arrays, hp)
        say(f"    worst {res['worst']:.3g}")
        assert res["ok"], res


def test_matmul_full_stream_sampled_outputs():
    """The small-matmul stream at its full size (1,920 projections of 32
    token rows, 604 MB of weights) in the launch configuration bench.py
    times (512-entry ring, four waves per workgroup, one unit per wave).
    Every pass writes the same outputs from the same inputs, so sampled
    output buffers are checked against the oracle run on that descriptor's
    own x and weights (downloaded from the GPU), four of each projection
    shape."""
    import torch
    s = W.make_matmul()
    recs = s.recs
    say(f"matmul full stream, {len(recs)} descriptors, ring 512, 4 waves, 1 unit per wave")
    pool = DevicePool.from_stream(s, fill="device")
    descs = to_descs(recs, pool.ptrs)
    ctx = G.gpuos_init(ring_entries=512, waves_per_wg=4, units_per_wave=1)
    try:
        rc, _, n = G.gpuos_submit_bursts(ctx, descs, np.asarray(s.bursts, np.uint32), G.GPUOS_SUBMIT_BLOCK)
        assert rc == 0 and n == len(descs)
        rc, es, st = G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 120_000_000_000)
        assert rc == 0, (rc, es, st)
    finally:
        assert G.gpuos_shutdown(ctx) == 0
    torch.cuda.current_stream().synchronize()
    per_pass = int(s.bursts[0])
    last = np.arange(len(recs) - per_pass, len(recs))
    rng = np.random.default_rng(41)
    pick = []
    for K, N in {(int(r["dim"][0]), int(r["dim"][1])) for r in recs[last]}:
        cand = last[(recs["dim"][last, 0] == K) & (recs["dim"][last, 1] == N)]
        pick += [int(i) for i in rng.choice(cand, size=min(4, len(cand)), replace=False)]
    say(f"  checking {len(pick)} projections of the last pass")
    bad = []
    for i in sorted(pick):
        r = recs[i:i + 1].copy()
        M, K, N = int(r["size"][0]), int(r["dim"][0, 0]), int(r["dim"][0, 1])
        x = pool.tensors[int(r["buf"][0, W.A])][: M * K * 2].cpu().numpy()
        wt = pool.tensors[int(r["buf"][0, W.B])][: N * K * 2].cpu().numpy()
        g_out = pool.tensors[int(r["buf"][0, W.OUT])][: M * N * 2].cpu().numpy()
        arrays = [x, wt, np.zeros(M * N * 2, np.uint8)]
        r["buf"][0, W.A], r["buf"][0, W.B], r["buf"][0, W.OUT] = 0, 1, 2
        r["off"][0, W.A] = r["off"][0, W.B] = r["off"][0, W.OUT] = 0
        p = oracle.Pool([a.copy() for a in arrays])
        hp = run_record_oracle(p, r[0], False)
        res = check_record(r[0], arrays, [x, wt, g_out], p.arrays, hp)
        if not res["ok"]:
            bad.append((i, K, N, res))
    assert not bad, bad[:3]
