"""GPU parity, one micro-op at a time, through the C ABI: every op body at
small shapes (several tiles, ragged tails, misaligned operands, special
values) against the oracle.  Bytes no record writes must stay identical."""
import numpy as np
import pytest

import workloads as W
from expr_programs import programs as _programs
from gpu_harness import check_record, run_gpu, run_oracle, say, untouched_equal
from oracle_util import bf16, rec

pytestmark = pytest.mark.gpu
RNG = np.random.default_rng(2024)


@pytest.fixture(scope="module")
def ctx():
    from persistent_micro_dispatch_amd import gpuos as G
    c = G.gpuos_init()
    yield c
    assert G.gpuos_shutdown(c) == 0


def _special_f32(n):
    x = (RNG.standard_normal(n) * 3).astype(np.float32)
    sp = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-40, 3e38, -3e38, 1.0, -1.0], np.float32)
    k = min(len(sp), n)
    x[:k] = sp[:k]
    return x


def _vals(n, dt):
    x = _special_f32(n)
    return x if dt == W.F32 else bf16(x)


def _run_and_check(ctx, arrays, recs):
    gpu = run_gpu(arrays, recs, ctx=ctx)
    orc, hps = run_oracle(arrays, recs, capture=True)
    inputs = [np.ascontiguousarray(a).view(np.uint8).reshape(-1) for a in arrays]
    results = [check_record(r, inputs, gpu, orc, hp) for r, hp in zip(recs, hps)]
    bad = [x for x in results if not x["ok"]]
    assert not bad, bad[:5]
    assert untouched_equal(recs, gpu, orc)
    return results


@pytest.mark.parametrize("dt", [W.F32, W.BF16])
@pytest.mark.parametrize("op", [W.OP_ADD, W.OP_MUL, W.OP_RELU, W.OP_GELU])
def test_elementwise(ctx, op, dt):
    say(f"elementwise op={W.OP_NAMES[op]} dt={dt}")
    sizes = [1, 7, 255, 256, 2047, 2048, 2049, 4095, 4097, 8192, 12345, 65536, 16383, 16389, 40000, 32771, 65541]
    recs, arrays = [], []
    for i, n in enumerate(sizes):
        cap = n + 16
        a, b, o = _vals(cap, dt), _vals(cap, dt), np.zeros_like(_vals(cap, dt))
        base = len(arrays)
        arrays += [a, b, o]
        es = W.DTYPE_BYTES[dt]
        sh = es if i % 3 == 2 else 0      # every third case misaligned by one element
        recs.append(rec(op, dtype=dt, size=n, a=(base, sh), b=(base + 1, sh), out=(base + 2, sh)))
    # in place: out = a
    a = _vals(5000, dt)
    arrays.append(a)
    recs.append(rec(op, dtype=dt, size=5000, a=len(arrays) - 1, b=len(arrays) - 1, out=len(arrays) - 1))
    res = _run_and_check(ctx, arrays, np.concatenate(recs))
    say("  worst", max(r["worst"] for r in res))


@pytest.mark.parametrize("dt", [W.F32, W.BF16])
def test_gelu_dense_sweep(ctx, dt):
    """GELU over a dense grid of [-14, 14], every fp32 value in the last few
    ulps on both sides of -3 (where the body switches from its fp32 path to
    the one with a double-precision exponent), the tails where the result
    becomes subnormal and underflows, and the specials."""
    say(f"gelu sweep dt={dt}")
    grid = np.linspace(-14.0, 14.0, 1 << 16, dtype=np.float32)
    m3 = np.float32(-3.0)
    near = np.concatenate([m3 + np.arange(-64, 65, dtype=np.float32) * np.spacing(m3),
                           np.nextafter(m3, np.float32(0)) - np.arange(8, dtype=np.float32) * 1e-7])
    tails = -np.geomspace(9.0, 1e4, 2048).astype(np.float32)
    sp = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45, 1e-38, -1e-38, 3e38, -3e38], np.float32)
    x = np.concatenate([grid, near, tails, -tails, sp]).astype(np.float32)
    xs = x if dt == W.F32 else bf16(x)
    arrays = [xs, np.zeros_like(xs)]
    res = _run_and_check(ctx, arrays, rec(W.OP_GELU, dtype=dt, size=len(x), a=0, out=1))
    say("  worst", max(r["worst"] for r in res))


def test_bf16_rounding_ties_through_add(ctx):
    """bf16 add of pairs whose exact fp32 sums fall exactly half-way between
    two bf16 values (both parities), just above and below half-way, and
    overflow to infinity: the rounding of the fp32 result to bf16 decides
    every bit, and must equal the oracle's round-to-nearest-even."""
    say("bf16 rounding ties")
    base = np.ldexp(np.float32(1) + np.arange(128, dtype=np.float32) / 128, np.arange(-20, 20)[:, None]).astype(
        np.float32).reshape(-1)                               # every bf16 significand, many exponents
    ulp = np.ldexp(np.float32(1), (np.frexp(base)[1] - 8)).astype(np.float32)   # bf16 ulp of base
    a_parts, b_parts = [], []
    for frac in (0.5, 0.5 + 2.0 ** -8, 0.5 - 2.0 ** -8, 0.25, 0.75, 1.5):
        a_parts.append(base)
        b_parts.append((ulp * np.float32(frac)).astype(np.float32))
    a = np.concatenate(a_parts + [np.float32([3.3895e38, -3.3895e38])])
    b = np.concatenate(b_parts + [np.float32([1.5e36, -1.5e36])])
    # b must be a bf16 value itself for the test to be about the sum's rounding
    ab, bb = bf16(a), bf16(b)
    arrays = [ab, bb, np.zeros_like(ab)]
    _run_and_check(ctx, arrays, rec(W.OP_ADD, dtype=W.BF16, size=len(a), a=0, b=1, out=2))


@pytest.mark.parametrize("op", [W.OP_SUM, W.OP_MAX, W.OP_MIN, W.OP_SOFTMAX, W.OP_LAYERNORM])
@pytest.mark.parametrize("dt", [W.F32, W.BF16])
def test_rows(ctx, op, dt):
    say(f"rows op={W.OP_NAMES[op]} dt={dt}")
    recs, arrays = [], []
    for rows, h in [(1, 768), (3, 1024), (64, 2048), (5, 4096), (2, 100), (3, 5000), (1, 1), (37, 256),
                    (21, 768)]:
        x = (RNG.standard_normal(rows * h) * 2).astype(np.float32)
        if op in (W.OP_MAX, W.OP_MIN) and rows * h > 10:
            x[3] = -0.0
            x[4] = 0.0
        xs = x if dt == W.F32 else bf16(x)
        g = (1 + 0.1 * RNG.standard_normal(h)).astype(np.float32)
        b = (0.1 * RNG.standard_normal(h)).astype(np.float32)
        gs, bs = (g, b) if dt == W.F32 else (bf16(g), bf16(b))
        red = op in (W.OP_SUM, W.OP_MAX, W.OP_MIN)
        o = np.zeros(rows if red else rows * h, xs.dtype)
        base = len(arrays)
        arrays += [xs, gs, bs, o]
        recs.append(rec(op, dtype=dt, size=rows, dim=(h,), fparam=(1e-5,), a=base, aux0=base + 1,
                        aux1=base + 2, out=base + 3))
    res = _run_and_check(ctx, arrays, np.concatenate(recs))
    say("  worst", max(r["worst"] for r in res))


def test_rows_special_values(ctx):
    x = np.array([[1.0, np.nan, -2.0, 3.0] * 256, [-0.0] * 1024, [0.0, -0.0] * 512], np.float32).reshape(-1)
    arrays = [x, np.zeros(3, np.float32), np.zeros(3, np.float32)]
    recs = np.concatenate([rec(W.OP_MAX, size=3, dim=(1024,), a=0, out=1),
                           rec(W.OP_MIN, size=3, dim=(1024,), a=0, out=2)])
    _run_and_check(ctx, arrays, recs)


@pytest.mark.parametrize("dt,half", [(W.BF16, False), (W.BF16, True), (W.F32, False)])
def test_rope(ctx, dt, half):
    say(f"rope dt={dt} half={half}")
    recs, arrays = [], []
    for B, H, D, lens in [(1, 32, 128, [1]), (3, 8, 128, [2, 100, 4096]), (8, 32, 128, list(RNG.integers(1, 4097, 8))),
                          (2, 4, 64, [7, 3000]), (1, 2, 256, [1234])]:
        q = _vals(B * H * D, dt)
        k = _vals(B * H * D, dt)
        if dt == W.F32:
            q = (RNG.standard_normal(B * H * D)).astype(np.float32)
            k = (RNG.standard_normal(B * H * D)).astype(np.float32)
        else:
            q, k = bf16(RNG.standard_normal(B * H * D)), bf16(RNG.standard_normal(B * H * D))
        base = len(arrays)
        arrays += [q, k]
        recs.append(rec(W.OP_ROPE, dtype=dt, size=B, dim=(H, D), fparam=(10000.0,), lens=lens,
                        flags=W.FLAG_ROPE_HALF if half else 0, a=base, b=base + 1))
    _run_and_check(ctx, arrays, np.concatenate(recs))


def test_kv_append(ctx):
    recs, arrays = [], []
    for B, H, D, C, lens in [(1, 32, 128, 4096, [4096]), (8, 32, 128, 512, list(RNG.integers(1, 513, 8))),
                             (3, 4, 64, 100, [1, 50, 100])]:
        k, v = bf16(RNG.standard_normal(B * H * D)), bf16(RNG.standard_normal(B * H * D))
        K, V = bf16(RNG.standard_normal(B * H * C * D)), bf16(RNG.standard_normal(B * H * C * D))
        base = len(arrays)
        arrays += [k, v, K, V]
        recs.append(rec(W.OP_KV_APPEND, dtype=W.BF16, size=B, dim=(H, D, C), lens=lens, a=base, b=base + 1,
                        aux0=base + 2, aux1=base + 3))
    _run_and_check(ctx, arrays, np.concatenate(recs))


@pytest.mark.parametrize("out_dt", [W.F32, W.BF16])
def test_sdpa(ctx, out_dt):
    say(f"sdpa out={out_dt}")
    recs, arrays = [], []
    for B, H, D, C, lens in [(1, 4, 128, 4096, [1]), (2, 4, 128, 4096, [255, 257]), (1, 2, 128, 4096, [4096]),
                             (8, 2, 128, 2048, list(RNG.integers(1, 2049, 8))), (2, 3, 64, 600, [256, 513]),
                             (3, 1, 128, 300, [300, 1, 129]), (1, 2, 128, 16384, [16384]),
                             (2, 1, 128, 9000, [8500, 7937]), (1, 3, 64, 10000, [9000])]:
        q = bf16(RNG.standard_normal(B * H * D))
        K, V = bf16(RNG.standard_normal(B * H * C * D)), bf16(RNG.standard_normal(B * H * C * D))
        o = np.zeros(B * H * D, np.float32 if out_dt == W.F32 else np.uint16)
        base = len(arrays)
        arrays += [q, K, V, o]
        recs.append(rec(W.OP_SDPA, dtype=W.BF16, out_dtype=out_dt, size=B, dim=(H, D, C), lens=lens,
                        a=base, aux0=base + 1, aux1=base + 2, out=base + 3))
    res = _run_and_check(ctx, arrays, np.concatenate(recs))
    say("  worst", max(r["worst"] for r in res))


@pytest.mark.parametrize("dt,out_dt", [(W.BF16, W.BF16), (W.F32, W.F32), (W.BF16, W.F32)])
def test_gemv(ctx, dt, out_dt):
    say(f"gemv dt={dt} out={out_dt}")
    recs, arrays = [], []
    for K, N in [(1024, 3072), (3072, 1024), (100, 77), (64, 512), (65, 513), (1, 8), (1000, 200),
                 (4100, 72)]:
        x = RNG.standard_normal(K).astype(np.float32)
        Wm = (RNG.standard_normal(K * N) * 0.02).astype(np.float32)
        if dt == W.BF16:
            x, Wm = bf16(x), bf16(Wm)
        o = np.zeros(N, np.float32 if out_dt == W.F32 else np.uint16)
        base = len(arrays)
        arrays += [x, Wm, o]
        recs.append(rec(W.OP_GEMV, dtype=dt, out_dtype=out_dt, dim=(K, N), a=base, b=base + 1, out=base + 2))
    res = _run_and_check(ctx, arrays, np.concatenate(recs))
    say("  worst", max(r["worst"] for r in res))


def test_copy_and_nop(ctx):
    recs, arrays = [], []
    for n, sh in [(1, 0), (15, 1), (16384, 0), (100000, 3), (0, 0)]:
        a = RNG.integers(0, 255, n + 8).astype(np.uint8)
        base = len(arrays)
        arrays += [a, np.zeros(n + 8, np.uint8)]
        recs.append(rec(W.OP_COPY, size=n, a=(base, sh), out=(base + 1, sh)))
    recs.append(rec(W.OP_NOP))
    _run_and_check(ctx, arrays, np.concatenate(recs))


def test_empty_descriptors(ctx):
    """Element-wise and row ops of size 0 (one unit each that does nothing)
    complete and write nothing; the ordinary descriptors after them still run."""
    say("empty descriptors: element-wise and row ops of size 0, then ordinary ones")
    recs, arrays = [], []
    for dt in (W.F32, W.BF16):
        es = W.DTYPE_BYTES[dt]
        base = len(arrays)
        arrays += [_vals(4096, dt), _vals(4096, dt), RNG.integers(0, 255, 4096 * es).astype(np.uint8),
                   _vals(4096, dt) if dt == W.F32 else bf16(1.0 + 0.1 * RNG.standard_normal(4096).astype(np.float32)),
                   _vals(4096, dt)]
        for op in (W.OP_ADD, W.OP_MUL, W.OP_RELU, W.OP_GELU):
            recs.append(rec(op, dtype=dt, size=0, a=base, b=base + 1, out=base + 2))
        for op in (W.OP_SUM, W.OP_MAX, W.OP_MIN, W.OP_SOFTMAX):
            recs.append(rec(op, dtype=dt, size=0, dim=(1024,), a=base, out=base + 2))
        recs.append(rec(W.OP_LAYERNORM, dtype=dt, size=0, dim=(1024,), fparam=(1e-5,), a=base, aux0=base + 3,
                        aux1=base + 4, out=base + 2))
        # ordinary work after the empty descriptors, on the same output
        recs.append(rec(W.OP_ADD, dtype=dt, size=777, a=base, b=base + 1, out=(base + 2, es * 100)))
        recs.append(rec(W.OP_SOFTMAX, dtype=dt, size=2, dim=(1024,), a=(base, es * 1024), out=(base + 2, es * 2048)))
    _run_and_check(ctx, arrays, np.concatenate(recs))


def test_large_descriptors(ctx):
    """Descriptors of hundreds of units (completion counted by one per-slot counter)."""
    say("large descriptors: copy 8 MiB + 37 B, add/mul 1M + 3 elements")
    recs, arrays = [], []
    n = (8 << 20) + 37
    a = RNG.integers(0, 255, n + 8).astype(np.uint8)
    arrays += [a, np.zeros(n + 8, np.uint8)]
    recs.append(rec(W.OP_COPY, size=n, a=0, out=1))
    for op, dt in [(W.OP_ADD, W.F32), (W.OP_MUL, W.BF16), (W.OP_GELU, W.F32)]:
        m = (1 << 20) + 3
        base = len(arrays)
        arrays += [_vals(m, dt), _vals(m, dt), np.zeros_like(_vals(m, dt))]
        recs.append(rec(op, dtype=dt, size=m, a=base, b=base + 1, out=base + 2))
    _run_and_check(ctx, arrays, np.concatenate(recs))


def test_batch_of_many_units_published_in_prefixes(ctx):
    """One batch of more units than several publication steps (the fetcher
    publishes a large batch 2,048 units at a time): a copy of 96 MiB + 5 B
    (3,073 units) and an fp32 add of 8M + 1 elements (4,097 units) submitted
    together, both exact."""
    say("one batch of about 7,000 units: copy 96 MiB + 5 B, add 8M + 1")
    n = (96 << 20) + 5
    a = RNG.integers(0, 255, n).astype(np.uint8)
    m = (8 << 20) + 1
    x, y = _vals(m, W.F32), _vals(m, W.F32)
    arrays = [a, np.zeros(n, np.uint8), x, y, np.zeros(m, np.float32)]
    recs = np.concatenate([rec(W.OP_COPY, size=n, a=0, out=1), rec(W.OP_ADD, dtype=W.F32, size=m, a=2, b=3, out=4)])
    _run_and_check(ctx, arrays, recs)


# ------------------------------------------------ injected element-wise programs
@pytest.mark.parametrize("dt", [W.F32, W.BF16])
def test_expr_programs(ctx, dt):
    from persistent_micro_dispatch_amd import gpuos as G
    say(f"expr programs dt={dt}")
    recs, arrays = [], []
    for k, (name, (prog, exact)) in enumerate(_programs().items()):
        op_id = 80 + k
        assert G.gpuos_register_expr(ctx, op_id, prog) == 0
        unary = not any((int(w) & 0xFF) == W.X_LDB for w in prog[1:1 + (int(prog[0]) & 0xFF)])
        for n, sh in [(1, 0), (777, 0), (2053, 1), (70001, 0)]:
            if exact:
                a, b = _vals(n + sh, dt), _vals(n + sh, dt)[::-1].copy()
            else:
                a = (RNG.standard_normal(n + sh)).astype(np.float32)
                b = (RNG.standard_normal(n + sh)).astype(np.float32)
                if dt == W.BF16:
                    a, b = bf16(a), bf16(b)
            base = len(arrays)
            arrays += [a, b, np.zeros_like(a), prog]
            roles = dict(a=(base, sh * a.itemsize), out=(base + 2, sh * a.itemsize), aux2=base + 3)
            if not unary:
                roles["b"] = (base + 1, sh * a.itemsize)
            recs.append(rec(W.OP_EXPR, dtype=dt, size=n, dim=(0, 0, len(prog), op_id), **roles))
    res = _run_and_check(ctx, arrays, np.concatenate(recs))
    say("  worst", max(r["worst"] for r in res))


def test_expr_reregistration_flips_between_descriptors(ctx):
    """Descriptors submitted before a re-registration run the old program,
    those after it the new one (the dual-slot table with a version flip)."""
    from persistent_micro_dispatch_amd import gpuos as G
    from workloads.gpu import DevicePool, to_descs
    X, P = W.xins, W.program
    p1 = P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_ADD, 0, 1, 2)])
    p2 = P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_MUL, 0, 1, 2)])
    n = 50000
    a = (RNG.standard_normal(n)).astype(np.float32)
    b = (RNG.standard_normal(n)).astype(np.float32)
    arrays = [a, b, np.zeros_like(a), np.zeros_like(a), p1, p2]
    r1 = rec(W.OP_EXPR, size=n, dim=(0, 0, len(p1), 90), a=0, b=1, out=2, aux2=4)
    r2 = rec(W.OP_EXPR, size=n, dim=(0, 0, len(p2), 90), a=0, b=1, out=3, aux2=5)
    pool = DevicePool(arrays)
    d = to_descs(np.concatenate([r1, r2]), pool.ptrs)
    assert G.gpuos_register_expr(ctx, 90, p1) == 0
    rc, _ = G.gpuos_submit(ctx, d[:1], G.GPUOS_SUBMIT_BLOCK)
    assert rc == 0
    assert G.gpuos_register_expr(ctx, 90, p2) == 0  # the first may still be running
    rc, _ = G.gpuos_submit(ctx, d[1:], G.GPUOS_SUBMIT_BLOCK)
    assert rc == 0
    assert G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 30_000_000_000)[0] == 0
    assert np.array_equal(pool.download(2).view(np.float32), a + b)
    assert np.array_equal(pool.download(3).view(np.float32), a * b)


# ------------------------------------------------ grouped-query attention
@pytest.mark.parametrize("out_dt", [W.F32, W.BF16])
def test_sdpa_grouped_kv_heads(ctx, out_dt):
    say(f"sdpa gqa out={out_dt}")
    recs, arrays = [], []
    for B, H, Hkv, D, C, lens in [(2, 8, 2, 128, 600, [300, 17]), (1, 32, 8, 128, 4096, [4096]),
                                  (3, 4, 1, 64, 700, [1, 256, 700]), (8, 32, 8, 128, 512, list(RNG.integers(1, 513, 8))),
                                  (2, 16, 1, 128, 1100, [1025, 31]), (1, 8, 2, 128, 40, [33])]:
        q = bf16(RNG.standard_normal(B * H * D))
        K, V = bf16(RNG.standard_normal(B * Hkv * C * D)), bf16(RNG.standard_normal(B * Hkv * C * D))
        o = np.zeros(B * H * D, np.float32 if out_dt == W.F32 else np.uint16)
        base = len(arrays)
        arrays += [q, K, V, o]
        recs.append(rec(W.OP_SDPA, dtype=W.BF16, out_dtype=out_dt, size=B, dim=(H, D, C, Hkv), lens=lens,
                        a=base, aux0=base + 1, aux1=base + 2, out=base + 3))
    res = _run_and_check(ctx, arrays, np.concatenate(recs))
    say("  worst", max(r["worst"] for r in res))


@pytest.mark.parametrize("dt,half", [(W.BF16, False), (W.F32, False), (W.BF16, True)])
def test_rope_fewer_key_heads(ctx, dt, half):
    say(f"rope gqa dt={dt} half={half}")
    recs, arrays = [], []
    for B, H, Hk, D, lens in [(3, 32, 8, 128, [1, 77, 4096]), (1, 6, 2, 64, [1234]), (2, 8, 1, 128, [9, 10])]:
        if dt == W.F32:
            q = RNG.standard_normal(B * H * D).astype(np.float32)
            k = RNG.standard_normal(B * Hk * D).astype(np.float32)
        else:
            q, k = bf16(RNG.standard_normal(B * H * D)), bf16(RNG.standard_normal(B * Hk * D))
        base = len(arrays)
        arrays += [q, k]
        recs.append(rec(W.OP_ROPE, dtype=dt, size=B, dim=(H, D, 0, Hk), fparam=(10000.0,), lens=lens,
                        flags=W.FLAG_ROPE_HALF if half else 0, a=base, b=base + 1))
    _run_and_check(ctx, arrays, np.concatenate(recs))


# ------------------------------------------------ attention masking
def _mask(B, C, lens, kind):
    """fp32 [B, C] additive masks: random finite values, padding (-inf on a
    random subset), a causal-like band, and rows with every key masked."""
    m = np.zeros((B, C), np.float32)
    for b in range(B):
        L = int(lens[b])
        if kind == "random":
            m[b] = (RNG.standard_normal(C) * 2).astype(np.float32)
        elif kind == "padding":
            m[b, RNG.random(C) < 0.3] = -np.inf
            m[b, L - 1] = 0.0
        elif kind == "band":
            m[b, : max(0, L - 100)] = -np.inf   # only the last 100 keys
        elif kind == "all":
            m[b] = -np.inf if b % 2 == 0 else 0.0
    return m.reshape(-1)


@pytest.mark.parametrize("out_dt", [W.F32, W.BF16])
@pytest.mark.parametrize("kind", ["random", "padding", "band", "all"])
def test_sdpa_masked(ctx, out_dt, kind):
    say(f"sdpa masked ({kind}) out={out_dt}")
    recs, arrays = [], []
    for B, H, Hkv, D, C, lens in [(2, 8, 2, 128, 600, [300, 17]), (1, 32, 8, 128, 4096, [4096]),
                                  (3, 4, 4, 64, 700, [1, 256, 700]), (4, 8, 8, 128, 3000, [3000, 2049, 1500, 64])]:
        q = bf16(RNG.standard_normal(B * H * D))
        K, V = bf16(RNG.standard_normal(B * Hkv * C * D)), bf16(RNG.standard_normal(B * Hkv * C * D))
        o = np.zeros(B * H * D, np.float32 if out_dt == W.F32 else np.uint16)
        base = len(arrays)
        arrays += [q, K, V, o, _mask(B, C, lens, kind)]
        recs.append(rec(W.OP_SDPA, dtype=W.BF16, out_dtype=out_dt, size=B, dim=(H, D, C, Hkv), lens=lens,
                        flags=W.FLAG_SDPA_MASK, a=base, aux0=base + 1, aux1=base + 2, out=base + 3, aux2=base + 4))
    res = _run_and_check(ctx, arrays, np.concatenate(recs))
    say("  worst", max(r["worst"] for r in res))


# ------------------------------------------------ small matmul (matrix cores)
@pytest.mark.parametrize("out_dt", [W.F32, W.BF16])
def test_matmul(ctx, out_dt):
    say(f"matmul out={out_dt}")
    recs, arrays = [], []
    for M, K, N in [(1, 1024, 3072), (16, 1024, 3072), (33, 3072, 1024), (64, 256, 100), (7, 32, 17),
                    (64, 4096, 64), (2, 1056, 300), (48, 512, 1000), (32, 3072, 1000), (32, 2048, 130)]:
        x = bf16(RNG.standard_normal(M * K))
        wt = bf16(0.05 * RNG.standard_normal(N * K))
        y = np.zeros(M * N, np.float32 if out_dt == W.F32 else np.uint16)
        base = len(arrays)
        arrays += [x, wt, y]
        recs.append(rec(W.OP_MATMUL, dtype=W.BF16, out_dtype=out_dt, size=M, dim=(K, N), a=base, b=base + 1,
                        out=base + 2))
    res = _run_and_check(ctx, arrays, np.concatenate(recs))
    say("  worst", max(r["worst"] for r in res), "plain", max(r["plain"] for r in res))


# ------------------------------------------------ paged KV caches
def _paged_case(B, Hkv, D, PS, MP, extra):
    """A pool of B*MP+extra pages (NaN-filled, so a read of an unmapped page
    shows) and a block table giving every batch row its own random pages."""
    NP = B * MP + extra
    pool_k = bf16(RNG.standard_normal(NP * Hkv * PS * D))
    pool_v = bf16(RNG.standard_normal(NP * Hkv * PS * D))
    table = RNG.permutation(NP)[:B * MP].astype(np.int32)
    unmapped = np.setdiff1d(np.arange(NP), table)
    for p in (pool_k, pool_v):
        p.reshape(NP, -1)[unmapped] = 0x7FC0  # bf16 NaN
    return pool_k, pool_v, table, NP


@pytest.mark.parametrize("out_dt", [W.F32, W.BF16])
@pytest.mark.parametrize("masked", [False, True])
def test_sdpa_paged(ctx, out_dt, masked):
    say(f"sdpa paged out={out_dt} masked={masked}")
    recs, arrays = [], []
    for B, H, Hkv, D, PS, MP, lens in [(2, 8, 8, 128, 64, 8, [512, 17]), (1, 32, 8, 128, 1024, 4, [4096]),
                                       (3, 4, 1, 64, 256, 3, [1, 256, 700]),
                                       (8, 32, 8, 128, 128, 4, list(RNG.integers(1, 513, 8))),
                                       (4, 16, 16, 128, 64, 40, [2560, 65, 1000, 63])]:
        pk, pv, table, NP = _paged_case(B, Hkv, D, PS, MP, extra=3)
        q = bf16(RNG.standard_normal(B * H * D))
        o = np.zeros(B * H * D, np.float32 if out_dt == W.F32 else np.uint16)
        base = len(arrays)
        arrays += [q, pk, pv, o, table]
        roles = dict(a=base, aux0=base + 1, aux1=base + 2, out=base + 3, b=base + 4)
        fl = W.FLAG_KV_PAGED
        if masked:
            mask = np.where(RNG.random(B * MP * PS) < 0.25, -np.inf, RNG.standard_normal(B * MP * PS))
            mask.reshape(B, -1)[:, 0] = 0.0  # every row keeps a key
            arrays.append(mask.astype(np.float32))
            roles["aux2"] = base + 5
            fl |= W.FLAG_SDPA_MASK
        recs.append(rec(W.OP_SDPA, dtype=W.BF16, out_dtype=out_dt, size=W.paged_size(B, MP, NP),
                        dim=(H, D, PS, Hkv), lens=lens, flags=fl, **roles))
    res = _run_and_check(ctx, arrays, np.concatenate(recs))
    say("  worst", max(r["worst"] for r in res))


def test_kv_append_paged(ctx):
    say("kv append paged")
    recs, arrays = [], []
    for B, H, D, PS, MP, lens in [(2, 8, 128, 64, 8, [512, 1]), (8, 8, 128, 128, 4, list(RNG.integers(1, 513, 8))),
                                  (3, 4, 64, 1024, 2, [1024, 1025, 2048]), (1, 2, 36, 64, 3, [100])]:
        pk, pv, table, NP = _paged_case(B, H, D, PS, MP, extra=2)
        k, v = bf16(RNG.standard_normal(B * H * D)), bf16(RNG.standard_normal(B * H * D))
        base = len(arrays)
        arrays += [k, v, pk, pv, table]
        recs.append(rec(W.OP_KV_APPEND, dtype=W.BF16, size=W.paged_size(B, MP, NP), dim=(H, D, PS), lens=lens,
                        flags=W.FLAG_KV_PAGED, a=base, b=base + 1, aux0=base + 2, aux1=base + 3, aux2=base + 4))
    _run_and_check(ctx, arrays, np.concatenate(recs))


def test_paged_decode_stream_verify(ctx):
    """A short decode stream on paged caches (64-position pages placed at
    random per row), in verify mode: RoPE, append through the table and
    attention over the pages, against the oracle step by step; the final
    pools bit for bit.  It runs on this module's context: a second context
    would launch a second resident executor, which cannot be placed while
    the first holds the CUs."""
    from gpu_harness import verify_stream
    s = W.make_decode(steps=3, layers=2, capacity=512, l_min=100, n_triples=8, n_out=8, page_size=64)
    say(f"paged decode verify, {len(s)} descriptors")
    res = verify_stream([b.host_bytes() for b in s.buffers], s.recs, bursts=s.bursts, ctx=ctx)
    assert not res["fails"], res["fails"][:3]
    assert res["kv_ok"]


def test_sdpa_paged_entries_outside_the_pool(ctx):
    """Block-table entries outside the pool (too large, negative) drop that
    page's keys, in units that span several pages and in units within one."""
    say("sdpa paged, entries outside the pool")
    recs, arrays = [], []
    for B, H, Hkv, D, PS, MP, lens in [(2, 8, 8, 128, 64, 40, [2560, 700]), (3, 16, 4, 128, 256, 8, [2048, 1500, 300]),
                                       (1, 4, 4, 64, 1024, 2, [2000])]:
        pk, pv, table, NP = _paged_case(B, Hkv, D, PS, MP, extra=1)
        t = table.reshape(B, MP).copy()
        t[0, 1] = NP + 5          # one page of row 0 outside the pool
        if B > 1:
            t[1, 0] = -3          # the first page of row 1
        q = bf16(RNG.standard_normal(B * H * D))
        o = np.zeros(B * H * D, np.float32)
        base = len(arrays)
        arrays += [q, pk, pv, o, t.reshape(-1).astype(np.int32)]
        recs.append(rec(W.OP_SDPA, dtype=W.BF16, out_dtype=W.F32, size=W.paged_size(B, MP, NP), dim=(H, D, PS, Hkv),
                        lens=lens, flags=W.FLAG_KV_PAGED, a=base, aux0=base + 1, aux1=base + 2, out=base + 3,
                        b=base + 4))
    res = _run_and_check(ctx, arrays, np.concatenate(recs))
    say("  worst", max(r["worst"] for r in res))
