"""Pins of the CPU oracle to facts outside itself.

Each test checks an oracle function against a closed form, an invariant, a
brute-force computation or an independent library routine (numpy / torch in
float64), chosen so that a dropped term, a wrong sign or index or a
transposed operand in the oracle fails at least one of them.  None of these
tests touches the GPU.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle_util import bf16, bf16_val, f32_bits, rec, run

RNG = np.random.default_rng(12345)


# ---------------------------------------------------------------------------
# bf16 rounding (round to nearest, ties to even) -- pinned to torch's own
# fp32 -> bf16 conversion on fp32-representable inputs, over every exponent.
# ---------------------------------------------------------------------------
def test_bf16_round_matches_torch_on_fp32_values():
    bits = RNG.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32)
    # add exact ties and neighbours of ties for many exponents
    hi = (RNG.integers(0, 2 ** 16, 20_000, dtype=np.uint64).astype(np.uint32) << 16)
    bits = np.concatenate([bits, hi | 0x8000, hi | 0x7FFF, hi | 0x8001, hi])
    vals = bits.view(np.float32)
    vals = vals[~np.isnan(vals)]
    ref = bf16(vals)
    got = np.array([oracle.round_bf16(float(v)) for v in vals[:60_000]], np.uint16)
    assert np.array_equal(got, ref[:60_000])


def test_bf16_round_special_cases():
    assert oracle.round_bf16(0.0) == 0x0000
    assert oracle.round_bf16(-0.0) == 0x8000
    assert oracle.round_bf16(float("inf")) == 0x7F80
    assert oracle.round_bf16(float("-inf")) == 0xFF80
    assert (oracle.round_bf16(float("nan")) & 0x7FC0) == 0x7FC0
    # 1 + 2^-8 is exactly half way between 1 and 1 + 2^-7: ties to even -> 1
    assert oracle.round_bf16(1.0 + 2 ** -8) == 0x3F80
    # 1 + 3*2^-8 is half way between 1+2^-7 (odd) and 1+2^-6 (even) -> up
    assert oracle.round_bf16(1.0 + 3 * 2 ** -8) == 0x3F82
    # just above a tie rounds up (a double that fp32 could not hold)
    assert oracle.round_bf16(1.0 + 2 ** -8 + 2 ** -40) == 0x3F81
    # largest finite bf16 and the overflow threshold
    maxf = (2 - 2 ** -7) * 2.0 ** 127
    assert oracle.round_bf16(maxf) == 0x7F7F
    assert oracle.round_bf16((2 - 2 ** -8) * 2.0 ** 127) == 0x7F80
    # smallest subnormal 2^-133, and half of it rounds to zero (even)
    assert oracle.round_bf16(2.0 ** -133) == 0x0001
    assert oracle.round_bf16(2.0 ** -134) == 0x0000
    assert oracle.round_bf16(3 * 2.0 ** -134) == 0x0002


def test_bf16_decode_is_exact_widening():
    h = np.arange(0, 65536, 97, dtype=np.uint16)
    got = np.array([oracle.bf16_to_float(int(x)) for x in h])
    ref = bf16_val(h).astype(np.float64)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


# ---------------------------------------------------------------------------
# add / mul: bit-exact IEEE results
# ---------------------------------------------------------------------------
def _specials_f32():
    return np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45,
                     1.1754942e-38, 3.4028235e38, -3.4028235e38, 0.5, 2.0], np.float32)


@pytest.mark.parametrize("op", [W.OP_ADD, W.OP_MUL])
def test_f32_binary_matches_numpy(op):
    n = 4096
    a = RNG.standard_normal(n).astype(np.float32) * np.float32(2.0) ** RNG.integers(-140, 120, n)
    b = RNG.standard_normal(n).astype(np.float32) * np.float32(2.0) ** RNG.integers(-140, 120, n)
    sp = _specials_f32()
    a[:len(sp) ** 2] = np.repeat(sp, len(sp))
    b[:len(sp) ** 2] = np.tile(sp, len(sp))
    a, b = a.astype(np.float32), b.astype(np.float32)
    o = np.zeros(n, np.float32)
    _, _, out = run(rec(op, size=n, a=0, b=1, out=2), [a, b, o])
    with np.errstate(all="ignore"):
        ref = a + b if op == W.OP_ADD else a * b
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(out), nan)
    assert np.array_equal(f32_bits(out)[~nan], f32_bits(ref)[~nan])


def test_f32_identities():
    x = RNG.standard_normal(1000).astype(np.float32)
    z, one, m1 = np.zeros_like(x), np.ones_like(x), -np.ones_like(x)
    o = np.zeros_like(x)
    r = run([rec(W.OP_ADD, size=1000, a=0, b=1, out=4)], [x, z, one, m1, o])[4]
    assert np.array_equal(f32_bits(r), f32_bits(x))
    r = run([rec(W.OP_MUL, size=1000, a=0, b=2, out=4)], [x, z, one, m1, o])[4]
    assert np.array_equal(f32_bits(r), f32_bits(x))
    r = run([rec(W.OP_MUL, size=1000, a=0, b=3, out=4)], [x, z, one, m1, o])[4]
    assert np.array_equal(f32_bits(r), f32_bits(-x))
    y = RNG.standard_normal(1000).astype(np.float32)
    r1 = run([rec(W.OP_ADD, size=1000, a=0, b=1, out=2)], [x, y, o])[2]
    r2 = run([rec(W.OP_ADD, size=1000, a=1, b=0, out=2)], [x, y, o])[2]
    assert np.array_equal(f32_bits(r1), f32_bits(r2))


@pytest.mark.parametrize("op", [W.OP_ADD, W.OP_MUL])
def test_bf16_binary_matches_torch_bf16(op):
    """Every bf16 value against 512 random bf16 partners: torch computes the
    bf16 op in fp32 and rounds once to bf16; since fp32 holds 2*8+2 bits this
    is the correctly rounded result, the same definition the oracle follows."""
    allv = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    partners = RNG.integers(0, 65536, 512).astype(np.uint16)
    a = np.repeat(allv, len(partners))
    b = np.tile(partners, len(allv))
    o = np.zeros_like(a)
    _, _, out = run(rec(op, dtype=W.BF16, size=len(a), a=0, b=1, out=2), [a, b, o])
    ta = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    tb = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
    ref = (ta + tb if op == W.OP_ADD else ta * tb).view(torch.int16).numpy().view(np.uint16)
    nan_ref = (ref & 0x7F80) == 0x7F80
    nan_ref &= (ref & 0x007F) != 0
    nan_out = ((out & 0x7F80) == 0x7F80) & ((out & 0x007F) != 0)
    assert np.array_equal(nan_ref, nan_out)
    assert np.array_equal(out[~nan_ref], ref[~nan_ref])


# ---------------------------------------------------------------------------
# ReLU
# ---------------------------------------------------------------------------
def test_relu_identities_and_specials():
    x = np.concatenate([RNG.standard_normal(2000), _specials_f32()]).astype(np.float32)
    n = len(x)
    o = np.zeros(n, np.float32)
    r = run(rec(W.OP_RELU, size=n, a=0, out=1), [x, o])[1]
    rr = run(rec(W.OP_RELU, size=n, a=0, out=1), [r, o])[1]
    assert np.array_equal(f32_bits(rr), f32_bits(r))           # idempotent
    rn = run(rec(W.OP_RELU, size=n, a=0, out=1), [-x, o])[1]
    fin = np.isfinite(x)
    assert np.array_equal((r - rn)[fin], x[fin])                  # relu(x)-relu(-x) = x
    assert f32_bits(r[x == 0]).max() == 0                          # +0 for both zeros
    assert np.isnan(r[np.isnan(x)]).all()
    assert np.all(r[x > 0] == x[x > 0])


# ---------------------------------------------------------------------------
# GELU (tanh approximation)
# ---------------------------------------------------------------------------
def _gelu_decimal(x: float) -> float:
    """tanh-approximation GELU from its literal definition, 0.5 x (1 + tanh(u))
    with tanh(u) = (e^{2u} - 1) / (e^{2u} + 1), in Python's decimal module with
    enough digits that the cancellation in 1 + tanh(u) for u << 0 leaves 50
    significant digits."""
    from decimal import Decimal, getcontext
    pi = Decimal("3.14159265358979323846264338327950288419716939937510582097494459230781640628620899")
    getcontext().prec = 80
    X = Decimal(x)
    u = (Decimal(2) / pi).sqrt() * (X + Decimal("0.044715") * X * X * X)
    lost = int(abs(float(u)) * 2 * 0.4343) + 10 if u < 0 else 0
    getcontext().prec = 80 + lost
    u = (Decimal(2) / pi).sqrt() * (X + Decimal("0.044715") * X * X * X)
    e2 = (2 * u).exp()
    th = (e2 - 1) / (e2 + 1)
    return float(Decimal("0.5") * X * (1 + th))


def test_gelu_matches_high_precision_reference():
    """Relative accuracy over the whole range, including x << 0 where the
    literal 1 + tanh(u) would cancel."""
    xs = list(np.linspace(-12, 12, 481)) + list(RNG.standard_normal(300) * 4) + [-30.0, -20.5, 1e-30, -1e-30]
    worst = 0.0
    for x in xs:
        ref = _gelu_decimal(float(x))
        got = oracle.gelu(float(x))
        if ref == 0.0:
            assert got == 0.0
            continue
        worst = max(worst, abs(got - ref) / abs(ref))
    assert worst < 1e-13, worst


def test_gelu_matches_torch_tanh_gelu_where_no_cancellation():
    x = np.concatenate([np.linspace(-2, 12, 2001), RNG.standard_normal(2000)])
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    got = np.array([oracle.gelu(v) for v in x])
    assert np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-300)) < 1e-12


def test_gelu_odd_identity_and_limits():
    for x in list(np.linspace(-8, 8, 321)) + [1e-6, 0.3, 17.0]:
        assert abs(oracle.gelu(x) - oracle.gelu(-x) - x) <= 1e-15 * max(1.0, abs(x))
    assert oracle.gelu(0.0) == 0.0
    assert abs(oracle.gelu(30.0) - 30.0) < 1e-12
    assert abs(oracle.gelu(-30.0)) < 1e-12
    # the sigmoid form x / (1 + exp(-2u)) is algebraically identical
    for x in np.linspace(-6, 6, 121):
        u = math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)
        assert abs(oracle.gelu(x) - x / (1 + math.exp(-2 * u))) <= 1e-15 * max(1.0, abs(x))


def test_gelu_record_rounds_once():
    x = RNG.standard_normal(3000).astype(np.float32)
    o = np.zeros_like(x)
    r = run(rec(W.OP_GELU, size=len(x), a=0, out=1), [x, o])[1]
    ref = torch.nn.functional.gelu(torch.from_numpy(x.astype(np.float64)), approximate="tanh")
    ref32 = ref.numpy().astype(np.float32)
    assert np.max(np.abs(r.astype(np.float64) - ref32.astype(np.float64))
                  / np.maximum(np.abs(ref32), 1e-30)) <= 2 ** -23


# ---------------------------------------------------------------------------
# sum / max / min along the last dimension
# ---------------------------------------------------------------------------
def test_sum_exact_on_integers_and_constants():
    rows, h = 8, 1024
    x = RNG.integers(-1000, 1000, (rows, h)).astype(np.float32)
    o = np.zeros(rows, np.float32)
    r = run(rec(W.OP_SUM, size=rows, dim=(h,), a=0, out=1), [x, o])[1]
    assert np.array_equal(r, x.sum(axis=1, dtype=np.int64).astype(np.float32))
    c = np.full((4, 4096), 0.75, np.float32)
    r = run(rec(W.OP_SUM, size=4, dim=(4096,), a=0, out=1), [c, np.zeros(4, np.float32)])[1]
    assert np.all(r == 3072.0)


def test_max_min_match_numpy_and_order_zeros():
    rows, h = 16, 768
    x = RNG.standard_normal((rows, h)).astype(np.float32) * 2
    o = np.zeros(rows, np.float32)
    mx = run(rec(W.OP_MAX, size=rows, dim=(h,), a=0, out=1), [x, o])[1]
    mn = run(rec(W.OP_MIN, size=rows, dim=(h,), a=0, out=1), [x, o])[1]
    assert np.array_equal(mx, x.max(axis=1)) and np.array_equal(mn, x.min(axis=1))
    z = np.array([[0.0, -0.0, -0.0], [-0.0, 0.0, -0.0], [-1.0, np.nan, 5.0]], np.float32)
    o = np.zeros(3, np.float32)
    mx = run(rec(W.OP_MAX, size=3, dim=(3,), a=0, out=1), [z, o])[1]
    mn = run(rec(W.OP_MIN, size=3, dim=(3,), a=0, out=1), [z, o])[1]
    assert f32_bits(mx[:2]).tolist() == [0, 0]                   # +0 is the max
    assert f32_bits(mn[:2]).tolist() == [0x80000000] * 2          # -0 is the min
    assert np.isnan(mx[2]) and np.isnan(mn[2])
    assert oracle.max2(1.0, float("nan")) != oracle.max2(1.0, float("nan"))


# ---------------------------------------------------------------------------
# softmax
# ---------------------------------------------------------------------------
def test_softmax_against_torch_and_closed_forms():
    rows, h = 4, 2048
    x = (RNG.standard_normal((rows, h)) * 2).astype(np.float32)
    o = np.zeros_like(x)
    y = run(rec(W.OP_SOFTMAX, size=rows, dim=(h,), a=0, out=1), [x, o])[1]
    ref = torch.softmax(torch.from_numpy(x.astype(np.float64)), dim=1).numpy()
    assert np.max(np.abs(y - ref) / ref) <= 2 ** -24 * 1.01
    assert np.all(np.abs(y.astype(np.float64).sum(axis=1) - 1) <= h * 2 ** -24)
    y2 = run(rec(W.OP_SOFTMAX, size=rows, dim=(h,), a=0, out=1), [x + np.float32(3.0), o])[1]
    assert np.max(np.abs(y2 - y) / y) < 1e-6                         # shift invariance
    for n in (1024, 2048, 4096):
        c = np.full((1, n), -0.3, np.float32)
        yc = run(rec(W.OP_SOFTMAX, size=1, dim=(n,), a=0, out=1), [c, np.zeros_like(c)])[1]
        assert np.all(yc == np.float32(1.0 / n))


# ---------------------------------------------------------------------------
# LayerNorm
# ---------------------------------------------------------------------------
def test_layernorm_closed_form_and_torch():
    rows, h, eps = 3, 1024, np.float32(1e-5)
    x = (RNG.standard_normal((rows, h)) * 2 + 0.5).astype(np.float32)
    g1, b0 = np.ones(h, np.float32), np.zeros(h, np.float32)
    o = np.zeros_like(x)
    y = run(rec(W.OP_LAYERNORM, size=rows, dim=(h,), fparam=(eps,), a=0, out=3, aux0=1, aux1=2),
            [x, g1, b0, o])[3].astype(np.float64)
    xd = x.astype(np.float64)
    var = xd.var(axis=1)
    assert np.all(np.abs(y.mean(axis=1)) < 1e-6)
    assert np.allclose(y.var(axis=1), var / (var + float(eps)), rtol=1e-6)
    g = (1 + 0.1 * RNG.standard_normal(h)).astype(np.float32)
    b = (0.1 * RNG.standard_normal(h)).astype(np.float32)
    y = run(rec(W.OP_LAYERNORM, size=rows, dim=(h,), fparam=(eps,), a=0, out=3, aux0=1, aux1=2),
            [x, g, b, o])[3]
    ref = torch.nn.functional.layer_norm(torch.from_numpy(xd), (h,), torch.from_numpy(g.astype(np.float64)),
                                         torch.from_numpy(b.astype(np.float64)), eps=float(eps)).numpy()
    assert np.max(np.abs(y - ref) / np.maximum(np.abs(ref), 1)) < 2 ** -23


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------
def _rope_complex(x, pos, theta, half=False):
    """Independent formulation: pairs as complex numbers times e^{i angle}."""
    B, H, D = x.shape
    i = np.arange(D // 2)
    freq = np.power(theta, -2.0 * i / D)
    if half:
        z = x[..., : D // 2] + 1j * x[..., D // 2:]
    else:
        z = x[..., 0::2] + 1j * x[..., 1::2]
    rot = z * np.exp(1j * pos[:, None, None] * freq[None, None, :])
    out = np.empty_like(x)
    if half:
        out[..., : D // 2], out[..., D // 2:] = rot.real, rot.imag
    else:
        out[..., 0::2], out[..., 1::2] = rot.real, rot.imag
    return out


@pytest.mark.parametrize("half", [False, True])
def test_rope_matches_complex_rotation_f32(half):
    B, H, D = 3, 4, 128
    q = RNG.standard_normal((B, H, D)).astype(np.float32)
    k = RNG.standard_normal((B, H, D)).astype(np.float32)
    lens = [1, 77, 4096]
    out = run(rec(W.OP_ROPE, size=B, dim=(H, D), fparam=(10000.0,), lens=lens,
                  flags=W.FLAG_ROPE_HALF if half else 0, a=0, b=1), [q, k])
    pos = np.array(lens, np.float64) - 1
    for got, x in zip(out, (q, k)):
        ref = _rope_complex(x.astype(np.float64), pos, 10000.0, half)
        assert np.max(np.abs(got - ref)) <= 2 ** -23 * np.max(np.abs(ref)) + 1e-12
        # position 0 (L = 1) is the identity, bit-exact
        assert np.array_equal(f32_bits(got[0]), f32_bits(x[0]))


def test_rope_relative_position_and_norm():
    H, D = 2, 128
    q = RNG.standard_normal((1, H, D))
    k = RNG.standard_normal((1, H, D))

    def rot(x, L):
        xx = x.astype(np.float32)
        out = run(rec(W.OP_ROPE, size=1, dim=(H, D), fparam=(10000.0,), lens=[L], a=0, b=1), [xx, xx.copy()])
        return out[0].astype(np.float64)
    for (m, n, t) in [(5, 9, 11), (100, 3, 40)]:
        d1 = np.sum(rot(q, m + 1) * rot(k, n + 1))
        d2 = np.sum(rot(q, m + t + 1) * rot(k, n + t + 1))
        assert abs(d1 - d2) < 1e-4
    r = rot(q, 300)
    qq = q.astype(np.float32).astype(np.float64)
    n0 = qq[..., 0::2] ** 2 + qq[..., 1::2] ** 2
    n1 = r[..., 0::2] ** 2 + r[..., 1::2] ** 2
    assert np.allclose(n0, n1, rtol=1e-6)


def test_rope_bf16_is_single_rounding_of_double():
    B, H, D = 2, 3, 128
    q = bf16(RNG.standard_normal((B, H, D)))
    k = bf16(RNG.standard_normal((B, H, D)))
    lens = [10, 3000]
    oq, ok = run(rec(W.OP_ROPE, dtype=W.BF16, size=B, dim=(H, D), fparam=(10000.0,), lens=lens, a=0, b=1),
                 [q, k])
    pos = np.array(lens, np.float64) - 1
    for got, x in ((oq, q), (ok, k)):
        ref = _rope_complex(bf16_val(x).astype(np.float64), pos, 10000.0)
        expect = np.array([oracle.round_bf16(v) for v in ref.reshape(-1)], np.uint16).reshape(ref.shape)
        # complex-exponential vs cos/sin evaluation differ by ~1e-16; a bf16
        # tie flip is possible only at exact midpoints
        mism = np.sum(got != expect)
        assert mism <= 2


# ---------------------------------------------------------------------------
# KV append
# ---------------------------------------------------------------------------
def test_kv_append_is_bit_copy_and_touches_one_row():
    B, H, D, C = 2, 3, 8, 16
    k = bf16(RNG.standard_normal((B, H, D)))
    v = bf16(RNG.standard_normal((B, H, D)))
    K0 = bf16(RNG.standard_normal((B, H, C, D)))
    V0 = bf16(RNG.standard_normal((B, H, C, D)))
    lens = [5, 16]
    _, _, K, V = run(rec(W.OP_KV_APPEND, dtype=W.BF16, size=B, dim=(H, D, C), lens=lens,
                         a=0, b=1, aux0=2, aux1=3), [k, v, K0, V0])
    for b, L in enumerate(lens):
        assert np.array_equal(K[b, :, L - 1], k[b]) and np.array_equal(V[b, :, L - 1], v[b])
        mask = np.ones(C, bool)
        mask[L - 1] = False
        assert np.array_equal(K[b][:, mask], K0[b][:, mask])
        assert np.array_equal(V[b][:, mask], V0[b][:, mask])


# ---------------------------------------------------------------------------
# decode SDPA
# ---------------------------------------------------------------------------
def _sdpa_torch(q, K, V, lens):
    B, H, D = q.shape
    out = np.zeros((B, H, D))
    for b, L in enumerate(lens):
        qq = torch.from_numpy(q[b][:, None, :])
        kk = torch.from_numpy(K[b][:, :L, :])
        vv = torch.from_numpy(V[b][:, :L, :])
        out[b] = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[:, 0, :].numpy()
    return out


def test_sdpa_matches_torch_brute_force():
    for (B, H, D, C) in [(1, 1, 4, 8), (2, 3, 8, 8), (3, 2, 128, 64)]:
        q = bf16(RNG.standard_normal((B, H, D)))
        K = bf16(RNG.standard_normal((B, H, C, D)))
        V = bf16(RNG.standard_normal((B, H, C, D)))
        lens = list(RNG.integers(1, C + 1, B))
        o = np.zeros((B, H, D), np.float32)
        got = run(rec(W.OP_SDPA, dtype=W.BF16, out_dtype=W.F32, size=B, dim=(H, D, C), lens=lens,
                      a=0, aux0=1, aux1=2, out=3), [q, K, V, o])[3]
        ref = _sdpa_torch(*(bf16_val(t).astype(np.float64) for t in (q, K, V)), lens)
        assert np.max(np.abs(got - ref)) <= 2 ** -23 * np.max(np.abs(ref)) + 1e-12


def test_sdpa_special_cases():
    B, H, D, C = 1, 2, 16, 32
    q = bf16(RNG.standard_normal((B, H, D)))
    K = bf16(RNG.standard_normal((B, H, C, D)))
    V = bf16(RNG.standard_normal((B, H, C, D)))
    o = np.zeros((B, H, D), np.float32)

    def sdpa(qq, KK, VV, L):
        return run(rec(W.OP_SDPA, dtype=W.BF16, out_dtype=W.F32, size=B, dim=(H, D, C), lens=[L],
                       a=0, aux0=1, aux1=2, out=3), [qq, KK, VV, o])[3]
    # L = 1: o = V_0
    assert np.array_equal(sdpa(q, K, V, 1), bf16_val(V[:, :, 0, :]))
    # q = 0: uniform weights -> mean of V over [0, L)
    L = 20
    got = sdpa(np.zeros_like(q), K, V, L)
    ref = bf16_val(V[:, :, :L, :]).astype(np.float64).mean(axis=2)
    assert np.max(np.abs(got - ref)) < 1e-6
    # identical keys: mean of V as well
    Ks = np.repeat(K[:, :, :1, :], C, axis=2)
    got = sdpa(q, Ks, V, L)
    assert np.max(np.abs(got - ref)) < 1e-6
    # permuting keys together with their values changes nothing
    perm = np.concatenate([RNG.permutation(L), np.arange(L, C)])
    a = sdpa(q, K, V, L)
    b = sdpa(q, K[:, :, perm, :], V[:, :, perm, :], L)
    assert np.max(np.abs(a - b)) < 1e-6


# ---------------------------------------------------------------------------
# GEMV
# ---------------------------------------------------------------------------
def test_gemv_exact_on_small_integers_and_against_numpy():
    K, N = 64, 48
    x = RNG.integers(-4, 5, K).astype(np.float32)
    Wm = RNG.integers(-4, 5, (K, N)).astype(np.float32)
    y = run(rec(W.OP_GEMV, dim=(K, N), a=0, b=1, out=2), [x, Wm, np.zeros(N, np.float32)])[2]
    assert np.array_equal(y, (x.astype(np.int64) @ Wm.astype(np.int64)).astype(np.float32))
    K, N = 1024, 96
    x = bf16(RNG.standard_normal(K))
    Wb = bf16(RNG.standard_normal((K, N)) * 0.02)
    y = run(rec(W.OP_GEMV, dtype=W.BF16, dim=(K, N), a=0, b=1, out=2), [x, Wb, np.zeros(N, np.uint16)])[2]
    ref = bf16_val(x).astype(np.float64) @ bf16_val(Wb).astype(np.float64)
    expect = np.array([oracle.round_bf16(v) for v in ref], np.uint16)
    assert np.sum(y != expect) == 0
    # transposed operand would fail this: a non-square W with distinct rows
    x = np.zeros(K, np.float32)
    x[3] = 1
    Wm = RNG.standard_normal((K, N)).astype(np.float32)
    y = run(rec(W.OP_GEMV, dim=(K, N), a=0, b=1, out=2), [x, Wm, np.zeros(N, np.float32)])[2]
    assert np.array_equal(y, Wm[3])


# ---------------------------------------------------------------------------
# copy, errors, stream semantics
# ---------------------------------------------------------------------------
def test_copy_and_bounds_errors():
    a = RNG.integers(0, 255, 1000).astype(np.uint8)
    o = np.zeros(1000, np.uint8)
    r = run(rec(W.OP_COPY, size=1000, a=0, out=1), [a, o])[1]
    assert np.array_equal(r, a)
    with pytest.raises(oracle.OracleError):
        run(rec(W.OP_COPY, size=1001, a=0, out=1), [a, o])
    with pytest.raises(oracle.OracleError):
        run(rec(99, size=1, a=0, out=1), [a, o])


def test_stream_is_sequential_with_aliasing():
    """A stream equals running its records one after another: y = (x + x) * x
    written in place, then relu, matches the hand-computed composition."""
    x = RNG.standard_normal(500).astype(np.float32)
    recs = [rec(W.OP_ADD, size=500, a=0, b=0, out=0),
            rec(W.OP_MUL, size=500, a=0, b=1, out=0),
            rec(W.OP_RELU, size=500, a=0, out=0)]
    y = run(recs, [x, x.copy()])[0]
    ref = np.maximum((x + x) * x, np.float32(0))
    ref[ref == 0] = 0.0
    assert np.array_equal(f32_bits(y), f32_bits(ref))


def test_pr1_prefix_matches_numpy_replay():
    """PR1 (add/mul/relu only) replayed independently with numpy fp32."""
    s = W.make_pr1()
    pool = oracle.Pool.from_stream(s)
    pool.run(s.recs)
    vals = [b.host_values().copy() for b in s.buffers]
    with np.errstate(all="ignore"):
        for r in s.recs:
            a = vals[r["buf"][W.A]]
            if r["op"] == W.OP_RELU:
                out = np.where(np.isnan(a), a, np.where(a > 0, a, np.float32(0)))
            else:
                b = vals[r["buf"][W.B]]
                out = a + b if r["op"] == W.OP_ADD else a * b
            vals[r["buf"][W.OUT]] = out.astype(np.float32)
    for i, v in enumerate(vals):
        got = pool.view(i, np.float32)
        nan = np.isnan(v)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(f32_bits(got)[~nan], f32_bits(v)[~nan])


# ------------------------------------------------ injected element-wise programs
P = W.program
X = W.xins


def _eval_vec(prog, a, b):
    return np.array([oracle.expr_eval(prog, float(x), float(y)) for x, y in zip(a, b)], np.float32)


def test_expr_exact_steps_equal_ieee_binary32():
    rng = np.random.default_rng(5)
    a = np.concatenate([rng.standard_normal(300), rng.standard_normal(100) * 1e-39, [0.0, -0.0, 1e38, -1e38]])
    a = a.astype(np.float32)
    b = np.concatenate([rng.standard_normal(300), rng.standard_normal(100) * 1e-39, [-0.0, 0.0, 1e38, 3e38]])
    b = b.astype(np.float32)
    lda_ldb = [X(W.X_LDA, 1), X(W.X_LDB, 2)]
    with np.errstate(all="ignore"):
        cases = [(W.X_ADD, a + b), (W.X_SUB, a - b), (W.X_MUL, a * b), (W.X_DIV, a / b)]
        for op, ref in cases:
            got = _eval_vec(P(lda_ldb + [X(op, 0, 1, 2)]), a, b)
            assert np.array_equal(f32_bits(got), f32_bits(ref)), op
        got = _eval_vec(P([X(W.X_LDA, 1), X(W.X_ABS, 1, 1), X(W.X_SQRT, 0, 1)]), a, b)
        assert np.array_equal(f32_bits(got), f32_bits(np.sqrt(np.abs(a))))
    got = _eval_vec(P([X(W.X_LDA, 1), X(W.X_NEG, 0, 1)]), a, b)
    assert np.array_equal(f32_bits(got), f32_bits(-a))


def test_expr_min_max_relu_match_the_op_definitions():
    v = np.array([1.0, -2.0, np.nan, 0.0, -0.0, np.inf, -np.inf, 3.5], np.float32)
    for x in v:
        for y in v:
            mx = oracle.expr_eval(P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_MAX, 0, 1, 2)]), float(x), float(y))
            mn = oracle.expr_eval(P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_MIN, 0, 1, 2)]), float(x), float(y))
            rmx, rmn = oracle.max2(float(x), float(y)), oracle.min2(float(x), float(y))
            assert (math.isnan(mx) and math.isnan(rmx)) or f32_bits(np.float32(mx)) == f32_bits(np.float32(rmx))
            assert (math.isnan(mn) and math.isnan(rmn)) or f32_bits(np.float32(mn)) == f32_bits(np.float32(rmn))
        r = oracle.expr_eval(P([X(W.X_LDA, 1), X(W.X_RELU, 0, 1)]), float(x), 0.0)
        rr = oracle.relu(float(x))
        assert (math.isnan(r) and math.isnan(rr)) or f32_bits(np.float32(r)) == f32_bits(np.float32(rr))


def test_expr_transcendentals_are_rounded_double_functions():
    x = np.linspace(-6, 6, 241).astype(np.float32)
    pos = np.abs(x) + np.float32(1e-3)
    for op, fn, arg in [(W.X_EXP, np.exp, x), (W.X_TANH, np.tanh, x), (W.X_LOG, np.log, pos),
                        (W.X_SIGMOID, lambda t: 1.0 / (1.0 + np.exp(-t)), x)]:
        got = _eval_vec(P([X(W.X_LDA, 1), X(op, 0, 1)]), arg, arg)
        ref = fn(arg.astype(np.float64))
        ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(got - ref) <= 0.5 * ulp * 1.0001 + 1e-45), op


def test_expr_constants_registers_and_composite_gelu():
    # registers start at zero; constants come from the program's tail
    assert oracle.expr_eval(P([X(W.X_ADD, 0, 1, 2)]), 5.0, 7.0) == 0.0
    assert oracle.expr_eval(P([X(W.X_CONST, 0, 0, 0, 1)], [2.0, -3.25]), 0.0, 0.0) == -3.25
    # tanh-GELU written as a program, step by step in binary32, stays within
    # a few binary32 ulps of the double definition where nothing cancels
    k, c = math.sqrt(2 / math.pi), 0.044715
    prog = P([X(W.X_LDA, 1), X(W.X_MUL, 2, 1, 1), X(W.X_MUL, 2, 2, 1), X(W.X_CONST, 3, 0, 0, 0),
              X(W.X_MUL, 2, 2, 3), X(W.X_ADD, 2, 2, 1), X(W.X_CONST, 3, 0, 0, 1), X(W.X_MUL, 2, 2, 3),
              X(W.X_TANH, 2, 2), X(W.X_CONST, 3, 0, 0, 2), X(W.X_ADD, 2, 2, 3), X(W.X_MUL, 2, 2, 1),
              X(W.X_CONST, 3, 0, 0, 3), X(W.X_MUL, 0, 2, 3)], [c, k, 1.0, 0.5])
    x = np.linspace(-2, 3, 101).astype(np.float32)
    got = _eval_vec(prog, x, x)
    ref = np.array([oracle.gelu(float(t)) for t in x])
    assert np.all(np.abs(got - ref) <= 8 * np.spacing(np.maximum(np.abs(ref), 1e-3).astype(np.float32)))


def test_expr_malformed_programs_are_rejected():
    good = [X(W.X_LDA, 0)]
    for words in [P([X(0, 0)]), P([X(W.X_RELU + 1, 0)]), P([X(W.X_LDA, 4)]), P([X(W.X_MOV, 0, 5)]),
                  P([X(W.X_CONST, 0, 0, 0, 1)], [1.0]), P(good)[:1], np.array([0], np.uint32),
                  np.array([33], np.uint32), P(good) | np.array([1 << 16, 0], np.uint32)]:
        with pytest.raises(ValueError):
            oracle.expr_eval(words, 1.0, 2.0)


def test_expr_record_matches_builtin_ops_bit_exactly():
    """A program a+b (a*b) on bf16 rounds the binary32 result to bf16, which
    equals one rounding of the exact result (24 >= 2*8+2), so it matches the
    built-in add (mul) record bit for bit; the same holds in fp32."""
    rng = np.random.default_rng(8)
    for dt in (W.F32, W.BF16):
        n = 1000
        a = rng.standard_normal(n).astype(np.float32)
        b = (rng.standard_normal(n) * np.exp(rng.uniform(-20, 20, n))).astype(np.float32)
        if dt == W.BF16:
            a, b = bf16(a), bf16(b)
        for op, xop in ((W.OP_ADD, W.X_ADD), (W.OP_MUL, W.X_MUL)):
            prog = P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(xop, 0, 1, 2)])
            zeros = np.zeros_like(a)
            arrays = [a, b, zeros.copy(), zeros.copy(), prog]
            recs = np.concatenate([rec(op, dtype=dt, size=n, a=0, b=1, out=2),
                                   rec(W.OP_EXPR, dtype=dt, size=n, dim=(0, 0, len(prog), 70), a=0, b=1, out=3,
                                       aux2=4)])
            out = run(recs, arrays)
            assert np.array_equal(out[2].view(np.uint8), out[3].view(np.uint8)), (dt, op)


# ------------------------------------------------ grouped-query attention
def test_sdpa_grouped_kv_heads_match_repeated_heads_and_torch():
    """Hkv key/value heads shared by H/Hkv query heads each: the same as
    multi-head attention with every key/value head repeated H/Hkv times
    (checked through the oracle's own MHA path and through torch)."""
    for (B, H, Hkv, D, C) in [(2, 8, 2, 8, 12), (1, 4, 1, 16, 9), (3, 6, 3, 128, 40)]:
        G = H // Hkv
        q = bf16(RNG.standard_normal((B, H, D)))
        K = bf16(RNG.standard_normal((B, Hkv, C, D)))
        V = bf16(RNG.standard_normal((B, Hkv, C, D)))
        lens = list(RNG.integers(1, C + 1, B))
        o = np.zeros((B, H, D), np.float32)
        got = run(rec(W.OP_SDPA, dtype=W.BF16, out_dtype=W.F32, size=B, dim=(H, D, C, Hkv), lens=lens,
                      a=0, aux0=1, aux1=2, out=3), [q, K, V, o])[3]
        Kr, Vr = np.repeat(K, G, axis=1), np.repeat(V, G, axis=1)
        mha = run(rec(W.OP_SDPA, dtype=W.BF16, out_dtype=W.F32, size=B, dim=(H, D, C), lens=lens,
                      a=0, aux0=1, aux1=2, out=3), [q, Kr, Vr, o])[3]
        assert np.array_equal(got, mha)
        ref = _sdpa_torch(*(bf16_val(t).astype(np.float64) for t in (q, Kr, Vr)), lens)
        assert np.max(np.abs(got - ref.reshape(got.shape))) <= 2 ** -23 * np.max(np.abs(ref)) + 1e-12


def test_rope_with_fewer_key_heads_rotates_each_tensor_by_its_own_heads():
    B, H, Hk, D = 2, 8, 2, 16
    lens = [5, 300]
    q = (RNG.standard_normal(B * H * D)).astype(np.float32)
    k = (RNG.standard_normal(B * Hk * D)).astype(np.float32)
    both = run(rec(W.OP_ROPE, dtype=W.F32, size=B, dim=(H, D, 0, Hk), fparam=(10000.0,), lens=lens, a=0, b=1),
               [q, k])
    q_only = run(rec(W.OP_ROPE, dtype=W.F32, size=B, dim=(H, D), fparam=(10000.0,), lens=lens, a=0, b=1),
                 [q, np.zeros_like(q)])[0]
    k_only = run(rec(W.OP_ROPE, dtype=W.F32, size=B, dim=(Hk, D), fparam=(10000.0,), lens=lens, a=0, b=1),
                 [np.zeros_like(k), k])[1]
    assert np.array_equal(both[0], q_only) and np.array_equal(both[1], k_only)


# ---------------------------------------------------------------------------
# Unrounded capture (orc_run_capture): the doubles it reports are the values
# the record rounds to its output type -- they round to exactly the stored
# bytes -- and they equal an independent double evaluation of each op.  A
# window that reports the wrong element, another op's value or a rounded
# value fails one of these.
# ---------------------------------------------------------------------------
def _capture(r, arrays, role=W.OUT, es=None, nbytes=None):
    pool = oracle.Pool([np.array(a, copy=True) for a in arrays])
    b, off = int(r["buf"][0, role]), int(r["off"][0, role])
    es = es or W.DTYPE_BYTES[int(r["out_dtype"][0])]
    nbytes = nbytes or pool.arrays[b].nbytes - off
    (hp,) = pool.run_capture(r, [(b, off, nbytes, es)])
    return hp, pool.arrays[b][off: off + nbytes]


@pytest.mark.parametrize("dt", [W.F32, W.BF16])
def test_capture_rounds_to_stored_output(dt):
    n = 4099
    x = RNG.standard_normal(n).astype(np.float32) * 3
    y = RNG.standard_normal(n).astype(np.float32)
    if dt == W.BF16:
        xa, ya = bf16(x), bf16(y)
    else:
        xa, ya = x, y
    gam = (1 + 0.1 * RNG.standard_normal(1024)).astype(np.float32)
    bet = (0.1 * RNG.standard_normal(1024)).astype(np.float32)
    if dt == W.BF16:
        gam, bet = bf16(gam), bf16(bet)
    cases = [
        rec(W.OP_GELU, dtype=dt, size=n, a=0, out=2),
        rec(W.OP_ADD, dtype=dt, size=n, a=0, b=1, out=2),
        rec(W.OP_SOFTMAX, dtype=dt, size=4, dim=(1024,), a=0, out=2),
        rec(W.OP_LAYERNORM, dtype=dt, size=4, dim=(1024,), fparam=(1e-5,), a=0, aux0=3, aux1=4, out=2),
        rec(W.OP_SUM, dtype=dt, size=4, dim=(1024,), a=0, out=2),
    ]
    for r in cases:
        arrays = [xa, ya, np.zeros_like(xa), gam, bet]
        hp, stored = _capture(r, arrays)
        m = ~np.isnan(hp)
        assert m.sum() > 0
        if dt == W.F32:
            assert np.array_equal(hp[m].astype(np.float32).view(np.uint32), stored.view(np.uint32)[m])
        else:
            assert np.array_equal(np.array([oracle.round_bf16(v) for v in hp[m]], np.uint16),
                                  stored.view(np.uint16)[m])
    # the values themselves, against independent double evaluations
    xd = bf16_val(xa).astype(np.float64) if dt == W.BF16 else x.astype(np.float64)
    hp, _ = _capture(cases[0], [xa, ya, np.zeros_like(xa), gam, bet])
    for i in range(0, n, 97):
        assert abs(hp[i] - _gelu_decimal(float(xd[i]))) <= 1e-14 * max(abs(hp[i]), 1e-300) + 1e-300
    hp, _ = _capture(cases[2], [xa, ya, np.zeros_like(xa), gam, bet])
    ref = torch.softmax(torch.tensor(xd[:4096].reshape(4, 1024)), dim=1).numpy().reshape(-1)
    assert np.allclose(hp[:4096], ref, rtol=1e-13, atol=0)


def test_capture_of_sdpa_and_gemv_match_torch_in_double():
    B, H, D, C = 2, 4, 64, 40
    q = bf16(RNG.standard_normal(B * H * D))
    K, V = bf16(RNG.standard_normal(B * H * C * D)), bf16(RNG.standard_normal(B * H * C * D))
    o = np.zeros(B * H * D, np.uint16)
    r = rec(W.OP_SDPA, dtype=W.BF16, out_dtype=W.BF16, size=B, dim=(H, D, C, H), lens=[40, 7],
            a=0, aux0=1, aux1=2, out=3)
    hp, _ = _capture(r, [q, K, V, o])
    ref = _sdpa_torch(bf16_val(q).astype(np.float64).reshape(B, H, D),
                      bf16_val(K).astype(np.float64).reshape(B, H, C, D),
                      bf16_val(V).astype(np.float64).reshape(B, H, C, D), [40, 7])
    assert np.allclose(hp, ref.reshape(-1), rtol=1e-12, atol=1e-12)
    Kd, Nd = 96, 40
    x = bf16(RNG.standard_normal(Kd))
    Wm = bf16(0.02 * RNG.standard_normal(Kd * Nd))
    r = rec(W.OP_GEMV, dtype=W.BF16, out_dtype=W.BF16, dim=(Kd, Nd), a=0, b=1, out=2)
    hp, _ = _capture(r, [x, Wm, np.zeros(Nd, np.uint16)])
    ref = bf16_val(x).astype(np.float64) @ bf16_val(Wm).astype(np.float64).reshape(Kd, Nd)
    assert np.allclose(hp, ref, rtol=1e-13, atol=1e-15)


def test_capture_of_inplace_rope_reports_both_tensors():
    B, H, Hk, D = 1, 2, 1, 8
    q = bf16(RNG.standard_normal(B * H * D))
    k = bf16(RNG.standard_normal(B * Hk * D))
    r = rec(W.OP_ROPE, dtype=W.BF16, size=B, dim=(H, D, 0, Hk), fparam=(10000.0,), lens=[5], a=0, b=1)
    pool = oracle.Pool([q.copy(), k.copy()])
    hq, hk = pool.run_capture(r, [(0, 0, q.nbytes, 2), (1, 0, k.nbytes, 2)])
    assert not np.isnan(hq).any() and not np.isnan(hk).any()
    ref_q = _rope_complex(bf16_val(q).astype(np.float64).reshape(B, H, D), np.array([4.0]), 10000.0)
    ref_k = _rope_complex(bf16_val(k).astype(np.float64).reshape(B, Hk, D), np.array([4.0]), 10000.0)
    assert np.allclose(hq, ref_q.reshape(-1), rtol=1e-12, atol=1e-14)
    assert np.allclose(hk, ref_k.reshape(-1), rtol=1e-12, atol=1e-14)
    assert np.array_equal(np.array([oracle.round_bf16(v) for v in hq], np.uint16), pool.arrays[0].view(np.uint16))


# ---------------------------------------------------------------------------
# decode SDPA with an additive mask [B, C] (record flag FLAG_SDPA_MASK)
# ---------------------------------------------------------------------------
def _sdpa_masked_case(B=3, H=4, Hkv=2, D=16, C=24, lens=(24, 9, 17), seed=5):
    rng = np.random.default_rng(seed)
    q = bf16(rng.standard_normal(B * H * D))
    K = bf16(rng.standard_normal(B * Hkv * C * D))
    V = bf16(rng.standard_normal(B * Hkv * C * D))
    return q, K, V, list(lens), (B, H, Hkv, D, C)


def _run_masked(q, K, V, lens, dims, mask):
    B, H, Hkv, D, C = dims
    o = np.zeros(B * H * D, np.float32)
    r = rec(W.OP_SDPA, dtype=W.BF16, out_dtype=W.F32, size=B, dim=(H, D, C, Hkv), lens=lens,
            flags=W.FLAG_SDPA_MASK if mask is not None else 0, a=0, aux0=1, aux1=2, out=3,
            **({"aux2": 4} if mask is not None else {}))
    arrays = [q, K, V, o] + ([np.asarray(mask, np.float32)] if mask is not None else [])
    return run(r, arrays)[3].reshape(B, H, D).astype(np.float64)


def test_sdpa_zero_mask_equals_no_mask():
    q, K, V, lens, dims = _sdpa_masked_case()
    B, H, Hkv, D, C = dims
    a = _run_masked(q, K, V, lens, dims, None)
    b = _run_masked(q, K, V, lens, dims, np.zeros(B * C))
    assert np.array_equal(a, b)


def test_sdpa_minus_inf_mask_equals_attention_over_the_kept_keys():
    q, K, V, lens, dims = _sdpa_masked_case()
    B, H, Hkv, D, C = dims
    rng = np.random.default_rng(8)
    keep = rng.random((B, C)) < 0.6
    keep[:, 0] = True  # at least one key per row
    mask = np.where(keep, 0.0, -np.inf)
    got = _run_masked(q, K, V, lens, dims, mask.reshape(-1))
    qf = bf16_val(q).astype(np.float64).reshape(B, H, D)
    Kf = bf16_val(K).astype(np.float64).reshape(B, Hkv, C, D)
    Vf = bf16_val(V).astype(np.float64).reshape(B, Hkv, C, D)
    for b in range(B):
        idx = [j for j in range(lens[b]) if keep[b, j]]
        Kk = np.repeat(Kf[b][:, idx], H // Hkv, axis=0)[None]
        Vk = np.repeat(Vf[b][:, idx], H // Hkv, axis=0)[None]
        ref = _sdpa_torch(qf[b][None], Kk, Vk, [len(idx)])[0]
        assert np.allclose(got[b], ref, rtol=1e-5, atol=1e-6), b


def test_sdpa_mask_shift_invariance_and_torch_attn_mask():
    import torch
    q, K, V, lens, dims = _sdpa_masked_case(seed=9)
    B, H, Hkv, D, C = dims
    rng = np.random.default_rng(10)
    mask = (rng.standard_normal((B, C)) * 3).astype(np.float32)
    got = _run_masked(q, K, V, lens, dims, mask.reshape(-1))
    shifted = _run_masked(q, K, V, lens, dims, (mask + np.float32(4.0)).reshape(-1))
    assert np.allclose(got, shifted, rtol=1e-5, atol=1e-6)
    qf = torch.tensor(bf16_val(q).astype(np.float64).reshape(B, H, 1, D))
    Kf = torch.tensor(np.repeat(bf16_val(K).astype(np.float64).reshape(B, Hkv, C, D), H // Hkv, axis=1))
    Vf = torch.tensor(np.repeat(bf16_val(V).astype(np.float64).reshape(B, Hkv, C, D), H // Hkv, axis=1))
    for b in range(B):
        L = lens[b]
        am = torch.tensor(mask[b, :L].astype(np.float64)).reshape(1, 1, 1, L)
        ref = torch.nn.functional.scaled_dot_product_attention(qf[b:b + 1], Kf[b:b + 1, :, :L], Vf[b:b + 1, :, :L],
                                                                attn_mask=am)[0, :, 0].numpy()
        assert np.allclose(got[b], ref, rtol=1e-5, atol=1e-6), b


def test_sdpa_fully_masked_row_is_nan():
    q, K, V, lens, dims = _sdpa_masked_case()
    B, H, Hkv, D, C = dims
    mask = np.zeros((B, C))
    mask[1, :] = -np.inf
    got = _run_masked(q, K, V, lens, dims, mask.reshape(-1))
    assert np.isnan(got[1]).all() and np.isfinite(got[0]).all() and np.isfinite(got[2]).all()


# ---------------------------------------------------------------------------
# small matmul: y[M, N] = x[M, K] . Wt[N, K]^T (weight in [out, in] layout)
# ---------------------------------------------------------------------------
def _matmul(x, wt, M, K, N, dt=W.BF16, out_dt=W.F32):
    y = np.zeros(M * N, np.float32 if out_dt == W.F32 else np.uint16)
    r = rec(W.OP_MATMUL, dtype=dt, out_dtype=out_dt, size=M, dim=(K, N), a=0, b=1, out=2)
    return run(r, [x, wt, y])[2]


def test_matmul_exact_on_small_integers_and_against_numpy():
    rng = np.random.default_rng(21)
    M, K, N = 5, 64, 7
    xi = rng.integers(-8, 9, M * K).astype(np.float32)
    wi = rng.integers(-8, 9, N * K).astype(np.float32)
    got = _matmul(bf16(xi), bf16(wi), M, K, N)
    ref = xi.reshape(M, K).astype(np.float64) @ wi.reshape(N, K).astype(np.float64).T
    assert np.array_equal(got.reshape(M, N), ref.astype(np.float32))  # exact: integers below 2^24
    xf, wf = bf16(rng.standard_normal(M * K)), bf16(rng.standard_normal(N * K))
    got = _matmul(xf, wf, M, K, N).reshape(M, N).astype(np.float64)
    ref = bf16_val(xf).astype(np.float64).reshape(M, K) @ bf16_val(wf).astype(np.float64).reshape(N, K).T
    assert np.allclose(got, ref, rtol=1e-6, atol=1e-6)


def test_matmul_weight_layout_is_transposed_and_m1_equals_gemv():
    """The weight is read as Wt[n, k] (not W[k, n]): with a non-square weight
    the transposed reading would differ; one row equals the vector-matrix
    product with W = Wt^T laid out [K, N]."""
    rng = np.random.default_rng(22)
    K, N = 32, 12
    x = bf16(rng.standard_normal(K))
    wt = bf16(rng.standard_normal(N * K))
    y = _matmul(x, wt, 1, K, N)
    w_kn = bf16_val(wt).reshape(N, K).T.copy()  # [K, N]
    g = np.zeros(N, np.float32)
    r = rec(W.OP_GEMV, dtype=W.BF16, out_dtype=W.F32, dim=(K, N), a=0, b=1, out=2)
    gemv = run(r, [x, W.to_bf16_bits(w_kn.astype(np.float32)).reshape(-1), g])[2]
    assert np.array_equal(y, gemv)
    wrong = bf16_val(x).astype(np.float64) @ bf16_val(wt).astype(np.float64).reshape(K, N)
    assert not np.allclose(y, wrong, rtol=1e-3)


def test_matmul_bf16_output_rounds_once():
    rng = np.random.default_rng(23)
    M, K, N = 3, 96, 10
    x, wt = bf16(rng.standard_normal(M * K)), bf16(rng.standard_normal(N * K))
    y32 = _matmul(x, wt, M, K, N, out_dt=W.F32)
    y16 = _matmul(x, wt, M, K, N, out_dt=W.BF16)
    exact = bf16_val(x).astype(np.float64).reshape(M, K) @ bf16_val(wt).astype(np.float64).reshape(N, K).T
    assert np.array_equal(y16, np.array([oracle.round_bf16(v) for v in exact.reshape(-1)], np.uint16))
    assert np.allclose(y32.reshape(M, N), exact, rtol=1e-6)


# ------------------------------------------------ paged KV caches
# Pinned against the contiguous-cache path (itself pinned to torch above):
# a pool that holds the contiguous caches' rows scattered to randomly placed
# pages, read through the block table, must give the same attention bit for
# bit, and an append through the table must land where the contiguous
# append does.
def _paged_layout(B=3, Hkv=2, D=16, PS=8, MP=4, extra_pages=5, seed=12):
    rng = np.random.default_rng(seed)
    NP = B * MP + extra_pages
    perm = rng.permutation(NP)[:B * MP].astype(np.int32)
    return perm.reshape(B, MP), NP


def _scatter(cache, table, NP, B, Hkv, C, D, PS, fill):
    """contiguous [B, Hkv, C, D] -> pool [NP, Hkv, PS, D] through the table"""
    c = cache.reshape(B, Hkv, C, D)
    pool = np.full((NP, Hkv, PS, D), fill, dtype=cache.dtype)
    for b in range(B):
        for i in range(C // PS):
            pool[table[b, i]] = c[b, :, i * PS:(i + 1) * PS, :]
    return pool.reshape(-1)


def _gather(pool, table, NP, B, Hkv, C, D, PS):
    p = pool.reshape(NP, Hkv, PS, D)
    out = np.zeros((B, Hkv, C, D), dtype=pool.dtype)
    for b in range(B):
        for i in range(C // PS):
            out[b, :, i * PS:(i + 1) * PS, :] = p[table[b, i]]
    return out.reshape(-1)


@pytest.mark.parametrize("masked", [False, True])
def test_paged_sdpa_equals_contiguous_sdpa(masked):
    B, H, Hkv, D, PS, MP = 3, 4, 2, 16, 8, 4
    C = PS * MP
    rng = np.random.default_rng(31)
    q = bf16(rng.standard_normal(B * H * D))
    K = bf16(rng.standard_normal(B * Hkv * C * D))
    V = bf16(rng.standard_normal(B * Hkv * C * D))
    lens = [C, 1, 19]
    table, NP = _paged_layout(B, Hkv, D, PS, MP)
    mask = np.where(rng.random(B * C) < 0.3, -np.inf, rng.standard_normal(B * C)).astype(np.float32)
    mask.reshape(B, C)[:, 0] = 0.0
    Kp = _scatter(K, table, NP, B, Hkv, C, D, PS, np.uint16(0x7FC0))  # NaN where no page is mapped
    Vp = _scatter(V, table, NP, B, Hkv, C, D, PS, np.uint16(0x7FC0))
    fl = W.FLAG_SDPA_MASK if masked else 0
    mk = {"aux2": 4} if masked else {}
    o = np.zeros(B * H * D, np.float32)
    ref = rec(W.OP_SDPA, dtype=W.BF16, out_dtype=W.F32, size=B, dim=(H, D, C, Hkv), lens=lens, flags=fl,
              a=0, aux0=1, aux1=2, out=3, **mk)
    got = rec(W.OP_SDPA, dtype=W.BF16, out_dtype=W.F32, size=W.paged_size(B, MP, NP), dim=(H, D, PS, Hkv),
              lens=lens, flags=fl | W.FLAG_KV_PAGED, a=0, aux0=1, aux1=2, out=3, b=5, **mk)
    a = run(ref, [q, K, V, o.copy(), mask])[3]
    b = run(got, [q, Kp, Vp, o.copy(), mask, table.reshape(-1)])[3]
    assert np.isfinite(a).all()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_paged_kv_append_equals_contiguous_append():
    B, H, D, PS, MP = 3, 2, 16, 8, 4
    C = PS * MP
    rng = np.random.default_rng(32)
    K = bf16(rng.standard_normal(B * H * C * D))
    V = bf16(rng.standard_normal(B * H * C * D))
    k = bf16(rng.standard_normal(B * H * D))
    v = bf16(rng.standard_normal(B * H * D))
    lens = [C, 1, 13]   # appends at the last row of the last page, the first row, mid-page
    table, NP = _paged_layout(B, H, D, PS, MP, seed=13)
    Kp, Vp = _scatter(K, table, NP, B, H, C, D, PS, 0), _scatter(V, table, NP, B, H, C, D, PS, 0)
    ref = rec(W.OP_KV_APPEND, dtype=W.BF16, size=B, dim=(H, D, C), lens=lens, a=0, b=1, aux0=2, aux1=3)
    got = rec(W.OP_KV_APPEND, dtype=W.BF16, size=W.paged_size(B, MP, NP), dim=(H, D, PS), lens=lens,
              flags=W.FLAG_KV_PAGED, a=0, b=1, aux0=2, aux1=3, aux2=4)
    _, _, Kr, Vr = run(ref, [k, v, K, V])
    _, _, Kg, Vg, _ = run(got, [k, v, Kp, Vp, table.reshape(-1)])
    assert np.array_equal(_gather(Kg, table, NP, B, H, C, D, PS), Kr)
    assert np.array_equal(_gather(Vg, table, NP, B, H, C, D, PS), Vr)
    # pages no row maps are untouched
    unused = np.setdiff1d(np.arange(NP), table.reshape(-1))
    assert np.array_equal(Kg.reshape(NP, -1)[unused], Kp.reshape(NP, -1)[unused])


def test_paged_table_entry_outside_the_pool():
    """A page number outside the pool: the append writes nothing there, and
    attention leaves that page's keys out (the same as masking them)."""
    B, H, Hkv, D, PS, MP = 2, 2, 2, 16, 8, 3
    C = PS * MP
    rng = np.random.default_rng(33)
    q = bf16(rng.standard_normal(B * H * D))
    K = bf16(rng.standard_normal(B * Hkv * C * D))
    V = bf16(rng.standard_normal(B * Hkv * C * D))
    table, NP = _paged_layout(B, Hkv, D, PS, MP, extra_pages=0, seed=14)
    Kp, Vp = _scatter(K, table, NP, B, Hkv, C, D, PS, 0), _scatter(V, table, NP, B, Hkv, C, D, PS, 0)
    bad = table.copy()
    bad[1, 1] = NP + 7
    bad[0, 2] = -1
    lens = [C, C]
    o = np.zeros(B * H * D, np.float32)
    got = rec(W.OP_SDPA, dtype=W.BF16, out_dtype=W.F32, size=W.paged_size(B, MP, NP), dim=(H, D, PS, Hkv),
              lens=lens, flags=W.FLAG_KV_PAGED, a=0, aux0=1, aux1=2, out=3, b=4)
    b_out = run(got, [q, Kp, Vp, o.copy(), bad.reshape(-1)])[3]
    mask = np.zeros((B, C), np.float32)
    mask[1, PS:2 * PS] = -np.inf
    mask[0, 2 * PS:3 * PS] = -np.inf
    a_out = _run_masked(q, K, V, lens, (B, H, Hkv, D, C), mask.reshape(-1))
    assert np.array_equal(b_out.reshape(B, H, D).astype(np.float64), a_out)
    k = bf16(rng.standard_normal(B * Hkv * D))
    app = rec(W.OP_KV_APPEND, dtype=W.BF16, size=W.paged_size(B, MP, NP), dim=(Hkv, D, PS), lens=[PS + 3, 2 * PS + 1],
              flags=W.FLAG_KV_PAGED, a=0, b=0, aux0=1, aux1=2, aux2=3)
    bad2 = table.copy()
    bad2[0, 1] = NP          # row 0 appends at position PS + 2: page index 1 -> outside
    _, Kg, _, _ = run(app, [k, Kp, Vp, bad2.reshape(-1)])
    # row 1 (position 2 PS, page table[1, 2]) was written; nothing else changed
    changed = np.nonzero(Kg.reshape(NP, -1) != Kp.reshape(NP, -1))[0]
    assert set(np.unique(changed)) == {int(table[1, 2])}
