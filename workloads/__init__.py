"""Seeded synthetic descriptor streams shaped like the GPUOS pages' workloads.

This module is shared by both sides of every parity check: the GPU harness
turns a stream into device descriptors, the oracle runs it on host arrays.
It holds no arithmetic of any micro-op.  Everything here is input
generation: a counter-based random generator, buffer initialisers and the
symbolic descriptor records that name buffers by index instead of pointer.

Random numbers come from SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014): z = seed + (i+1)*golden, then
two xor-shift-multiply rounds.  Uniforms take the top 53 (or 24) bits;
normals use the Box-Muller transform in double precision.  bf16 values are
produced from fp32 samples by torch's own float->bfloat16 conversion, so no
rounding routine of the method is involved.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

# ---------------------------------------------------------------------------
# Operation codes and dtypes of the symbolic stream.  The numbering is the
# public op-id numbering of the C ABI (gpuos.h); the oracle declares the same
# numbers on its own.
# ---------------------------------------------------------------------------
OP_NOP, OP_ADD, OP_MUL, OP_RELU, OP_GELU = 0, 1, 2, 3, 4
OP_SUM, OP_MAX, OP_MIN, OP_SOFTMAX, OP_LAYERNORM = 5, 6, 7, 8, 9
OP_ROPE, OP_KV_APPEND, OP_SDPA, OP_GEMV, OP_COPY = 10, 11, 12, 13, 14
OP_EXPR = 15  # injected element-wise program (program words in AUX2, dim[2] words, op id in dim[3])
OP_MATMUL = 16  # small matmul: y[M = size, N = dim[1]] = x[M, K = dim[0]] . Wt[N, K]^T
OP_NAMES = {
    OP_NOP: "nop", OP_ADD: "add", OP_MUL: "mul", OP_RELU: "relu", OP_GELU: "gelu",
    OP_SUM: "sum", OP_MAX: "max", OP_MIN: "min", OP_SOFTMAX: "softmax",
    OP_LAYERNORM: "layernorm", OP_ROPE: "rope", OP_KV_APPEND: "kv_append",
    OP_SDPA: "sdpa", OP_GEMV: "gemv", OP_COPY: "copy", OP_EXPR: "expr", OP_MATMUL: "matmul",
}

# Injected element-wise programs: instruction codes and encoding (the word
# layout of gpuos.h and of the oracle; data formatting only, no arithmetic).
(X_LDA, X_LDB, X_CONST, X_MOV, X_ADD, X_SUB, X_MUL, X_DIV, X_MIN, X_MAX, X_NEG, X_ABS,
 X_EXP, X_LOG, X_SQRT, X_TANH, X_SIGMOID, X_RELU) = range(1, 19)
X_EXACT = {X_LDA, X_LDB, X_CONST, X_MOV, X_ADD, X_SUB, X_MUL, X_DIV, X_MIN, X_MAX, X_NEG, X_ABS, X_SQRT,
           X_RELU}


def xins(op: int, d: int = 0, s1: int = 0, s2: int = 0, k: int = 0) -> int:
    return op | (d << 8) | (s1 << 12) | (s2 << 16) | (k << 20)


def program(instrs, consts=()) -> np.ndarray:
    """Program words: header, instructions, constants (fp32 bit patterns)."""
    c = np.asarray(consts, np.float32).view(np.uint32)
    return np.concatenate([np.array([len(instrs) | (len(c) << 8)], np.uint32),
                           np.asarray(instrs, np.uint32), c]).astype(np.uint32)


def program_is_exact(words) -> bool:
    """True when every instruction is one of the correctly rounded steps."""
    n = int(words[0]) & 0xFF
    return all((int(w) & 0xFF) in X_EXACT for w in words[1:1 + n])
F32, BF16 = 0, 1
I32 = 2  # int32 buffers (block tables of paged caches); never an op dtype
DTYPE_BYTES = {F32: 4, BF16: 2, I32: 4}
FLAG_ROPE_HALF = 1  # rotate-half pairing (x_i, x_{i+D/2}) instead of adjacent pairs
FLAG_SDPA_MASK = 2  # SDPA adds an fp32 mask [B, C] (AUX2) to the scaled scores
# KV_APPEND / SDPA on paged caches: pools of NP pages [heads, PS, D] and an
# int32 block table [B, MP] (AUX2 for KV_APPEND, B for SDPA); the record's
# size packs B (bits 0-15), MP (bits 16-31) and NP (bits 32-63), dim[2] = PS
FLAG_KV_PAGED = 4


def paged_size(b: int, mp: int, n_pages: int) -> int:
    return int(b) | (int(mp) << 16) | (int(n_pages) << 32)


def rec_rows(r) -> int:
    """Batch rows of an attention record (the low bits of size when paged)."""
    return int(r["size"]) & 0xFFFF if int(r["flags"]) & FLAG_KV_PAGED else int(r["size"])

# Operand roles: index into buf/off.
A, B, OUT, AUX0, AUX1, AUX2 = 0, 1, 2, 3, 4, 5

REC_DTYPE = np.dtype([
    ("op", "<i4"), ("dtype", "<i4"), ("out_dtype", "<i4"), ("flags", "<i4"),
    ("buf", "<i4", (6,)),
    ("off", "<i8", (6,)),
    ("size", "<i8"),
    ("dim", "<i4", (4,)),
    ("fparam", "<f4", (2,)),
    ("lens", "<i4", (8,)),
])
assert REC_DTYPE.itemsize == 152


# ---------------------------------------------------------------------------
# SplitMix64
# ---------------------------------------------------------------------------
_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, start: int, n: int) -> np.ndarray:
    """Outputs start..start+n-1 of the SplitMix64 sequence for `seed`."""
    with np.errstate(over="ignore"):
        i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


class Rng:
    """A counter over one SplitMix64 sequence."""

    def __init__(self, seed: int):
        self.seed = seed
        self.ctr = 0

    def raw(self, n: int) -> np.ndarray:
        out = splitmix64(self.seed, self.ctr, n)
        self.ctr += n
        return out

    def uniform(self, n: int) -> np.ndarray:
        """Doubles in [0, 1) with 53 random bits."""
        return (self.raw(n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)

    def uniform24(self, n: int) -> np.ndarray:
        """Doubles in [0, 1) with 24 random bits (exact in fp32)."""
        return (self.raw(n) >> np.uint64(40)).astype(np.float64) * (2.0 ** -24)

    def integers(self, k: int, n: int) -> np.ndarray:
        """Uniform integers in {0..k-1}."""
        return np.minimum((self.uniform(n) * k).astype(np.int64), k - 1)

    def normal(self, n: int) -> np.ndarray:
        """Standard normals by Box-Muller (one output per pair of draws)."""
        z = self.raw(2 * n)
        u1 = ((z[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)
        u2 = (z[1::2] >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
        return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)

    def scalar_int(self, lo: int, hi: int) -> int:
        """One integer uniform in [lo, hi]."""
        return lo + int(self.integers(hi - lo + 1, 1)[0])


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32/fp64 samples -> bf16 bit patterns (uint16) via torch's conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact widening: append 16 zero bits)."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# Buffers and streams
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class Buffer:
    """One pool buffer.  init = ("normal", std, mean) | ("uniform", lo, hi) |
    ("zeros",) | ("pages", n_pages) (int32: the first nelem entries of a
    random permutation of range(n_pages), a block table whose rows never
    share a page).  Values are drawn from SplitMix64 stream `seed`."""
    name: str
    dtype: int
    nelem: int
    init: tuple
    seed: int = 0

    @property
    def nbytes(self) -> int:
        return self.nelem * DTYPE_BYTES[self.dtype]

    def host_values(self) -> np.ndarray:
        """Materialise on the host: float32 array, or uint16 bf16 bits."""
        kind = self.init[0]
        if kind == "pages":
            n_pages = int(self.init[1])
            assert self.dtype == I32 and self.nelem <= n_pages
            rng = Rng(self.seed)
            perm = np.arange(n_pages, dtype=np.int64)
            u = rng.uniform24(n_pages)  # Fisher-Yates with the stream's uniforms
            for i in range(n_pages - 1, 0, -1):
                j = min(int(u[i] * (i + 1)), i)
                perm[i], perm[j] = perm[j], perm[i]
            return perm[:self.nelem].astype(np.int32)
        if kind == "zeros":
            v = np.zeros(self.nelem, np.float64)
        else:
            rng = Rng(self.seed)
            if kind == "normal":
                std, mean = self.init[1], (self.init[2] if len(self.init) > 2 else 0.0)
                v = rng.normal(self.nelem) * std + mean
            elif kind == "uniform":
                lo, hi = self.init[1], self.init[2]
                v = lo + (hi - lo) * rng.uniform24(self.nelem)
            else:
                raise ValueError(kind)
        if self.dtype == F32:
            return v.astype(np.float32)
        return to_bf16_bits(v.astype(np.float32))

    def host_bytes(self) -> np.ndarray:
        return self.host_values().view(np.uint8)


@dataclasses.dataclass
class Stream:
    """A symbolic descriptor stream over a pool of buffers."""
    name: str
    buffers: List[Buffer]
    recs: np.ndarray                 # REC_DTYPE records, in submission order
    bursts: np.ndarray               # burst sizes, sum == len(recs)
    meta: dict = dataclasses.field(default_factory=dict)

    def __len__(self) -> int:
        return len(self.recs)


def _new_recs(n: int) -> np.ndarray:
    r = np.zeros(n, REC_DTYPE)
    r["buf"] = -1
    return r


def _buffer_seed(stream_seed: int, idx: int) -> int:
    return (stream_seed * 1_000_003 + 7919 * (idx + 1)) & 0xFFFFFFFFFFFFFFFF


# ---------------------------------------------------------------------------
# PR1: 1,000 descriptors over 16 fp32 vectors of 4096 values U[-1,1];
# op uniform over {add, mul, relu}; operands and outputs uniform over the pool.
# ---------------------------------------------------------------------------
def make_pr1(seed: int = 1, n_desc: int = 1000, n_tensors: int = 16,
             n_elem: int = 4096) -> Stream:
    bufs = [Buffer(f"v{i}", F32, n_elem, ("uniform", -1.0, 1.0), _buffer_seed(seed, i))
            for i in range(n_tensors)]
    rng = Rng(seed)
    ops = np.array([OP_ADD, OP_MUL, OP_RELU])[rng.integers(3, n_desc)]
    a = rng.integers(n_tensors, n_desc)
    b = rng.integers(n_tensors, n_desc)
    o = rng.integers(n_tensors, n_desc)
    r = _new_recs(n_desc)
    r["op"] = ops
    r["dtype"] = F32
    r["out_dtype"] = F32
    r["buf"][:, A] = a
    r["buf"][:, B] = np.where(ops == OP_RELU, -1, b)
    r["buf"][:, OUT] = o
    r["size"] = n_elem
    return Stream("pr1", bufs, r, np.array([n_desc]), {"seed": seed})


# ---------------------------------------------------------------------------
# Element-wise stream: pool of 32 fp32 + 32 bf16 tensors of 65536 values
# N(0,1); per descriptor a dtype (50/50), n = floor(256 * 256**u) in
# [256, 65536], op uniform over {add, mul, relu, gelu}; 10% in place
# (out = a), otherwise out drawn from the other tensors of that dtype;
# bursts of 1..64.
# ---------------------------------------------------------------------------
def make_elementwise(seed: int = 2, n_desc: int = 100_000, n_per_dtype: int = 32,
                     n_elem: int = 65536, n_min: int = 256, inplace_p: float = 0.1,
                     ops: Sequence[int] = (OP_ADD, OP_MUL, OP_RELU, OP_GELU),
                     max_burst: int = 64) -> Stream:
    bufs = [Buffer(f"f{i}", F32, n_elem, ("normal", 1.0), _buffer_seed(seed, i))
            for i in range(n_per_dtype)]
    bufs += [Buffer(f"h{i}", BF16, n_elem, ("normal", 1.0), _buffer_seed(seed, 1000 + i))
             for i in range(n_per_dtype)]
    rng = Rng(seed)
    dt = rng.integers(2, n_desc)
    u = rng.uniform(n_desc)
    ratio = n_elem / n_min
    n = np.minimum(np.floor(n_min * ratio ** u).astype(np.int64), n_elem)
    op = np.asarray(ops)[rng.integers(len(ops), n_desc)]
    a = rng.integers(n_per_dtype, n_desc)
    b = rng.integers(n_per_dtype, n_desc)
    inplace = rng.uniform(n_desc) < inplace_p
    other = rng.integers(n_per_dtype - 1, n_desc)
    o = np.where(inplace, a, np.where(other >= a, other + 1, other))
    base = np.where(dt == BF16, n_per_dtype, 0)
    r = _new_recs(n_desc)
    r["op"] = op
    r["dtype"] = dt
    r["out_dtype"] = dt
    r["buf"][:, A] = base + a
    binary = (op == OP_ADD) | (op == OP_MUL)
    r["buf"][:, B] = np.where(binary, base + b, -1)
    r["buf"][:, OUT] = base + o
    r["size"] = n
    bursts = _bursts(rng, n_desc, max_burst)
    return Stream("elementwise", bufs, r, bursts, {"seed": seed})


def _bursts(rng: Rng, n: int, max_burst: int) -> np.ndarray:
    sizes = 1 + rng.integers(max_burst, n // 1 + 1)
    c = np.cumsum(sizes)
    k = int(np.searchsorted(c, n)) + 1
    sizes = sizes[:k].copy()
    sizes[-1] -= int(c[k - 1] - n)
    return sizes[sizes > 0]


# ---------------------------------------------------------------------------
# Row ops: rows in {1,2,4,...,64}, hidden in {768,1024,2048,4096},
# x ~ N(0, std 2); op uniform over {sum, max, min, softmax, layernorm};
# gamma ~ N(1, 0.1), beta ~ N(0, 0.1), eps = 1e-5.  Inputs are [rows, h]
# prefixes of random pool buffers of capacity [64, 4096]; outputs are
# consecutive slices of a rotating output arena.
# ---------------------------------------------------------------------------
ROW_HIDDEN = (768, 1024, 2048, 4096)


def make_rows(seed: int = 3, n_desc: int = 50_000, n_pool: int = 2048,
              max_rows: int = 64, max_hidden: int = 4096,
              arena_bytes: int = 256 << 20, dtype: int = F32,
              hidden: Sequence[int] = ROW_HIDDEN, max_burst: int = 64) -> Stream:
    esz = DTYPE_BYTES[dtype]
    bufs = [Buffer(f"x{i}", dtype, max_rows * max_hidden, ("normal", 2.0), _buffer_seed(seed, i))
            for i in range(n_pool)]
    g0 = len(bufs)
    for j, h in enumerate(hidden):
        bufs.append(Buffer(f"gamma{h}", dtype, h, ("normal", 0.1, 1.0), _buffer_seed(seed, 50_000 + j)))
        bufs.append(Buffer(f"beta{h}", dtype, h, ("normal", 0.1, 0.0), _buffer_seed(seed, 60_000 + j)))
    arena = len(bufs)
    bufs.append(Buffer("arena", dtype, arena_bytes // esz, ("zeros",)))
    rng = Rng(seed)
    log_rows = int(round(math.log2(max_rows)))
    rows = (1 << rng.integers(log_rows + 1, n_desc)).astype(np.int64)
    hidx = rng.integers(len(hidden), n_desc)
    hid = np.asarray(hidden, np.int64)[hidx]
    opset = np.array([OP_SUM, OP_MAX, OP_MIN, OP_SOFTMAX, OP_LAYERNORM])
    op = opset[rng.integers(5, n_desc)]
    src = rng.integers(n_pool, n_desc)
    r = _new_recs(n_desc)
    r["op"] = op
    r["dtype"] = dtype
    r["out_dtype"] = dtype
    r["buf"][:, A] = src
    r["size"] = rows
    r["dim"][:, 0] = hid
    is_ln = op == OP_LAYERNORM
    r["buf"][:, AUX0] = np.where(is_ln, g0 + 2 * hidx, -1)
    r["buf"][:, AUX1] = np.where(is_ln, g0 + 2 * hidx + 1, -1)
    r["fparam"][:, 0] = np.where(is_ln, np.float32(1e-5), 0)
    red = (op == OP_SUM) | (op == OP_MAX) | (op == OP_MIN)
    out_bytes = np.where(red, rows * esz, rows * hid * esz)
    # consecutive 256-byte-aligned slices of the arena, wrapping
    aligned = (out_bytes + 255) // 256 * 256
    offs = np.zeros(n_desc, np.int64)
    cur = 0
    for i in range(n_desc):
        if cur + aligned[i] > arena_bytes:
            cur = 0
        offs[i] = cur
        cur += int(aligned[i])
    r["buf"][:, OUT] = arena
    r["off"][:, OUT] = offs
    bursts = _bursts(rng, n_desc, max_burst)
    return Stream("rows", bufs, r, bursts, {"seed": seed, "arena": arena})


# ---------------------------------------------------------------------------
# Attention decoding: per step a batch B ~ U{1,2,4,8}; per layer RoPE on q,k
# at position L_b-1, KV append at L_b-1, single-query SDPA over [0, L_b).
# H heads, D head_dim, C cache capacity per sequence; lengths start
# U[L_min, C] and grow by one per step (a sequence that would exceed C is
# redrawn as a new request).  q, k, v cycle through a pool of triples.
# ---------------------------------------------------------------------------
def make_decode(seed: int = 4, steps: int = 2000, layers: int = 32, heads: int = 32,
                head_dim: int = 128, capacity: int = 4096, max_batch: int = 8,
                l_min: int = 128, n_triples: int = 256, theta: float = 10000.0,
                out_dtype: int = F32, n_out: int = 64,
                batches: Sequence[int] = (1, 2, 4, 8), kv_heads: int = 0, page_size: int = 0) -> Stream:
    """kv_heads (0: heads) below heads gives grouped-query attention: k, v
    and the caches have kv_heads heads, shared by heads/kv_heads queries.
    page_size > 0 stores each layer's caches as pools of max_batch *
    capacity / page_size pages of page_size positions, with a block table per
    layer that gives every batch row its own randomly placed pages (the same
    bytes as the contiguous caches, in paged layout)."""
    H, D, C, Bm = heads, head_dim, capacity, max_batch
    Hkv = kv_heads or H
    assert H % Hkv == 0
    PS = page_size
    MP = C // PS if PS else 0
    NP = Bm * MP
    assert not PS or C % PS == 0
    bufs: List[Buffer] = []
    kc0 = len(bufs)
    for l in range(layers):
        bufs.append(Buffer(f"K{l}", BF16, Bm * Hkv * C * D, ("normal", 1.0), _buffer_seed(seed, 10 * l)))
        bufs.append(Buffer(f"V{l}", BF16, Bm * Hkv * C * D, ("normal", 1.0), _buffer_seed(seed, 10 * l + 1)))
    tb0 = len(bufs)
    if PS:
        for l in range(layers):
            bufs.append(Buffer(f"T{l}", I32, Bm * MP, ("pages", NP), _buffer_seed(seed, 10 * l + 2)))
    tq = len(bufs)
    for t in range(n_triples):
        for j, nm in enumerate("qkv"):
            bufs.append(Buffer(f"{nm}{t}", BF16, Bm * (H if nm == "q" else Hkv) * D, ("normal", 1.0),
                               _buffer_seed(seed, 100_000 + 3 * t + j)))
    o0 = len(bufs)
    for i in range(n_out):
        bufs.append(Buffer(f"o{i}", out_dtype, Bm * H * D, ("zeros",)))
    rng = Rng(seed)
    lens = np.array([rng.scalar_int(l_min, C) for _ in range(Bm)], np.int64)
    recs = []
    tcount = 0
    for s in range(steps):
        Bsz = int(np.asarray(batches)[rng.integers(len(batches), 1)[0]])
        for b in range(Bsz):
            lens[b] += 1
            if lens[b] > C:
                lens[b] = rng.scalar_int(l_min, C)
        for l in range(layers):
            t = tcount % n_triples
            tcount += 1
            q, k, v = tq + 3 * t, tq + 3 * t + 1, tq + 3 * t + 2
            lens_row = np.zeros(8, np.int32)
            lens_row[:Bsz] = lens[:Bsz]
            rr = _new_recs(3)
            # RoPE on q and k in place
            rr[0]["op"] = OP_ROPE
            rr[0]["buf"][A], rr[0]["buf"][B] = q, k
            rr[0]["fparam"][0] = theta
            # KV append
            rr[1]["op"] = OP_KV_APPEND
            rr[1]["buf"][A], rr[1]["buf"][B] = k, v
            rr[1]["buf"][AUX0], rr[1]["buf"][AUX1] = kc0 + 2 * l, kc0 + 2 * l + 1
            # SDPA
            rr[2]["op"] = OP_SDPA
            rr[2]["buf"][A] = q
            rr[2]["buf"][AUX0], rr[2]["buf"][AUX1] = kc0 + 2 * l, kc0 + 2 * l + 1
            rr[2]["buf"][OUT] = o0 + (s * layers + l) % n_out
            rr[2]["out_dtype"] = out_dtype
            for x in rr:
                x["dtype"] = BF16
                if x["op"] != OP_SDPA:
                    x["out_dtype"] = BF16
                x["size"] = Bsz
                x["dim"][:] = (H, D, C, Hkv if Hkv != H else 0)
                x["lens"][:] = lens_row
            rr[1]["dim"][:] = (Hkv, D, C, 0)
            if PS:
                for x in rr[1:]:
                    x["flags"] |= FLAG_KV_PAGED
                    x["size"] = paged_size(Bsz, MP, NP)
                    x["dim"][2] = PS
                rr[1]["buf"][AUX2] = tb0 + l
                rr[2]["buf"][B] = tb0 + l
            recs.append(rr)
    r = np.concatenate(recs) if recs else _new_recs(0)
    bursts = np.full(steps * layers, 3) if steps else np.zeros(0, np.int64)
    return Stream("decode", bufs, r, bursts,
                  {"seed": seed, "kv_first": kc0, "layers": layers, "heads": H, "kv_heads": Hkv,
                   "head_dim": D, "capacity": C, "page_size": PS, "tables_first": tb0 if PS else None})


# ---------------------------------------------------------------------------
# Mixed decode pipeline: tokens through `layers` layers at hidden 1024 with
# 8 heads of 128, bf16.  Per layer: LN -> GEMV 1024x3072 (qkv) -> RoPE(q,k)
# -> KV append -> SDPA -> residual add -> LN -> GEMV 1024x3072 (up) -> GELU
# -> GEMV 3072x1024 (down) -> residual add.  Weights N(0, 0.02); gamma
# N(1, 0.1), beta N(0, 0.1); x per token N(0,1); L_0 ~ U[64, 2048], +1 per token.
# ---------------------------------------------------------------------------
def make_mixed(seed: int = 5, tokens: int = 500, layers: int = 32, hidden: int = 1024,
               heads: int = 8, head_dim: int = 128, ffn: int = 3072, capacity: int = 4096,
               l0_range=(64, 2048), theta: float = 10000.0, n_tok_pool: int = 64,
               eps: float = 1e-5) -> Stream:
    Hd, H, D, F, C = hidden, heads, head_dim, ffn, capacity
    assert H * D == Hd
    bufs: List[Buffer] = []

    def add(name, dtype, n, init, key):
        bufs.append(Buffer(name, dtype, n, init, _buffer_seed(seed, key)))
        return len(bufs) - 1

    W = []
    for l in range(layers):
        W.append(dict(
            wqkv=add(f"wqkv{l}", BF16, Hd * 3 * Hd, ("normal", 0.02), 100 * l + 1),
            wup=add(f"wup{l}", BF16, Hd * F, ("normal", 0.02), 100 * l + 2),
            wdown=add(f"wdown{l}", BF16, F * Hd, ("normal", 0.02), 100 * l + 3),
            g1=add(f"g1_{l}", BF16, Hd, ("normal", 0.1, 1.0), 100 * l + 4),
            b1=add(f"b1_{l}", BF16, Hd, ("normal", 0.1, 0.0), 100 * l + 5),
            g2=add(f"g2_{l}", BF16, Hd, ("normal", 0.1, 1.0), 100 * l + 6),
            b2=add(f"b2_{l}", BF16, Hd, ("normal", 0.1, 0.0), 100 * l + 7),
            kc=add(f"K{l}", BF16, H * C * D, ("normal", 1.0), 100 * l + 8),
            vc=add(f"V{l}", BF16, H * C * D, ("normal", 1.0), 100 * l + 9),
        ))
    xs = [add(f"xtok{i}", BF16, Hd, ("normal", 1.0), 900_000 + i) for i in range(n_tok_pool)]
    x = add("x", BF16, Hd, ("zeros",), 1)
    h = add("h", BF16, Hd, ("zeros",), 2)
    qkv = add("qkv", BF16, 3 * Hd, ("zeros",), 3)
    att = add("att", BF16, Hd, ("zeros",), 4)
    up = add("up", BF16, F, ("zeros",), 5)
    dn = add("down", BF16, Hd, ("zeros",), 6)
    rng = Rng(seed)
    L = rng.scalar_int(*l0_range)
    recs = []

    def rec(op, **kw):
        r = _new_recs(1)[0]
        r["op"] = op
        r["dtype"] = BF16
        r["out_dtype"] = BF16
        for k, v in kw.items():
            if k in ("a", "b", "out", "aux0", "aux1"):
                role = {"a": A, "b": B, "out": OUT, "aux0": AUX0, "aux1": AUX1}[k]
                bi, off = v if isinstance(v, tuple) else (v, 0)
                r["buf"][role] = bi
                r["off"][role] = off
            elif k == "dim":
                r["dim"][:len(v)] = v
            elif k == "fparam":
                r["fparam"][:len(v)] = v
            else:
                r[k] = v
        return r

    for t in range(tokens):
        L += 1
        if L > C:
            L = rng.scalar_int(*l0_range)
        lens_row = np.zeros(8, np.int32)
        lens_row[0] = L
        recs.append(rec(OP_COPY, a=xs[t % n_tok_pool], out=x, size=Hd * 2))
        for l in range(layers):
            w = W[l]
            recs.append(rec(OP_LAYERNORM, a=x, out=h, aux0=w["g1"], aux1=w["b1"], size=1,
                            dim=(Hd,), fparam=(eps,)))
            recs.append(rec(OP_GEMV, a=h, b=w["wqkv"], out=qkv, dim=(Hd, 3 * Hd)))
            r = rec(OP_ROPE, a=(qkv, 0), b=(qkv, Hd * 2), size=1, dim=(H, D, C), fparam=(theta,))
            r["lens"][:] = lens_row
            recs.append(r)
            r = rec(OP_KV_APPEND, a=(qkv, Hd * 2), b=(qkv, Hd * 4), aux0=w["kc"], aux1=w["vc"],
                    size=1, dim=(H, D, C))
            r["lens"][:] = lens_row
            recs.append(r)
            r = rec(OP_SDPA, a=(qkv, 0), aux0=w["kc"], aux1=w["vc"], out=att, size=1, dim=(H, D, C))
            r["lens"][:] = lens_row
            recs.append(r)
            recs.append(rec(OP_ADD, a=x, b=att, out=x, size=Hd))
            recs.append(rec(OP_LAYERNORM, a=x, out=h, aux0=w["g2"], aux1=w["b2"], size=1,
                            dim=(Hd,), fparam=(eps,)))
            recs.append(rec(OP_GEMV, a=h, b=w["wup"], out=up, dim=(Hd, F)))
            recs.append(rec(OP_GELU, a=up, out=up, size=F))
            recs.append(rec(OP_GEMV, a=up, b=w["wdown"], out=dn, dim=(F, Hd)))
            recs.append(rec(OP_ADD, a=x, b=dn, out=x, size=Hd))
    r = np.array(recs, dtype=REC_DTYPE) if recs else _new_recs(0)
    per_tok = 1 + 11 * layers
    bursts = np.full(tokens, per_tok) if tokens else np.zeros(0, np.int64)
    return Stream("mixed", bufs, r, bursts,
                  {"seed": seed, "layers": layers, "x": x, "ops_per_token": per_tok})


def make_matmul(seed: int = 6, passes: int = 20, layers: int = 32, rows: int = 32, hidden: int = 1024,
                ffn: int = 3072) -> Stream:
    """Small matmuls of batched decoding: `rows` tokens through the QKV
    (hidden -> 3 hidden), up (hidden -> ffn) and down (ffn -> hidden)
    projections of `layers` layers, bf16, weights N(0, 0.02) in the [out, in]
    layout (604 MB at the defaults, more than the 256 MB last-level cache),
    `passes` times.  Every projection reads the same token activations and
    writes its own output, so the descriptors are independent and the
    stream measures the operator's own rate."""
    Hd, F = hidden, ffn
    bufs: List[Buffer] = []

    def add(name, dtype, n, init, key):
        bufs.append(Buffer(name, dtype, n, init, _buffer_seed(seed, key)))
        return len(bufs) - 1
    xh = add("x_hidden", BF16, rows * Hd, ("normal", 1.0), 1)
    xf = add("x_ffn", BF16, rows * F, ("normal", 1.0), 2)
    shapes = (("qkv", Hd, 3 * Hd, xh), ("up", Hd, F, xh), ("down", F, Hd, xf))
    wts, outs = [], []
    for l in range(layers):
        for j, (nm, K, N, x) in enumerate(shapes):
            wts.append((add(f"w{nm}{l}", BF16, N * K, ("normal", 0.02), 100 * l + 10 + j), K, N, x))
            outs.append(add(f"y{nm}{l}", BF16, rows * N, ("zeros",), 100 * l + 20 + j))
    recs = _new_recs(passes * len(wts))
    i = 0
    for _ in range(passes):
        for (w, K, N, x), y in zip(wts, outs):
            r = recs[i]
            r["op"] = OP_MATMUL
            r["dtype"] = r["out_dtype"] = BF16
            r["size"] = rows
            r["dim"][:2] = (K, N)
            r["buf"][A], r["buf"][B], r["buf"][OUT] = x, w, y
            i += 1
    per_pass = len(wts)
    return Stream("matmul", bufs, recs, np.full(passes, per_pass),
                  {"seed": seed, "rows": rows, "layers": layers, "flops": 2 * rows * sum(K * N for (_, K, N, _) in wts) * passes})


# ---------------------------------------------------------------------------
# Byte ranges each record touches: used by tests and by harnesses that need
# to know which buffer bytes a descriptor writes.  These are the operands'
# extents as laid out by the generators above.
# ---------------------------------------------------------------------------
def output_ranges(r) -> list:
    """[(buf, byte_off, nbytes), ...] written by record r."""
    op = int(r["op"])
    es = DTYPE_BYTES[int(r["dtype"])]
    eo = DTYPE_BYTES[int(r["out_dtype"])]
    size = int(r["size"])
    d = [int(v) for v in r["dim"]]
    buf, off = r["buf"], r["off"]
    if op in (OP_ADD, OP_MUL, OP_RELU, OP_GELU, OP_EXPR):
        return [(int(buf[OUT]), int(off[OUT]), size * eo)]
    if op in (OP_SUM, OP_MAX, OP_MIN):
        return [(int(buf[OUT]), int(off[OUT]), size * eo)]
    if op in (OP_SOFTMAX, OP_LAYERNORM):
        return [(int(buf[OUT]), int(off[OUT]), size * d[0] * eo)]
    if op == OP_ROPE:
        hk = d[3] if d[3] else d[0]
        return [(int(buf[A]), int(off[A]), size * d[0] * d[1] * es), (int(buf[B]), int(off[B]), size * hk * d[1] * es)]
    if op == OP_KV_APPEND and int(r["flags"]) & FLAG_KV_PAGED:
        # the pages written depend on the block table: the whole pools
        n_pages = size >> 32
        pool = n_pages * d[0] * d[2] * d[1] * es
        return [(int(buf[AUX0]), int(off[AUX0]), pool), (int(buf[AUX1]), int(off[AUX1]), pool)]
    if op == OP_KV_APPEND:
        H, D, C = d[0], d[1], d[2]
        out = []
        for bb in range(size):
            pos = int(r["lens"][bb]) - 1
            for hh in range(H):
                row = ((bb * H + hh) * C + pos) * D * es
                out.append((int(buf[AUX0]), int(off[AUX0]) + row, D * es))
                out.append((int(buf[AUX1]), int(off[AUX1]) + row, D * es))
        return out
    if op == OP_SDPA:
        return [(int(buf[OUT]), int(off[OUT]), rec_rows(r) * d[0] * d[1] * eo)]
    if op == OP_GEMV:
        return [(int(buf[OUT]), int(off[OUT]), d[1] * eo)]
    if op == OP_MATMUL:
        return [(int(buf[OUT]), int(off[OUT]), size * d[1] * eo)]
    if op == OP_COPY:
        return [(int(buf[OUT]), int(off[OUT]), size)]
    return []


def algorithmic_bytes(recs: np.ndarray) -> np.ndarray:
    """Bytes each record must move at minimum: every operand read once and
    every output written once (per-op formulas of the measurement plan)."""
    op = recs["op"]
    es = np.where(recs["dtype"] == BF16, 2, 4).astype(np.int64)
    eo = np.where(recs["out_dtype"] == BF16, 2, 4).astype(np.int64)
    n = recs["size"].astype(np.int64)
    n = np.where(recs["flags"] & FLAG_KV_PAGED, n & 0xFFFF, n)  # paged attention: batch rows
    d0, d1 = recs["dim"][:, 0].astype(np.int64), recs["dim"][:, 1].astype(np.int64)
    out = np.zeros(len(recs), np.int64)
    m = (op == OP_ADD) | (op == OP_MUL) | ((op == OP_EXPR) & (recs["buf"][:, B] >= 0))
    out[m] = (2 * es[m] + eo[m]) * n[m]
    m = (op == OP_EXPR) & (recs["buf"][:, B] < 0)
    out[m] = (es[m] + eo[m]) * n[m]
    m = (op == OP_RELU) | (op == OP_GELU)
    out[m] = (es[m] + eo[m]) * n[m]
    m = (op == OP_SUM) | (op == OP_MAX) | (op == OP_MIN)
    out[m] = es[m] * n[m] * d0[m] + eo[m] * n[m]
    m = op == OP_SOFTMAX
    out[m] = (es[m] + eo[m]) * n[m] * d0[m]
    m = op == OP_LAYERNORM
    out[m] = (es[m] + eo[m]) * n[m] * d0[m] + 2 * es[m] * d0[m]
    d3 = recs["dim"][:, 3].astype(np.int64)
    hk = np.where(d3 > 0, d3, d0)  # key/value heads (grouped-query attention)
    m = op == OP_ROPE
    out[m] = 2 * n[m] * (d0[m] + hk[m]) * d1[m] * es[m]
    m = op == OP_KV_APPEND
    out[m] = 4 * n[m] * d0[m] * d1[m] * es[m]
    m = op == OP_SDPA
    if m.any():
        L = recs["lens"][m].astype(np.int64)
        bmask = np.arange(8)[None, :] < n[m][:, None]
        keys = (L * bmask).sum(axis=1)
        out[m] = (n[m] * d0[m] * d1[m] * (es[m] + eo[m])) + 2 * keys * hk[m] * d1[m] * es[m]
    m = op == OP_GEMV
    out[m] = es[m] * d0[m] + es[m] * d0[m] * d1[m] + eo[m] * d1[m]
    m = op == OP_COPY
    out[m] = 2 * n[m]
    m = op == OP_MATMUL
    out[m] = es[m] * n[m] * d0[m] + es[m] * d1[m] * d0[m] + eo[m] * n[m] * d1[m]
    return out
