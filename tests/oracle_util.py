"""Helpers for driving the oracle on hand-built pools in the CPU pin tests."""
import numpy as np

import oracle
import workloads as W


def rec(op, dtype=W.F32, out_dtype=None, size=0, dim=(), fparam=(), lens=(), flags=0, **roles):
    r = np.zeros(1, W.REC_DTYPE)
    r["buf"] = -1
    r["op"] = op
    r["dtype"] = dtype
    r["out_dtype"] = dtype if out_dtype is None else out_dtype
    r["flags"] = flags
    r["size"] = size
    r["dim"][0, :len(dim)] = dim
    r["fparam"][0, :len(fparam)] = fparam
    r["lens"][0, :len(lens)] = lens
    idx = {"a": W.A, "b": W.B, "out": W.OUT, "aux0": W.AUX0, "aux1": W.AUX1, "aux2": W.AUX2}
    for k, v in roles.items():
        bi, off = v if isinstance(v, tuple) else (v, 0)
        r["buf"][0, idx[k]] = bi
        r["off"][0, idx[k]] = off
    return r


def run(recs, arrays):
    """Run records on copies of `arrays`; return the resulting arrays with
    their original dtypes."""
    dts = [a.dtype for a in arrays]
    shapes = [a.shape for a in arrays]
    pool = oracle.Pool([np.array(a, copy=True) for a in arrays])
    pool.run(np.concatenate(recs) if isinstance(recs, list) else recs)
    return [pool.arrays[i].view(dts[i]).reshape(shapes[i]) for i in range(len(arrays))]


def f32_bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def bf16(x):
    """fp32 values -> bf16 bits via torch (a library conversion, not the oracle's)."""
    return W.to_bf16_bits(np.asarray(x, np.float32))


def bf16_val(bits):
    return W.bf16_bits_to_f32(np.asarray(bits, np.uint16))
