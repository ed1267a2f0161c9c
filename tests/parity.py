"""Comparison metrics between the HIP path and the oracle.

Tolerances (per op, from the stated bars: bit-exact for add/mul/relu/max/
min/KV append/copy; max relative error 1e-5 fp32 / 1e-2 bf16 for GELU,
softmax, LayerNorm and sum; 2e-3 for decode SDPA with fp32 accumulation).
A plain |g-r|/|r| is ill-posed where an output crosses zero, so each
toleranced op uses the denominator its arithmetic fixes:
  GELU       |g-r| <= tol * max(|r|, 2^-126)
  softmax    |g-r| <= tol * |r|              (outputs are strictly positive)
  LayerNorm  |g-r| <= tol * max(|r|, 1)      (outputs are unit-scale)
  sum        |g-r| <= tol * sum|x_i|         (summation condition number)
  SDPA       |g_d-r_d| <= tol * sum_j p_j |V_jd|
  GEMV       |g_n-r_n| <= tol * sum_k |x_k W_kn|
  matmul     |g_mn-r_mn| <= tol * sum_k |x_mk Wt_nk|
  RoPE       within one bf16 ulp of the exact double result
Toleranced outputs are compared with the oracle's unrounded double (the
value it would round to the output type), so a bf16 output carries its own
rounding only, with no second rounding of the reference and no extra
allowance.  RoPE is compared with the rounded oracle value (its bar is one
bf16 ulp of it).
"""
from __future__ import annotations

import numpy as np

import workloads as W

TOL = {"f32": 1e-5, "bf16": 1e-2, "sdpa": 2e-3}


def as_float(raw: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == W.F32:
        return raw.view(np.float32).astype(np.float64)
    return W.bf16_bits_to_f32(raw.view(np.uint16)).astype(np.float64)


def bits_equal(g: np.ndarray, r: np.ndarray, dtype: int) -> np.ndarray:
    """Element-wise bit equality, NaN compared as a class."""
    if dtype == W.F32:
        gi, ri = g.view(np.uint32), r.view(np.uint32)
        gn = (gi & 0x7FFFFFFF) > 0x7F800000
        rn = (ri & 0x7FFFFFFF) > 0x7F800000
    else:
        gi, ri = g.view(np.uint16), r.view(np.uint16)
        gn = (gi & 0x7FFF) > 0x7F80
        rn = (ri & 0x7FFF) > 0x7F80
    return np.where(gn | rn, gn & rn, gi == ri)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    a = np.abs(x).astype(np.float64)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def rel_check(g: np.ndarray, r: np.ndarray, denom: np.ndarray, tol: float):
    """Returns (ok mask, worst ratio)."""
    err = np.abs(g - r)
    both_nan = np.isnan(g) & np.isnan(r)
    same_inf = np.isinf(g) & np.isinf(r) & (np.sign(g) == np.sign(r))
    ratio = np.where(both_nan | same_inf, 0.0, err / np.maximum(denom, 1e-300))
    ratio = np.where(np.isnan(ratio), np.inf, ratio)
    return ratio <= tol, float(np.max(ratio)) if ratio.size else 0.0
