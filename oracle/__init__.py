"""Python loader for the CPU oracle (gpuos_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product library.  It shares no
code with the HIP path.  It builds liboracle.so with gcc (no -ffast-math, no
FMA contraction) and runs symbolic record streams on host copies of a pool.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gpuos_oracle.c")
# GPUOS_ORACLE_LIB names another build of the same source (the sanitizer
# test loads an AddressSanitizer build this way)
LIB = os.environ.get("GPUOS_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so in place."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared",
               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
               "-o", LIB + ".tmp", SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(LIB + ".tmp", LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if "GPUOS_ORACLE_LIB" not in os.environ and (not os.path.exists(LIB) or
                                                     os.path.getmtime(LIB) < os.path.getmtime(SRC)):
            build(force=True)
        L = ctypes.CDLL(LIB)
        L.orc_run.restype = ctypes.c_int64
        L.orc_run.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                              ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
        L.orc_round_bf16.restype = ctypes.c_uint16
        L.orc_round_bf16.argtypes = [ctypes.c_double]
        L.orc_bf16_to_double.restype = ctypes.c_double
        L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        for nm in ("orc_relu", "orc_gelu"):
            getattr(L, nm).restype = ctypes.c_double
            getattr(L, nm).argtypes = [ctypes.c_double]
        for nm in ("orc_max2", "orc_min2"):
            getattr(L, nm).restype = ctypes.c_double
            getattr(L, nm).argtypes = [ctypes.c_double, ctypes.c_double]
        L.orc_expr_eval.restype = ctypes.c_float
        L.orc_expr_eval.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_float,
                                    ctypes.POINTER(ctypes.c_int32)]
        L.orc_record_size.restype = ctypes.c_int32
        L.orc_run_capture.restype = ctypes.c_int64
        L.orc_run_capture.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


class Pool:
    """Host copies of a stream's buffers (uint8 arrays)."""

    def __init__(self, arrays: Sequence[np.ndarray]):
        self.arrays: List[np.ndarray] = [np.ascontiguousarray(a).view(np.uint8).reshape(-1)
                                         for a in arrays]
        self._refresh()

    @classmethod
    def from_stream(cls, stream) -> "Pool":
        return cls([b.host_bytes() for b in stream.buffers])

    def _refresh(self):
        n = len(self.arrays)
        self._ptrs = (ctypes.c_void_p * n)(*[a.ctypes.data for a in self.arrays])
        self._sizes = np.array([a.nbytes for a in self.arrays], np.int64)

    def copy(self) -> "Pool":
        return Pool([a.copy() for a in self.arrays])

    def run(self, recs: np.ndarray) -> None:
        """Execute records in order, in place on this pool."""
        recs = np.ascontiguousarray(recs)
        assert recs.dtype.itemsize == lib().orc_record_size()
        err = ctypes.c_int32(0)
        rc = lib().orc_run(recs.ctypes.data, len(recs), ctypes.cast(self._ptrs, ctypes.c_void_p),
                           self._sizes.ctypes.data, len(self.arrays), ctypes.byref(err))
        if rc != 0:
            raise OracleError(f"record {-rc - 1} failed with oracle error {err.value}")

    def run_capture(self, rec: np.ndarray, windows) -> List[np.ndarray]:
        """Execute one record in place and return, for each output window
        (buffer, byte offset, bytes, element bytes) -- at most two -- the
        unrounded double of every element the record stored there (NaN where
        it stored nothing)."""
        rec = np.ascontiguousarray(np.asarray(rec).reshape(1))
        assert rec.dtype.itemsize == lib().orc_record_size() and len(windows) <= 2
        outs = [np.full(int(nb) // int(es), np.nan) for (_, _, nb, es) in windows]
        nw = len(windows)
        wb = np.array([w[0] for w in windows] + [0] * (2 - nw), np.int32)
        wo = np.array([w[1] for w in windows] + [0] * (2 - nw), np.int64)
        wn = np.array([w[2] for w in windows] + [0] * (2 - nw), np.int64)
        optr = (ctypes.c_void_p * 2)(*([o.ctypes.data for o in outs] + [None] * (2 - nw)))
        err = ctypes.c_int32(0)
        rc = lib().orc_run_capture(rec.ctypes.data, ctypes.cast(self._ptrs, ctypes.c_void_p),
                                   self._sizes.ctypes.data, len(self.arrays), ctypes.byref(err), nw,
                                   wb.ctypes.data, wo.ctypes.data, wn.ctypes.data,
                                   ctypes.cast(optr, ctypes.c_void_p))
        if rc != 0:
            raise OracleError(f"record failed with oracle error {err.value}")
        return outs

    def view(self, buf: int, dtype, off: int = 0, count: int = -1) -> np.ndarray:
        a = self.arrays[buf][off:]
        v = a.view(np.uint8)
        itemsize = np.dtype(dtype).itemsize
        if count < 0:
            count = v.nbytes // itemsize
        return v[: count * itemsize].view(dtype)


def round_bf16(x: float) -> int:
    return int(lib().orc_round_bf16(float(x)))


def bf16_to_float(h: int) -> float:
    return float(lib().orc_bf16_to_double(int(h)))


def relu(x: float) -> float:
    return lib().orc_relu(float(x))


def gelu(x: float) -> float:
    return lib().orc_gelu(float(x))


def max2(a: float, b: float) -> float:
    return lib().orc_max2(float(a), float(b))


def expr_eval(program, a: float, b: float) -> float:
    """One element of an injected element-wise program (binary32 steps);
    raises ValueError for a malformed program."""
    w = np.ascontiguousarray(np.asarray(program, np.uint32))
    err = ctypes.c_int32(0)
    v = lib().orc_expr_eval(w.ctypes.data, len(w), a, b, ctypes.byref(err))
    if err.value:
        raise ValueError("malformed program")
    return v


def min2(a: float, b: float) -> float:
    return lib().orc_min2(float(a), float(b))
