"""ctypes binding of libgpuos.so (include/gpuos.h), names as in the C ABI.

Argument marshalling only: every step of the dispatch path runs in the HIP
library.  If the library has not been built this module raises; there is no
fallback implementation.
"""
from __future__ import annotations

import atexit
import ctypes
import os
from typing import Optional, Tuple

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("GPUOS_LIB") or os.path.join(_PKG, "libgpuos.so")

# ---- constants (mirror include/gpuos.h) ----
GPUOS_OK, GPUOS_E_INVAL, GPUOS_E_FULL, GPUOS_E_NOOP = 0, -1, -2, -3
GPUOS_E_TIMEOUT, GPUOS_E_DEVICE, GPUOS_E_HIP, GPUOS_E_STATE = -4, -5, -6, -7
GPUOS_ST_OK, GPUOS_ST_BAD_OP, GPUOS_ST_BAD_SHAPE, GPUOS_ST_SPIN = 0, 1, 2, 3
(GPUOS_OP_NOP, GPUOS_OP_ADD, GPUOS_OP_MUL, GPUOS_OP_RELU, GPUOS_OP_GELU, GPUOS_OP_SUM, GPUOS_OP_MAX,
 GPUOS_OP_MIN, GPUOS_OP_SOFTMAX, GPUOS_OP_LAYERNORM, GPUOS_OP_ROPE, GPUOS_OP_KV_APPEND, GPUOS_OP_SDPA,
 GPUOS_OP_GEMV, GPUOS_OP_COPY, GPUOS_OP_EXPR, GPUOS_OP_MATMUL, GPUOS_OP_JIT) = range(18)
GPUOS_KIND_COUNT = 18
GPUOS_KIND_EMPTY = 0xFFFFFFFF
GPUOS_MAX_OPS = 256
(GPUOS_X_LDA, GPUOS_X_LDB, GPUOS_X_CONST, GPUOS_X_MOV, GPUOS_X_ADD, GPUOS_X_SUB, GPUOS_X_MUL, GPUOS_X_DIV,
 GPUOS_X_MIN, GPUOS_X_MAX, GPUOS_X_NEG, GPUOS_X_ABS, GPUOS_X_EXP, GPUOS_X_LOG, GPUOS_X_SQRT, GPUOS_X_TANH,
 GPUOS_X_SIGMOID, GPUOS_X_RELU) = range(1, 19)
GPUOS_EXPR_MAX_INSTR, GPUOS_EXPR_MAX_CONSTS = 32, 16
GPUOS_OP_USER = 64
GPUOS_F32, GPUOS_BF16 = 0, 1
GPUOS_F_ROPE_HALF = 1 << 8
GPUOS_F_SDPA_MASK = 1 << 9
GPUOS_F_KV_PAGED = 1 << 10
GPUOS_INIT_LOOPBACK = 1
GPUOS_INIT_TRACE = 2
GPUOS_INIT_JIT = 4
GPUOS_JIT_MAX_VGPRS, GPUOS_JIT_MAX_AGPRS, GPUOS_JIT_MAX_SGPRS, GPUOS_JIT_MAX_STACK = 96, 32, 102, 0
GPUOS_SUBMIT_BLOCK, GPUOS_SUBMIT_NOHAZARD, GPUOS_SUBMIT_SERIAL = 1, 2, 4
GPUOS_SEQ_ALL = 0xFFFFFFFFFFFFFFFF

ERR_NAMES = {0: "OK", -1: "E_INVAL", -2: "E_FULL", -3: "E_NOOP", -4: "E_TIMEOUT",
             -5: "E_DEVICE", -6: "E_HIP", -7: "E_STATE"}


def flags(in_dtype: int, out_dtype: Optional[int] = None) -> int:
    return int(in_dtype) | (int(in_dtype if out_dtype is None else out_dtype) << 4)


DESC_DTYPE = np.dtype([
    ("op_id", "<u4"), ("flags", "<u4"), ("seq", "<u8"),
    ("input_a", "<u8"), ("input_b", "<u8"), ("output", "<u8"), ("size", "<u8"),
    ("dim", "<u4", (4,)), ("aux", "<u8", (3,)),
    ("dep_delta", "<u2", (6,)), ("dep_range", "<u2"), ("table_version", "<u2"),
    ("param", "<u4", (6,)),
])
assert DESC_DTYPE.itemsize == 128


def new_descs(n: int) -> np.ndarray:
    return np.zeros(n, DESC_DTYPE)


def set_param_f(d: np.ndarray, idx: int, val) -> None:
    """Write float parameter word `idx` (0..5) of descriptor(s) d."""
    d["param"][..., idx] = np.asarray(val, np.float32).view(np.uint32)


def set_lens(d: np.ndarray, lens) -> None:
    """Write per-batch lengths lens[0..7] (uint16) into param words 0..3."""
    L = np.zeros(d.shape + (8,), np.uint16)
    lens = np.asarray(lens)
    L[..., : lens.shape[-1]] = lens
    d["param"][..., 0:4] = L.view(np.uint32).reshape(d.shape + (4,))


class GpuosError(RuntimeError):
    def __init__(self, fn: str, rc: int):
        super().__init__(f"{fn} failed: {ERR_NAMES.get(rc, rc)} ({rc})")
        self.rc = rc


class InitParams(ctypes.Structure):
    _fields_ = [("device", ctypes.c_int32), ("ring_entries", ctypes.c_uint32),
                ("num_wgs", ctypes.c_uint32), ("waves_per_wg", ctypes.c_uint32),
                ("backoff_max", ctypes.c_uint32), ("flags", ctypes.c_uint32),
                ("hip_stream", ctypes.c_void_p), ("scratch_bytes", ctypes.c_uint64),
                ("unit_queue_log2", ctypes.c_uint32), ("spin_limit_ms", ctypes.c_uint32),
                ("units_per_wave", ctypes.c_uint32), ("idle_exit_ms", ctypes.c_uint32)]


class Stats(ctypes.Structure):
    _fields_ = [("submitted", ctypes.c_uint64), ("completed", ctypes.c_uint64),
                ("full_rejections", ctypes.c_uint64), ("launches", ctypes.c_uint64),
                ("last_launch_ms", ctypes.c_float), ("total_launch_ms", ctypes.c_float),
                ("units", ctypes.c_uint64), ("fetch_batches", ctypes.c_uint64),
                ("fetched", ctypes.c_uint64), ("dep_waits", ctypes.c_uint64),
                ("num_wgs", ctypes.c_uint32), ("waves_per_wg", ctypes.c_uint32),
                ("ring_entries", ctypes.c_uint32), ("cu_count", ctypes.c_uint32),
                ("next_seq", ctypes.c_uint64), ("deps_explicit", ctypes.c_uint64),
                ("deps_range", ctypes.c_uint64), ("ns_submit", ctypes.c_uint64),
                ("ns_blocked", ctypes.c_uint64), ("ns_annotate", ctypes.c_uint64),
                ("idle_exits", ctypes.c_uint64)]


_lib = None
EXPORTS = [
    "gpuos_abi_version", "gpuos_init", "gpuos_register_op", "gpuos_submit", "gpuos_submit_bursts", "gpuos_sync",
    "gpuos_query", "gpuos_pause", "gpuos_resume", "gpuos_shutdown", "gpuos_stats_get",
    "gpuos_loopback_order", "gpuos_eager_submit", "gpuos_eager_scratch_bytes", "gpuos_graph_build",
    "gpuos_graph_launch", "gpuos_graph_destroy", "gpuos_null_launch_bench", "gpuos_latency_bench", "gpuos_trace_read",
    "gpuos_hbm_probe", "gpuos_register_expr", "gpuos_ring_peek",
    "gpuos_eager_submit_static", "gpuos_hbm_probe_grid", "gpuos_register_jit", "gpuos_jit_source",
]


class JitInfo(ctypes.Structure):
    _fields_ = [("compile_ms", ctypes.c_double), ("load_ms", ctypes.c_double), ("flip_ms", ctypes.c_double),
                ("vgprs", ctypes.c_uint32), ("agprs", ctypes.c_uint32), ("sgprs", ctypes.c_uint32),
                ("stack_bytes", ctypes.c_uint32), ("code_bytes", ctypes.c_uint64), ("reused", ctypes.c_uint32),
                ("pad", ctypes.c_uint32)]

TRACE_DTYPE = np.dtype([("seq", "<u8"), ("tile", "<u4"), ("hw", "<u4"), ("t_claim", "<u8"), ("t_ready", "<u8"),
                        ("t_body", "<u8"), ("t_done", "<u8"), ("unit", "<u8"), ("pad", "<u8")])


def lib():
    """Load libgpuos.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    # One HIP runtime per process: torch ships its own libamdhip64.so.7, and
    # whichever copy is loaded first serves every library that needs that
    # soname.  Loading torch first binds libgpuos.so to torch's runtime, the
    # same one torch's allocations and streams come from; loading libgpuos.so
    # first would leave torch on a runtime it was not built with (its GPU
    # initialisation then fails).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    vp, u32, u64, i64 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int64
    sig = {
        "gpuos_abi_version": ([], ctypes.c_int),
        "gpuos_init": ([ctypes.POINTER(InitParams), ctypes.POINTER(vp)], ctypes.c_int),
        "gpuos_register_op": ([vp, u32, u32, vp, u32], ctypes.c_int),
        "gpuos_submit": ([vp, vp, u32, u32, ctypes.POINTER(u64)], ctypes.c_int),
        "gpuos_submit_bursts": ([vp, vp, vp, u32, u32, ctypes.POINTER(u64), ctypes.POINTER(u64)], ctypes.c_int),
        "gpuos_sync": ([vp, u64, i64, ctypes.POINTER(u64), ctypes.POINTER(u32)], ctypes.c_int),
        "gpuos_query": ([vp, u64], ctypes.c_int),
        "gpuos_pause": ([vp, i64], ctypes.c_int),
        "gpuos_resume": ([vp], ctypes.c_int),
        "gpuos_shutdown": ([vp], ctypes.c_int),
        "gpuos_stats_get": ([vp, ctypes.POINTER(Stats)], ctypes.c_int),
        "gpuos_loopback_order": ([vp, vp, u64, ctypes.POINTER(u64)], ctypes.c_int),
        "gpuos_eager_submit": ([vp, u32, vp, vp, u64], ctypes.c_int),
        "gpuos_eager_scratch_bytes": ([vp, u32], u64),
        "gpuos_graph_build": ([vp, u32, vp, vp, u64, ctypes.POINTER(vp)], ctypes.c_int),
        "gpuos_graph_launch": ([vp, vp], ctypes.c_int),
        "gpuos_graph_destroy": ([vp], ctypes.c_int),
        "gpuos_trace_read": ([vp, vp, u64, ctypes.POINTER(u64)], ctypes.c_int),
        "gpuos_latency_bench": ([vp, vp, u32, vp], ctypes.c_int),
        "gpuos_null_launch_bench": ([vp, u32, ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
        "gpuos_hbm_probe": ([vp, vp, u64, u32, u32, vp, ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
        "gpuos_register_expr": ([vp, u32, vp, u32], ctypes.c_int),
        "gpuos_ring_peek": ([vp, u64, vp, vp], ctypes.c_int),
        "gpuos_eager_submit_static": ([vp, u32, vp], ctypes.c_int),
        "gpuos_hbm_probe_grid": ([vp, vp, u64, u32, u32, u32, vp, ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
        "gpuos_register_jit": ([vp, u32, vp, u32, ctypes.POINTER(JitInfo)], ctypes.c_int),
        "gpuos_jit_source": ([vp, u32, vp, u64, ctypes.POINTER(u64)], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def _check(fn: str, rc: int) -> int:
    if rc != GPUOS_OK:
        raise GpuosError(fn, rc)
    return rc


def _descs_ptr(descs: np.ndarray):
    assert descs.dtype == DESC_DTYPE and descs.flags["C_CONTIGUOUS"]
    return descs.ctypes.data


# ---------------------------------------------------------------- functions
def gpuos_abi_version() -> int:
    return lib().gpuos_abi_version()


# Contexts not yet shut down.  A resident executor kernel never finishes by
# itself, and the HIP runtime waits for running kernels when the process
# exits, so contexts left open (an exception, a forgotten shutdown) are shut
# down at interpreter exit.
_LIVE = set()


def _shutdown_live():
    for c in list(_LIVE):
        gpuos_shutdown(c)


atexit.register(_shutdown_live)


def gpuos_init(device: int = 0, ring_entries: int = 0, num_wgs: int = 0, waves_per_wg: int = 0,
               backoff_max: int = 0, flags: int = 0, hip_stream: int = 0, scratch_bytes: int = 0,
               unit_queue_log2: int = 0, spin_limit_ms: int = 0, units_per_wave: int = 0,
               idle_exit_ms: int = 0) -> int:
    p = InitParams(device, ring_entries, num_wgs, waves_per_wg, backoff_max, flags,
                   hip_stream or None, scratch_bytes, unit_queue_log2, spin_limit_ms, units_per_wave,
                   idle_exit_ms)
    out = ctypes.c_void_p()
    _check("gpuos_init", lib().gpuos_init(ctypes.byref(p), ctypes.byref(out)))
    _LIVE.add(out.value)
    return out.value


def gpuos_register_op(ctx: int, op_id: int, kind: int, consts=None) -> int:
    buf, n = None, 0
    if consts is not None:
        arr = np.ascontiguousarray(np.asarray(consts, np.float32).reshape(-1))
        buf, n = arr.ctypes.data, arr.nbytes
    return lib().gpuos_register_op(ctx, op_id, kind, buf, n)


def gpuos_register_expr(ctx: int, op_id: int, program) -> int:
    """Bind op_id to an element-wise program (uint32 words, gpuos.h layout)."""
    w = np.ascontiguousarray(np.asarray(program, np.uint32).reshape(-1))
    return lib().gpuos_register_expr(ctx, op_id, w.ctypes.data if len(w) else None, len(w))


def gpuos_register_jit(ctx: int, op_id: int, program) -> Tuple[int, dict]:
    """Bind op_id to the program compiled at run time.  Returns (rc, info)
    with the compile, load and flip times and the code's resources."""
    w = np.ascontiguousarray(np.asarray(program, np.uint32).reshape(-1))
    info = JitInfo()
    rc = lib().gpuos_register_jit(ctx, op_id, w.ctypes.data if len(w) else None, len(w), ctypes.byref(info))
    return rc, {k: getattr(info, k) for k, _ in JitInfo._fields_ if k != "pad"}


def gpuos_jit_source(program) -> Tuple[int, str]:
    """The HIP source gpuos_register_jit compiles for `program`."""
    w = np.ascontiguousarray(np.asarray(program, np.uint32).reshape(-1))
    n = ctypes.c_uint64(0)
    rc = lib().gpuos_jit_source(w.ctypes.data if len(w) else None, len(w), None, 0, ctypes.byref(n))
    if rc != GPUOS_OK:
        return rc, ""
    buf = ctypes.create_string_buffer(n.value + 1)
    rc = lib().gpuos_jit_source(w.ctypes.data, len(w), buf, n.value + 1, ctypes.byref(n))
    return rc, buf.value.decode()


def gpuos_submit(ctx: int, descs: np.ndarray, flags: int = 0) -> Tuple[int, int]:
    """Returns (rc, first_seq)."""
    first = ctypes.c_uint64(0)
    rc = lib().gpuos_submit(ctx, _descs_ptr(descs), len(descs), flags, ctypes.byref(first))
    return rc, first.value


def gpuos_submit_bursts(ctx: int, descs: np.ndarray, bursts: np.ndarray, flags: int = 0) -> Tuple[int, int, int]:
    """Returns (rc, first_seq, n_submitted)."""
    b = np.ascontiguousarray(bursts, dtype=np.uint32)
    assert int(b.sum()) <= len(descs)
    first, n = ctypes.c_uint64(0), ctypes.c_uint64(0)
    rc = lib().gpuos_submit_bursts(ctx, _descs_ptr(descs), b.ctypes.data, len(b), flags, ctypes.byref(first),
                                   ctypes.byref(n))
    return rc, first.value, n.value


def gpuos_sync(ctx: int, upto: int = GPUOS_SEQ_ALL, timeout_ns: int = -1) -> Tuple[int, int, int]:
    """Returns (rc, err_seq, err_status)."""
    es, st = ctypes.c_uint64(0), ctypes.c_uint32(0)
    rc = lib().gpuos_sync(ctx, upto, timeout_ns, ctypes.byref(es), ctypes.byref(st))
    return rc, es.value, st.value


def gpuos_query(ctx: int, seq: int) -> int:
    return lib().gpuos_query(ctx, seq)


def gpuos_pause(ctx: int, timeout_ns: int = -1) -> int:
    return lib().gpuos_pause(ctx, timeout_ns)


def gpuos_resume(ctx: int) -> int:
    return lib().gpuos_resume(ctx)


def gpuos_shutdown(ctx: int) -> int:
    _LIVE.discard(ctx)
    return lib().gpuos_shutdown(ctx)


def gpuos_stats_get(ctx: int) -> dict:
    s = Stats()
    _check("gpuos_stats_get", lib().gpuos_stats_get(ctx, ctypes.byref(s)))
    return {k: getattr(s, k) for k, _ in Stats._fields_}


def gpuos_loopback_order(ctx: int) -> np.ndarray:
    n = ctypes.c_uint64(0)
    _check("gpuos_loopback_order", lib().gpuos_loopback_order(ctx, None, 0, ctypes.byref(n)))
    out = np.zeros(n.value, np.uint64)
    _check("gpuos_loopback_order", lib().gpuos_loopback_order(ctx, out.ctypes.data, n.value, ctypes.byref(n)))
    return out


def gpuos_eager_scratch_bytes(descs: np.ndarray) -> int:
    return int(lib().gpuos_eager_scratch_bytes(_descs_ptr(descs), len(descs)))


def gpuos_eager_submit(descs: np.ndarray, hip_stream: int, scratch: int, scratch_bytes: int) -> int:
    return lib().gpuos_eager_submit(_descs_ptr(descs), len(descs), hip_stream or None, scratch or None,
                                    scratch_bytes)


GPUOS_EAGER_STATIC_SCRATCH_BYTES = 16 << 20


def gpuos_eager_submit_static(descs: np.ndarray, hip_stream: int) -> int:
    """gpuos_eager_submit with the library's static scratch (no allocation)."""
    return lib().gpuos_eager_submit_static(_descs_ptr(descs), len(descs), hip_stream or None)


def gpuos_graph_build(descs: np.ndarray, hip_stream: int, scratch: int, scratch_bytes: int) -> int:
    ge = ctypes.c_void_p()
    _check("gpuos_graph_build", lib().gpuos_graph_build(_descs_ptr(descs), len(descs), hip_stream or None,
                                                        scratch or None, scratch_bytes, ctypes.byref(ge)))
    return ge.value


def gpuos_graph_launch(graph_exec: int, hip_stream: int) -> int:
    return lib().gpuos_graph_launch(graph_exec, hip_stream or None)


def gpuos_graph_destroy(graph_exec: int) -> int:
    return lib().gpuos_graph_destroy(graph_exec)


def gpuos_null_launch_bench(hip_stream: int, n: int) -> Tuple[float, float]:
    a, s = ctypes.c_double(0), ctypes.c_double(0)
    _check("gpuos_null_launch_bench",
           lib().gpuos_null_launch_bench(hip_stream or None, n, ctypes.byref(a), ctypes.byref(s)))
    return a.value, s.value


def gpuos_latency_bench(ctx: int, descs: np.ndarray) -> np.ndarray:
    """Closed-loop latency (us) of each descriptor, submitted alone and waited for."""
    out = np.zeros(len(descs), np.float64)
    _check("gpuos_latency_bench", lib().gpuos_latency_bench(ctx, _descs_ptr(descs), len(descs), out.ctypes.data))
    return out


def gpuos_hbm_probe(src: int, dst: int, nbytes: int, mode: int, reps: int, hip_stream: int) -> float:
    """Achievable GB/s: mode 0 reads nbytes at src, mode 1 copies src -> dst."""
    g = ctypes.c_double(0)
    _check("gpuos_hbm_probe", lib().gpuos_hbm_probe(src, dst, nbytes, mode, reps, hip_stream or None, ctypes.byref(g)))
    return g.value


def gpuos_ring_peek(ctx: int, seq: int) -> Tuple[int, np.ndarray, np.ndarray]:
    """(rc, descriptor as committed, 56 side dependency deltas)."""
    d = new_descs(1)
    ex = np.zeros(56, np.uint16)
    rc = lib().gpuos_ring_peek(ctx, seq, d.ctypes.data, ex.ctypes.data)
    return rc, d[0], ex


def gpuos_hbm_probe_grid(src: int, dst: int, nbytes: int, mode: int, reps: int, workgroups: int,
                         hip_stream: int) -> float:
    g = ctypes.c_double(0)
    _check("gpuos_hbm_probe_grid", lib().gpuos_hbm_probe_grid(src, dst, nbytes, mode, reps, workgroups,
                                                                hip_stream or None, ctypes.byref(g)))
    return g.value


def gpuos_trace_read(ctx: int, max_records: int = 1 << 20) -> np.ndarray:
    """Trace of the last finished launch (records with t_done == 0 are unused)."""
    out = np.zeros(max_records, TRACE_DTYPE)
    n = ctypes.c_uint64(0)
    _check("gpuos_trace_read", lib().gpuos_trace_read(ctx, out.ctypes.data, max_records, ctypes.byref(n)))
    return out[out["t_done"] != 0]
