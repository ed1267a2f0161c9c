"""PyTorch integration: route eligible aten ops to the persistent executor.

The GPUOS digest page (section 3 Q2, "PyTorch integration") intercepts
operations with a TorchDispatch hook and decides per operation, with a
four-dimensional filter, whether it goes to the ring or down PyTorch's normal
path (hybrid execution):
  1. operation type -- element-wise ops, small reductions and cache updates
     first;
  2. tensor size -- small tensors gain the most;
  3. execution context -- operations of high-frequency inner loops first;
  4. current load -- when the ring is full, fall back to a normal launch.
Operations the filter refuses (large GEMMs, anything without a body here)
run as usual.

Here:
  1. the aten ops with an executor body: add/mul (same shape and dtype,
     alpha 1, also in place), relu, gelu(tanh), softmax and sum/amax/amin
     over the last dimension, contiguous same-size copy_ (cache updates),
     and small bf16 matmuls x[M, K] @ W^T with M <= 64 (mm with the weight
     given as the transpose of a contiguous [N, K] tensor, which is what a
     linear layer without bias calls); fp32 or bf16, contiguous, on the
     context's device;
  2. at most `max_elems` elements per operand (for a matmul, of the
     activation: the weights of a small matmul are read once either way);
  3. an op is routed once its (op, shapes, dtype) key has been seen
     `hot_after` times inside the mode (a recurring inner-loop op), so
     one-off calls stay on the normal path;
  4. each routed op is submitted without blocking; E_FULL sends it to the
     normal path instead.
Ordering between the two paths is kept per storage: a normal op that
touches storage an in-flight routed op uses waits for the executor first
(gpuos_sync), and a routed op that touches storage a normal op wrote waits
for torch's stream first.  Routed ops keep references to their tensors
until the executor has completed them, so the caching allocator cannot hand
that memory out early.

This module marshals arguments only: every routed operation runs in the
executor's kernels (libgpuos.so); nothing is computed here.  While the mode
is active, do not empty torch's allocator cache (it would free device memory
under a resident kernel).
"""
from __future__ import annotations

import collections
from dataclasses import dataclass, field
from typing import Any, Dict, List, Optional, Tuple

import torch
from torch.utils._python_dispatch import TorchDispatchMode

from . import gpuos as G

aten = torch.ops.aten
_DT = {torch.float32: G.GPUOS_F32, torch.bfloat16: G.GPUOS_BF16}

# aten op -> executor kind and the shape rule it follows
_ELEMENTWISE_BINARY = {aten.add.Tensor: G.GPUOS_OP_ADD, aten.mul.Tensor: G.GPUOS_OP_MUL,
                       aten.add_.Tensor: G.GPUOS_OP_ADD, aten.mul_.Tensor: G.GPUOS_OP_MUL}
_ELEMENTWISE_UNARY = {aten.relu.default: G.GPUOS_OP_RELU, aten.relu_.default: G.GPUOS_OP_RELU,
                      aten.gelu.default: G.GPUOS_OP_GELU, aten.gelu_.default: G.GPUOS_OP_GELU}
_INPLACE = {aten.add_.Tensor, aten.mul_.Tensor, aten.relu_.default, aten.gelu_.default}
_ROW_REDUCE = {aten.sum.dim_IntList: G.GPUOS_OP_SUM, aten.amax.default: G.GPUOS_OP_MAX,
               aten.amin.default: G.GPUOS_OP_MIN}
# ops that neither read nor write tensor data (metadata or fresh allocation)
_NO_DATA = {aten.empty.memory_format, aten.empty_strided.default, aten.empty_like.default,
            aten.detach.default, aten.alias.default, aten.lift_fresh.default}


@dataclass
class Decision:
    route: bool
    reason: str                 # why not, or the kind's name when routed
    kind: int = -1
    inputs: Tuple = ()          # tensors read
    out: Optional[torch.Tensor] = None   # the output when it exists already (in place, copy_)
    out_shape: Tuple = ()
    out_dtype: Any = None
    rows: int = 0
    h: int = 0


@dataclass
class RouteStats:
    routed: collections.Counter = field(default_factory=collections.Counter)
    fallback: collections.Counter = field(default_factory=collections.Counter)


class RoutingFilter:
    """The four-dimensional filter (pure host logic, no device calls)."""

    def __init__(self, max_elems: int = 1 << 20, hot_after: int = 2, device_type: str = "cuda"):
        self.max_elems = max_elems
        self.hot_after = hot_after
        self.device_type = device_type
        self.seen: collections.Counter = collections.Counter()

    def _tensor_ok(self, t) -> Optional[str]:
        if not isinstance(t, torch.Tensor):
            return "not a tensor"
        if t.device.type != self.device_type:
            return "device"
        if t.dtype not in _DT:
            return "dtype"
        if not t.is_contiguous():
            return "layout"
        if t.numel() > self.max_elems:
            return "size"
        return None

    def decide(self, func, args, kwargs) -> Decision:
        kwargs = kwargs or {}
        d = self._op_type(func, args, kwargs)
        if not d.route:
            return d
        # dimension 2: size (checked per operand in _tensor_ok) and
        # dimension 3: execution context (a recurring key)
        key = (func, tuple(tuple(t.shape) for t in d.inputs), d.inputs[0].dtype)
        self.seen[key] += 1
        if self.seen[key] < self.hot_after:
            return Decision(False, "cold")
        return d

    # dimension 1: operation type (and the operand shapes its body takes)
    def _op_type(self, func, args, kwargs) -> Decision:
        if func in _ELEMENTWISE_BINARY:
            if len(args) < 2 or kwargs.get("alpha", 1) != 1:
                return Decision(False, "op form")
            a, b = args[0], args[1]
            for t in (a, b):
                why = self._tensor_ok(t)
                if why:
                    return Decision(False, why)
            if a.shape != b.shape:
                return Decision(False, "broadcast")
            if a.dtype != b.dtype or a.device != b.device:
                return Decision(False, "mixed operands")
            out = a if func in _INPLACE else None
            return Decision(True, "elementwise", _ELEMENTWISE_BINARY[func], (a, b), out, tuple(a.shape), a.dtype)
        if func in _ELEMENTWISE_UNARY:
            a = args[0]
            why = self._tensor_ok(a)
            if why:
                return Decision(False, why)
            if func in (aten.gelu.default, aten.gelu_.default) and kwargs.get("approximate", "none") != "tanh":
                return Decision(False, "gelu variant")
            out = a if func in _INPLACE else None
            return Decision(True, "elementwise", _ELEMENTWISE_UNARY[func], (a,), out, tuple(a.shape), a.dtype)
        if func in _ROW_REDUCE:
            a = args[0]
            why = self._tensor_ok(a)
            if why:
                return Decision(False, why)
            dims = args[1] if len(args) > 1 else kwargs.get("dim")
            keep = args[2] if len(args) > 2 else kwargs.get("keepdim", False)
            if a.dim() == 0 or dims is None or len(dims) != 1 or dims[0] % a.dim() != a.dim() - 1:
                return Decision(False, "reduction dims")
            if kwargs.get("dtype") not in (None, a.dtype) or (len(args) > 3 and args[3] not in (None, a.dtype)):
                return Decision(False, "dtype")
            h = a.shape[-1]
            if h == 0:
                return Decision(False, "empty rows")
            shape = tuple(a.shape[:-1]) + ((1,) if keep else ())
            return Decision(True, "reduction", _ROW_REDUCE[func], (a,), None, shape, a.dtype, a.numel() // h, h)
        if func is aten._softmax.default:
            a, dim, half = args[0], args[1], args[2]
            why = self._tensor_ok(a)
            if why:
                return Decision(False, why)
            if a.dim() == 0 or dim % a.dim() != a.dim() - 1 or half:
                return Decision(False, "softmax dim")
            h = a.shape[-1]
            if h == 0:
                return Decision(False, "empty rows")
            return Decision(True, "softmax", G.GPUOS_OP_SOFTMAX, (a,), None, tuple(a.shape), a.dtype, a.numel() // h, h)
        if func is aten.mm.default:
            a, b = args[0], args[1]
            why = self._tensor_ok(a)
            if why:
                return Decision(False, why)
            if not isinstance(b, torch.Tensor) or b.device != a.device or b.dtype != a.dtype:
                return Decision(False, "mixed operands")
            if a.dtype != torch.bfloat16 or a.dim() != 2 or b.dim() != 2 or not b.t().is_contiguous():
                return Decision(False, "matmul form")
            M, K = a.shape
            N = b.shape[1]
            if M == 0 or M > 64 or K == 0 or K % 32 != 0 or N == 0 or b.shape[0] != K:
                return Decision(False, "matmul size")
            return Decision(True, "small matmul", G.GPUOS_OP_MATMUL, (a, b), None, (M, N), a.dtype, M, K)
        if func is aten.copy_.default:
            dst, src = args[0], args[1]
            for t in (dst, src):
                why = self._tensor_ok(t)
                if why:
                    return Decision(False, why)
            if dst.dtype != src.dtype or dst.numel() != src.numel() or (len(args) > 2 and args[2]):
                return Decision(False, "copy form")
            return Decision(True, "cache update", G.GPUOS_OP_COPY, (src,), dst, tuple(dst.shape), dst.dtype)
        return Decision(False, "op type")


def _storages(args) -> List[int]:
    out = []
    for a in args:
        if isinstance(a, torch.Tensor):
            out.append(a.untyped_storage().data_ptr())
        elif isinstance(a, (list, tuple)):
            out += _storages(a)
    return out


class GpuosMode(TorchDispatchMode):
    """Route eligible aten ops to a gpuos context (created on entry unless
    one is given; shut down on exit if created here).  `stats` counts routed
    ops by kind and normal-path ops by reason.

    A context created here has one executor wave per workgroup unless `init`
    says otherwise: the PyTorch kernels of the ops that take the normal path
    run beside the resident executor, and with one wave per CU three SIMDs of
    every CU stay free for them whatever registers they need (an executor
    wave on every SIMD leaves each only what the executor does not use)."""

    def __init__(self, ctx: Optional[int] = None, filter: Optional[RoutingFilter] = None, **init):
        super().__init__()
        self.ctx = ctx
        self.own = ctx is None
        self.init = {"waves_per_wg": 1, **init}
        self.filter = filter or RoutingFilter()
        self.stats = RouteStats()
        self.inflight: collections.deque = collections.deque()  # (seq, tensors kept alive)
        self.gpu_storages: Dict[int, int] = {}   # storage -> last seq of a routed op using it
        self.torch_storages: set = set()         # storages written by normal ops not yet synced
        self.torch_all_dirty = True              # tensors made before entry: unknown state

    # ------------------------------------------------------------ lifecycle
    def __enter__(self):
        if self.ctx is None:
            self.ctx = G.gpuos_init(**self.init)
        return super().__enter__()

    def __exit__(self, *exc):
        try:
            self.flush()
        finally:
            r = super().__exit__(*exc)
            if self.own and self.ctx is not None:
                G.gpuos_shutdown(self.ctx)
                self.ctx = None
        return r

    def flush(self):
        """Wait for every routed op and release their tensors."""
        if self.inflight:
            rc, es, st = G.gpuos_sync(self.ctx, G.GPUOS_SEQ_ALL, 120_000_000_000)
            if rc != G.GPUOS_OK:
                raise G.GpuosError("gpuos_sync", rc)
        self.inflight.clear()
        self.gpu_storages.clear()

    def _retire(self):
        while self.inflight and G.gpuos_query(self.ctx, self.inflight[0][0]) == 1:
            self.inflight.popleft()

    # ------------------------------------------------------------- dispatch
    def __torch_dispatch__(self, func, types, args=(), kwargs=None):
        kwargs = kwargs or {}
        if func in _NO_DATA or func.is_view:
            return func(*args, **kwargs)
        d = self.filter.decide(func, args, kwargs)
        if d.route:
            out = self._submit(d)
            if out is not None:
                self.stats.routed[d.reason] += 1
                return out
            self.stats.fallback["ring full"] += 1
        else:
            self.stats.fallback[d.reason] += 1
        return self._normal(func, args, kwargs)

    def _normal(self, func, args, kwargs):
        touched = _storages(list(args) + list(kwargs.values()))
        self._retire()
        if self.inflight:
            oldest = self.inflight[0][0]
            if any(self.gpu_storages.get(s, -1) >= oldest for s in touched):
                self.flush()
        res = func(*args, **kwargs)
        # what this op wrote is pending on torch's stream: its outputs and,
        # for ops with in-place or out= forms, its arguments
        self.torch_storages.update(_storages([res]))
        if func._schema.is_mutable:
            self.torch_storages.update(touched)
        return res

    def _submit(self, d: Decision) -> Optional[torch.Tensor]:
        out = d.out if d.out is not None else torch.empty(d.out_shape, dtype=d.out_dtype,
                                                          device=d.inputs[0].device)
        tensors = list(d.inputs) + [out]
        st = _storages(tensors)
        if self.torch_all_dirty or any(s in self.torch_storages for s in st):
            if out.device.type == "cuda":
                torch.cuda.current_stream(out.device).synchronize()
            self.torch_storages.clear()
            self.torch_all_dirty = False
        desc = G.new_descs(1)
        dt = _DT[d.inputs[0].dtype]
        desc["op_id"] = d.kind
        desc["flags"] = G.flags(dt)
        desc["input_a"] = d.inputs[0].data_ptr()
        if len(d.inputs) > 1:
            desc["input_b"] = d.inputs[1].data_ptr()
        desc["output"] = out.data_ptr()
        if d.kind == G.GPUOS_OP_COPY:
            desc["size"] = out.numel() * out.element_size()
        elif d.kind == G.GPUOS_OP_MATMUL:
            # b is the transposed view of the [N, K] weight: its storage is Wt
            desc["size"] = d.rows
            desc["dim"][0, 0] = d.h
            desc["dim"][0, 1] = d.out_shape[1]
        elif d.rows:
            desc["size"] = d.rows
            desc["dim"][0, 0] = d.h
        else:
            desc["size"] = out.numel()
        self._retire()
        rc, seq = G.gpuos_submit(self.ctx, desc, 0)
        if rc == G.GPUOS_E_FULL:
            return None
        if rc != G.GPUOS_OK:
            raise G.GpuosError("gpuos_submit", rc)
        self.inflight.append((seq, tensors))
        for s in st:
            self.gpu_storages[s] = seq
        return out
