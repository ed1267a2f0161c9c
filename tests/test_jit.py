"""Compiled operator injection on the host (no GPU): the source template,
program validation, the compile with hipRTC and the resource check against
the budget the executor reserves, the reuse of compiled code, the refusal
on contexts made without GPUOS_INIT_JIT, the compiler the code comes from,
the resources of the executor build that calls injected code, and a
loopback stream through injected op ids."""
import os
import re
import subprocess

import numpy as np
import pytest

import workloads as W
from persistent_micro_dispatch_amd import gpuos as G

X, P = W.xins, W.program
ADD = P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_ADD, 0, 1, 2)])
TANH = P([X(W.X_LDA, 1), X(W.X_TANH, 0, 1)])


def test_source_substitutes_the_program():
    prog = P([X(W.X_LDA, 1), X(W.X_CONST, 2, 0, 0, 0), X(W.X_MUL, 0, 1, 2), X(W.X_SQRT, 3, 0),
              X(W.X_MAX, 0, 0, 3)], [2.5])
    rc, src = G.gpuos_jit_source(prog)
    assert rc == 0
    body = src[src.index("float f(float a, float b)"):src.index("return r0;")]
    steps = re.findall(r"\{ const float t = (.*?); (r\d) = t; \}", body)
    assert steps == [("a", "r1"), ("__uint_as_float(0x40200000u)", "r2"), ("r1 * r2", "r0"),
                     ("sqrtf(r0)", "r3"), ("tmax(r0, r3)", "r0")]
    assert "#define USES_B false" in src and "#define TILE_BYTES 4096u" in src
    assert "#define USES_B true" in G.gpuos_jit_source(ADD)[1]
    for name in ("gpuos_jit_f32", "gpuos_jit_bf16", "gpuos_jit_f32_addr", "gpuos_jit_bf16_addr", "gpuos_jit_probe"):
        assert name in src


@pytest.mark.parametrize("bad", [
    [],                                                   # empty
    [0],                                                  # no instructions
    [1],                                                  # missing instruction word
    P([X(W.X_LDA, 4)]),                                   # register out of range
    P([X(W.X_CONST, 0, 0, 0, 1)], [1.0]),                 # constant index past the table
    P([X(19, 0, 1)]),                                     # unknown op
    [33] + [X(W.X_LDA, 0)] * 33,                          # too many instructions
])
def test_malformed_programs_are_refused(bad):
    assert G.gpuos_jit_source(bad)[0] == G.GPUOS_E_INVAL
    ctx = G.gpuos_init(flags=G.GPUOS_INIT_LOOPBACK | G.GPUOS_INIT_JIT)
    try:
        assert G.gpuos_register_jit(ctx, 100, bad)[0] == G.GPUOS_E_INVAL
    finally:
        G.gpuos_shutdown(ctx)


def test_register_refused_without_jit_flag_and_out_of_range():
    ctx = G.gpuos_init(flags=G.GPUOS_INIT_LOOPBACK)
    try:
        assert G.gpuos_register_jit(ctx, 100, ADD)[0] == G.GPUOS_E_INVAL
    finally:
        G.gpuos_shutdown(ctx)
    ctx = G.gpuos_init(flags=G.GPUOS_INIT_LOOPBACK | G.GPUOS_INIT_JIT)
    try:
        assert G.gpuos_register_jit(ctx, 256, ADD)[0] == G.GPUOS_E_NOOP
        # the kind itself cannot be bound with register_op
        assert G.gpuos_register_op(ctx, 100, G.GPUOS_OP_JIT) == G.GPUOS_E_INVAL
    finally:
        G.gpuos_shutdown(ctx)
    # the build that calls injected code holds one unit per wave
    with pytest.raises(G.GpuosError):
        G.gpuos_init(flags=G.GPUOS_INIT_LOOPBACK | G.GPUOS_INIT_JIT, units_per_wave=2)


def test_compile_fits_budget_and_is_reused(tmp_path):
    dump = tmp_path / "jit.co"
    os.environ["GPUOS_JIT_DUMP"] = str(dump)
    ctx = G.gpuos_init(flags=G.GPUOS_INIT_LOOPBACK | G.GPUOS_INIT_JIT)
    try:
        rc, info = G.gpuos_register_jit(ctx, 100, TANH)
        assert rc == 0, info
        assert 0 < info["vgprs"] <= G.GPUOS_JIT_MAX_VGPRS
        assert info["agprs"] <= G.GPUOS_JIT_MAX_AGPRS
        assert 0 < info["sgprs"] <= G.GPUOS_JIT_MAX_SGPRS
        assert info["stack_bytes"] == 0 and info["reused"] == 0 and info["code_bytes"] > 0
        assert info["compile_ms"] > 0
        rc, again = G.gpuos_register_jit(ctx, 101, TANH)
        assert rc == 0 and again["reused"] == 1 and again["compile_ms"] == 0
    finally:
        del os.environ["GPUOS_JIT_DUMP"]
        G.gpuos_shutdown(ctx)
    # the code object was made by the same compiler as the executor
    llvm = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin")
    com = subprocess.run([os.path.join(llvm, "llvm-readelf"), "-p", ".comment", str(dump)],
                         capture_output=True, text=True, check=True).stdout
    hipcc = subprocess.run(["hipcc", "--version"], capture_output=True, text=True, check=True).stdout
    ver = re.search(r"AMD clang version \S+ \(\S+ (\S+ \d+ \w+)\)", hipcc).group(1)
    assert ver in com, (ver, com)


def test_executor_build_holds_the_injected_code_budget():
    from persistent_micro_dispatch_amd import _build
    obj = os.path.join(_build.BUILD, "gpuos_device.hip.o")
    if not os.path.exists(obj):
        pytest.skip("library not built in this tree")
    res = _build.jit_kernel_resources(obj)
    total, agpr, sgpr = int(res["vgpr_count"]), int(res["agpr_count"]), int(res["sgpr_count"])
    assert total - agpr >= G.GPUOS_JIT_MAX_VGPRS and agpr >= G.GPUOS_JIT_MAX_AGPRS
    assert sgpr >= G.GPUOS_JIT_MAX_SGPRS and total <= _build.EXECUTOR_MAX_REGS
    assert res["uses_dynamic_stack"] == "true"


def test_loopback_stream_through_injected_op_ids():
    """Descriptors of an injected op id are ordered by the same hazard
    tracking as built-in ones (the loopback consumer checks the order)."""
    ctx = G.gpuos_init(flags=G.GPUOS_INIT_LOOPBACK | G.GPUOS_INIT_JIT, ring_entries=64)
    try:
        assert G.gpuos_register_jit(ctx, 130, ADD)[0] == 0
        d = G.new_descs(300)
        base = 1 << 40
        for i in range(300):
            d[i]["op_id"] = 130
            d[i]["flags"] = G.flags(G.GPUOS_F32)
            d[i]["size"] = 1000
            d[i]["input_a"] = base + (i % 7) * 8192
            d[i]["input_b"] = base + ((i + 3) % 7) * 8192
            d[i]["output"] = base + ((i * 5) % 7) * 8192
        rc, first = G.gpuos_submit(ctx, d[:64], G.GPUOS_SUBMIT_BLOCK)
        assert rc == 0
        for i in range(64, 300, 64):
            assert G.gpuos_submit(ctx, d[i:i + 64], G.GPUOS_SUBMIT_BLOCK)[0] == 0
        assert G.gpuos_sync(ctx, G.GPUOS_SEQ_ALL, 10_000_000_000)[0] == 0
        order = G.gpuos_loopback_order(ctx)
        assert len(order) == 300
        pos = {int(s): k for k, s in enumerate(order)}
        ranges = [(int(x["input_a"]), int(x["input_b"]), int(x["output"])) for x in d]
        for j in range(300):
            for i in range(j):
                ai, bi, oi = ranges[i]
                aj, bj, oj = ranges[j]
                if oi in (aj, bj, oj) or oj in (ai, bi):
                    assert pos[first + i] < pos[first + j], (i, j)
    finally:
        G.gpuos_shutdown(ctx)
