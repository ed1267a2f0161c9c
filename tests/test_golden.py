"""Hand-derived fixtures under tests/golden/ checked against the oracle:
bf16 rounding cases worked out from the format's definition, and
element-wise programs evaluated by hand where every step is exact."""
import os

import numpy as np

import oracle
import workloads as W

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    for ln in open(os.path.join(HERE, name)):
        ln = ln.strip()
        if ln and not ln.startswith("#"):
            yield ln.split(None, 2) if name.startswith("bf16") else ln.split(None, 4)


def test_bf16_rounding_cases():
    n = 0
    for v, bits, _why in _rows("bf16_rounding.txt"):
        assert oracle.round_bf16(float.fromhex(v)) == int(bits, 16), (v, bits)
        n += 1
    assert n >= 15


def _programs():
    X, P = W.xins, W.program
    return {
        "a_plus_b": P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_ADD, 0, 1, 2)]),
        "diff_over_absb1": P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_SUB, 0, 1, 2), X(W.X_ABS, 3, 2),
                              X(W.X_CONST, 2, 0, 0, 0), X(W.X_ADD, 3, 3, 2), X(W.X_DIV, 0, 0, 3)], [1.0]),
        "max_a_negb_half": P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_NEG, 2, 2), X(W.X_MAX, 0, 1, 2),
                              X(W.X_CONST, 3, 0, 0, 0), X(W.X_MUL, 0, 0, 3)], [0.5]),
        "sqrt_absa_relu_b": P([X(W.X_LDA, 1), X(W.X_ABS, 1, 1), X(W.X_SQRT, 1, 1), X(W.X_LDB, 2),
                               X(W.X_RELU, 2, 2), X(W.X_ADD, 0, 1, 2)]),
        "min_a_2_times_a": P([X(W.X_LDA, 1), X(W.X_CONST, 2, 0, 0, 0), X(W.X_MIN, 0, 1, 2),
                              X(W.X_MUL, 0, 0, 1)], [2.0]),
    }


def test_expr_programs_by_hand():
    progs = _programs()
    n = 0
    for name, a, b, want, _why in _rows("expr_programs.txt"):
        got = np.float32(oracle.expr_eval(progs[name], float.fromhex(a), float.fromhex(b)))
        exp = np.float32(float.fromhex(want))
        assert got.view(np.uint32) == exp.view(np.uint32), (name, a, b, got, exp)
        n += 1
    assert n >= 9


def test_pr1_final_pool_digest():
    """The oracle still produces the recorded final PR1 pool (the recorded
    digest was written by tests/golden/make_pr1_digest.py from the oracle)."""
    import sys
    sys.path.insert(0, HERE)
    from make_pr1_digest import digest
    s = W.make_pr1()
    p = oracle.Pool([b.host_bytes() for b in s.buffers])
    p.run(s.recs)
    want = open(os.path.join(HERE, "pr1_final_pool.sha256")).read().split()[0]
    assert digest(p.arrays) == want
