"""Element-wise programs (gpuos_register_expr / gpuos_register_jit format)
shared by the GPU tests of interpreted and compiled injection: name ->
(program words, True if every step is correctly rounded, so results are
bit-exact)."""
import workloads as W


def programs():
    X, P = W.xins, W.program
    return {
        "a+b": (P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_ADD, 0, 1, 2)]), True),
        "(a-b)/(|b|+1)": (P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_SUB, 0, 1, 2), X(W.X_ABS, 3, 2),
                             X(W.X_CONST, 2, 0, 0, 0), X(W.X_ADD, 3, 3, 2), X(W.X_DIV, 0, 0, 3)], [1.0]), True),
        "max(a,-b)*0.5": (P([X(W.X_LDA, 1), X(W.X_LDB, 2), X(W.X_NEG, 2, 2), X(W.X_MAX, 0, 1, 2),
                             X(W.X_CONST, 3, 0, 0, 0), X(W.X_MUL, 0, 0, 3)], [0.5]), True),
        "sqrt|a|+relu(b)": (P([X(W.X_LDA, 1), X(W.X_ABS, 1, 1), X(W.X_SQRT, 1, 1), X(W.X_LDB, 2),
                               X(W.X_RELU, 2, 2), X(W.X_ADD, 0, 1, 2)]), True),
        "min(a,2)*a": (P([X(W.X_LDA, 1), X(W.X_CONST, 2, 0, 0, 0), X(W.X_MIN, 0, 1, 2), X(W.X_MUL, 0, 0, 1)],
                         [2.0]), True),
        "sigmoid(a)*b": (P([X(W.X_LDA, 1), X(W.X_SIGMOID, 1, 1), X(W.X_LDB, 2), X(W.X_MUL, 0, 1, 2)]), False),
        "tanh(a)+b/2": (P([X(W.X_LDA, 1), X(W.X_TANH, 1, 1), X(W.X_LDB, 2), X(W.X_CONST, 3, 0, 0, 0),
                           X(W.X_MUL, 2, 2, 3), X(W.X_ADD, 0, 1, 2)], [0.5]), False),
        "exp(-a^2)": (P([X(W.X_LDA, 1), X(W.X_MUL, 1, 1, 1), X(W.X_NEG, 1, 1), X(W.X_EXP, 0, 1)]), False),
        "log(1+|a|)": (P([X(W.X_LDA, 1), X(W.X_ABS, 1, 1), X(W.X_CONST, 2, 0, 0, 0), X(W.X_ADD, 1, 1, 2),
                          X(W.X_LOG, 0, 1)], [1.0]), False),
        "gelu (14 steps)": (P([X(W.X_LDA, 1), X(W.X_MUL, 2, 1, 1), X(W.X_MUL, 2, 2, 1), X(W.X_CONST, 3, 0, 0, 0),
                               X(W.X_MUL, 2, 2, 3), X(W.X_ADD, 2, 2, 1), X(W.X_CONST, 3, 0, 0, 1),
                               X(W.X_MUL, 2, 2, 3), X(W.X_TANH, 2, 2), X(W.X_CONST, 3, 0, 0, 2),
                               X(W.X_ADD, 2, 2, 3), X(W.X_MUL, 2, 2, 1), X(W.X_CONST, 3, 0, 0, 3),
                               X(W.X_MUL, 0, 2, 3)], [0.044715, 0.7978845608028654, 1.0, 0.5]), False),
    }
