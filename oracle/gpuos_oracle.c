/*
 * gpuos_oracle.c -- CPU oracle for the persistent micro-op dispatch path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The product path never
 * calls it, and it shares no code, header, table or constant with the HIP
 * library: it declares its own record layout, op numbering and bf16 helpers.
 *
 * What it computes.  GPUOS ("GPUOS: A GPU Operating System Primitive for
 * Transparent Operation Fusion", digest page, sections 2 and 3 Q2) replaces
 * one kernel launch per micro-op by a device-side function call; dispatch
 * changes nothing numerically.  The result of a descriptor stream is
 * therefore exactly the result of running each micro-op, in submission
 * order, one after the other.  This file is that definition: a sequential
 * interpreter over a stream of records, each naming its operands as
 * (buffer index, byte offset) in a host pool.
 *
 * Arithmetic.  Floating-point ops are evaluated in double and rounded once
 * to the output type (fp32 by the C cast, which rounds to nearest even;
 * bf16 by round_bf16 below).  For add and mul of fp32 or bf16 operands this
 * equals the correctly rounded single-precision operation, because double
 * carries at least 2p+2 bits for p = 24 and p = 8 (Figueroa, "When is double
 * rounding innocuous?", 1995).  Build without -ffast-math and without
 * flush-to-zero.
 *
 * Operator list (digest page, section 3 Q2, "Operator library"): add, mul,
 * ReLU, GELU, softmax, LayerNorm; vector-matrix products; SDPA and rotary
 * embeddings; KV-cache update; sum, max and min over small dimensions.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - relu(-0) = +0 and relu(NaN) = NaN.
 *  - max/min propagate NaN and order -0 below +0.
 *  - GELU is the tanh approximation with sqrt(2/pi) and 0.044715; where
 *    1 + tanh(u) would cancel (u < -1/2) the exact identity
 *    1 + tanh(u) = 2 / (1 + e^(-2u)) is used instead.
 *  - LayerNorm uses the biased variance and adds eps inside the root.
 *  - RoPE rotates adjacent pairs (x_2i, x_2i+1) by pos * theta^(-2i/D)
 *    (rotate-half pairing with flag 1); pos = L_b - 1.
 *  - KV append writes K[b,h,L_b-1,:] and V[b,h,L_b-1,:]; the cache is
 *    [B, H, C, D].  SDPA attends one query over keys [0, L_b).
 *  - GEMV: y[n] = sum_k x[k] W[k,n] with W row-major [K, N].
 *  - Small matmul: y[m,n] = sum_k x[m,k] Wt[n,k], x row-major [M, K] and the
 *    weight Wt row-major [N, K] (a linear layer's [out, in] layout).
 *  - An injected operator (the pages' run-time operator injection, digest
 *    page section 3 Q2 "Dynamic Operator Table") is an element-wise program
 *    on four binary32 registers, applied per element; its definition is the
 *    program run step by step in binary32 (orc_expr_eval below).
 *
 * Parity pins: every function here is checked in the CPU test suite against
 * closed forms, invariants, brute force or library routines.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- record layout (152 bytes), as written by the stream generator ---- */
typedef struct {
    int32_t op, dtype, out_dtype, flags;
    int32_t buf[6];   /* a, b, out, aux0, aux1, aux2; -1 = none */
    int64_t off[6];   /* byte offsets into those buffers */
    int64_t size;
    int32_t dim[4];
    float fparam[2];
    int32_t lens[8];
} orc_rec;

enum { ORC_NOP = 0, ORC_ADD, ORC_MUL, ORC_RELU, ORC_GELU, ORC_SUM, ORC_MAX, ORC_MIN,
       ORC_SOFTMAX, ORC_LAYERNORM, ORC_ROPE, ORC_KV_APPEND, ORC_SDPA, ORC_GEMV, ORC_COPY, ORC_EXPR,
       ORC_MATMUL };
enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { R_A = 0, R_B, R_OUT, R_AUX0, R_AUX1, R_AUX2 };

/* error codes returned (negated) by orc_run together with the record index */
#define ORC_E_BOUNDS 1
#define ORC_E_OP 2
#define ORC_E_DTYPE 3

/* ------------------------------------------------------------------------ */
/* bf16: 1 sign bit, 8 exponent bits, 7 fraction bits (the top half of an   */
/* IEEE binary32).  Decoding appends 16 zero bits.  Encoding rounds a double */
/* to the nearest bf16 value, ties to even, written out from the definition: */
/* find the spacing q of bf16 values around |x|, round |x|/q to an integer.  */
/* ------------------------------------------------------------------------ */
double orc_bf16_to_double(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

uint16_t orc_round_bf16(double x) {
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return (uint16_t)(sign | 0x7FC0);
    double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80);
    if (a == 0.0) return sign;
    double q;                                  /* spacing of bf16 values at a */
    if (a >= ldexp(1.0, -126)) {
        int e;
        frexp(a, &e);                          /* a = m * 2^e, m in [0.5, 1) */
        q = ldexp(1.0, (e - 1) - 7);           /* 8 significant bits */
    } else {
        q = ldexp(1.0, -133);                  /* subnormal spacing */
    }
    double t = a / q;                          /* exact: q is a power of two */
    double fl = floor(t);
    double fr = t - fl;
    if (fr > 0.5 || (fr == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    double r = fl * q;
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);  /* overflow */
    float f = (float)r;                        /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

/* ---- element access by dtype ---- */
static double ld(const uint8_t* p, int dt, int64_t i) {
    if (dt == ORC_F32) { float f; memcpy(&f, p + 4 * i, 4); return (double)f; }
    uint16_t h; memcpy(&h, p + 2 * i, 2); return orc_bf16_to_double(h);
}

/* Observation windows (set only by orc_run_capture): every value an op
 * stores into a window is also written there as the double it computed,
 * before rounding to the output type.  Comparisons of a rounded GPU result
 * against the exact value then carry no second rounding.  This observes the
 * arithmetic and changes none of it. */
typedef struct { const uint8_t* base; int64_t nbytes; double* out; } cap_t;
static cap_t cap_win[2];
static int cap_n = 0;

static void st(uint8_t* p, int dt, int64_t i, double v) {
    const int64_t es = dt == ORC_F32 ? 4 : 2;
    for (int w = 0; w < cap_n; ++w) {
        const uint8_t* q = p + es * i;
        if (q >= cap_win[w].base && q < cap_win[w].base + cap_win[w].nbytes)
            cap_win[w].out[(q - cap_win[w].base) / es] = v;
    }
    if (dt == ORC_F32) { float f = (float)v; memcpy(p + 4 * i, &f, 4); }
    else { uint16_t h = orc_round_bf16(v); memcpy(p + 2 * i, &h, 2); }
}

static int esize(int dt) { return dt == ORC_F32 ? 4 : 2; }

/* ---- scalar definitions (exported for the pins) ---- */
double orc_relu(double x) {
    if (isnan(x)) return x;
    return x > 0.0 ? x : 0.0;                  /* -0 and negatives give +0 */
}

/* GELU, tanh approximation: 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3).
 * For u < -1/2 the sum 1 + tanh(u) cancels in double (at x = -7 it keeps
 * only a few digits, below about x = -8.5 none), so there it is evaluated
 * with the exact identity 1 + tanh(u) = 2 / (1 + e^(-2u)). */
double orc_gelu(double x) {
    const double k = sqrt(2.0 / M_PI);
    const double u = k * (x + 0.044715 * x * x * x);
    const double t = u >= -0.5 ? 1.0 + tanh(u) : 2.0 / (1.0 + exp(-2.0 * u));
    return 0.5 * x * t;
}

/* max/min under a total order on non-NaN values with -0 < +0; NaN wins */
static int lt_total(double a, double b) {
    if (a == 0.0 && b == 0.0) return signbit(a) && !signbit(b);
    return a < b;
}
double orc_max2(double a, double b) {
    if (isnan(a)) return a;
    if (isnan(b)) return b;
    return lt_total(a, b) ? b : a;
}
double orc_min2(double a, double b) {
    if (isnan(a)) return a;
    if (isnan(b)) return b;
    return lt_total(b, a) ? b : a;
}

/* ---- injected element-wise programs ----
 * Program words: w[0] = number of instructions (bits 0-7) | number of
 * constants (bits 8-15); then one word per instruction: operation (bits
 * 0-7), destination register (8-11), sources (12-15, 16-19), constant index
 * (20-27); then the constants as binary32 bit patterns.  Registers r0..r3
 * start at 0; r0 is the result.  Every step yields a binary32 value: + - *
 * / and sqrt are the correctly rounded operations (computed in double and
 * rounded once, which is innocuous for these, Figueroa 1995); exp, log,
 * tanh and the logistic function are the double functions rounded once to
 * binary32; min/max as orc_min2/orc_max2; relu as orc_relu; neg and abs
 * flip and clear the sign. */
enum { X_LDA = 1, X_LDB, X_CONST, X_MOV, X_ADD, X_SUB, X_MUL, X_DIV, X_MIN, X_MAX, X_NEG, X_ABS,
       X_EXP, X_LOG, X_SQRT, X_TANH, X_SIGMOID, X_RELU, X_END };

static float to_f32(double v) { return (float)v; }

/* Evaluate the program for one element; *err = 1 for a malformed program. */
float orc_expr_eval(const uint32_t* w, int64_t n_words, float a, float b, int32_t* err) {
    float R[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    *err = 1;
    if (n_words < 1) return 0.0f;
    const uint32_t ni = w[0] & 0xFFu, nk = (w[0] >> 8) & 0xFFu;
    if (ni < 1 || ni > 32 || nk > 16 || (w[0] >> 16) != 0 || n_words != 1 + (int64_t)ni + nk) return 0.0f;
    for (uint32_t i = 0; i < ni; ++i) {
        const uint32_t ins = w[1 + i];
        const uint32_t op = ins & 0xFFu, d = (ins >> 8) & 0xFu, s1 = (ins >> 12) & 0xFu, s2 = (ins >> 16) & 0xFu;
        const uint32_t k = (ins >> 20) & 0xFFu;
        if (op < X_LDA || op >= X_END || d > 3 || s1 > 3 || s2 > 3 || (ins >> 28) != 0) return 0.0f;
        if (op == X_CONST && k >= nk) return 0.0f;
        const double x = R[s1], y = R[s2];
        float v;
        switch (op) {
            case X_LDA: v = a; break;
            case X_LDB: v = b; break;
            case X_CONST: memcpy(&v, &w[1 + ni + k], 4); break;
            case X_MOV: v = R[s1]; break;
            case X_ADD: v = to_f32(x + y); break;
            case X_SUB: v = to_f32(x - y); break;
            case X_MUL: v = to_f32(x * y); break;
            case X_DIV: v = to_f32(x / y); break;
            case X_MIN: v = to_f32(orc_min2(x, y)); break;
            case X_MAX: v = to_f32(orc_max2(x, y)); break;
            case X_NEG: v = -R[s1]; break;
            case X_ABS: v = fabsf(R[s1]); break;
            case X_EXP: v = to_f32(exp(x)); break;
            case X_LOG: v = to_f32(log(x)); break;
            case X_SQRT: v = to_f32(sqrt(x)); break;
            case X_TANH: v = to_f32(tanh(x)); break;
            case X_SIGMOID: v = to_f32(1.0 / (1.0 + exp(-x))); break;
            default: v = to_f32(orc_relu(x)); break; /* X_RELU */
        }
        R[d] = v;
    }
    *err = 0;
    return R[0];
}

/* ---- pool access with bounds checks ---- */
typedef struct {
    uint8_t** base;
    const int64_t* nbytes;
    int32_t nbuf;
} pool_t;

static uint8_t* span(const pool_t* P, const orc_rec* r, int role, int64_t nbytes) {
    int32_t b = r->buf[role];
    if (b < 0 || b >= P->nbuf) return NULL;
    int64_t off = r->off[role];
    if (off < 0 || nbytes < 0 || off + nbytes > P->nbytes[b]) return NULL;
    return P->base[b] + off;
}

/* ---- the micro-ops ---- */
static int op_binary(const pool_t* P, const orc_rec* r) {
    int64_t n = r->size;
    int di = r->dtype, dout = r->out_dtype;
    const uint8_t* a = span(P, r, R_A, n * esize(di));
    const uint8_t* b = span(P, r, R_B, n * esize(di));
    uint8_t* o = span(P, r, R_OUT, n * esize(dout));
    if (!a || !b || !o) return ORC_E_BOUNDS;
    /* elementwise, so in-place aliasing of o with a or b is harmless */
    for (int64_t i = 0; i < n; ++i) {
        double x = ld(a, di, i), y = ld(b, di, i);
        st(o, dout, i, r->op == ORC_ADD ? x + y : x * y);
    }
    return 0;
}

static int op_unary(const pool_t* P, const orc_rec* r) {
    int64_t n = r->size;
    int di = r->dtype, dout = r->out_dtype;
    const uint8_t* a = span(P, r, R_A, n * esize(di));
    uint8_t* o = span(P, r, R_OUT, n * esize(dout));
    if (!a || !o) return ORC_E_BOUNDS;
    for (int64_t i = 0; i < n; ++i) {
        double x = ld(a, di, i);
        st(o, dout, i, r->op == ORC_RELU ? orc_relu(x) : orc_gelu(x));
    }
    return 0;
}

/* sum / max / min along the last dimension: [rows, h] -> [rows] */
static int op_reduce(const pool_t* P, const orc_rec* r) {
    int64_t rows = r->size, h = r->dim[0];
    int di = r->dtype, dout = r->out_dtype;
    const uint8_t* x = span(P, r, R_A, rows * h * esize(di));
    uint8_t* o = span(P, r, R_OUT, rows * esize(dout));
    if (!x || !o || h <= 0) return ORC_E_BOUNDS;
    for (int64_t i = 0; i < rows; ++i) {
        double acc = ld(x, di, i * h);
        for (int64_t j = 1; j < h; ++j) {
            double v = ld(x, di, i * h + j);
            if (r->op == ORC_SUM) acc += v;
            else if (r->op == ORC_MAX) acc = orc_max2(acc, v);
            else acc = orc_min2(acc, v);
        }
        st(o, dout, i, acc);
    }
    return 0;
}

/* softmax along the last dimension: y = exp(x - max x) / sum exp(x - max x) */
static int op_softmax(const pool_t* P, const orc_rec* r) {
    int64_t rows = r->size, h = r->dim[0];
    int di = r->dtype, dout = r->out_dtype;
    const uint8_t* x = span(P, r, R_A, rows * h * esize(di));
    uint8_t* o = span(P, r, R_OUT, rows * h * esize(dout));
    if (!x || !o || h <= 0) return ORC_E_BOUNDS;
    double* e = (double*)malloc(sizeof(double) * h);
    if (!e) return ORC_E_BOUNDS;
    for (int64_t i = 0; i < rows; ++i) {
        double m = -INFINITY;
        for (int64_t j = 0; j < h; ++j) { double v = ld(x, di, i * h + j); if (v > m) m = v; }
        double s = 0.0;
        for (int64_t j = 0; j < h; ++j) { e[j] = exp(ld(x, di, i * h + j) - m); s += e[j]; }
        for (int64_t j = 0; j < h; ++j) st(o, dout, i * h + j, e[j] / s);
    }
    free(e);
    return 0;
}

/* LayerNorm along the last dimension, biased variance, eps inside the root:
 * y = (x - mu) / sqrt(var + eps) * gamma + beta */
static int op_layernorm(const pool_t* P, const orc_rec* r) {
    int64_t rows = r->size, h = r->dim[0];
    int di = r->dtype, dout = r->out_dtype;
    const uint8_t* x = span(P, r, R_A, rows * h * esize(di));
    const uint8_t* g = span(P, r, R_AUX0, h * esize(di));
    const uint8_t* b = span(P, r, R_AUX1, h * esize(di));
    uint8_t* o = span(P, r, R_OUT, rows * h * esize(dout));
    if (!x || !g || !b || !o || h <= 0) return ORC_E_BOUNDS;
    double eps = (double)r->fparam[0];
    double* row = (double*)malloc(sizeof(double) * h);
    if (!row) return ORC_E_BOUNDS;
    for (int64_t i = 0; i < rows; ++i) {
        double mu = 0.0;
        for (int64_t j = 0; j < h; ++j) { row[j] = ld(x, di, i * h + j); mu += row[j]; }
        mu /= (double)h;
        double var = 0.0;
        for (int64_t j = 0; j < h; ++j) { double d = row[j] - mu; var += d * d; }
        var /= (double)h;
        double inv = 1.0 / sqrt(var + eps);
        for (int64_t j = 0; j < h; ++j)
            st(o, dout, i * h + j, (row[j] - mu) * inv * ld(g, di, j) + ld(b, di, j));
    }
    free(row);
    return 0;
}

/* Rotary embedding in place on q and k ([B, H, D] each) at pos = L_b - 1:
 * pair i (i < D/2) turns by angle pos * theta^(-2i/D). */
/* RoPE on q [B, H, D] and k [B, Hk, D]; Hk = dim[3] (0: H) is the number
 * of key heads, fewer than the query heads under grouped-query attention. */
static int op_rope(const pool_t* P, const orc_rec* r) {
    int64_t B = r->size, H = r->dim[0], D = r->dim[1], Hk = r->dim[3] > 0 ? r->dim[3] : r->dim[0];
    int dt = r->dtype;
    if (D <= 0 || (D & 1) || B > 8 || Hk > H) return ORC_E_BOUNDS;
    uint8_t* q = span(P, r, R_A, B * H * D * esize(dt));
    uint8_t* k = span(P, r, R_B, B * Hk * D * esize(dt));
    if (!q || !k) return ORC_E_BOUNDS;
    double theta = r->fparam[0] != 0.0f ? (double)r->fparam[0] : 10000.0;
    int half = (r->flags & 1) != 0;
    for (int64_t b = 0; b < B; ++b) {
        double pos = (double)(r->lens[b] - 1);
        for (int64_t h = 0; h < H; ++h) {
            for (int t = 0; t < 2; ++t) {
                if (t == 1 && h >= Hk) continue;
                uint8_t* v = t == 0 ? q : k;
                int64_t base = (b * (t == 0 ? H : Hk) + h) * D;
                for (int64_t i = 0; i < D / 2; ++i) {
                    int64_t i0 = half ? i : 2 * i, i1 = half ? i + D / 2 : 2 * i + 1;
                    double ang = pos * pow(theta, -2.0 * (double)i / (double)D);
                    double c = cos(ang), s = sin(ang);
                    double x0 = ld(v, dt, base + i0), x1 = ld(v, dt, base + i1);
                    st(v, dt, base + i0, x0 * c - x1 * s);
                    st(v, dt, base + i1, x0 * s + x1 * c);
                }
            }
        }
    }
    return 0;
}

/* Paged caches (record flag 4): the cache is a pool of NP pages, page p
 * holding positions of H heads as [H, PS, D]; the block table (int32,
 * [B, MP]) gives the page of position j of batch row b as table[b][j / PS]
 * and its row as j % PS.  The record's size packs B (bits 0-15), MP (bits
 * 16-31) and NP (bits 32-63); dim[2] is PS.  paged_row returns the element
 * offset of position j, head h, of row b in the pool, or -1 if the table
 * entry is outside [0, NP). */
static int64_t paged_row(const uint8_t* table, int64_t MP, int64_t NP, int64_t H, int64_t PS, int64_t D,
                         int64_t b, int64_t h, int64_t j) {
    int32_t page;
    memcpy(&page, table + (b * MP + j / PS) * 4, 4);
    if (page < 0 || page >= NP) return -1;
    return (((int64_t)page * H + h) * PS + j % PS) * D;
}

/* KV append into paged caches: position L_b - 1 of every head of row b */
static int op_kv_append_paged(const pool_t* P, const orc_rec* r) {
    int64_t B = r->size & 0xFFFF, MP = (r->size >> 16) & 0xFFFF, NP = r->size >> 32;
    int64_t H = r->dim[0], D = r->dim[1], PS = r->dim[2];
    int es = esize(r->dtype);
    if (B > 8 || MP < 1 || NP < 1 || PS < 1) return ORC_E_BOUNDS;
    const uint8_t* k = span(P, r, R_A, B * H * D * es);
    const uint8_t* v = span(P, r, R_B, B * H * D * es);
    uint8_t* K = span(P, r, R_AUX0, NP * H * PS * D * es);
    uint8_t* V = span(P, r, R_AUX1, NP * H * PS * D * es);
    const uint8_t* table = span(P, r, R_AUX2, B * MP * 4);
    if (!k || !v || !K || !V || !table) return ORC_E_BOUNDS;
    for (int64_t b = 0; b < B; ++b) {
        int64_t pos = r->lens[b] - 1;
        if (pos < 0 || pos >= MP * PS) return ORC_E_BOUNDS;
        for (int64_t h = 0; h < H; ++h) {
            int64_t at = paged_row(table, MP, NP, H, PS, D, b, h, pos);
            if (at < 0) continue;  /* a page outside the pool: nothing is written */
            memcpy(K + at * es, k + (b * H + h) * D * es, (size_t)(D * es));
            memcpy(V + at * es, v + (b * H + h) * D * es, (size_t)(D * es));
        }
    }
    return 0;
}

/* KV append: K[b,h,L_b-1,:] = k[b,h,:], V[b,h,L_b-1,:] = v[b,h,:] (bit copy) */
static int op_kv_append(const pool_t* P, const orc_rec* r) {
    if (r->flags & 4) return op_kv_append_paged(P, r);
    int64_t B = r->size, H = r->dim[0], D = r->dim[1], C = r->dim[2];
    int es = esize(r->dtype);
    if (B > 8) return ORC_E_BOUNDS;
    const uint8_t* k = span(P, r, R_A, B * H * D * es);
    const uint8_t* v = span(P, r, R_B, B * H * D * es);
    uint8_t* K = span(P, r, R_AUX0, B * H * C * D * es);
    uint8_t* V = span(P, r, R_AUX1, B * H * C * D * es);
    if (!k || !v || !K || !V) return ORC_E_BOUNDS;
    for (int64_t b = 0; b < B; ++b) {
        int64_t pos = r->lens[b] - 1;
        if (pos < 0 || pos >= C) return ORC_E_BOUNDS;
        for (int64_t h = 0; h < H; ++h) {
            int64_t dst = ((b * H + h) * C + pos) * D * es, src = (b * H + h) * D * es;
            memcpy(K + dst, k + src, (size_t)(D * es));
            memcpy(V + dst, v + src, (size_t)(D * es));
        }
    }
    return 0;
}

/* Single-query SDPA: for each (b, h), s_j = scale * q . K_j for j < L_b,
 * p = softmax(s), o = sum_j p_j V_j.  scale defaults to 1/sqrt(D).  The
 * caches hold Hkv = dim[3] (0: H) heads [B, Hkv, C, D]; query head h reads
 * key/value head h / (H / Hkv) (grouped-query attention; Hkv = 1 is
 * multi-query attention).  Attention masking (record flag 2): s_j gets
 * mask[b, j] added, an fp32 mask [B, C] in aux2 shared by all heads; a row
 * whose scores are all -inf is softmax over nothing and gives NaN. */
static int op_sdpa(const pool_t* P, const orc_rec* r) {
    /* paged caches (flag 4): the caches are pools of NP pages [Hkv, PS, D],
     * the block table is in b, and a row holds C = MP * PS positions */
    const int paged = (r->flags & 4) != 0;
    int64_t B = paged ? (r->size & 0xFFFF) : r->size, H = r->dim[0], D = r->dim[1];
    int64_t MP = paged ? (r->size >> 16) & 0xFFFF : 0, NP = paged ? r->size >> 32 : 0, PS = r->dim[2];
    int64_t C = paged ? MP * PS : r->dim[2];
    int64_t Hkv = r->dim[3] > 0 ? r->dim[3] : H;
    int dt = r->dtype, dout = r->out_dtype;
    if (B > 8 || H % Hkv != 0) return ORC_E_BOUNDS;
    if (paged && (MP < 1 || NP < 1 || PS < 1)) return ORC_E_BOUNDS;
    const int64_t G = H / Hkv;
    const int64_t cache = paged ? NP * Hkv * PS * D : B * Hkv * C * D;
    const uint8_t* q = span(P, r, R_A, B * H * D * esize(dt));
    const uint8_t* K = span(P, r, R_AUX0, cache * esize(dt));
    const uint8_t* V = span(P, r, R_AUX1, cache * esize(dt));
    uint8_t* o = span(P, r, R_OUT, B * H * D * esize(dout));
    const uint8_t* table = paged ? span(P, r, R_B, B * MP * 4) : NULL;
    if (!q || !K || !V || !o || (paged && !table)) return ORC_E_BOUNDS;
    const uint8_t* mask = NULL;
    if (r->flags & 2) {
        mask = span(P, r, R_AUX2, B * C * 4);
        if (!mask) return ORC_E_BOUNDS;
    }
    double scale = r->fparam[1] != 0.0f ? (double)r->fparam[1] : 1.0 / sqrt((double)D);
    double* s = (double*)malloc(sizeof(double) * (size_t)(C > 0 ? C : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)D);
    if (!s || !acc) { free(s); free(acc); return ORC_E_BOUNDS; }
    int rc = 0;
    for (int64_t b = 0; b < B && !rc; ++b) {
        int64_t L = r->lens[b];
        if (L < 1 || L > C) { rc = ORC_E_BOUNDS; break; }
        for (int64_t h = 0; h < H; ++h) {
            int64_t kv = (b * Hkv + h / G) * C * D, qo = (b * H + h) * D;
            double m = -INFINITY;
            for (int64_t j = 0; j < L; ++j) {
                /* key j: row j of the (b, head) cache, or its place in a page;
                 * a page outside the pool leaves key j out */
                int64_t kj = paged ? paged_row(table, MP, NP, Hkv, PS, D, b, h / G, j) : kv + j * D;
                if (kj < 0) { s[j] = -INFINITY; continue; }
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d) dot += ld(q, dt, qo + d) * ld(K, dt, kj + d);
                s[j] = dot * scale;
                if (mask) s[j] += ld(mask, ORC_F32, b * C + j);
                if (s[j] > m) m = s[j];
            }
            double z = 0.0;
            for (int64_t j = 0; j < L; ++j) { s[j] = exp(s[j] - m); z += s[j]; }
            for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
            for (int64_t j = 0; j < L; ++j) {
                double p = s[j] / z;
                int64_t kj = paged ? paged_row(table, MP, NP, Hkv, PS, D, b, h / G, j) : kv + j * D;
                if (kj < 0) continue;  /* a key left out has no value row */
                for (int64_t d = 0; d < D; ++d) acc[d] += p * ld(V, dt, kj + d);
            }
            for (int64_t d = 0; d < D; ++d) st(o, dout, qo + d, acc[d]);
        }
    }
    free(s);
    free(acc);
    return rc;
}

/* y[n] = sum_k x[k] * W[k, n], W row-major [K, N] */
static int op_gemv(const pool_t* P, const orc_rec* r) {
    int64_t K = r->dim[0], N = r->dim[1];
    int dt = r->dtype, dout = r->out_dtype;
    const uint8_t* x = span(P, r, R_A, K * esize(dt));
    const uint8_t* W = span(P, r, R_B, K * N * esize(dt));
    uint8_t* y = span(P, r, R_OUT, N * esize(dout));
    if (!x || !W || !y) return ORC_E_BOUNDS;
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) acc += ld(x, dt, k) * ld(W, dt, k * N + n);
        st(y, dout, n, acc);
    }
    return 0;
}

/* small matmul: y[m, n] = sum_k x[m, k] * Wt[n, k]; x [M = size, K = dim[0]],
 * Wt [N = dim[1], K], both row-major */
static int op_matmul(const pool_t* P, const orc_rec* r) {
    int64_t M = r->size, K = r->dim[0], N = r->dim[1];
    int dt = r->dtype, dout = r->out_dtype;
    const uint8_t* x = span(P, r, R_A, M * K * esize(dt));
    const uint8_t* Wt = span(P, r, R_B, N * K * esize(dt));
    uint8_t* y = span(P, r, R_OUT, M * N * esize(dout));
    if (!x || !Wt || !y) return ORC_E_BOUNDS;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += ld(x, dt, m * K + k) * ld(Wt, dt, n * K + k);
            st(y, dout, m * N + n, acc);
        }
    return 0;
}

/* injected program: a, b, out of `size` elements; the program's dim[2]
 * words in aux2 (at the record's aux2 offset); no b -> b reads a */
static int op_expr(const pool_t* P, const orc_rec* r) {
    int64_t n = r->size, nw = r->dim[2];
    int di = r->dtype, dout = r->out_dtype;
    const uint8_t* a = span(P, r, R_A, n * esize(di));
    const uint8_t* b = r->buf[R_B] >= 0 ? span(P, r, R_B, n * esize(di)) : a;
    uint8_t* o = span(P, r, R_OUT, n * esize(dout));
    const uint8_t* pw = span(P, r, R_AUX2, nw * 4);
    if (!a || !b || !o || !pw || nw < 1 || nw > 64) return ORC_E_BOUNDS;
    uint32_t w[64];
    memcpy(w, pw, (size_t)nw * 4);
    for (int64_t i = 0; i < n; ++i) {
        int32_t err = 0;
        const float v = orc_expr_eval(w, nw, (float)ld(a, di, i), (float)ld(b, di, i), &err);
        if (err) return ORC_E_OP;
        st(o, dout, i, (double)v);
    }
    return 0;
}

static int op_copy(const pool_t* P, const orc_rec* r) {
    const uint8_t* a = span(P, r, R_A, r->size);
    uint8_t* o = span(P, r, R_OUT, r->size);
    if (!a || !o) return ORC_E_BOUNDS;
    memmove(o, a, (size_t)r->size);
    return 0;
}

static int run_one(const pool_t* P, const orc_rec* r) {
    if ((r->dtype != ORC_F32 && r->dtype != ORC_BF16) ||
        (r->out_dtype != ORC_F32 && r->out_dtype != ORC_BF16))
        return ORC_E_DTYPE;
    switch (r->op) {
        case ORC_NOP: return 0;
        case ORC_ADD: case ORC_MUL: return op_binary(P, r);
        case ORC_RELU: case ORC_GELU: return op_unary(P, r);
        case ORC_SUM: case ORC_MAX: case ORC_MIN: return op_reduce(P, r);
        case ORC_SOFTMAX: return op_softmax(P, r);
        case ORC_LAYERNORM: return op_layernorm(P, r);
        case ORC_ROPE: return op_rope(P, r);
        case ORC_KV_APPEND: return op_kv_append(P, r);
        case ORC_SDPA: return op_sdpa(P, r);
        case ORC_GEMV: return op_gemv(P, r);
        case ORC_COPY: return op_copy(P, r);
        case ORC_EXPR: return op_expr(P, r);
        case ORC_MATMUL: return op_matmul(P, r);
        default: return ORC_E_OP;
    }
}

/* Run records [0, n) in order on the pool.  Returns 0, or -(1 + index) of
 * the first record that failed; *err receives its error code. */
int64_t orc_run(const orc_rec* recs, int64_t n, uint8_t** bufs, const int64_t* nbytes,
                int32_t nbuf, int32_t* err) {
    pool_t P = {bufs, nbytes, nbuf};
    for (int64_t i = 0; i < n; ++i) {
        int rc = run_one(&P, &recs[i]);
        if (rc) { if (err) *err = rc; return -(1 + i); }
    }
    if (err) *err = 0;
    return 0;
}

/* Run one record like orc_run and also report, for up to two output
 * windows (buffer index win_buf[w], byte offset win_off[w], win_bytes[w]
 * bytes), the unrounded double of every element the record stores there
 * into out[w][element], elements counted in the stored type.  Elements the record does not
 * store keep what the caller put in out[w].  Returns like orc_run. */
int64_t orc_run_capture(const orc_rec* rec, uint8_t** bufs, const int64_t* nbytes, int32_t nbuf,
                        int32_t* err, int32_t n_win, const int32_t* win_buf, const int64_t* win_off,
                        const int64_t* win_bytes, double** out) {
    if (n_win < 0 || n_win > 2) { if (err) *err = ORC_E_BOUNDS; return -1; }
    for (int w = 0; w < n_win; ++w) {
        if (win_buf[w] < 0 || win_buf[w] >= nbuf || win_off[w] < 0 || win_bytes[w] < 0 ||
            win_off[w] + win_bytes[w] > nbytes[win_buf[w]]) {
            if (err) *err = ORC_E_BOUNDS;
            return -1;
        }
        cap_win[w].base = bufs[win_buf[w]] + win_off[w];
        cap_win[w].nbytes = win_bytes[w];
        cap_win[w].out = out[w];
    }
    cap_n = n_win;
    const int64_t rc = orc_run(rec, 1, bufs, nbytes, nbuf, err);
    cap_n = 0;
    return rc;
}

int32_t orc_record_size(void) { return (int32_t)sizeof(orc_rec); }
