// Micro-op bodies for CDNA4 (gfx950).  Each body runs one work unit (a
// tile of one descriptor) on one wave64; the executor and the eager
// baseline kernels call the same functions.
//
// Operator list: GPUOS digest page, section 3 Q2 ("Operator library"):
// element-wise add/mul/ReLU/GELU, softmax, LayerNorm, vector-matrix
// products, SDPA, rotary embeddings, KV-cache update, sum/max/min.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gpuos_internal.h"

namespace gpuos {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Wave-uniform view of one work unit.
struct Unit {
    uint64_t seq;
    uint32_t kind, flags, tile, ntiles;
    uint64_t a, b, out, size;
    uint32_t dim[4];
    uint64_t aux0, aux1, aux2;
    float pf[6];      // param words as floats
    uint64_t lensw[2];  // lens[0..7], packed (see lens_at)
    float p0;         // table default parameter
    uint8_t* scratch; // this descriptor's scratch (physical), or null
};

// ------------------------------------------------------------------ scalars
__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16, round to nearest even on the bit pattern; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) | 0x0040u) & 0xFFFFu;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// double -> bf16 with one rounding: round to odd into fp32 (24 >= 8 + 2
// bits), then to nearest even (Boldo and Melquiond, "Emulation of FMA and
// correctly rounded sums: proved algorithms using rounding to odd", 2008).
__device__ __forceinline__ uint32_t d2bf(double x) {
    float f = (float)x;
    if (f == f && !isinf(f) && (double)f != x) {
        uint32_t u = __float_as_uint(f);
        if (fabs((double)f) > fabs(x)) u -= 1u;  // neighbour toward zero
        f = __uint_as_float(u | 1u);
    }
    return f2bf(f);
}

template <uint32_t DT>
__device__ __forceinline__ float ld_elem(const uint8_t* p, uint64_t i) {
    if constexpr (DT == GPUOS_F32) return ((const float*)p)[i];
    else return bf2f(((const uint16_t*)p)[i]);
}
template <uint32_t DT>
__device__ __forceinline__ void st_elem(uint8_t* p, uint64_t i, float v);

__device__ __forceinline__ float relu_f(float x) { return x > 0.0f ? x : (x != x ? x : 0.0f); }

// GELU, tanh approximation, evaluated as x / (1 + exp(-2u)) with
// u = sqrt(2/pi) (x + 0.044715 x^3) (the same function; no cancellation).
// For |x| < 3 (|2u| < 7) fp32 arithmetic keeps the relative error near
// 1e-6.  Beyond that the exponent a = -2u is formed in double and split as
// k ln2 + r with |r| <= ln2/2, so only r goes through the fp32 exp; for
// a > 0 (x < 0) the result x e^{-a} / (1 + e^{-a}) is formed as a normal
// float and scaled by 2^-k last, so results in the denormal range are
// rounded only once.
__device__ __forceinline__ float gelu_wide(float x) {
    const double xd = (double)x;
    const double a = -2.0 * 0.7978845608028654 * (xd + 0.044715 * xd * xd * xd);
    if (a != a) return x;                    // NaN input
    if (a > 300.0) return x * 0.0f;          // below every denormal: -0 (NaN for -inf)
    if (a < -300.0) return x;                // exp(-2u) = 0
    const double k = rint(a * 1.4426950408889634);
    const float r = (float)(a - k * 0.6931471805599453);
    if (a > 0.0) {
        const float er = expf(-r);                 // e^{-r} in [0.7, 1.42]
        const float t = ldexpf(er, -(int)k);       // e^{-a}
        return ldexpf(x * er / (1.0f + t), -(int)k);
    }
    return x / (1.0f + ldexpf(expf(r), (int)k));
}
__device__ __forceinline__ float gelu_f(float x) {
    if (!(fabsf(x) < 3.0f)) return gelu_wide(x);   // also NaN and infinities
    const float a = -1.5957691216057308f * (x + 0.044715f * x * x * x);
    return x / (1.0f + expf(a));
}

// max / min under a total order: NaN wins, -0 < +0.
__device__ __forceinline__ float tmax(float a, float b) {
    if (a != a) return a;
    if (b != b) return b;
    if (a == b) return (__float_as_uint(a) & 0x80000000u) ? b : a;
    return a < b ? b : a;
}
__device__ __forceinline__ float tmin(float a, float b) {
    if (a != a) return a;
    if (b != b) return b;
    if (a == b) return (__float_as_uint(a) & 0x80000000u) ? a : b;
    return a < b ? a : b;
}

// ------------------------------------------------------------ wave helpers
__device__ __forceinline__ float wsum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}
__device__ __forceinline__ float wmaxf(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}
__device__ __forceinline__ float wtmax(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = tmax(v, __shfl_xor(v, m, 64));
    return v;
}
__device__ __forceinline__ float wtmin(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = tmin(v, __shfl_xor(v, m, 64));
    return v;
}

// Stores of op outputs are device-scope write-through (cache policy SC1): the
// eight XCD L2s are not coherent, and a release fence on gfx950 has to write
// back every dirty line of the issuing XCD's L2.  Writing results through
// keeps that fence cheap and leaves nothing stale for readers on other XCDs.
// 128-bit stores go through a raw buffer resource built on the unit's base
// pointer (the per-lane offset stays below 2 GiB); narrower stores use
// relaxed agent-scope atomic stores, which compile to the same SC1 stores.
constexpr int CPOL_SC1 = 16;
struct WBuf {
    __amdgpu_buffer_rsrc_t r;
};
__device__ __forceinline__ WBuf wbuf(const void* base) {
    return WBuf{__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000)};
}
__device__ __forceinline__ void wst16(WBuf b, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, b.r, (int)off, 0, CPOL_SC1);
}
__device__ __forceinline__ void wst32(void* p, uint32_t v) {
    __hip_atomic_store((uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wst16b(void* p, uint16_t v) {
    __hip_atomic_store((uint16_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wst8(void* p, uint8_t v) {
    __hip_atomic_store((uint8_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wst64(void* p, uint64_t v) {
    __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wstf(void* p, float v) { wst32(p, __float_as_uint(v)); }

__device__ __forceinline__ u32x4 ld16(const uint8_t* p) { return *(const u32x4*)p; }

template <uint32_t DT>
__device__ __forceinline__ void st_elem(uint8_t* p, uint64_t i, float v) {
    if constexpr (DT == GPUOS_F32) wstf(p + 4 * i, v);
    else wst16b(p + 2 * i, (uint16_t)f2bf(v));
}

// 16 bytes -> VE floats
template <uint32_t DT>
__device__ __forceinline__ void unpack(u32x4 v, float* f) {
    if constexpr (DT == GPUOS_F32) {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    } else {
        f[0] = bf2f(v.x & 0xFFFFu); f[1] = bf2f(v.x >> 16);
        f[2] = bf2f(v.y & 0xFFFFu); f[3] = bf2f(v.y >> 16);
        f[4] = bf2f(v.z & 0xFFFFu); f[5] = bf2f(v.z >> 16);
        f[6] = bf2f(v.w & 0xFFFFu); f[7] = bf2f(v.w >> 16);
    }
}
template <uint32_t DT>
__device__ __forceinline__ u32x4 pack(const float* f) {
    u32x4 v;
    if constexpr (DT == GPUOS_F32) {
        v.x = __float_as_uint(f[0]); v.y = __float_as_uint(f[1]);
        v.z = __float_as_uint(f[2]); v.w = __float_as_uint(f[3]);
    } else {
        v.x = f2bf(f[0]) | (f2bf(f[1]) << 16); v.y = f2bf(f[2]) | (f2bf(f[3]) << 16);
        v.z = f2bf(f[4]) | (f2bf(f[5]) << 16); v.w = f2bf(f[6]) | (f2bf(f[7]) << 16);
    }
    return v;
}

// ------------------------------------------------------------ element-wise
template <uint32_t K>
__device__ __forceinline__ float ew_op(float x, float y) {
    if constexpr (K == GPUOS_OP_ADD) return x + y;
    else if constexpr (K == GPUOS_OP_MUL) return x * y;
    else if constexpr (K == GPUOS_OP_RELU) return relu_f(x);
    else return gelu_f(x);
}

// One tile of ew_tile_bytes(K) per operand (8 chunks of 16 bytes per lane,
// 2 for GELU), all loads issued before any compute.  The ragged tail (fewer than one
// chunk) and misaligned operands take an element loop.
template <uint32_t K, uint32_t DT>
__device__ __forceinline__ void ew_tile(const Unit& u, uint32_t lane) {
    constexpr uint32_t ES = DT == GPUOS_F32 ? 4u : 2u;
    constexpr uint32_t TILE = ew_tile_bytes(K) / ES;
    constexpr uint32_t VE = 16u / ES;
    constexpr uint32_t CH = TILE / VE / 64u;
    constexpr bool BIN = (K == GPUOS_OP_ADD || K == GPUOS_OP_MUL);
    const uint64_t start = (uint64_t)u.tile * TILE;
    if (start >= u.size) return;
    const uint64_t end = u.size - start < TILE ? u.size : start + TILE;
    const uint8_t* A = (const uint8_t*)u.a;
    const uint8_t* B = (const uint8_t*)u.b;
    uint8_t* O = (uint8_t*)u.out;
    const bool aligned = (((u.a | u.out | (BIN ? u.b : 0ull)) & 15ull) == 0);
    if (aligned) {
        const WBuf ob = wbuf(O + start * ES);
        u32x4 va[CH], vb[CH];
#pragma unroll
        for (uint32_t c = 0; c < CH; ++c) {
            const uint64_t idx = start + (uint64_t)(lane + 64u * c) * VE;
            if (idx + VE <= end) {
                va[c] = ld16(A + idx * ES);
                if constexpr (BIN) vb[c] = ld16(B + idx * ES);
            }
        }
#pragma unroll
        for (uint32_t c = 0; c < CH; ++c) {
            const uint64_t idx = start + (uint64_t)(lane + 64u * c) * VE;
            if (idx + VE <= end) {
                float x[VE], y[VE], o[VE];
                unpack<DT>(va[c], x);
                if constexpr (BIN) unpack<DT>(vb[c], y);
#pragma unroll
                for (uint32_t e = 0; e < VE; ++e) o[e] = ew_op<K>(x[e], BIN ? y[e] : 0.0f);
                wst16(ob, (uint32_t)((idx - start) * ES), pack<DT>(o));
            }
        }
        const uint64_t rem = start + ((end - start) / VE) * VE;
        if (rem + lane < end) {
            const uint64_t i = rem + lane;
            st_elem<DT>(O, i, ew_op<K>(ld_elem<DT>(A, i), BIN ? ld_elem<DT>(B, i) : 0.0f));
        }
    } else {
        for (uint64_t i = start + lane; i < end; i += 64u)
            st_elem<DT>(O, i, ew_op<K>(ld_elem<DT>(A, i), BIN ? ld_elem<DT>(B, i) : 0.0f));
    }
}

// bf16 ReLU acts on the bit pattern (no rounding involved); fp32 uses relu_f.
template <>
__device__ __forceinline__ void ew_tile<GPUOS_OP_RELU, GPUOS_BF16>(const Unit& u, uint32_t lane) {
    constexpr uint32_t TILE = EW_TILE_BYTES / 2u;
    const uint64_t start = (uint64_t)u.tile * TILE;
    if (start >= u.size) return;
    const uint64_t end = u.size - start < TILE ? u.size : start + TILE;
    const uint16_t* A = (const uint16_t*)u.a;
    uint16_t* O = (uint16_t*)u.out;
    auto r16 = [](uint32_t h) -> uint32_t {
        if ((h & 0x7FFFu) > 0x7F80u) return h;  // NaN
        return (h & 0x8000u) ? 0u : h;          // negatives and -0 -> +0
    };
    if (((u.a | u.out) & 15ull) == 0) {
        const WBuf ob = wbuf(O + start);
        u32x4 va[8];
#pragma unroll
        for (uint32_t c = 0; c < 8; ++c) {
            const uint64_t idx = start + (uint64_t)(lane + 64u * c) * 8u;
            if (idx + 8 <= end) va[c] = ld16((const uint8_t*)(A + idx));
        }
#pragma unroll
        for (uint32_t c = 0; c < 8; ++c) {
            const uint64_t idx = start + (uint64_t)(lane + 64u * c) * 8u;
            if (idx + 8 <= end) {
                u32x4 v = va[c], o;
                o.x = r16(v.x & 0xFFFFu) | (r16(v.x >> 16) << 16);
                o.y = r16(v.y & 0xFFFFu) | (r16(v.y >> 16) << 16);
                o.z = r16(v.z & 0xFFFFu) | (r16(v.z >> 16) << 16);
                o.w = r16(v.w & 0xFFFFu) | (r16(v.w >> 16) << 16);
                wst16(ob, (uint32_t)((idx - start) * 2u), o);
            }
        }
        const uint64_t rem = start + ((end - start) / 8u) * 8u;
        if (rem + lane < end) wst16b(O + rem + lane, (uint16_t)r16(A[rem + lane]));
    } else {
        for (uint64_t i = start + lane; i < end; i += 64u) wst16b(O + i, (uint16_t)r16(A[i]));
    }
}

// ------------------------------------------------------------------ rows
// One row of [rows, h] per unit.  Rows up to ROW_MAX_CACHED elements with
// 16-byte alignment are held in registers (64 values per lane); others
// stream from memory in several passes.
template <uint32_t K, uint32_t DT>
__device__ __forceinline__ void row_tile(const Unit& u, uint32_t lane) {
    constexpr uint32_t ES = DT == GPUOS_F32 ? 4u : 2u;
    constexpr uint32_t VE = 16u / ES;
    constexpr uint32_t KMAX = ROW_MAX_CACHED / VE / 64u;
    constexpr bool RED = (K == GPUOS_OP_SUM || K == GPUOS_OP_MAX || K == GPUOS_OP_MIN);
    const uint64_t r = u.tile;
    if (r >= u.size) return;
    const uint32_t h = u.dim[0];
    const uint8_t* X = (const uint8_t*)u.a + r * h * ES;
    uint8_t* O = (uint8_t*)u.out + (RED ? r * ES : r * h * ES);
    const uint8_t* G = (const uint8_t*)u.aux0;
    const uint8_t* Bt = (const uint8_t*)u.aux1;
    float eps = 1e-5f;
    if constexpr (K == GPUOS_OP_LAYERNORM) eps = u.pf[0] != 0.0f ? u.pf[0] : (u.p0 != 0.0f ? u.p0 : 1e-5f);
    const float inv_h = 1.0f / (float)h;
    uint64_t amask = (uint64_t)X | (RED ? 0ull : (uint64_t)O);
    if constexpr (K == GPUOS_OP_LAYERNORM) amask |= u.aux0 | u.aux1;
    const bool cached = h <= ROW_MAX_CACHED && (h % VE) == 0 && (amask & 15ull) == 0;
    if (cached) {
        const WBuf ob = wbuf(O);
        const uint32_t nch = h / VE;
        float v[KMAX][VE];
        u32x4 raw[KMAX];
#pragma unroll
        for (uint32_t k = 0; k < KMAX; ++k) {
            const uint32_t c = lane + 64u * k;
            if (c < nch) raw[k] = ld16(X + (uint64_t)c * 16u);
        }
        float acc = RED && K != GPUOS_OP_SUM ? __uint_as_float(0x7FC00000u) : 0.0f;
        bool first = true;
        float mx = -INFINITY;
#pragma unroll
        for (uint32_t k = 0; k < KMAX; ++k) {
            const uint32_t c = lane + 64u * k;
            if (c < nch) {
                unpack<DT>(raw[k], v[k]);
#pragma unroll
                for (uint32_t e = 0; e < VE; ++e) {
                    const float x = v[k][e];
                    if constexpr (K == GPUOS_OP_SUM || K == GPUOS_OP_LAYERNORM) acc += x;
                    else if constexpr (K == GPUOS_OP_MAX) acc = first ? x : tmax(acc, x);
                    else if constexpr (K == GPUOS_OP_MIN) acc = first ? x : tmin(acc, x);
                    else mx = fmaxf(mx, x);
                    first = false;
                }
            }
        }
        if constexpr (K == GPUOS_OP_SUM) {
            acc = wsum(acc);
            if (lane == 0) st_elem<DT>(O, 0, acc);
        } else if constexpr (K == GPUOS_OP_MAX || K == GPUOS_OP_MIN) {
            // lanes that saw no element hold a placeholder: replace it by an
            // element of the row so it never wins
            const float ref = __shfl(acc, 0, 64);  // lane 0 always has an element (h >= VE)
            if (first) acc = ref;
            acc = K == GPUOS_OP_MAX ? wtmax(acc) : wtmin(acc);
            if (lane == 0) st_elem<DT>(O, 0, acc);
        } else if constexpr (K == GPUOS_OP_SOFTMAX) {
            mx = wmaxf(mx);
            float s = 0.0f;
#pragma unroll
            for (uint32_t k = 0; k < KMAX; ++k) {
                const uint32_t c = lane + 64u * k;
                if (c < nch) {
#pragma unroll
                    for (uint32_t e = 0; e < VE; ++e) { v[k][e] = expf(v[k][e] - mx); s += v[k][e]; }
                }
            }
            s = wsum(s);
#pragma unroll
            for (uint32_t k = 0; k < KMAX; ++k) {
                const uint32_t c = lane + 64u * k;
                if (c < nch) {
                    float o[VE];
#pragma unroll
                    for (uint32_t e = 0; e < VE; ++e) o[e] = v[k][e] / s;
                    wst16(ob, c * 16u, pack<DT>(o));
                }
            }
        } else {  // LAYERNORM
            const float mean = wsum(acc) * inv_h;
            float q = 0.0f;
#pragma unroll
            for (uint32_t k = 0; k < KMAX; ++k) {
                const uint32_t c = lane + 64u * k;
                if (c < nch) {
#pragma unroll
                    for (uint32_t e = 0; e < VE; ++e) { const float d = v[k][e] - mean; q += d * d; }
                }
            }
            const float var = wsum(q) * inv_h;
            const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
            for (uint32_t k = 0; k < KMAX; ++k) {
                const uint32_t c = lane + 64u * k;
                if (c < nch) {
                    float g[VE], bb[VE], o[VE];
                    unpack<DT>(ld16(G + (uint64_t)c * 16u), g);
                    unpack<DT>(ld16(Bt + (uint64_t)c * 16u), bb);
#pragma unroll
                    for (uint32_t e = 0; e < VE; ++e) o[e] = (v[k][e] - mean) * rstd * g[e] + bb[e];
                    wst16(ob, c * 16u, pack<DT>(o));
                }
            }
        }
        return;
    }
    // streaming path
    if constexpr (RED) {
        float acc = 0.0f;
        bool has = false;
        for (uint32_t i = lane; i < h; i += 64u) {
            const float x = ld_elem<DT>(X, i);
            if constexpr (K == GPUOS_OP_SUM) acc += x;
            else if constexpr (K == GPUOS_OP_MAX) acc = has ? tmax(acc, x) : x;
            else acc = has ? tmin(acc, x) : x;
            has = true;
        }
        if constexpr (K == GPUOS_OP_SUM) {
            acc = wsum(acc);
        } else {
            const float ref = __shfl(acc, 0, 64);  // lane 0 has element 0
            if (!has) acc = ref;
            acc = K == GPUOS_OP_MAX ? wtmax(acc) : wtmin(acc);
        }
        if (lane == 0) st_elem<DT>(O, 0, acc);
    } else if constexpr (K == GPUOS_OP_SOFTMAX) {
        float mx = -INFINITY;
        for (uint32_t i = lane; i < h; i += 64u) mx = fmaxf(mx, ld_elem<DT>(X, i));
        mx = wmaxf(mx);
        float s = 0.0f;
        for (uint32_t i = lane; i < h; i += 64u) s += expf(ld_elem<DT>(X, i) - mx);
        s = wsum(s);
        for (uint32_t i = lane; i < h; i += 64u) st_elem<DT>(O, i, expf(ld_elem<DT>(X, i) - mx) / s);
    } else {  // LAYERNORM
        float s = 0.0f;
        for (uint32_t i = lane; i < h; i += 64u) s += ld_elem<DT>(X, i);
        const float mean = wsum(s) * inv_h;
        float q = 0.0f;
        for (uint32_t i = lane; i < h; i += 64u) { const float d = ld_elem<DT>(X, i) - mean; q += d * d; }
        const float rstd = 1.0f / sqrtf(wsum(q) * inv_h + eps);
        for (uint32_t i = lane; i < h; i += 64u)
            st_elem<DT>(O, i, (ld_elem<DT>(X, i) - mean) * rstd * ld_elem<DT>(G, i) + ld_elem<DT>(Bt, i));
    }
}

// ------------------------------------------------------------------ RoPE
// Unit = one batch row b: every head of q and k, rotated at pos = L_b - 1.
// The angle pos * theta^(-2i/D) and its sine and cosine are evaluated in
// double, as is the rotation; the result is rounded once to the dtype.
template <uint32_t DT>
__device__ __forceinline__ void rope_tile(const Unit& u, uint32_t lane) {
    const uint32_t b = u.tile;
    const uint32_t H = u.dim[0], D = u.dim[1];
    const bool half = (u.flags & GPUOS_F_ROPE_HALF) != 0;
    const double theta = u.pf[4] != 0.0f ? (double)u.pf[4] : (u.p0 != 0.0f ? (double)u.p0 : 10000.0);
    const double pos = (double)((int)lens_at(u.lensw, b) - 1);
    for (uint32_t pi = lane; pi < D / 2; pi += 64u) {
        const double fr = pow(theta, -2.0 * (double)pi / (double)D);
        double s, c;
        sincos(pos * fr, &s, &c);
        const uint32_t i0 = half ? pi : 2u * pi, i1 = half ? pi + D / 2 : 2u * pi + 1u;
        for (uint32_t t = 0; t < 2; ++t) {
            uint8_t* P = (uint8_t*)(t == 0 ? u.a : u.b);
            for (uint32_t hh = 0; hh < H; ++hh) {
                const uint64_t base = ((uint64_t)b * H + hh) * D;
                const double x0 = (double)ld_elem<DT>(P, base + i0);
                const double x1 = (double)ld_elem<DT>(P, base + i1);
                const double y0 = x0 * c - x1 * s;
                const double y1 = x0 * s + x1 * c;
                if constexpr (DT == GPUOS_F32) {
                    wstf(P + 4 * (base + i0), (float)y0);
                    wstf(P + 4 * (base + i1), (float)y1);
                } else {
                    wst16b(P + 2 * (base + i0), (uint16_t)d2bf(y0));
                    wst16b(P + 2 * (base + i1), (uint16_t)d2bf(y1));
                }
            }
        }
    }
}

// -------------------------------------------------------------- KV append
// Unit = one batch row b: K[b, h, L_b-1, :] = k[b, h, :] and the same for V.
__device__ __forceinline__ void kv_tile(const Unit& u, uint32_t lane) {
    const uint32_t b = u.tile;
    const uint32_t H = u.dim[0], D = u.dim[1], C = u.dim[2];
    const uint32_t ES = esz(dt_in(u.flags));
    const uint64_t pos = (uint64_t)lens_at(u.lensw, b) - 1;
    const uint64_t RB = (uint64_t)D * ES;
    for (uint32_t t = 0; t < 2; ++t) {
        const uint8_t* src = (const uint8_t*)(t == 0 ? u.a : u.b) + (uint64_t)b * H * RB;
        uint8_t* dst = (uint8_t*)(t == 0 ? u.aux0 : u.aux1);
        if (((uint64_t)src & 15ull) == 0 && ((uint64_t)dst & 15ull) == 0 && (RB & 15ull) == 0) {
            const uint64_t cpr = RB / 16u, total = cpr * H;
            for (uint64_t j = lane; j < total; j += 64u) {
                const uint64_t hh = j / cpr, off = (j % cpr) * 16u;
                const u32x4 v = ld16(src + hh * RB + off);
                uint8_t* d = dst + (((uint64_t)b * H + hh) * C + pos) * RB + off;
                wst64(d, (uint64_t)v.x | ((uint64_t)v.y << 32));
                wst64(d + 8, (uint64_t)v.z | ((uint64_t)v.w << 32));
            }
        } else {
            const uint64_t total = RB * H / 2u;  // 2-byte words (ES is 2 or 4)
            for (uint64_t j = lane; j < total; j += 64u) {
                const uint64_t byte = j * 2u, hh = byte / RB, off = byte % RB;
                wst16b(dst + (((uint64_t)b * H + hh) * C + pos) * RB + off, *(const uint16_t*)(src + hh * RB + off));
            }
        }
    }
}

// ------------------------------------------------------------ decode SDPA
// Unit = (b, h, split of SDPA_KT keys).  One key row of D bf16 is DV = D/8
// lanes x 16 bytes, so one load instruction covers RPI = 64/DV keys.  Keys
// are consumed in chunks of 8 instructions with a running max (online
// softmax); each unit produces (max, sum of exp, unnormalised P.V) for its
// keys, and when a head has several splits the last unit to finish merges
// them (the split softmax of flash-decoding).  Dense MFMA does not apply:
// one query per head makes q.K^T and P.V matrix-vector products with no reuse.
template <uint32_t DV, uint32_t DTO>
__device__ __forceinline__ void sdpa_tile(const Unit& u, uint32_t lane) {
    constexpr uint32_t D = DV * 8u;
    constexpr uint32_t RPI = 64u / DV;
    constexpr uint32_t NIT = SDPA_KT / RPI;
    constexpr uint32_t PSTRIDE = D + 4u;  // floats per partial record: m, l, pad, pad, acc[D]
    const uint32_t H = u.dim[0], C = u.dim[2];
    const uint32_t Bn = (uint32_t)u.size;
    uint32_t t = u.tile, base = 0, b = 0, ns = 1, L = 0;
    for (b = 0; b < Bn; ++b) {
        L = lens_at(u.lensw, b);
        ns = (L + SDPA_KT - 1) / SDPA_KT;
        const uint32_t nu = H * ns;
        if (t < base + nu) break;
        base += nu;
    }
    if (b >= Bn) return;
    const uint32_t local = t - base, h = local / ns, sp = local % ns;
    const uint32_t k0 = sp * SDPA_KT;
    const uint32_t nk = min(L - k0, SDPA_KT);
    const uint64_t bh = (uint64_t)b * H + h;
    const float scale = u.pf[4] != 0.0f ? u.pf[4] : (u.p0 != 0.0f ? u.p0 : 1.0f / sqrtf((float)D));
    const uint32_t g = lane / DV, c = lane % DV;
    const uint8_t* Kp = (const uint8_t*)u.aux0 + (bh * C + k0) * D * 2u + c * 16u;
    const uint8_t* Vp = (const uint8_t*)u.aux1 + (bh * C + k0) * D * 2u + c * 16u;
    float q[8];
    unpack<GPUOS_BF16>(ld16((const uint8_t*)u.a + bh * D * 2u + c * 16u), q);
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] *= scale;
    float m = -INFINITY, lsum = 0.0f;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (uint32_t i0 = 0; i0 < NIT && i0 * RPI < nk; i0 += 8) {
        u32x4 kv[8], vv[8];
#pragma unroll
        for (uint32_t j = 0; j < 8; ++j) {
            const uint32_t key = (i0 + j) * RPI + g;
            if (key < nk) kv[j] = ld16(Kp + (uint64_t)key * D * 2u);
        }
#pragma unroll
        for (uint32_t j = 0; j < 8; ++j) {
            const uint32_t key = (i0 + j) * RPI + g;
            if (key < nk) vv[j] = ld16(Vp + (uint64_t)key * D * 2u);
        }
        float s[8];
        float cm = -INFINITY;
#pragma unroll
        for (uint32_t j = 0; j < 8; ++j) {
            const uint32_t key = (i0 + j) * RPI + g;
            float kf[8], d = 0.0f;
            if (key < nk) {
                unpack<GPUOS_BF16>(kv[j], kf);
#pragma unroll
                for (int e = 0; e < 8; ++e) d += q[e] * kf[e];
            }
#pragma unroll
            for (uint32_t mm = DV / 2; mm >= 1; mm >>= 1) d += __shfl_xor(d, mm, 64);
            s[j] = key < nk ? d : -INFINITY;
            cm = fmaxf(cm, s[j]);
        }
#pragma unroll
        for (uint32_t mm = DV; mm < 64; mm <<= 1) cm = fmaxf(cm, __shfl_xor(cm, mm, 64));
        const float mn = fmaxf(m, cm);          // finite: the chunk has at least one key
        const float alpha = expf(m - mn);       // 0 on the first chunk (m = -inf)
        lsum *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
        for (uint32_t j = 0; j < 8; ++j) {
            const uint32_t key = (i0 + j) * RPI + g;
            if (key < nk) {
                const float p = expf(s[j] - mn);
                float vf[8];
                unpack<GPUOS_BF16>(vv[j], vf);
                lsum += p;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += p * vf[e];
            }
        }
        m = mn;
    }
#pragma unroll
    for (uint32_t mm = DV; mm < 64; mm <<= 1) {
        lsum += __shfl_xor(lsum, mm, 64);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], mm, 64);
    }
    constexpr uint32_t ESO = DTO == GPUOS_F32 ? 4u : 2u;
    uint8_t* O = (uint8_t*)u.out + bh * D * ESO;
    if (ns == 1) {
        if (g == 0) {
            float o[8];
            const float inv = 1.0f / lsum;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = acc[e] * inv;
            const WBuf ob = wbuf(O);
            if constexpr (DTO == GPUOS_F32) {
                wst16(ob, c * 32u, pack<GPUOS_F32>(o));
                wst16(ob, c * 32u + 16u, pack<GPUOS_F32>(o + 4));
            } else {
                wst16(ob, c * 16u, pack<GPUOS_BF16>(o));
            }
        }
        return;
    }
    // several splits: publish this partial, the last arriver merges
    float* part = (float*)(u.scratch + COUNTER_AREA) + (uint64_t)t * PSTRIDE;
    if (g == 0) {
        const WBuf pb = wbuf(part);
        wst16(pb, (4u + 8u * c) * 4u, pack<GPUOS_F32>(acc));
        wst16(pb, (8u + 8u * c) * 4u, pack<GPUOS_F32>(acc + 4));
    }
    if (lane == 0) { wstf(part, m); wstf(part + 1, lsum); }
    uint32_t* ctr = (uint32_t*)u.scratch + bh;
    uint32_t prev = 0;
    if (lane == 0) prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    prev = (uint32_t)__builtin_amdgcn_readlane((int)prev, 0);
    if (prev != ns - 1) return;
    // merge: M = max m_i, Ls = sum l_i e^{m_i - M}, o = sum acc_i e^{m_i - M} / Ls
    const float* p0 = (const float*)(u.scratch + COUNTER_AREA) + (uint64_t)(t - sp) * PSTRIDE;
    float M = -INFINITY;
    for (uint32_t i = 0; i < ns; ++i) M = fmaxf(M, p0[(uint64_t)i * PSTRIDE]);
    float Ls = 0.0f;
    constexpr uint32_t DPL = D / 64u;  // dims per lane
    float o[DPL];
#pragma unroll
    for (uint32_t e = 0; e < DPL; ++e) o[e] = 0.0f;
    for (uint32_t i = 0; i < ns; ++i) {
        const float* pi = p0 + (uint64_t)i * PSTRIDE;
        const float w = expf(pi[0] - M);
        Ls += pi[1] * w;
#pragma unroll
        for (uint32_t e = 0; e < DPL; ++e) o[e] += pi[4 + lane * DPL + e] * w;
    }
    const float inv = 1.0f / Ls;
#pragma unroll
    for (uint32_t e = 0; e < DPL; ++e) {
        const uint32_t d = lane * DPL + e;
        st_elem<DTO>(O, d, o[e] * inv);
    }
    if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ GEMV
// Unit = (column block of 64 lanes x 16 bytes, k-split of GEMV_KC rows of W).
// x[k] for the split is loaded once (lane k) and broadcast with readlane.
// With several k-splits each unit writes fp32 partial sums and the last unit
// of a column block adds them in split order (a fixed order).
template <uint32_t DT, uint32_t DTO>
__device__ __forceinline__ void gemv_tile(const Unit& u, uint32_t lane) {
    constexpr uint32_t ES = DT == GPUOS_F32 ? 4u : 2u;
    constexpr uint32_t VE = 16u / ES;
    constexpr uint32_t CPB = 64u * VE;
    const uint32_t K = u.dim[0], N = u.dim[1];
    const uint32_t ncb = (N + CPB - 1) / CPB, nks = (K + GEMV_KC - 1) / GEMV_KC;
    const uint32_t cb = u.tile % ncb, ks = u.tile / ncb;
    const uint32_t kb = ks * GEMV_KC, kn = min(K - kb, GEMV_KC);
    const uint8_t* X = (const uint8_t*)u.a;
    const uint8_t* Wm = (const uint8_t*)u.b;
    const float xv = lane < kn ? ld_elem<DT>(X, kb + lane) : 0.0f;
    const uint32_t c0 = cb * CPB + lane * VE;
    float acc[VE];
#pragma unroll
    for (uint32_t e = 0; e < VE; ++e) acc[e] = 0.0f;
    const bool vec = (N % VE) == 0 && ((uint64_t)Wm & 15ull) == 0;
    if (vec) {
        const bool mine = c0 < N;
        const uint8_t* wp = Wm + ((uint64_t)kb * N + c0) * ES;
        uint32_t r = 0;
        for (; r + 8 <= kn; r += 8) {
            u32x4 w[8];
#pragma unroll
            for (uint32_t j = 0; j < 8; ++j)
                if (mine) w[j] = ld16(wp + (uint64_t)(r + j) * N * ES);
#pragma unroll
            for (uint32_t j = 0; j < 8; ++j) {
                const float xr = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(xv), r + j));
                if (mine) {
                    float wf[VE];
                    unpack<DT>(w[j], wf);
#pragma unroll
                    for (uint32_t e = 0; e < VE; ++e) acc[e] += xr * wf[e];
                }
            }
        }
        for (; r < kn; ++r) {
            const float xr = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(xv), r));
            if (mine) {
                float wf[VE];
                unpack<DT>(ld16(wp + (uint64_t)r * N * ES), wf);
#pragma unroll
                for (uint32_t e = 0; e < VE; ++e) acc[e] += xr * wf[e];
            }
        }
    } else {
        // element path: lane handles columns cb*CPB + lane + 64 e
        for (uint32_t r = 0; r < kn; ++r) {
            const float xr = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(xv), r));
#pragma unroll
            for (uint32_t e = 0; e < VE; ++e) {
                const uint32_t col = cb * CPB + lane + 64u * e;
                if (col < N) acc[e] += xr * ld_elem<DT>(Wm, (uint64_t)(kb + r) * N + col);
            }
        }
    }
    // column of acc[e]
    auto col_of = [&](uint32_t e) -> uint32_t { return vec ? c0 + e : cb * CPB + lane + 64u * e; };
    uint8_t* Y = (uint8_t*)u.out;
    if (nks == 1) {
#pragma unroll
        for (uint32_t e = 0; e < VE; ++e) {
            const uint32_t col = col_of(e);
            if (col < N) st_elem<DTO>(Y, col, acc[e]);
        }
        return;
    }
    float* part = (float*)(u.scratch + COUNTER_AREA);
#pragma unroll
    for (uint32_t e = 0; e < VE; ++e) {
        const uint32_t col = col_of(e);
        if (col < N) wstf(part + (uint64_t)ks * N + col, acc[e]);
    }
    uint32_t* ctr = (uint32_t*)u.scratch + cb;
    uint32_t prev = 0;
    if (lane == 0) prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    prev = (uint32_t)__builtin_amdgcn_readlane((int)prev, 0);
    if (prev != nks - 1) return;
#pragma unroll
    for (uint32_t e = 0; e < VE; ++e) {
        const uint32_t col = col_of(e);
        if (col < N) {
            float s = 0.0f;
            for (uint32_t k = 0; k < nks; ++k) s += part[(uint64_t)k * N + col];
            st_elem<DTO>(Y, col, s);
        }
    }
    if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ COPY
__device__ __forceinline__ void copy_tile(const Unit& u, uint32_t lane) {
    const uint64_t start = (uint64_t)u.tile * COPY_TILE_BYTES;
    if (start >= u.size) return;
    const uint64_t end = u.size - start < COPY_TILE_BYTES ? u.size : start + COPY_TILE_BYTES;
    const uint8_t* A = (const uint8_t*)u.a;
    uint8_t* O = (uint8_t*)u.out;
    if (((u.a | u.out) & 15ull) == 0) {
        const WBuf ob = wbuf(O + start);
        u32x4 v[16];
#pragma unroll
        for (uint32_t k = 0; k < 16; ++k) {
            const uint64_t off = start + (uint64_t)(lane + 64u * k) * 16u;
            if (off + 16 <= end) v[k] = ld16(A + off);
        }
#pragma unroll
        for (uint32_t k = 0; k < 16; ++k) {
            const uint64_t off = start + (uint64_t)(lane + 64u * k) * 16u;
            if (off + 16 <= end) wst16(ob, (uint32_t)(off - start), v[k]);
        }
        const uint64_t rem = start + ((end - start) / 16u) * 16u;
        for (uint64_t i = rem + lane; i < end; i += 64u) wst8(O + i, A[i]);
    } else {
        for (uint64_t i = start + lane; i < end; i += 64u) wst8(O + i, A[i]);
    }
}

// ------------------------------------------------------------- dispatch
// Wave-uniform switch on the resolved kind (indirect calls would force a
// conservative register and stack budget on AMDGPU).
__device__ __forceinline__ void run_unit(const Unit& u, uint32_t lane) {
    const uint32_t di = dt_in(u.flags), dout = dt_out(u.flags);
    const bool bf = di == GPUOS_BF16;
    switch (u.kind) {
        case GPUOS_OP_NOP: break;
        case GPUOS_OP_ADD: bf ? ew_tile<GPUOS_OP_ADD, GPUOS_BF16>(u, lane) : ew_tile<GPUOS_OP_ADD, GPUOS_F32>(u, lane); break;
        case GPUOS_OP_MUL: bf ? ew_tile<GPUOS_OP_MUL, GPUOS_BF16>(u, lane) : ew_tile<GPUOS_OP_MUL, GPUOS_F32>(u, lane); break;
        case GPUOS_OP_RELU: bf ? ew_tile<GPUOS_OP_RELU, GPUOS_BF16>(u, lane) : ew_tile<GPUOS_OP_RELU, GPUOS_F32>(u, lane); break;
        case GPUOS_OP_GELU: bf ? ew_tile<GPUOS_OP_GELU, GPUOS_BF16>(u, lane) : ew_tile<GPUOS_OP_GELU, GPUOS_F32>(u, lane); break;
        case GPUOS_OP_SUM: bf ? row_tile<GPUOS_OP_SUM, GPUOS_BF16>(u, lane) : row_tile<GPUOS_OP_SUM, GPUOS_F32>(u, lane); break;
        case GPUOS_OP_MAX: bf ? row_tile<GPUOS_OP_MAX, GPUOS_BF16>(u, lane) : row_tile<GPUOS_OP_MAX, GPUOS_F32>(u, lane); break;
        case GPUOS_OP_MIN: bf ? row_tile<GPUOS_OP_MIN, GPUOS_BF16>(u, lane) : row_tile<GPUOS_OP_MIN, GPUOS_F32>(u, lane); break;
        case GPUOS_OP_SOFTMAX: bf ? row_tile<GPUOS_OP_SOFTMAX, GPUOS_BF16>(u, lane) : row_tile<GPUOS_OP_SOFTMAX, GPUOS_F32>(u, lane); break;
        case GPUOS_OP_LAYERNORM: bf ? row_tile<GPUOS_OP_LAYERNORM, GPUOS_BF16>(u, lane) : row_tile<GPUOS_OP_LAYERNORM, GPUOS_F32>(u, lane); break;
        case GPUOS_OP_ROPE: bf ? rope_tile<GPUOS_BF16>(u, lane) : rope_tile<GPUOS_F32>(u, lane); break;
        case GPUOS_OP_KV_APPEND: kv_tile(u, lane); break;
        case GPUOS_OP_SDPA:
            if (u.dim[1] == 128u) {
                dout == GPUOS_F32 ? sdpa_tile<16, GPUOS_F32>(u, lane) : sdpa_tile<16, GPUOS_BF16>(u, lane);
            } else {
                dout == GPUOS_F32 ? sdpa_tile<8, GPUOS_F32>(u, lane) : sdpa_tile<8, GPUOS_BF16>(u, lane);
            }
            break;
        case GPUOS_OP_GEMV:
            if (bf) dout == GPUOS_F32 ? gemv_tile<GPUOS_BF16, GPUOS_F32>(u, lane) : gemv_tile<GPUOS_BF16, GPUOS_BF16>(u, lane);
            else dout == GPUOS_F32 ? gemv_tile<GPUOS_F32, GPUOS_F32>(u, lane) : gemv_tile<GPUOS_F32, GPUOS_BF16>(u, lane);
            break;
        case GPUOS_OP_COPY: copy_tile(u, lane); break;
        default: break;
    }
}

}  // namespace gpuos
