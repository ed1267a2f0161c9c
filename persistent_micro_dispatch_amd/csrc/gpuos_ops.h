// Micro-op bodies for CDNA4 (gfx950).  Each body runs one work unit (a
// tile of one descriptor) on one wave64; the executor and the eager
// baseline kernels call the same functions.
//
// Operator list: GPUOS digest page, section 3 Q2 ("Operator library"):
// element-wise add/mul/ReLU/GELU, softmax, LayerNorm, vector-matrix
// products, SDPA, rotary embeddings, KV-cache update, sum/max/min.
//
// Memory access rules that every body follows:
//  - Operand pointers arrive in descriptors, so the compiler cannot see that
//    they are global; left generic they become flat instructions, which also
//    count on the LDS/scalar counter: every shuffle or scalar load would then
//    wait for all outstanding loads, and a guarded flat load is preceded by a
//    full wait.  All loads and stores of op data name the global address
//    space, or go through a buffer resource.
//  - Loads and stores of op data are device-scope (cache policy SC1): loads
//    are coherent across the eight XCDs, whose L2s are not, and stores are
//    written through.  A unit therefore needs no cache invalidation before
//    it reads what a unit on another XCD wrote, and no L2 write-back after
//    it writes: waiting for its own stores (stores_done) publishes them.
//  - A body issues all loads of a batch before it uses any of them, so one
//    wave keeps 8-32 KiB in flight; stores come after.
//  - Ragged ends use buffer resources bounded to the valid bytes: 16-byte
//    loads beyond the bound return zero and stores beyond it are dropped,
//    without a divergent branch around the access.
//  - Reductions inside 8- or 16-lane groups use DPP lane moves; across the
//    four 16-lane rows of the wave, readlane.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gpuos_internal.h"
#include "rope_math.h"

namespace gpuos {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(1))) const u32x4 gc_u32x4;
typedef __attribute__((address_space(1))) const uint32_t gc_u32;
typedef __attribute__((address_space(1))) const uint16_t gc_u16;
typedef __attribute__((address_space(1))) const uint8_t gc_u8;
typedef __attribute__((address_space(1))) uint64_t g_u64;
typedef __attribute__((address_space(1))) uint32_t g_u32;
typedef __attribute__((address_space(1))) uint16_t g_u16;
typedef __attribute__((address_space(1))) uint8_t g_u8;

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
    uint64_t prog;    // EXPR: the program (device memory), else 0
};

// ------------------------------------------------------------------ scalars
__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.  gfx950
// converts two floats per instruction (v_cvt_pk_bf16_f32, under the default
// round-to-nearest-even mode); over all 2^32 inputs it matches rounding the
// bit pattern (add 0x7FFF plus the lowest kept bit, truncate), NaN aside.
typedef __bf16 bf16v2 __attribute__((ext_vector_type(2)));
typedef float f32v2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f2bf2(float lo, float hi) {
    const f32v2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16v2));
}
__device__ __forceinline__ uint32_t f2bf(float f) { return f2bf2(f, 0.0f) & 0xFFFFu; }

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

// ------------------------------------------------------------ global memory
// Device-coherent scalar loads (relaxed agent-scope atomic loads compile to
// SC1 global loads).
__device__ __forceinline__ uint32_t ld4(const uint8_t* p) {
    return __hip_atomic_load((g_u32*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld2(const uint8_t* p) {
    return __hip_atomic_load((g_u16*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld1(const uint8_t* p) {
    return __hip_atomic_load((g_u8*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <uint32_t DT>
__device__ __forceinline__ float ld_elem(const uint8_t* p, uint64_t i) {
    if constexpr (DT == GPUOS_F32) return __uint_as_float(ld4(p + 4 * i));
    else return bf2f(ld2(p + 2 * i));
}

// Stores of op outputs are device-scope write-through (cache policy SC1): the
// eight XCD L2s are not coherent, and a release fence on gfx950 has to write
// back every dirty line of the issuing XCD's L2.  Writing results through
// keeps that fence cheap and leaves nothing stale for readers on other XCDs.
// Narrow stores are relaxed agent-scope atomic stores, which compile to the
// same SC1 global stores.
__device__ __forceinline__ void wst32(void* p, uint32_t v) {
    __hip_atomic_store((g_u32*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wst16b(void* p, uint16_t v) {
    __hip_atomic_store((g_u16*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wst8(void* p, uint8_t v) {
    __hip_atomic_store((g_u8*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wst64(void* p, uint64_t v) {
    __hip_atomic_store((g_u64*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wstf(void* p, float v) { wst32(p, __float_as_uint(v)); }

template <uint32_t DT>
__device__ __forceinline__ void st_elem(uint8_t* p, uint64_t i, float v) {
    if constexpr (DT == GPUOS_F32) wstf(p + 4 * i, v);
    else wst16b(p + 2 * i, (uint16_t)f2bf(v));
}

// Wait until every store this wave issued is acknowledged at device scope
// (gfx9 counts stores in vmcnt).  With write-through stores this makes them
// visible to every XCD, in place of a release fence, which on gfx950 would
// also write back the whole L2 of the issuing XCD.  The memory clobber keeps
// the compiler from moving memory accesses across the wait.
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ------------------------------------------------------- buffer resources
// A window of `nbytes` at `base` (raw buffer, stride 0).  Word 3 selects the
// 32-bit data format that raw buffer instructions require on gfx9-family
// parts.  Offsets are 32-bit: callers keep windows below 2 GiB.
#ifndef GPUOS_GEMV_DOT2
#define GPUOS_GEMV_DOT2 1
#endif
constexpr bool GEMV_DOT2 = GPUOS_GEMV_DOT2;
constexpr int CPOL_SC1 = 16;
// Data read once per descriptor and never again soon (attention's keys and
// values, a vector-matrix product's weights) is loaded with the
// non-temporal hint as well, so that it does not displace cached data
// (decode stream +4.6%).  Element-wise operands and every store keep plain
// SC1: non-temporal stores lengthened the dependent-op latency by 7%.
constexpr int CPOL_NT = 2;
#ifndef GPUOS_STREAM_CPOL
#define GPUOS_STREAM_CPOL (16 | 2)
#endif
constexpr int CPOL_LD = CPOL_SC1, CPOL_ST = CPOL_SC1, CPOL_STREAM = GPUOS_STREAM_CPOL;
struct RBuf {
    __amdgpu_buffer_rsrc_t r;
};
struct WBuf {
    __amdgpu_buffer_rsrc_t r;
};
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mkrsrc(const void* base, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}
__device__ __forceinline__ RBuf rbuf(const void* base, uint32_t nbytes) { return RBuf{mkrsrc(base, nbytes)}; }
__device__ __forceinline__ WBuf wbuf(const void* base, uint32_t nbytes = 0x7FFFFFFFu) {
    return WBuf{mkrsrc(base, nbytes)};
}
__device__ __forceinline__ u32x4 rld16(RBuf b, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(b.r, (int)off, 0, CPOL_LD);
}
__device__ __forceinline__ u32x4 rld16s(RBuf b, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(b.r, (int)off, 0, CPOL_STREAM);
}
__device__ __forceinline__ uint32_t rld4(RBuf b, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(b.r, (int)off, 0, CPOL_LD);
}
__device__ __forceinline__ void wst16(WBuf b, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, b.r, (int)off, 0, CPOL_ST);
}

// Two bf16 in one dword.  The argument is taken by value: a bit cast applied
// directly to a vector component expression (v.y) reads component 0 with
// this compiler.
__device__ __forceinline__ bf16x2 as_bf2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// 16 bytes -> VE floats
template <uint32_t DT>
__device__ __forceinline__ void unpack(u32x4 v, float* f) {
    if constexpr (DT == GPUOS_F32) {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    } else {
        f[0] = bf2f(v.x & 0xFFFFu); f[1] = __uint_as_float(v.x & 0xFFFF0000u);
        f[2] = bf2f(v.y & 0xFFFFu); f[3] = __uint_as_float(v.y & 0xFFFF0000u);
        f[4] = bf2f(v.z & 0xFFFFu); f[5] = __uint_as_float(v.z & 0xFFFF0000u);
        f[6] = bf2f(v.w & 0xFFFFu); f[7] = __uint_as_float(v.w & 0xFFFF0000u);
    }
}
template <uint32_t DT>
__device__ __forceinline__ u32x4 pack(const float* f) {
    u32x4 v;
    if constexpr (DT == GPUOS_F32) {
        v.x = __float_as_uint(f[0]); v.y = __float_as_uint(f[1]);
        v.z = __float_as_uint(f[2]); v.w = __float_as_uint(f[3]);
    } else {
        v.x = f2bf2(f[0], f[1]); v.y = f2bf2(f[2], f[3]);
        v.z = f2bf2(f[4], f[5]); v.w = f2bf2(f[6], f[7]);
    }
    return v;
}

__device__ __forceinline__ float relu_f(float x) { return x > 0.0f ? x : (x != x ? x : 0.0f); }

// GELU, tanh approximation, evaluated as x / (1 + exp(-2u)) with
// u = sqrt(2/pi) (x + 0.044715 x^3) (the same function; no cancellation).
// For x > -3 the exponent a = -2u stays below 7.3, and fp32 arithmetic with
// the hardware exp2 and reciprocal keeps the relative error below 1.1e-6
// (largest over every fp32 x > -3, against a double evaluation; the result's
// sensitivity to an absolute error in a is at most 1).  For x <= -3 the
// result is about x e^{-a} with a large, so a must be exact to well below
// 1e-5 in absolute terms: there a is formed in double and split as
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
    if (!(x > -3.0f)) return gelu_wide(x);   // also NaN and -inf
    // a = -2 sqrt(2/pi) (x + 0.044715 x^3) = x (-1.5957691 - 0.0713548 x^2);
    // +inf gives a = -inf, e = 0 and the result +inf
    const float a = x * fmaf(-0.0713548162726f, x * x, -1.5957691216057308f);
    const float e = __builtin_amdgcn_exp2f(a * 1.44269504f);
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// max / min under a total order: NaN wins, -0 < +0.
// Written as selects, not early returns: the returns became divergent
// branches around every element.  Equal operands are identical bit
// patterns unless they are +0 and -0, so AND of the bits picks +0 for max and
// OR picks -0 for min.  -inf (max) and +inf (min) are identities.
__device__ __forceinline__ float tmax(float a, float b) {
    const float m = a < b ? b : a;
    const float z = __uint_as_float(__float_as_uint(a) & __float_as_uint(b));
    const float r = a == b ? z : m;
    return a != a ? a : (b != b ? b : r);
}
__device__ __forceinline__ float tmin(float a, float b) {
    const float m = a < b ? a : b;
    const float z = __uint_as_float(__float_as_uint(a) | __float_as_uint(b));
    const float r = a == b ? z : m;
    return a != a ? a : (b != b ? b : r);
}

// ------------------------------------------------------------ wave helpers
// DPP lane moves (gfx9 encodings): quad_perm [1,0,3,2] and [2,3,0,1] swap
// neighbours and pairs; half-mirror reverses each 8 lanes, mirror each 16.
// After xor1, xor2 every lane holds its quad's value; half-mirror then pairs
// quad 0 with quad 1 of each 8, mirror pairs the two 8s of each 16.  Each
// step combines a lane with a partner that holds the mirror-image partial,
// so every lane of the group ends with the same, bit-identical result.
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float rlf(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
struct OpAdd { __device__ float operator()(float a, float b) const { return a + b; } };
struct OpMax { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };
struct OpTMax { __device__ float operator()(float a, float b) const { return tmax(a, b); } };
struct OpTMin { __device__ float operator()(float a, float b) const { return tmin(a, b); } };

// combine over groups of G (8 or 16) consecutive lanes; all lanes active
template <int G, class F>
__device__ __forceinline__ float gred(float v, F f) {
    v = f(v, dpp<DPP_XOR1>(v));
    v = f(v, dpp<DPP_XOR2>(v));
    v = f(v, dpp<DPP_HALF_MIRROR>(v));
    if constexpr (G == 16) v = f(v, dpp<DPP_MIRROR>(v));
    return v;
}
// combine over the wave: 16-lane groups, then the four rows in a fixed order
template <class F>
__device__ __forceinline__ float wred(float v, F f) {
    v = gred<16>(v, f);
    return f(f(rlf(v, 0), rlf(v, 16)), f(rlf(v, 32), rlf(v, 48)));
}
__device__ __forceinline__ float wsum(float v) { return wred(v, OpAdd{}); }
__device__ __forceinline__ float wmaxf(float v) { return wred(v, OpMax{}); }
__device__ __forceinline__ float wtmax(float v) { return wred(v, OpTMax{}); }
__device__ __forceinline__ float wtmin(float v) { return wred(v, OpTMin{}); }

// ------------------------------------------------------------ element-wise
template <uint32_t K>
__device__ __forceinline__ float ew_op(float x, float y) {
    if constexpr (K == GPUOS_OP_ADD) return x + y;
    else if constexpr (K == GPUOS_OP_MUL) return x * y;
    else if constexpr (K == GPUOS_OP_RELU) return relu_f(x);
    else return gelu_f(x);
}

// bf16 ReLU acts on the bit pattern (no rounding involved)
__device__ __forceinline__ uint32_t relu_bf16(uint32_t h) {
    if ((h & 0x7FFFu) > 0x7F80u) return h;  // NaN
    return (h & 0x8000u) ? 0u : h;          // negatives and -0 -> +0
}
// Both halves of a dword at once: a half is NaN exactly when its magnitude
// plus 0x7F carries into bit 15 (magnitudes are at most 0x7FFF, so no carry
// crosses into the other half); halves with the sign set and not NaN become
// +0, through a mask spread from bit 15 over the half by a multiply.
__device__ __forceinline__ uint32_t relu_bf16x2(uint32_t v) {
    const uint32_t nan = ((v & 0x7FFF7FFFu) + 0x007F007Fu) & 0x80008000u;
    const uint32_t z = v & 0x80008000u & ~nan;
    return v & ~((z >> 15) * 0xFFFFu);
}
__device__ __forceinline__ u32x4 relu_bf16x8(u32x4 v) {
    return u32x4{relu_bf16x2(v.x), relu_bf16x2(v.y), relu_bf16x2(v.z), relu_bf16x2(v.w)};
}

// One tile of ew_tile_bytes(K, false) per operand: CH chunks of 16 bytes
// per lane (4 for add/mul/ReLU, 2 for GELU), all loads issued first.  The
// elements after the last whole chunk (fewer than one chunk) are one per
// lane.  Misaligned operands take an element loop.
template <uint32_t K, uint32_t DT>
__device__ __forceinline__ void ew_tile(const Unit& u, uint32_t tile, uint32_t lane) {
    constexpr uint32_t ES = DT == GPUOS_F32 ? 4u : 2u;
    constexpr uint32_t TILE = ew_tile_bytes(K, false) / ES;
    constexpr uint32_t VE = 16u / ES;
    constexpr uint32_t CH = TILE / VE / 64u;
    constexpr bool BIN = (K == GPUOS_OP_ADD || K == GPUOS_OP_MUL);
    constexpr bool RELU16 = (K == GPUOS_OP_RELU && DT == GPUOS_BF16);
    const uint64_t start = (uint64_t)tile * TILE;
    if (start >= u.size) return;
    const uint32_t cnt = (uint32_t)(u.size - start < TILE ? u.size - start : TILE);
    const uint8_t* A = (const uint8_t*)u.a + start * ES;
    const uint8_t* B = (const uint8_t*)u.b + start * ES;
    uint8_t* O = (uint8_t*)u.out + start * ES;
    const bool aligned = (((u.a | u.out | (BIN ? u.b : 0ull)) & 15ull) == 0);
    if (aligned) {
        const uint32_t full = cnt / VE;  // whole 16-byte chunks
        const RBuf ra = rbuf(A, full * 16u);
        const RBuf rb = rbuf(BIN ? B : A, full * 16u);
        const WBuf ob = wbuf(O, full * 16u);
        u32x4 va[CH], vb[CH];
#pragma unroll
        for (uint32_t c = 0; c < CH; ++c) {
            va[c] = rld16(ra, (lane + 64u * c) * 16u);
            if constexpr (BIN) vb[c] = rld16(rb, (lane + 64u * c) * 16u);
        }
        const uint32_t rem = full * VE;
        const bool tl = rem + lane < cnt;
        float xt = 0.0f, yt = 0.0f;
        if (tl) {
            xt = ld_elem<DT>(A, rem + lane);
            if constexpr (BIN) yt = ld_elem<DT>(B, rem + lane);
        }
#pragma unroll
        for (uint32_t c = 0; c < CH; ++c) {
            u32x4 o;
            if constexpr (RELU16) {
                o = relu_bf16x8(va[c]);
            } else {
                float x[VE], y[VE], r[VE];
                unpack<DT>(va[c], x);
                if constexpr (BIN) unpack<DT>(vb[c], y);
#pragma unroll
                for (uint32_t e = 0; e < VE; ++e) r[e] = ew_op<K>(x[e], BIN ? y[e] : 0.0f);
                o = pack<DT>(r);
            }
            wst16(ob, (lane + 64u * c) * 16u, o);  // chunks past `full` are dropped
        }
        if (tl) {
            if constexpr (RELU16) wst16b(O + 2u * (rem + lane), (uint16_t)relu_bf16(ld2(A + 2u * (rem + lane))));
            else st_elem<DT>(O, rem + lane, ew_op<K>(xt, yt));
        }
    } else {
        for (uint32_t i = lane; i < cnt; i += 64u) {
            if constexpr (RELU16) wst16b(O + 2u * i, (uint16_t)relu_bf16(ld2(A + 2u * i)));
            else st_elem<DT>(O, i, ew_op<K>(ld_elem<DT>(A, i), BIN ? ld_elem<DT>(B, i) : 0.0f));
        }
    }
}

// ------------------------------------------------------------ EXPR ops
// An element-wise program bound with gpuos_register_expr, interpreted per
// element on four fp32 registers.  The program (at most PROG_WORDS words)
// is read once per unit, word i into lane i with device-scope loads, and
// every instruction is then taken from a lane with readlane, so decoding is
// wave-uniform.  Tiles are laid out as for the built-in element-wise ops,
// but chunks are interpreted in a loop (the next chunk's loads issued before
// the current one is used) rather than unrolled: the interpreter is inlined
// once per element count, which keeps the executor's code small.
//
// exp, log, tanh and the logistic function use the hardware's exp2 and log2
// instructions (about 1 ulp) with the argument scaled in two parts, so their
// error stays near 1e-7 relative (absolute where the result is near 0).
__device__ __forceinline__ float xexp(float x) {
    // e^x = 2^t * 2^r with t = fl(x log2 e), r the rounding error of t plus
    // the low part of log2 e; |r| is tiny, so 2^r = 1 + r ln 2
    // (results below 2^-126 are formed as 2^(t+64) * 2^-64: the
    // instruction does not produce subnormals)
    const float t = x * 1.44269504f;
    const float r = fmaf(x, 1.44269504f, -t) + x * 1.9259629e-8f;
    const bool sub = t < -126.0f;
    const float p = __builtin_amdgcn_exp2f(sub ? t + 64.0f : t) * fmaf(r, 0.693147181f, 1.0f);
    return sub ? p * 5.42101086e-20f : p;
}
__device__ __forceinline__ float xlog(float x) {
    // subnormal arguments are scaled by 2^24 first
    const bool sub = x > 0.0f && x < 1.17549435e-38f;
    return __builtin_amdgcn_logf(sub ? x * 16777216.0f : x) * 0.693147181f - (sub ? 16.6355324f : 0.0f);
}
__device__ __forceinline__ float xtanh(float x) {
    const float e = xexp(2.0f * fabsf(x));
    const float t = 1.0f - 2.0f / (e + 1.0f);
    return x != x ? x : copysignf(t, x);
}
struct XRegs4 {
    float r[4];
};
__device__ __forceinline__ float xsel(const XRegs4& R, uint32_t i) {
    return i == 0 ? R.r[0] : i == 1 ? R.r[1] : i == 2 ? R.r[2] : R.r[3];
}
__device__ __forceinline__ void xput(XRegs4& R, uint32_t i, float v) {
    R.r[0] = i == 0 ? v : R.r[0];
    R.r[1] = i == 1 ? v : R.r[1];
    R.r[2] = i == 2 ? v : R.r[2];
    R.r[3] = i == 3 ? v : R.r[3];
}
__device__ __forceinline__ float xop(uint32_t op, float x, float y, float a, float b, float k) {
    switch (op) {
        case GPUOS_X_LDA: return a;
        case GPUOS_X_LDB: return b;
        case GPUOS_X_CONST: return k;
        case GPUOS_X_MOV: return x;
        case GPUOS_X_ADD: return x + y;
        case GPUOS_X_SUB: return x - y;
        case GPUOS_X_MUL: return x * y;
        case GPUOS_X_DIV: return x / y;
        case GPUOS_X_MIN: return tmin(x, y);
        case GPUOS_X_MAX: return tmax(x, y);
        case GPUOS_X_NEG: return __uint_as_float(__float_as_uint(x) ^ 0x80000000u);
        case GPUOS_X_ABS: return __uint_as_float(__float_as_uint(x) & 0x7FFFFFFFu);
        case GPUOS_X_EXP: return xexp(x);
        case GPUOS_X_LOG: return xlog(x);
        case GPUOS_X_SQRT: return sqrtf(x);
        case GPUOS_X_TANH: return xtanh(x);
        case GPUOS_X_SIGMOID: return 1.0f / (1.0f + xexp(-x));
        default: return x > 0.0f ? x : (x != x ? x : 0.0f);  // RELU (the host admits no other op)
    }
}
// Run the program on N elements; pw holds program word `lane` in each lane.
template <uint32_t N>
__device__ __forceinline__ void xrun(uint32_t pw, uint32_t ni, const float* a, const float* b, float* out) {
    XRegs4 R[N];
#pragma unroll
    for (uint32_t e = 0; e < N; ++e) R[e] = XRegs4{{0.0f, 0.0f, 0.0f, 0.0f}};
    for (uint32_t i = 0; i < ni; ++i) {
        const uint32_t w = (uint32_t)__builtin_amdgcn_readlane((int)pw, (int)(PROG_INSTR + i));
        const uint32_t op = w & 0xFFu, d = (w >> 8) & 3u, s1 = (w >> 12) & 3u, s2 = (w >> 16) & 3u;
        const float k = __uint_as_float(
            (uint32_t)__builtin_amdgcn_readlane((int)pw, (int)(PROG_CONST + ((w >> 20) & (GPUOS_EXPR_MAX_CONSTS - 1)))));
#pragma unroll
        for (uint32_t e = 0; e < N; ++e) xput(R[e], d, xop(op, xsel(R[e], s1), xsel(R[e], s2), a[e], b[e], k));
    }
#pragma unroll
    for (uint32_t e = 0; e < N; ++e) out[e] = R[e].r[0];
}

template <uint32_t DT>
__device__ __forceinline__ void expr_tile(const Unit& u, uint32_t lane) {
    constexpr uint32_t ES = DT == GPUOS_F32 ? 4u : 2u;
    constexpr uint32_t VE = 16u / ES;
    const uint32_t pw = lane < PROG_WORDS ? ld4((const uint8_t*)u.prog + 4u * lane) : 0u;
    const uint32_t w0 = (uint32_t)__builtin_amdgcn_readlane((int)pw, 0);
    const uint32_t ni = w0 & 0xFFu;
    const uint32_t tb = expr_tile_bytes(ni << 8, ew_big(u.size, ES));
    const uint32_t TILE = tb / ES, CH = tb / 16u / 64u;
    const uint64_t start = (uint64_t)u.tile * TILE;
    if (start >= u.size) return;
    const uint32_t cnt = (uint32_t)(u.size - start < TILE ? u.size - start : TILE);
    const bool useb = u.b != 0;
    const uint8_t* A = (const uint8_t*)u.a + start * ES;
    const uint8_t* B = useb ? (const uint8_t*)u.b + start * ES : A;
    uint8_t* O = (uint8_t*)u.out + start * ES;
    const bool aligned = (((u.a | u.out | u.b) & 15ull) == 0);
    if (aligned) {
        const uint32_t full = cnt / VE;  // whole 16-byte chunks
        const RBuf ra = rbuf(A, full * 16u), rb = rbuf(B, full * 16u);
        const WBuf ob = wbuf(O, full * 16u);
        const uint32_t rem = full * VE;
        const bool tl = rem + lane < cnt;
        float xt = 0.0f, yt = 0.0f;
        if (tl) {
            xt = ld_elem<DT>(A, rem + lane);
            yt = ld_elem<DT>(B, rem + lane);
        }
        u32x4 na = rld16(ra, lane * 16u), nb = rld16(rb, lane * 16u);
#pragma unroll 1
        for (uint32_t c = 0; c < CH; ++c) {
            const u32x4 ca = na, cb = nb;
            // the next chunk (past the tile: outside the window, reads zero)
            na = rld16(ra, (lane + 64u * (c + 1)) * 16u);
            nb = rld16(rb, (lane + 64u * (c + 1)) * 16u);
            __builtin_amdgcn_sched_barrier(0);
            float x[VE], y[VE], r[VE];
            unpack<DT>(ca, x);
            unpack<DT>(cb, y);
            xrun<VE>(pw, ni, x, y, r);
            wst16(ob, (lane + 64u * c) * 16u, pack<DT>(r));  // chunks past `full` are dropped
        }
        if (tl) {
            float r;
            xrun<1>(pw, ni, &xt, &yt, &r);
            st_elem<DT>(O, rem + lane, r);
        }
    } else {
        for (uint32_t i = lane; i < cnt; i += 64u) {
            const float x = ld_elem<DT>(A, i), y = ld_elem<DT>(B, i);
            float r;
            xrun<1>(pw, ni, &x, &y, &r);
            st_elem<DT>(O, i, r);
        }
    }
}

// ------------------------------------------------------------------ rows
// A unit is rows_per_unit(h) consecutive rows of [rows, h], done one after
// another.  Rows up to ROW_MAX_CACHED elements with 16-byte alignment are
// held in registers (up to 16 chunks of 16 bytes per lane, loaded in one
// batch together with LayerNorm's gamma and beta for the first LN_PRE
// chunks; the rest of gamma and beta is loaded after the statistics); others
// stream from memory in several passes.
template <uint32_t K, uint32_t DT>
__device__ __forceinline__ void row_one(const Unit& u, uint64_t r, uint32_t lane) {
    constexpr uint32_t ES = DT == GPUOS_F32 ? 4u : 2u;
    constexpr uint32_t VE = 16u / ES;
    constexpr uint32_t KMAX = ROW_MAX_CACHED / VE / 64u;
    constexpr bool RED = (K == GPUOS_OP_SUM || K == GPUOS_OP_MAX || K == GPUOS_OP_MIN);
    constexpr bool LN = (K == GPUOS_OP_LAYERNORM);
    constexpr uint32_t LN_PRE = KMAX / 2;
    const uint32_t h = u.dim[0];
    const uint8_t* X = (const uint8_t*)u.a + r * h * ES;
    uint8_t* O = (uint8_t*)u.out + (RED ? r * ES : r * h * ES);
    const uint8_t* G = (const uint8_t*)u.aux0;
    const uint8_t* Bt = (const uint8_t*)u.aux1;
    float eps = 1e-5f;
    if constexpr (LN) eps = u.pf[0] != 0.0f ? u.pf[0] : (u.p0 != 0.0f ? u.p0 : 1e-5f);
    const float inv_h = 1.0f / (float)h;
    uint64_t amask = (uint64_t)X | (RED ? 0ull : (uint64_t)O);
    if constexpr (LN) amask |= u.aux0 | u.aux1;
    const bool cached = h <= ROW_MAX_CACHED && (h % VE) == 0 && (amask & 15ull) == 0;
    if (cached) {
        const uint32_t nch = h / VE;
        const uint32_t kn = (nch + 63u) / 64u;  // chunk rounds in use (wave-uniform)
        const RBuf rx = rbuf(X, h * ES);
        u32x4 raw[KMAX], rg[LN ? LN_PRE : 1], rbb[LN ? LN_PRE : 1];
#pragma unroll
        for (uint32_t k = 0; k < KMAX; ++k)
            if (k < kn) raw[k] = rld16(rx, (lane + 64u * k) * 16u);
        const RBuf rgm = rbuf(G, LN ? h * ES : 0u), rbt = rbuf(Bt, LN ? h * ES : 0u);
        if constexpr (LN) {
#pragma unroll
            for (uint32_t k = 0; k < LN_PRE; ++k)
                if (k < kn) {
                    rg[k] = rld16(rgm, (lane + 64u * k) * 16u);
                    rbb[k] = rld16(rbt, (lane + 64u * k) * 16u);
                }
        }
        float v[KMAX][VE];
        float acc = K == GPUOS_OP_MAX ? -INFINITY : (K == GPUOS_OP_MIN ? INFINITY : 0.0f), mx = -INFINITY;
#pragma unroll
        for (uint32_t k = 0; k < KMAX; ++k) {
            if (k < kn) {
                const bool valid = lane + 64u * k < nch;  // chunks past the row read as zero
                unpack<DT>(raw[k], v[k]);
#pragma unroll
                for (uint32_t e = 0; e < VE; ++e) {
                    const float x = v[k][e];
                    if constexpr (K == GPUOS_OP_SUM || LN) {
                        acc += x;
                    } else if constexpr (K == GPUOS_OP_MAX || K == GPUOS_OP_MIN) {
                        const float c = K == GPUOS_OP_MAX ? tmax(acc, x) : tmin(acc, x);
                        acc = valid ? c : acc;
                    } else {
                        mx = valid ? fmaxf(mx, x) : mx;
                    }
                }
            }
        }
        const WBuf ob = wbuf(O, RED ? ES : h * ES);
        if constexpr (K == GPUOS_OP_SUM) {
            acc = wsum(acc);
            if (lane == 0) st_elem<DT>(O, 0, acc);
        } else if constexpr (K == GPUOS_OP_MAX || K == GPUOS_OP_MIN) {
            // lanes that saw no element hold the identity
            acc = K == GPUOS_OP_MAX ? wtmax(acc) : wtmin(acc);
            if (lane == 0) st_elem<DT>(O, 0, acc);
        } else if constexpr (K == GPUOS_OP_SOFTMAX) {
            mx = wmaxf(mx);
            float s = 0.0f;
#pragma unroll
            for (uint32_t k = 0; k < KMAX; ++k) {
                if (k < kn) {
                    const bool valid = lane + 64u * k < nch;
#pragma unroll
                    for (uint32_t e = 0; e < VE; ++e) {
                        v[k][e] = valid ? expf(v[k][e] - mx) : 0.0f;
                        s += v[k][e];
                    }
                }
            }
            s = wsum(s);
#pragma unroll
            for (uint32_t k = 0; k < KMAX; ++k) {
                if (k < kn) {
                    float o[VE];
#pragma unroll
                    for (uint32_t e = 0; e < VE; ++e) o[e] = v[k][e] / s;
                    wst16(ob, (lane + 64u * k) * 16u, pack<DT>(o));
                }
            }
        } else {  // LAYERNORM: two-pass variance from the registers
            const float mean = wsum(acc) * inv_h;
            float q = 0.0f;
#pragma unroll
            for (uint32_t k = 0; k < KMAX; ++k) {
                if (k < kn) {
                    const bool valid = lane + 64u * k < nch;
#pragma unroll
                    for (uint32_t e = 0; e < VE; ++e) {
                        const float d = v[k][e] - mean;
                        q += valid ? d * d : 0.0f;
                    }
                }
            }
            const float var = wsum(q) * inv_h;
            const float rstd = 1.0f / sqrtf(var + eps);
            u32x4 lg[KMAX - LN_PRE], lb[KMAX - LN_PRE];
#pragma unroll
            for (uint32_t k = LN_PRE; k < KMAX; ++k)
                if (k < kn) {
                    lg[k - LN_PRE] = rld16(rgm, (lane + 64u * k) * 16u);
                    lb[k - LN_PRE] = rld16(rbt, (lane + 64u * k) * 16u);
                }
#pragma unroll
            for (uint32_t k = 0; k < KMAX; ++k) {
                if (k < kn) {
                    float g[VE], bb[VE], o[VE];
                    unpack<DT>(k < LN_PRE ? rg[k < LN_PRE ? k : 0] : lg[k < LN_PRE ? 0 : k - LN_PRE], g);
                    unpack<DT>(k < LN_PRE ? rbb[k < LN_PRE ? k : 0] : lb[k < LN_PRE ? 0 : k - LN_PRE], bb);
#pragma unroll
                    for (uint32_t e = 0; e < VE; ++e) o[e] = (v[k][e] - mean) * rstd * g[e] + bb[e];
                    wst16(ob, (lane + 64u * k) * 16u, pack<DT>(o));
                }
            }
        }
        return;
    }
    // streaming path
    if constexpr (RED) {
        float acc = K == GPUOS_OP_MAX ? -INFINITY : (K == GPUOS_OP_MIN ? INFINITY : 0.0f);
        for (uint32_t i = lane; i < h; i += 64u) {
            const float x = ld_elem<DT>(X, i);
            if constexpr (K == GPUOS_OP_SUM) acc += x;
            else if constexpr (K == GPUOS_OP_MAX) acc = tmax(acc, x);
            else acc = tmin(acc, x);
        }
        if constexpr (K == GPUOS_OP_SUM) {
            acc = wsum(acc);
        } else {
            acc = K == GPUOS_OP_MAX ? wtmax(acc) : wtmin(acc);  // lanes without elements hold the identity
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


template <uint32_t K, uint32_t DT>
__device__ __forceinline__ void row_tile(const Unit& u, uint32_t lane) {
    const uint32_t g = rows_per_unit(u.dim[0], DT);
    const uint64_t r0 = (uint64_t)u.tile * g;
    const uint64_t r1 = r0 + g < u.size ? r0 + g : u.size;
    for (uint64_t r = r0; r < r1; ++r) row_one<K, DT>(u, r, lane);
}

// ------------------------------------------------------------------ RoPE
// Unit = one batch row b and a group of heads (rope_heads_per_unit), of both
// q and k, rotated at pos = L_b - 1.  The angle pos * theta^(-2i/D), its sine
// and cosine (rope_math.h, a few double ulps) and the rotation are evaluated
// in double and rounded once to the dtype, so the result is the correctly
// rounded rotation except where the exact value lies within a few double
// ulps of a rounding boundary.
//
// Fast path (adjacent pairs, a head's row of D elements = CPR chunks of 16
// bytes with CPR dividing 64, 16-byte aligned operands): the unit's heads
// are exactly one load instruction per tensor; lane l holds column chunk
// l % CPR of head l / CPR, so it computes the angles of its VE/2 pairs once.
template <uint32_t DT>
__device__ __forceinline__ void rope_tile(const Unit& u, uint32_t lane) {
    constexpr uint32_t ES = DT == GPUOS_F32 ? 4u : 2u;
    constexpr uint32_t VE = 16u / ES;
    const uint32_t H = u.dim[0], D = u.dim[1];
    const uint32_t Hk = u.dim[3] ? u.dim[3] : H;  // k's heads (fewer under grouped-query attention)
    const uint32_t RH = rope_heads_per_unit(D, DT);
    const uint32_t ng = (H + RH - 1) / RH;
    const uint32_t b = u.tile / ng, h0 = (u.tile - b * ng) * RH;
    const uint32_t hn = min(RH, H - h0);
    const bool half = (u.flags & GPUOS_F_ROPE_HALF) != 0;
    const double theta = u.pf[4] != 0.0f ? (double)u.pf[4] : (u.p0 != 0.0f ? (double)u.p0 : 10000.0);
    const double pos = (double)((int)lens_at(u.lensw, b) - 1);
    const double l2t = rmath::log2_d(theta);
    const uint32_t RB = D * ES;
    const uint32_t CPR = RB / 16u;
    const bool fast = !half && (RB % 16u) == 0 && CPR > 0 && CPR <= 64u && (64u % CPR) == 0 &&
                      ((u.a | u.b) & 15ull) == 0 && (uint64_t)H * RB < 0x80000000ull;
    if (fast) {
        // here RH = 64 / CPR: one row per (lane / CPR), rows past H read zero
        // and their stores are dropped by the window
        const uint32_t cc = lane % CPR, sub = lane / CPR;
        uint8_t* P0 = (uint8_t*)u.a + (uint64_t)b * H * RB;
        uint8_t* P1 = (uint8_t*)u.b + (uint64_t)b * Hk * RB;
        const WBuf w0 = wbuf(P0, H * RB), w1 = wbuf(P1, Hk * RB);  // rows past Hk: dropped
        const RBuf r0 = rbuf(P0, H * RB), r1 = rbuf(P1, Hk * RB);
        const uint32_t off = ((h0 + sub) * CPR + cc) * 16u;
        const u32x4 v0 = rld16(r0, off), v1 = rld16(r1, off);
        double cs[VE / 2], sn[VE / 2];
#pragma unroll
        for (uint32_t j = 0; j < VE / 2; ++j)
            rmath::sincos_d(rmath::rope_angle(pos, l2t, cc * (VE / 2) + j, D), &sn[j], &cs[j]);
#pragma unroll
        for (uint32_t t = 0; t < 2; ++t) {
            float x[VE];
            unpack<DT>(t == 0 ? v0 : v1, x);
            u32x4 o;
            if constexpr (DT == GPUOS_F32) {
                float y[VE];
#pragma unroll
                for (uint32_t j = 0; j < VE / 2; ++j) {
                    const double x0 = x[2 * j], x1 = x[2 * j + 1];
                    y[2 * j] = (float)(x0 * cs[j] - x1 * sn[j]);
                    y[2 * j + 1] = (float)(x0 * sn[j] + x1 * cs[j]);
                }
                o = pack<GPUOS_F32>(y);
            } else {
                uint32_t hb[VE];
#pragma unroll
                for (uint32_t j = 0; j < VE / 2; ++j) {
                    const double x0 = x[2 * j], x1 = x[2 * j + 1];
                    hb[2 * j] = d2bf(x0 * cs[j] - x1 * sn[j]);
                    hb[2 * j + 1] = d2bf(x0 * sn[j] + x1 * cs[j]);
                }
                o.x = hb[0] | (hb[1] << 16); o.y = hb[2] | (hb[3] << 16);
                o.z = hb[4] | (hb[5] << 16); o.w = hb[6] | (hb[7] << 16);
            }
            if (t == 0) wst16(w0, off, o);
            else wst16(w1, off, o);
        }
        return;
    }
    // general path: one pair per lane per step, heads [h0, h0 + hn)
    for (uint32_t pi = lane; pi < D / 2; pi += 64u) {
        double s, c;
        rmath::sincos_d(rmath::rope_angle(pos, l2t, pi, D), &s, &c);
        const uint32_t i0 = half ? pi : 2u * pi, i1 = half ? pi + D / 2 : 2u * pi + 1u;
        for (uint32_t t = 0; t < 2; ++t) {
            uint8_t* P = (uint8_t*)(t == 0 ? u.a : u.b);
            const uint32_t Ht = t == 0 ? H : Hk;
            for (uint32_t hh = h0; hh < h0 + hn && hh < Ht; ++hh) {
                const uint64_t base = ((uint64_t)b * Ht + hh) * D;
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
// Paged caches: row pos = L_b - 1 of batch row b lives on page
// table[b][pos / PS] at row pos % PS; that page holds [H, PS, D], so the
// destinations of all heads lie in one window of H * PS rows.  A page
// number outside the pool writes nothing.
__device__ __forceinline__ void kv_tile_paged(const Unit& u, uint32_t b, uint32_t lane) {
    const uint32_t H = u.dim[0], D = u.dim[1], PS = u.dim[2];
    const uint32_t MP = __float_as_uint(u.pf[5]);
    const uint32_t ES = esz(dt_in(u.flags));
    const uint32_t pos = lens_at(u.lensw, b) - 1u;
    const uint32_t pg = ld4((const uint8_t*)u.aux2 + ((uint64_t)b * MP + pos / PS) * 4u);
    if ((uint64_t)pg >= kv_pages(u.size)) return;
    const uint64_t RB = (uint64_t)D * ES;
    const uint64_t page_bytes = (uint64_t)H * PS * RB;
    const uint64_t rowoff = (uint64_t)(pos % PS) * RB;
    for (uint32_t t = 0; t < 2; ++t) {
        const uint8_t* src = (const uint8_t*)(t == 0 ? u.a : u.b) + (uint64_t)b * H * RB;
        uint8_t* dst = (uint8_t*)(t == 0 ? u.aux0 : u.aux1) + (uint64_t)pg * page_bytes + rowoff;
        if (RB % 16u == 0 && (((uint64_t)src | (uint64_t)dst) & 15ull) == 0 && page_bytes < (1ull << 31)) {
            const uint32_t cpr = (uint32_t)(RB / 16u), total = cpr * H;
            const RBuf rs = rbuf(src, total * 16u);
            const WBuf wd = wbuf(dst, (uint32_t)(page_bytes - rowoff));
            for (uint32_t j = lane; j < total; j += 64u) {
                const uint32_t hh = j / cpr;
                wst16(wd, (uint32_t)((uint64_t)hh * PS * RB) + (j % cpr) * 16u, rld16(rs, j * 16u));
            }
        } else {
            for (uint64_t j = lane; j < RB * H / 2u; j += 64u) {  // 2-byte words
                const uint64_t byte = j * 2u, hh = byte / RB, off = byte % RB;
                wst16b(dst + hh * PS * RB + off, (uint16_t)ld2(src + hh * RB + off));
            }
        }
    }
}

// Unit = one batch row b: K[b, h, L_b-1, :] = k[b, h, :] and the same for V.
// Fast path: rows a multiple of 16 bytes, aligned, and the strided window of
// destination rows below 2 GiB; 8 chunks per lane of each tensor are loaded
// before any store.
__device__ __forceinline__ void kv_tile(const Unit& u, uint32_t lane) {
    constexpr uint32_t NI = 8;
    const uint32_t b = u.tile;
    if (kv_paged(u.flags)) {
        kv_tile_paged(u, b, lane);
        return;
    }
    const uint32_t H = u.dim[0], D = u.dim[1], C = u.dim[2];
    const uint32_t ES = esz(dt_in(u.flags));
    const uint64_t pos = (uint64_t)lens_at(u.lensw, b) - 1;
    const uint64_t RB = (uint64_t)D * ES;
    const uint64_t span = ((uint64_t)H - 1) * C * RB + RB;
    const bool fast = (RB % 16u) == 0 && ((u.a | u.b | u.aux0 | u.aux1) & 15ull) == 0 && span < (1ull << 31) &&
                      (uint64_t)H * RB < (1ull << 31);
    if (fast) {
        const uint32_t cpr = (uint32_t)(RB / 16u), total = cpr * H;
        const uint8_t* s0 = (const uint8_t*)u.a + (uint64_t)b * H * RB;
        const uint8_t* s1 = (const uint8_t*)u.b + (uint64_t)b * H * RB;
        const uint64_t dbase = ((uint64_t)b * H * C + pos) * RB;
        const RBuf r0 = rbuf(s0, total * 16u), r1 = rbuf(s1, total * 16u);
        const WBuf w0 = wbuf((const uint8_t*)u.aux0 + dbase, (uint32_t)span);
        const WBuf w1 = wbuf((const uint8_t*)u.aux1 + dbase, (uint32_t)span);
        for (uint32_t j0 = 0; j0 < total; j0 += NI * 64u) {
            u32x4 v0[NI], v1[NI];
#pragma unroll
            for (uint32_t i = 0; i < NI; ++i) {
                const uint32_t j = j0 + i * 64u + lane;
                v0[i] = rld16(r0, j * 16u);
                v1[i] = rld16(r1, j * 16u);
            }
#pragma unroll
            for (uint32_t i = 0; i < NI; ++i) {
                const uint32_t j = j0 + i * 64u + lane;
                if (j < total) {
                    const uint32_t hh = j / cpr, off = (uint32_t)((uint64_t)hh * C * RB) + (j % cpr) * 16u;
                    wst16(w0, off, v0[i]);
                    wst16(w1, off, v1[i]);
                }
            }
        }
        return;
    }
    for (uint32_t t = 0; t < 2; ++t) {
        const uint8_t* src = (const uint8_t*)(t == 0 ? u.a : u.b) + (uint64_t)b * H * RB;
        uint8_t* dst = (uint8_t*)(t == 0 ? u.aux0 : u.aux1);
        const uint64_t total = RB * H / 2u;  // 2-byte words (ES is 2 or 4)
        for (uint64_t j = lane; j < total; j += 64u) {
            const uint64_t byte = j * 2u, hh = byte / RB, off = byte % RB;
            wst16b(dst + (((uint64_t)b * H + hh) * C + pos) * RB + off, (uint16_t)ld2(src + hh * RB + off));
        }
    }
}

// ------------------------------------------------------------ decode SDPA
// Unit = (b, h, split of kt = sdpa_keys_per_unit keys: 1024, halved down to 64
// while the op would give fewer than 256 units).  One key row of D bf16 is DV = D/8
// lanes x 16 bytes, so one load instruction covers RPI = 64/DV keys and the
// wave reads keys in chunks of 8 instructions (8 RPI keys, 16 KiB of K and V
// for D = 128).  The next chunk's loads are issued before the current chunk
// is used, so two chunks are in flight.  Scores are bf16 dot products (exact
// products, fp32 sums) reduced inside each DV-lane group with DPP, kept in
// the log2 domain (scale * log2 e folded in), with a running max (online
// softmax); each unit produces (max, sum of 2^(s - max), unnormalised P.V)
// for its keys, and when a head has several splits the last unit to finish
// merges them (the split softmax of flash-decoding).  Keys past L read as
// zero through the bounded buffer window and get weight 0.  Dense MFMA does
// not apply: one query per head makes q.K^T and P.V matrix-vector products
// with no reuse.  Attention masking: with GPUOS_F_SDPA_MASK an fp32 mask
// [B, C] (aux2, per batch row and key, the same for every head) is added to
// the scaled scores; the chunk's mask values are loaded with its keys.  A
// key with mask -inf gets weight 0; a chunk or split whose keys are all
// masked adds nothing (its running max stays -inf and is not subtracted
// from itself), and a row with every key masked gives NaN, as softmax over
// nothing does.
template <uint32_t DTO, uint32_t D>
__device__ __forceinline__ void sdpa_merge_splits(const Unit& u, uint32_t lane, uint32_t b, uint32_t h0, uint32_t gp,
                                                  uint32_t ns, uint32_t mbase);

template <uint32_t DV, uint32_t DTO, uint32_t GP>
__device__ __forceinline__ void sdpa_tile(const Unit& u, uint32_t lane) {
    constexpr uint32_t D = DV * 8u;
    constexpr uint32_t RPI = 64u / DV;
    constexpr uint32_t NI = 8u;  // load instructions per chunk
    constexpr uint32_t CK = NI * RPI;     // keys per chunk
    constexpr uint32_t PSTRIDE = D + 4u;  // floats per partial record: m, l, pad, pad, acc[D]
    const bool paged = kv_paged(u.flags);
    const uint32_t H = u.dim[0], PS = u.dim[2];
    const uint32_t MP = __float_as_uint(u.pf[5]);  // paged: table row length
    const uint32_t C = paged ? MP * PS : u.dim[2];  // positions per batch row
    const uint32_t Hkv = u.dim[3] ? u.dim[3] : H;
    const uint32_t Bn = (uint32_t)u.size;
    const uint32_t kt = sdpa_keys_per_unit(Bn, H, u.lensw);
    const uint32_t HG = H / GP;  // units per (b, split): groups of GP query heads
    // unit -> (b, head group, split); mbase numbers the per-head splits of
    // earlier batch rows (the partial records and counters are per head)
    uint32_t t = u.tile, base = 0, mbase = 0, b = 0, ns = 1, L = 0;
    for (b = 0; b < Bn; ++b) {
        L = lens_at(u.lensw, b);
        ns = (L + kt - 1) / kt;
        const uint32_t nu = HG * ns;
        if (t < base + nu) break;
        base += nu;
        mbase += H * ns;
    }
    if (b >= Bn) return;
    const uint32_t local = t - base, hg = local / ns, sp = local % ns;
    const uint32_t h0 = hg * GP;  // the unit's first query head; all GP share a key/value head
    const uint64_t bkv = (uint64_t)b * Hkv + h0 / (H / Hkv);
    const uint32_t k0 = sp * kt;
    const uint32_t nk = min(L - k0, kt);
    const float scale = u.pf[4] != 0.0f ? u.pf[4] : (u.p0 != 0.0f ? u.p0 : 1.0f / sqrtf((float)D));
    const float sl2 = scale * 1.4426950408889634f;  // scores in the log2 domain
    const uint32_t g = lane / DV, c = lane % DV;
    // the unit's keys: a stretch of one (b, key/value head) row; or, with
    // paged caches, of up to kt / PS pages, whose numbers lane i holds (page
    // k0 / PS + i of the row) and each chunk of keys (one page holds a
    // whole number of chunks) reads through its page's window
    const RBuf rk = rbuf((const uint8_t*)u.aux0 + (bkv * C + k0) * D * 2u, paged ? 0u : nk * D * 2u);
    const RBuf rv = rbuf((const uint8_t*)u.aux1 + (bkv * C + k0) * D * 2u, paged ? 0u : nk * D * 2u);
    const uint64_t hkv = bkv - (uint64_t)b * Hkv, NP = kv_pages(u.size);
    uint32_t ptab = 0;
    if (paged && lane < (nk + PS - 1) / PS) ptab = ld4((const uint8_t*)u.b + ((uint64_t)b * MP + k0 / PS + lane) * 4u);
    const bool masked = (u.flags & GPUOS_F_SDPA_MASK) != 0u;
    const RBuf rm = rbuf((const uint8_t*)u.aux2 + ((uint64_t)b * C + k0) * 4u, masked ? nk * 4u : 0u);
    bf16x2 qv[GP][4];
#pragma unroll
    for (uint32_t gi = 0; gi < GP; ++gi) {
        const uint64_t bh = (uint64_t)b * H + h0 + gi;
        const u32x4 qr = rld16(rbuf((const uint8_t*)u.a + bh * D * 2u, D * 2u), c * 16u);
        qv[gi][0] = as_bf2(qr.x); qv[gi][1] = as_bf2(qr.y); qv[gi][2] = as_bf2(qr.z); qv[gi][3] = as_bf2(qr.w);
    }
    float m[GP], lsum[GP], acc[GP][8];
#pragma unroll
    for (uint32_t gi = 0; gi < GP; ++gi) {
        m[gi] = -INFINITY;
        lsum[gi] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[gi][e] = 0.0f;
    }
    const uint32_t nch = (nk + CK - 1) / CK;
    // returns false for a chunk on a page outside the pool (its keys drop out)
    auto load = [&](u32x4* kv, u32x4* vv, float* mk, uint32_t ci) -> bool {
        RBuf ck = rk, cv = rv;
        uint32_t cbase = ci * CK * D * 2u;
        bool live = true;
        if (paged) {
            const uint32_t key0 = k0 + ci * CK;  // chunks past the unit read nothing
            const uint32_t pg = (uint32_t)__builtin_amdgcn_readlane((int)ptab, (int)((key0 / PS - k0 / PS) & 63u));
            live = pg < NP;
            const uint32_t keys = ci < nch && live ? min(CK, nk - ci * CK) : 0u;
            const uint64_t at = (((uint64_t)pg * Hkv + hkv) * PS + key0 % PS) * D * 2u;
            ck = rbuf((const uint8_t*)u.aux0 + at, keys * D * 2u);
            cv = rbuf((const uint8_t*)u.aux1 + at, keys * D * 2u);
            cbase = 0;
        }
#pragma unroll
        for (uint32_t j = 0; j < NI; ++j) {
            const uint32_t off = cbase + ((j * RPI + g) * D) * 2u + c * 16u;
            kv[j] = rld16s(ck, off);
            vv[j] = rld16s(cv, off);
        }
        if (masked) {
#pragma unroll
            for (uint32_t j = 0; j < NI; ++j) mk[j] = __uint_as_float(rld4(rm, (ci * CK + j * RPI + g) * 4u));
        }
        return live;
    };
    auto consume = [&](const u32x4* kv, const u32x4* vv, const float* mk, uint32_t ci, bool live) {
        float s[GP][NI];
        float mn[GP];
#pragma unroll
        for (uint32_t gi = 0; gi < GP; ++gi) {
            float cm = -INFINITY;
#pragma unroll
            for (uint32_t j = 0; j < NI; ++j) {
                float d = 0.0f;
                d = __builtin_amdgcn_fdot2_f32_bf16(qv[gi][0], as_bf2(kv[j].x), d, false);
                d = __builtin_amdgcn_fdot2_f32_bf16(qv[gi][1], as_bf2(kv[j].y), d, false);
                d = __builtin_amdgcn_fdot2_f32_bf16(qv[gi][2], as_bf2(kv[j].z), d, false);
                d = __builtin_amdgcn_fdot2_f32_bf16(qv[gi][3], as_bf2(kv[j].w), d, false);
                d = gred<DV>(d, OpAdd{}) * sl2;
                if (masked) d += mk[j] * 1.4426950408889634f;  // the mask, in the log2 domain too
                const bool valid = live && ci * CK + j * RPI + g < nk;
                s[gi][j] = valid ? d : -INFINITY;
                cm = fmaxf(cm, s[gi][j]);
            }
            // chunk max over the RPI key groups of the wave
            if constexpr (DV == 16) {
                cm = fmaxf(fmaxf(rlf(cm, 0), rlf(cm, 16)), fmaxf(rlf(cm, 32), rlf(cm, 48)));
            } else {
#pragma unroll
                for (uint32_t mm = DV; mm < 64; mm <<= 1) cm = fmaxf(cm, __shfl_xor(cm, mm, 64));
            }
            mn[gi] = fmaxf(m[gi], cm);  // -inf only while every key so far is masked
            // 0 on the first chunk with a live key (m = -inf); 1 while nothing is live
            const float alpha = mn[gi] == -INFINITY ? 1.0f : exp2f(m[gi] - mn[gi]);
            lsum[gi] *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[gi][e] *= alpha;
            m[gi] = mn[gi];
        }
#pragma unroll
        for (uint32_t j = 0; j < NI; ++j) {
            float vf[8];
            unpack<GPUOS_BF16>(vv[j], vf);
#pragma unroll
            for (uint32_t gi = 0; gi < GP; ++gi) {
                const float p = s[gi][j] == -INFINITY ? 0.0f : exp2f(s[gi][j] - mn[gi]);  // 0 past L, or masked
                lsum[gi] += p;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[gi][e] += p * vf[e];
            }
        }
    };
    // The scheduling barriers keep the compiler from sinking the next chunk's
    // loads below the use of the current one (it would to save registers).
    u32x4 ka[NI], va[NI], kb[NI], vb[NI];
    float ma[NI], mb[NI];
    bool la = load(ka, va, ma, 0), lb = true;
    for (uint32_t ci = 0; ci < nch; ci += 2) {
        lb = load(kb, vb, mb, ci + 1);  // past the last chunk: outside the window, reads nothing
        __builtin_amdgcn_sched_barrier(0);
        consume(ka, va, ma, ci, la);
        if (ci + 1 < nch) {
            la = load(ka, va, ma, ci + 2);
            __builtin_amdgcn_sched_barrier(0);
            consume(kb, vb, mb, ci + 1, lb);
        }
    }
    constexpr uint32_t ESO = DTO == GPUOS_F32 ? 4u : 2u;
    float* parts = (float*)(u.scratch + COUNTER_AREA);
    // per head: combine the RPI key groups (lanes with equal c), then store
    // the output (one split) or this split's partial record
#pragma unroll
    for (uint32_t gi = 0; gi < GP; ++gi) {
#pragma unroll
        for (uint32_t mm = DV; mm < 64; mm <<= 1) {
            lsum[gi] += __shfl_xor(lsum[gi], mm, 64);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[gi][e] += __shfl_xor(acc[gi][e], mm, 64);
        }
        const uint64_t bh = (uint64_t)b * H + h0 + gi;
        if (ns == 1) {
            if (g == 0) {
                uint8_t* O = (uint8_t*)u.out + bh * D * ESO;
                float o[8];
                const float inv = 1.0f / lsum[gi];
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = acc[gi][e] * inv;
                const WBuf ob = wbuf(O);
                if constexpr (DTO == GPUOS_F32) {
                    wst16(ob, c * 32u, pack<GPUOS_F32>(o));
                    wst16(ob, c * 32u + 16u, pack<GPUOS_F32>(o + 4));
                } else {
                    wst16(ob, c * 16u, pack<GPUOS_BF16>(o));
                }
            }
        } else {
            float* part = parts + ((uint64_t)mbase + (uint64_t)(h0 + gi) * ns + sp) * PSTRIDE;
            if (g == 0) {
                const WBuf pb = wbuf(part);
                wst16(pb, (4u + 8u * c) * 4u, pack<GPUOS_F32>(acc[gi]));
                wst16(pb, (8u + 8u * c) * 4u, pack<GPUOS_F32>(acc[gi] + 4));
            }
            if (lane == 0) { wstf(part, m[gi]); wstf(part + 1, lsum[gi]); }
        }
    }
    if (ns == 1) return;
    sdpa_merge_splits<DTO, D>(u, lane, b, h0, GP, ns, mbase);
}

// The split softmax of flash-decoding: each of the `gp` heads from h0 on
// counts this split (its partial record already stored); the last split of
// a head to arrive merges the head's ns records into the output.
template <uint32_t DTO, uint32_t D>
__device__ __forceinline__ void sdpa_merge_splits(const Unit& u, uint32_t lane, uint32_t b, uint32_t h0, uint32_t gp,
                                                  uint32_t ns, uint32_t mbase) {
    constexpr uint32_t PSTRIDE = D + 4u;
    constexpr uint32_t ESO = DTO == GPUOS_F32 ? 4u : 2u;
    const uint32_t H = u.dim[0];
    float* parts = (float*)(u.scratch + COUNTER_AREA);
    stores_done();  // the partials are published before they are counted
    // per head: count this split; the last arriver merges the head's splits
#pragma unroll 1
    for (uint32_t gi = 0; gi < gp; ++gi) {
        const uint32_t head = h0 + gi;
        const uint64_t bh = (uint64_t)b * H + head;
        uint32_t* ctr = (uint32_t*)u.scratch + bh;
        uint32_t prev = 0;
        if (lane == 0) prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        prev = (uint32_t)__builtin_amdgcn_readlane((int)prev, 0);
        if (prev != ns - 1) continue;
        uint8_t* O = (uint8_t*)u.out + bh * D * ESO;
        // merge (log2 domain): M = max m_i, Ls = sum l_i 2^{m_i - M}, o = sum acc_i 2^{m_i - M} / Ls.
        // Lane i < ns reads split i's (m, l).  A record's acc is CH = D/4
        // chunks of 16 bytes, so one load instruction covers SPI = 64/CH
        // splits: lane l reads chunk l % CH of split l / CH (+ SPI per
        // instruction), up to 16 instructions in flight; each lane adds its
        // splits in order, then the SPI lane groups are added in a fixed tree.
        const uint8_t* p0 = (const uint8_t*)(parts + ((uint64_t)mbase + (uint64_t)head * ns) * PSTRIDE);
        constexpr uint32_t CH = D / 4u;
        constexpr uint32_t SPI = 64u / CH;
        constexpr uint32_t NB = 16;  // load instructions per batch
        float mi = -INFINITY, li = 0.0f;
        if (lane < ns) {
            mi = __uint_as_float(ld4(p0 + (uint64_t)lane * PSTRIDE * 4u));
            li = __uint_as_float(ld4(p0 + (uint64_t)lane * PSTRIDE * 4u + 4u));
        }
        const float M = wmaxf(mi);
        const float wi = lane < ns ? exp2f(mi - M) : 0.0f;
        const float Ls = wsum(li * wi);
        const uint32_t jj = lane / CH, cc = lane % CH;
        const RBuf rp = rbuf(p0, ns * PSTRIDE * 4u);  // splits past ns read zero
        float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (uint32_t i0 = 0; i0 < ns; i0 += NB * SPI) {
            u32x4 v[NB];
#pragma unroll
            for (uint32_t k = 0; k < NB; ++k)
                if (i0 + k * SPI < ns) v[k] = rld16(rp, ((i0 + k * SPI + jj) * PSTRIDE + 4u + 4u * cc) * 4u);
#pragma unroll
            for (uint32_t k = 0; k < NB; ++k) {
                if (i0 + k * SPI < ns) {
                    const float w = __shfl(wi, (int)((i0 + k * SPI + jj) & 63u), 64);  // 0 past ns
                    o[0] += w * __uint_as_float(v[k].x);
                    o[1] += w * __uint_as_float(v[k].y);
                    o[2] += w * __uint_as_float(v[k].z);
                    o[3] += w * __uint_as_float(v[k].w);
                }
            }
        }
#pragma unroll
        for (uint32_t mm = CH; mm < 64; mm <<= 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] += __shfl_xor(o[e], (int)mm, 64);
        }
        if (lane < CH) {
            const float inv = 1.0f / Ls;
#pragma unroll
            for (uint32_t e = 0; e < 4; ++e) st_elem<DTO>(O, 4u * cc + e, o[e] * inv);
        }
        if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// LDS for the value chunk of sdpa_gqa_tile: one 32-key chunk per wave of a
// workgroup of up to four waves (one array for every instantiation)
constexpr uint32_t SDPA_VCHUNK_BYTES = 32u * 288u;
__shared__ uint64_t sdpa_vlds[4u * SDPA_VCHUNK_BYTES / 8u];

// --------------------------------------- decode SDPA, grouped heads (MFMA)
// GP = 4 query heads that share one key/value head (D = 128), on the matrix
// cores.  With four queries per key row the vector-ALU form does four dot
// products and four weighted sums per 512 bytes of K and V, which bounds it
// well below the memory system; here both contractions run as
// v_mfma_f32_16x16x32_bf16, the four heads taking 4 of the 16 rows.
// The unit (b, head group, split of kt keys) and its split records are those
// of sdpa_tile; keys come in chunks of CK = 32, the next chunk's loads
// issued before the current chunk is used.
//  - Scores: S^T[key, h] = K Q^T per 16-key block, K as the A operand (lane
//    l: key row l % 16, dims 8 (l / 16) + 32 s) and Q^T as B (lane l: head
//    l % 16, the same dims; rows past GP read zero).  K comes in as V does,
//    whole rows per load instruction, and goes through the wave's LDS area
//    into that layout: loaded in the operand layout directly, each
//    instruction took half of sixteen 128-byte lines, and the grouped decode
//    stream ran about 11% slower.  Lane (h = l % 16, q = l / 16) then holds
//    head h's scores of keys 4q + i and 16 + 4q + i (i < 4): its head's
//    softmax needs only the exchange over q.
//  - P.V: O[h, d] += P[h, key] V[key, d] per 16-column tile of d.  A matrix
//    product may number its contraction index in any order that both
//    operands share: key slot 8q + j of P is the j-th score lane (h, q)
//    holds, so P is used where it was computed.  V comes in with coalesced
//    loads (16 bytes of one key row per lane) and is written to LDS as rows;
//    the LDS transpose read (ds_read_b64_tr_b16) then gives each lane four
//    keys at one d: in each 16-lane group, lane i receives element i % 4 of
//    the 8 bytes that lanes 4e + i / 4 (e < 4) point at, so lane p of group
//    q points at row key(slot 8q + e), columns d0 + 4 (p % 4) .. +4, two
//    reads per tile.  Rows are 288 bytes apart, which spreads the 16 rows of
//    a read over the banks evenly.
//  - P has 24 significant bits; it goes in as a bf16 high part and a bf16
//    low part (two MFMAs), so the weights keep 16 bits, as the fp32 FMAs of
//    the vector form keep more than the 2e-3 bar needs.  Products of bf16
//    are exact in the fp32 accumulators.
//  - O accumulates in the C tiles (lane l < 16 holds heads 0..3 of column
//    l).  A head's reference max moves only when a chunk's max exceeds it by
//    more than 8 (log2 domain), so weights stay below 2^8 and the rescaling
//    of its accumulator rows (and sum) is rare after the first chunk; the
//    result is the same softmax, and partial records carry the reference
//    max they were computed with.
// Masking, paged caches and keys past L are handled as in sdpa_tile.
template <uint32_t DTO>
__device__ __forceinline__ void sdpa_gqa_tile(const Unit& u, uint32_t lane) {
    constexpr uint32_t D = 128u, GP = 4u, CK = 32u;
    constexpr uint32_t PSTRIDE = D + 4u;
    constexpr uint32_t VRS = 288u;  // bytes per key row of the LDS value chunk
    constexpr uint32_t KRS = 272u;  // ... of the key chunk, staged in the same place first
    constexpr uint32_t ESO = DTO == GPUOS_F32 ? 4u : 2u;
    static_assert(CK * VRS == SDPA_VCHUNK_BYTES && CK * KRS <= SDPA_VCHUNK_BYTES, "chunk sizes");
    __attribute__((address_space(3))) uint8_t* vl =
        (__attribute__((address_space(3))) uint8_t*)sdpa_vlds + (threadIdx.x >> 6) * SDPA_VCHUNK_BYTES;
    const bool paged = kv_paged(u.flags);
    const uint32_t H = u.dim[0], PS = u.dim[2];
    const uint32_t MP = __float_as_uint(u.pf[5]);
    const uint32_t C = paged ? MP * PS : u.dim[2];
    const uint32_t Hkv = u.dim[3] ? u.dim[3] : H;
    const uint32_t Bn = (uint32_t)u.size;
    const uint32_t kt = sdpa_keys_per_unit(Bn, H, u.lensw);
    const uint32_t HG = H / GP;
    uint32_t t = u.tile, base = 0, mbase = 0, b = 0, ns = 1, L = 0;
    for (b = 0; b < Bn; ++b) {
        L = lens_at(u.lensw, b);
        ns = (L + kt - 1) / kt;
        const uint32_t nu = HG * ns;
        if (t < base + nu) break;
        base += nu;
        mbase += H * ns;
    }
    if (b >= Bn) return;
    const uint32_t local = t - base, hg = local / ns, sp = local % ns;
    const uint32_t h0 = hg * GP;
    const uint64_t bkv = (uint64_t)b * Hkv + h0 / (H / Hkv);
    const uint32_t k0 = sp * kt;
    const uint32_t nk = min(L - k0, kt);
    const float scale = u.pf[4] != 0.0f ? u.pf[4] : (u.p0 != 0.0f ? u.p0 : 1.0f / sqrtf((float)D));
    const float sl2 = scale * 1.4426950408889634f;
    const uint32_t r16 = lane % 16u, q = lane / 16u;
    const RBuf rk = rbuf((const uint8_t*)u.aux0 + (bkv * C + k0) * D * 2u, paged ? 0u : nk * D * 2u);
    const RBuf rv = rbuf((const uint8_t*)u.aux1 + (bkv * C + k0) * D * 2u, paged ? 0u : nk * D * 2u);
    const uint64_t hkv = bkv - (uint64_t)b * Hkv, NP = kv_pages(u.size);
    uint32_t ptab = 0;
    if (paged && lane < (nk + PS - 1) / PS) ptab = ld4((const uint8_t*)u.b + ((uint64_t)b * MP + k0 / PS + lane) * 4u);
    const bool masked = (u.flags & GPUOS_F_SDPA_MASK) != 0u;
    const RBuf rm = rbuf((const uint8_t*)u.aux2 + ((uint64_t)b * C + k0) * 4u, masked ? nk * 4u : 0u);
    // Q^T (B operand of the scores): rows past the GP heads fall outside the window
    const RBuf rq = rbuf((const uint8_t*)u.a + ((uint64_t)b * H + h0) * D * 2u, GP * D * 2u);
    u32x4 qb[4];
#pragma unroll
    for (uint32_t s = 0; s < 4; ++s) qb[s] = rld16(rq, (r16 * D + 8u * q + 32u * s) * 2u);
    float m = -INFINITY, lsum = 0.0f;
    f32x4 oacc[8];
#pragma unroll
    for (uint32_t i = 0; i < 8; ++i) oacc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t nch = (nk + CK - 1) / CK;
    // K in the operand layout (block kb of 16 keys, dims step s), V as rows
    // (instruction j: key row 4j + q, bytes 16 (l % 16)), the mask of keys
    // 16 kb + 4q .. +3; false for a chunk on a page outside the pool
    auto load = [&](u32x4* kv, u32x4* vv, u32x4* mk, uint32_t ci) -> bool {
        RBuf ck = rk, cv = rv;
        uint32_t cbase = ci * CK * D * 2u;
        bool live = true;
        if (paged) {
            const uint32_t key0 = k0 + ci * CK;
            const uint32_t pg = (uint32_t)__builtin_amdgcn_readlane((int)ptab, (int)((key0 / PS - k0 / PS) & 63u));
            live = pg < NP;
            const uint32_t keys = ci < nch && live ? min(CK, nk - ci * CK) : 0u;
            const uint64_t at = (((uint64_t)pg * Hkv + hkv) * PS + key0 % PS) * D * 2u;
            ck = rbuf((const uint8_t*)u.aux0 + at, keys * D * 2u);
            cv = rbuf((const uint8_t*)u.aux1 + at, keys * D * 2u);
            cbase = 0;
        }
#pragma unroll
        for (uint32_t j = 0; j < 8; ++j) {
            kv[j] = rld16s(ck, cbase + (j * 4u + q) * D * 2u + r16 * 16u);
            vv[j] = rld16s(cv, cbase + (j * 4u + q) * D * 2u + r16 * 16u);
        }
        if (masked) {
#pragma unroll
            for (uint32_t kb = 0; kb < 2; ++kb) mk[kb] = rld16(rm, (ci * CK + kb * 16u + 4u * q) * 4u);
        }
        return live;
    };
    auto consume = [&](const u32x4* kv, const u32x4* vv, const u32x4* mk, uint32_t ci, bool live) {
        // K rows into LDS, then back in the operand layout (row kb 16 + l % 16,
        // dims 8 (l / 16) + 32 s); rows KRS bytes apart put the 8 lanes of
        // each quarter-wave of a read on distinct banks
#pragma unroll
        for (uint32_t j = 0; j < 8; ++j)
            *(__attribute__((address_space(3))) u32x4*)(vl + (j * 4u + q) * KRS + r16 * 16u) = kv[j];
        u32x4 ko[8];
#pragma unroll
        for (uint32_t kb = 0; kb < 2; ++kb)
#pragma unroll
            for (uint32_t s = 0; s < 4; ++s)
                ko[kb * 4u + s] = *(const __attribute__((address_space(3))) u32x4*)(
                    vl + (kb * 16u + r16) * KRS + (8u * q + 32u * s) * 2u);
        f32x4 st[2];
#pragma unroll
        for (uint32_t kb = 0; kb < 2; ++kb) {
            st[kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (uint32_t s = 0; s < 4; ++s)
                st[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ko[kb * 4u + s]),
                                                                 __builtin_bit_cast(bf16x8, qb[s]), st[kb], 0, 0, 0);
        }
        // the value rows go to LDS while the scores are finished
#pragma unroll
        for (uint32_t j = 0; j < 8; ++j) {
            __attribute__((address_space(3))) uint64_t* w =
                (__attribute__((address_space(3))) uint64_t*)(vl + (j * 4u + q) * VRS + r16 * 16u);
            w[0] = (uint64_t)vv[j].x | ((uint64_t)vv[j].y << 32);
            w[1] = (uint64_t)vv[j].z | ((uint64_t)vv[j].w << 32);
        }
        float sv[8], cm = -INFINITY;
#pragma unroll
        for (uint32_t kb = 0; kb < 2; ++kb) {
            float mv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (masked) {
                mv[0] = __uint_as_float(mk[kb].x); mv[1] = __uint_as_float(mk[kb].y);
                mv[2] = __uint_as_float(mk[kb].z); mv[3] = __uint_as_float(mk[kb].w);
            }
#pragma unroll
            for (uint32_t i = 0; i < 4; ++i) {
                float x = st[kb][i] * sl2;
                if (masked) x += mv[i] * 1.4426950408889634f;  // the mask, in the log2 domain too
                const bool valid = live && ci * CK + kb * 16u + 4u * q + i < nk;
                sv[kb * 4u + i] = valid ? x : -INFINITY;
                cm = fmaxf(cm, sv[kb * 4u + i]);
            }
        }
        cm = fmaxf(cm, __shfl_xor(cm, 16, 64));  // this head's other key groups
        cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
        // the reference max moves to this chunk's max when that is more than
        // 8 above it (always from -inf: m + 8 is -inf); the old sum and
        // accumulators are scaled by alpha = 2^(m - cm), 0 from -inf
        const bool move = cm > m + 8.0f;
        const float alpha = move ? exp2f(m - cm) : 1.0f;
        if (move) m = cm;  // -inf only while every key so far is masked
        float p[8], ps = 0.0f;
#pragma unroll
        for (uint32_t j = 0; j < 8; ++j) {
            p[j] = sv[j] == -INFINITY ? 0.0f : exp2f(sv[j] - m);  // 0 past L, or masked; below 2^8
            ps += p[j];
        }
        lsum = lsum * alpha + ps;
        if (__ballot(move) != 0ull) {
            // row i of the accumulators (lanes 0..15) is head i
#pragma unroll
            for (uint32_t i = 0; i < 4; ++i) {
                const float a = rlf(alpha, (int)i);
#pragma unroll
                for (uint32_t tt = 0; tt < 8; ++tt) oacc[tt][i] *= a;
            }
        }
        u32x4 ph, pl;
        uint32_t* phw = (uint32_t*)&ph;
        uint32_t* plw = (uint32_t*)&pl;
#pragma unroll
        for (uint32_t e = 0; e < 4; ++e) {
            const uint32_t hi = f2bf2(p[2 * e], p[2 * e + 1]);
            phw[e] = hi;
            plw[e] = f2bf2(p[2 * e] - bf2f(hi & 0xFFFFu), p[2 * e + 1] - __uint_as_float(hi & 0xFFFF0000u));
        }
        // B operand of tile tt: slot 8q + j is key 16 (j / 4) + 4q + j % 4,
        // column 16 tt + l % 16; lane p of group q points at row 4q + p / 4
        // (then 16 + 4q + p / 4), columns 16 tt + 4 (p % 4) .. +4
        const uint32_t ra = (4u * q + r16 / 4u) * VRS + 8u * (r16 % 4u);
#pragma unroll
        for (uint32_t tt = 0; tt < 8; ++tt) {
            const v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vl + ra + 32u * tt));
            const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vl + ra + 16u * VRS + 32u * tt));
            const u32x4 vb = __builtin_shufflevector(__builtin_bit_cast(u32x2, x0), __builtin_bit_cast(u32x2, x1), 0, 1, 2, 3);
            oacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ph),
                                                               __builtin_bit_cast(bf16x8, vb), oacc[tt], 0, 0, 0);
            oacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pl),
                                                               __builtin_bit_cast(bf16x8, vb), oacc[tt], 0, 0, 0);
        }
    };
    u32x4 ka[8], va[8], kb2[8], vb2[8], ma[2], mb[2];
    bool la = load(ka, va, ma, 0), lb = true;
    for (uint32_t ci = 0; ci < nch; ci += 2) {
        lb = load(kb2, vb2, mb, ci + 1);  // past the last chunk: outside the window, reads nothing
        __builtin_amdgcn_sched_barrier(0);
        consume(ka, va, ma, ci, la);
        if (ci + 1 < nch) {
            la = load(ka, va, ma, ci + 2);
            __builtin_amdgcn_sched_barrier(0);
            consume(kb2, vb2, mb, ci + 1, lb);
        }
    }
    // each head's sum over its four key groups; lanes 0..3 then hold heads 0..3
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    float* parts = (float*)(u.scratch + COUNTER_AREA);
#pragma unroll
    for (uint32_t i = 0; i < GP; ++i) {
        const float li = rlf(lsum, (int)i), mi = rlf(m, (int)i);
        const uint64_t bh = (uint64_t)b * H + h0 + i;
        if (ns == 1) {
            if (q == 0) {
                uint8_t* O = (uint8_t*)u.out + bh * D * ESO;
                const float inv = 1.0f / li;
#pragma unroll
                for (uint32_t tt = 0; tt < 8; ++tt) st_elem<DTO>(O, 16u * tt + r16, oacc[tt][i] * inv);
            }
        } else {
            float* part = parts + ((uint64_t)mbase + (uint64_t)(h0 + i) * ns + sp) * PSTRIDE;
            if (q == 0) {
#pragma unroll
                for (uint32_t tt = 0; tt < 8; ++tt) wstf(part + 4u + 16u * tt + r16, oacc[tt][i]);
            }
            if (lane == 0) { wstf(part, mi); wstf(part + 1, li); }
        }
    }
    if (ns == 1) return;
    sdpa_merge_splits<DTO, D>(u, lane, b, h0, GP, ns, mbase);
}

// ------------------------------------------------------------------ GEMV
// y[1,N] = x[1,K] W[K,N], W row-major.  Unit = (column block, k-split):
// 16 lanes x 16 bytes cover CPB = 16 VE columns of one row, the four 16-lane
// rows of the wave take four rows of W per load instruction, and a unit
// walks GEMV_KC (128) rows in batches of 64 (16 instructions, 16 KiB of bf16 W),
// the next batch loaded before the current one is used.  x[k] comes from a
// per-batch load of 64 values (one per lane) moved to the using lanes with a
// lane permute.  The four row groups are summed at the end in a fixed
// order; with several k-splits each unit writes fp32 partial sums and the
// last unit of a column block adds them in split order.
template <uint32_t DT, uint32_t DTO>
__device__ __forceinline__ void gemv_tile(const Unit& u, uint32_t lane) {
    constexpr uint32_t ES = DT == GPUOS_F32 ? 4u : 2u;
    constexpr uint32_t VE = 16u / ES;
    constexpr uint32_t CPB = 16u * VE;
    constexpr uint32_t RB = 64u;  // rows per batch
    const uint32_t K = u.dim[0], N = u.dim[1];
    const uint32_t ncb = (N + CPB - 1) / CPB, nks = (K + GEMV_KC - 1) / GEMV_KC;
    const uint32_t cb = u.tile % ncb, ks = u.tile / ncb;
    const uint32_t kb = ks * GEMV_KC, kn = min(K - kb, GEMV_KC);
    const uint8_t* X = (const uint8_t*)u.a;
    const uint8_t* Wm = (const uint8_t*)u.b;
    const uint32_t g = lane / 16u, cl = lane % 16u;
    const uint32_t c0 = cb * CPB + cl * VE;  // first column of this lane
    float acc[VE];
#pragma unroll
    for (uint32_t e = 0; e < VE; ++e) acc[e] = 0.0f;
    const uint64_t rowb = (uint64_t)N * ES;
    const bool vec = (N % VE) == 0 && ((uint64_t)Wm & 15ull) == 0 && (uint64_t)kn * rowb < (1ull << 31);
    if (vec) {
        // window: rows kb .. kb+kn-1 of the column block; columns past N in the
        // last block read neighbouring valid memory (never stored) or zero
        const uint8_t* wbase = Wm + (uint64_t)kb * rowb + (uint64_t)cb * CPB * ES;
        const uint32_t wlen = (uint32_t)((uint64_t)(kn - 1) * rowb + (uint64_t)(N - cb * CPB) * ES);
        const RBuf rw = rbuf(wbase, wlen);
        const RBuf rx = rbuf(X + (uint64_t)kb * ES, kn * ES);
        const uint32_t nb = (kn + RB - 1) / RB;
        auto loadw = [&](u32x4* w, uint32_t bi) {
#pragma unroll
            for (uint32_t i = 0; i < 16; ++i) {
                const uint32_t r = bi * RB + i * 4u + g;
                // rows past kn fall outside the window (zero)
                w[i] = rld16s(rw, r < kn ? r * (uint32_t)rowb + cl * 16u : 0xFFFFFFF0u);
            }
        };
        auto loadx = [&](uint32_t bi) -> float {
            const uint32_t r = bi * RB + lane;
            if constexpr (DT == GPUOS_F32) {
                return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rx.r, (int)(r * 4u), 0, CPOL_SC1));
            } else {
                return bf2f(__builtin_amdgcn_raw_buffer_load_b16(rx.r, (int)(r * 2u), 0, CPOL_SC1));
            }
        };
        auto consume = [&](const u32x4* w, float xv) {
            if constexpr (DT == GPUOS_BF16 && GEMV_DOT2) {
                // rows r and r + 4 (loads i and i + 1) paired for the bf16
                // dot instruction: per column, a permute packs the two
                // weights and one dot adds both products to the column's sum
#pragma unroll
                for (uint32_t i = 0; i < 16; i += 2) {
                    const float x1 = __shfl(xv, (int)(i * 4u + g), 64);
                    const float x2 = __shfl(xv, (int)((i + 1u) * 4u + g), 64);
                    const bf16x2 xb = as_bf2(f2bf2(x1, x2));  // exact: both are bf16 values
                    const uint32_t a[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
                    const uint32_t b[4] = {w[i + 1].x, w[i + 1].y, w[i + 1].z, w[i + 1].w};
#pragma unroll
                    for (uint32_t k = 0; k < 4; ++k) {
                        const uint32_t lo = __builtin_amdgcn_perm(b[k], a[k], 0x05040100u);
                        const uint32_t hi = __builtin_amdgcn_perm(b[k], a[k], 0x07060302u);
                        acc[2 * k] = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(lo), xb, acc[2 * k], false);
                        acc[2 * k + 1] = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(hi), xb, acc[2 * k + 1], false);
                    }
                }
            } else {
#pragma unroll
                for (uint32_t i = 0; i < 16; ++i) {
                    const float xr = __shfl(xv, (int)(i * 4u + g), 64);
                    float wf[VE];
                    unpack<DT>(w[i], wf);
#pragma unroll
                    for (uint32_t e = 0; e < VE; ++e) acc[e] += xr * wf[e];
                }
            }
        };
        u32x4 wa[16], wb[16];
        float xa = loadx(0), xb = 0.0f;
        loadw(wa, 0);
        for (uint32_t bi = 0; bi < nb; bi += 2) {
            if (bi + 1 < nb) { xb = loadx(bi + 1); loadw(wb, bi + 1); }
            __builtin_amdgcn_sched_barrier(0);  // keep the prefetch above the use
            consume(wa, xa);
            if (bi + 1 < nb) {
                if (bi + 2 < nb) { xa = loadx(bi + 2); loadw(wa, bi + 2); }
                __builtin_amdgcn_sched_barrier(0);
                consume(wb, xb);
            }
        }
        // sum the four row groups (lanes cl, cl+16, cl+32, cl+48) in a fixed order
#pragma unroll
        for (uint32_t e = 0; e < VE; ++e) {
            const float a1 = __shfl_xor(acc[e], 16, 64);
            const float s01 = (g & 1u) ? a1 + acc[e] : acc[e] + a1;  // same value in both lanes
            const float s23 = __shfl_xor(s01, 32, 64);
            acc[e] = (g & 2u) ? s23 + s01 : s01 + s23;
        }
    } else {
        // element path: lane handles columns cb*CPB + cl + 16 e, rows kb + g + 4 i
        for (uint32_t r = g; r < kn; r += 4u) {
            const float xr = ld_elem<DT>(X, kb + r);
#pragma unroll
            for (uint32_t e = 0; e < VE; ++e) {
                const uint32_t col = cb * CPB + cl + 16u * e;
                if (col < N) acc[e] += xr * ld_elem<DT>(Wm, (uint64_t)(kb + r) * N + col);
            }
        }
#pragma unroll
        for (uint32_t e = 0; e < VE; ++e) {
            const float a1 = __shfl_xor(acc[e], 16, 64);
            const float s01 = (g & 1u) ? a1 + acc[e] : acc[e] + a1;
            const float s23 = __shfl_xor(s01, 32, 64);
            acc[e] = (g & 2u) ? s23 + s01 : s01 + s23;
        }
    }
    // lanes of row group 0 hold the column sums
    auto col_of = [&](uint32_t e) -> uint32_t { return vec ? c0 + e : cb * CPB + cl + 16u * e; };
    uint8_t* Y = (uint8_t*)u.out;
    if (nks == 1) {
        if (g == 0) {
#pragma unroll
            for (uint32_t e = 0; e < VE; ++e) {
                const uint32_t col = col_of(e);
                if (col < N) st_elem<DTO>(Y, col, acc[e]);
            }
        }
        return;
    }
    float* part = (float*)(u.scratch + COUNTER_AREA);
    if (g == 0) {
#pragma unroll
        for (uint32_t e = 0; e < VE; ++e) {
            const uint32_t col = col_of(e);
            if (col < N) wstf(part + (uint64_t)ks * N + col, acc[e]);
        }
    }
    uint32_t* ctr = (uint32_t*)u.scratch + cb;
    uint32_t prev = 0;
    stores_done();  // this unit's partial is published before it is counted
    if (lane == 0) prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = (uint32_t)__builtin_amdgcn_readlane((int)prev, 0);
    if (prev != nks - 1) return;
    // merge: each of the 64 lanes sums its NCL = CPB/64 columns over the
    // splits in split order, the loads of up to 16 splits of all its columns
    // in flight together
    const uint8_t* pb = (const uint8_t*)part;
    constexpr uint32_t MAXS = 16;
    constexpr uint32_t NCL = CPB / 64u;
    const uint32_t cend = min(N, (cb + 1u) * CPB);
    float sm[NCL];
#pragma unroll
    for (uint32_t q = 0; q < NCL; ++q) sm[q] = 0.0f;
    for (uint32_t k0 = 0; k0 < nks; k0 += MAXS) {
        float pv[MAXS][NCL];
#pragma unroll
        for (uint32_t k = 0; k < MAXS; ++k) {
#pragma unroll
            for (uint32_t q = 0; q < NCL; ++q) {
                const uint32_t col = cb * CPB + lane + 64u * q;
                pv[k][q] = k0 + k < nks && col < cend ? __uint_as_float(ld4(pb + ((uint64_t)(k0 + k) * N + col) * 4u)) : 0.0f;
            }
        }
#pragma unroll
        for (uint32_t k = 0; k < MAXS; ++k) {
#pragma unroll
            for (uint32_t q = 0; q < NCL; ++q)
                if (k0 + k < nks) sm[q] += pv[k][q];
        }
    }
#pragma unroll
    for (uint32_t q = 0; q < NCL; ++q) {
        const uint32_t col = cb * CPB + lane + 64u * q;
        if (col < cend) st_elem<DTO>(Y, col, sm[q]);
    }
    if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- MATMUL
// y[M,N] = x[M,K] Wt[N,K]^T, the weight in the [out, in] layout of a linear
// layer; bf16 inputs, M <= 64 (the pages' "small matmuls").  At M rows per
// weight element the product is dense enough for the matrix cores: fp32
// vector FMAs would cap it near 20 flop per byte of weights, while the
// weights stream from HBM.  Unit = (block of NB = 16 NT output columns,
// k-split of MM_KC = 1024), with NT = 8 column tiles and MT <= 2 row tiles
// at M <= 32 and NT = 4, MT <= 4 above (the same 16 accumulator tiles;
// every unit reads all of x beside its weight slice, so the wider units
// read x half as often).  Per step of 32 k each MFMA takes, for one 16-row
// tile of x and one 16-column tile of Wt, one 16-byte piece of a row per
// lane (lane l: row l % 16, k offset 8 (l / 16)), the operand layout of
// v_mfma_f32_16x16x32_bf16, into fp32 accumulators (lane l holds rows
// 4 (l / 16) + i, column l % 16 of each 16x16 tile).  x is loaded in that
// layout; the weights come in whole 128-byte lines and reach it through
// LDS (below).  Rows past M and columns past N read zero through the
// bounded windows.  With several k-splits each unit writes fp32
// partial tiles and the last unit of a column block adds them in split
// order.
template <uint32_t DTO, uint32_t MTMAX, uint32_t NT>
__device__ __forceinline__ void matmul_tile(const Unit& u, uint32_t lane) {
    constexpr uint32_t NB = 16u * NT;
    const uint32_t M = (uint32_t)u.size, K = u.dim[0], N = u.dim[1];
    const uint32_t ncb = (N + NB - 1) / NB, nks = (K + MM_KC - 1) / MM_KC;
    const uint32_t cb = u.tile % ncb, ks = u.tile / ncb;
    const uint32_t kb = ks * MM_KC, kn = min(K - kb, MM_KC);  // a multiple of 32
    const uint32_t MT = (M + 15u) / 16u;                       // row tiles in use (wave-uniform)
    const uint32_t r16 = lane % 16u, kg = lane / 16u;
    const uint32_t ncol = min(N - cb * NB, NB);
    const RBuf rx = rbuf((const uint8_t*)u.a, M * K * 2u);
    const RBuf rw = rbuf((const uint8_t*)u.b + (uint64_t)cb * NB * K * 2u, ncol * K * 2u);
    f32x4 acc[MTMAX][NT];
#pragma unroll
    for (uint32_t mt = 0; mt < MTMAX; ++mt)
#pragma unroll
        for (uint32_t nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t nst = kn / 32u;
    {
        // The weights come in whole 128-byte lines and go through the
        // wave's LDS area into the operand layout.
        // Per double step of 64 k and group of four tiles, each tile takes
        // two loads of 8 rows x 128 bytes (lane l: row 8 h + l / 8, bytes
        // 16 (l % 8)), written to LDS with rows WRS bytes apart and read
        // back per step (lane l: row l % 16, bytes 16 (4 s + l / 16)).  The
        // operand-layout loads took half of sixteen lines per instruction,
        // and the small-matmul stream ran about 11% slower with them (no
        // non-temporal hint here: with those loads it had evicted the other
        // half of each line before the next step read it, 1.77x the weight
        // bytes from memory).
        // The registers that staged a group take the next group's loads at
        // once, so as many bytes are in flight as before; x comes per
        // double step, the next one's loads issued with the last group.
        constexpr uint32_t GT = 4u, NG = NT / GT, WRS = 144u;
        static_assert(NT % GT == 0 && GT * 16u * WRS <= SDPA_VCHUNK_BYTES, "weight staging fits the wave's LDS area");
        __attribute__((address_space(3))) uint8_t* wl =
            (__attribute__((address_space(3))) uint8_t*)sdpa_vlds + (threadIdx.x >> 6) * SDPA_VCHUNK_BYTES;
        const uint32_t nds = (nst + 1u) / 2u, nit = nds * NG;
        // past the last step of an odd count the loads read the next k (or
        // nothing, past the window) and their products are skipped
        auto load_w = [&](u32x4* R, uint32_t it) {
            const uint32_t k = kb + (it / NG) * 64u + (lane % 8u) * 8u;
            const uint32_t t0 = (it % NG) * GT;
#pragma unroll
            for (uint32_t tt = 0; tt < GT; ++tt)
#pragma unroll
                for (uint32_t h = 0; h < 2; ++h)
                    R[2u * tt + h] = rld16(rw, (((t0 + tt) * 16u + 8u * h + lane / 8u) * K + k) * 2u);
        };
        auto load_x = [&](u32x4* X, uint32_t d) {
#pragma unroll
            for (uint32_t s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (uint32_t t = 0; t < MTMAX; ++t)
                    X[s2 * MTMAX + t] = rld16(rx, ((t * 16u + r16) * K + kb + d * 64u + s2 * 32u + kg * 8u) * 2u);
        };
        u32x4 R[2 * GT], O[2 * GT], xa[2 * MTMAX], xb[2 * MTMAX];
        auto dstep = [&](uint32_t d, const u32x4* X, u32x4* Xn) {
#pragma unroll
            for (uint32_t g = 0; g < NG; ++g) {
                const uint32_t it = d * NG + g;
#pragma unroll
                for (uint32_t tt = 0; tt < GT; ++tt)
#pragma unroll
                    for (uint32_t h = 0; h < 2; ++h)
                        *(__attribute__((address_space(3))) u32x4*)(wl + (tt * 16u + 8u * h + lane / 8u) * WRS +
                                                                    (lane % 8u) * 16u) = R[2u * tt + h];
                if (it + 1 < nit) load_w(R, it + 1);
                if (g == NG - 1 && d + 1 < nds) load_x(Xn, d + 1);
                __builtin_amdgcn_sched_barrier(0);  // keep the prefetch above the use
#pragma unroll
                for (uint32_t tt = 0; tt < GT; ++tt)
#pragma unroll
                    for (uint32_t s2 = 0; s2 < 2; ++s2)
                        O[2u * tt + s2] = *(const __attribute__((address_space(3))) u32x4*)(
                            wl + (tt * 16u + r16) * WRS + (4u * s2 + kg) * 16u);
#pragma unroll
                for (uint32_t s2 = 0; s2 < 2; ++s2) {
                    if (2u * d + s2 >= nst) break;
#pragma unroll
                    for (uint32_t mt = 0; mt < MTMAX; ++mt) {
                        if (mt >= MT) break;
#pragma unroll
                        for (uint32_t tt = 0; tt < GT; ++tt)
                            acc[mt][g * GT + tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, X[s2 * MTMAX + mt]), __builtin_bit_cast(bf16x8, O[2u * tt + s2]),
                                acc[mt][g * GT + tt], 0, 0, 0);
                    }
                }
            }
        };
        load_w(R, 0);
        load_x(xa, 0);
        for (uint32_t d = 0; d < nds; d += 2) {
            dstep(d, xa, xb);
            if (d + 1 < nds) dstep(d + 1, xb, xa);
        }
    }
    uint8_t* Y = (uint8_t*)u.out;
    float* part = (float*)(u.scratch + COUNTER_AREA);
#pragma unroll
    for (uint32_t mt = 0; mt < MTMAX; ++mt) {
        if (mt >= MT) break;
#pragma unroll
        for (uint32_t nt = 0; nt < NT; ++nt) {
            const uint32_t n = cb * NB + nt * 16u + r16;
#pragma unroll
            for (uint32_t i = 0; i < 4; ++i) {
                const uint32_t m = mt * 16u + kg * 4u + i;
                if (m < M && n < N) {
                    if (nks == 1) st_elem<DTO>(Y, (uint64_t)m * N + n, acc[mt][nt][i]);
                    else wstf(part + ((uint64_t)ks * M + m) * N + n, acc[mt][nt][i]);
                }
            }
        }
    }
    if (nks == 1) return;
    uint32_t* ctr = (uint32_t*)u.scratch + cb;
    uint32_t prev = 0;
    stores_done();  // this unit's partial tiles are published before they are counted
    if (lane == 0) prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = (uint32_t)__builtin_amdgcn_readlane((int)prev, 0);
    if (prev != nks - 1) return;
    // merge: lane c owns columns cb * NB + c + 64 g and adds their M rows
    // over the splits in split order; the loads of 8 rows x 8 splits are in
    // flight at once (the row loop does not wait for one row's loads before
    // the next)
    constexpr uint32_t MR = 8, MS = 8;
    const RBuf rp = rbuf(part, (uint32_t)((uint64_t)nks * M * N * 4u));
#pragma unroll 1
    for (uint32_t cg = 0; cg < NB / 64u; ++cg) {
        const uint32_t col = cb * NB + cg * 64u + lane;
        for (uint32_t m0 = 0; m0 < M; m0 += MR) {
            float sm[MR];
#pragma unroll
            for (uint32_t i = 0; i < MR; ++i) sm[i] = 0.0f;
            for (uint32_t k0 = 0; k0 < nks; k0 += MS) {
                float pv[MR][MS];
#pragma unroll
                for (uint32_t i = 0; i < MR; ++i)
#pragma unroll
                    for (uint32_t k = 0; k < MS; ++k) {
                        // splits past nks, rows past M and columns past N are
                        // sent outside the window (reads zero, never added)
                        const bool in = k0 + k < nks && m0 + i < M && col < N;
                        pv[i][k] = __uint_as_float(rld4(rp, in ? (uint32_t)((((uint64_t)(k0 + k) * M + m0 + i) * N + col) * 4u)
                                                              : 0xFFFFFFF0u));
                    }
#pragma unroll
                for (uint32_t i = 0; i < MR; ++i)
#pragma unroll
                    for (uint32_t k = 0; k < MS; ++k)
                        if (k0 + k < nks) sm[i] += pv[i][k];
            }
#pragma unroll
            for (uint32_t i = 0; i < MR; ++i)
                if (m0 + i < M && col < N) st_elem<DTO>(Y, (uint64_t)(m0 + i) * N + col, sm[i]);
        }
    }
    if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ COPY
// COPY_TILE_BYTES per unit: 32 chunks of 16 bytes per lane, all loads first.
__device__ __forceinline__ void copy_tile(const Unit& u, uint32_t lane) {
    constexpr uint32_t NC = COPY_TILE_BYTES / 1024u;
    const uint64_t start = (uint64_t)u.tile * COPY_TILE_BYTES;
    if (start >= u.size) return;
    const uint32_t cnt = (uint32_t)(u.size - start < COPY_TILE_BYTES ? u.size - start : COPY_TILE_BYTES);
    const uint8_t* A = (const uint8_t*)u.a + start;
    uint8_t* O = (uint8_t*)u.out + start;
    if (((u.a | u.out) & 15ull) == 0) {
        const uint32_t full = cnt & ~15u;
        const RBuf ra = rbuf(A, full);
        const WBuf ob = wbuf(O, full);
        u32x4 v[NC];
#pragma unroll
        for (uint32_t k = 0; k < NC; ++k) v[k] = rld16(ra, (lane + 64u * k) * 16u);
#pragma unroll
        for (uint32_t k = 0; k < NC; ++k) wst16(ob, (lane + 64u * k) * 16u, v[k]);
        if (full + lane < cnt) wst8(O + full + lane, (uint8_t)ld1(A + full + lane));
    } else {
        for (uint32_t i = lane; i < cnt; i += 64u) wst8(O + i, (uint8_t)ld1(A + i));
    }
}

// add/mul/ReLU: a unit of a big op (see ew_big) is two consecutive tiles
template <uint32_t K, uint32_t DT>
__device__ __forceinline__ void ew_unit(const Unit& u, uint32_t lane) {
    constexpr uint32_t ES = DT == GPUOS_F32 ? 4u : 2u;
    constexpr uint32_t S = EW_TILE_BYTES_BIG / EW_TILE_BYTES;
    if (ew_big(u.size, ES)) {
#pragma unroll 1
        for (uint32_t j = 0; j < S; ++j) ew_tile<K, DT>(u, u.tile * S + j, lane);
    } else {
        ew_tile<K, DT>(u, u.tile, lane);
    }
}
template <uint32_t K>
__device__ __forceinline__ void ew_dispatch(const Unit& u, uint32_t lane, bool bf) {
    if (bf) ew_unit<K, GPUOS_BF16>(u, lane);
    else ew_unit<K, GPUOS_F32>(u, lane);
}

// ------------------------------------------------------------- dispatch
// Wave-uniform switch on the resolved kind (indirect calls would force a
// conservative register and stack budget on AMDGPU).
__device__ __forceinline__ void run_unit(const Unit& u, uint32_t lane) {
    const uint32_t di = dt_in(u.flags), dout = dt_out(u.flags);
    const bool bf = di == GPUOS_BF16;
    switch (u.kind) {
        case GPUOS_OP_NOP: break;
        case GPUOS_OP_ADD: ew_dispatch<GPUOS_OP_ADD>(u, lane, bf); break;
        case GPUOS_OP_MUL: ew_dispatch<GPUOS_OP_MUL>(u, lane, bf); break;
        case GPUOS_OP_RELU: ew_dispatch<GPUOS_OP_RELU>(u, lane, bf); break;
        case GPUOS_OP_GELU: bf ? ew_tile<GPUOS_OP_GELU, GPUOS_BF16>(u, u.tile, lane) : ew_tile<GPUOS_OP_GELU, GPUOS_F32>(u, u.tile, lane); break;
        case GPUOS_OP_EXPR: bf ? expr_tile<GPUOS_BF16>(u, lane) : expr_tile<GPUOS_F32>(u, lane); break;
        case GPUOS_OP_SUM: bf ? row_tile<GPUOS_OP_SUM, GPUOS_BF16>(u, lane) : row_tile<GPUOS_OP_SUM, GPUOS_F32>(u, lane); break;
        case GPUOS_OP_MAX: bf ? row_tile<GPUOS_OP_MAX, GPUOS_BF16>(u, lane) : row_tile<GPUOS_OP_MAX, GPUOS_F32>(u, lane); break;
        case GPUOS_OP_MIN: bf ? row_tile<GPUOS_OP_MIN, GPUOS_BF16>(u, lane) : row_tile<GPUOS_OP_MIN, GPUOS_F32>(u, lane); break;
        case GPUOS_OP_SOFTMAX: bf ? row_tile<GPUOS_OP_SOFTMAX, GPUOS_BF16>(u, lane) : row_tile<GPUOS_OP_SOFTMAX, GPUOS_F32>(u, lane); break;
        case GPUOS_OP_LAYERNORM: bf ? row_tile<GPUOS_OP_LAYERNORM, GPUOS_BF16>(u, lane) : row_tile<GPUOS_OP_LAYERNORM, GPUOS_F32>(u, lane); break;
        case GPUOS_OP_ROPE: bf ? rope_tile<GPUOS_BF16>(u, lane) : rope_tile<GPUOS_F32>(u, lane); break;
        case GPUOS_OP_KV_APPEND: kv_tile(u, lane); break;
        case GPUOS_OP_SDPA:
            if (u.dim[1] == 128u) {
                if (sdpa_heads_per_unit(u.dim[0], u.dim[3], 128u) == 4u)
                    dout == GPUOS_F32 ? sdpa_gqa_tile<GPUOS_F32>(u, lane) : sdpa_gqa_tile<GPUOS_BF16>(u, lane);
                else
                    dout == GPUOS_F32 ? sdpa_tile<16, GPUOS_F32, 1>(u, lane) : sdpa_tile<16, GPUOS_BF16, 1>(u, lane);
            } else {
                dout == GPUOS_F32 ? sdpa_tile<8, GPUOS_F32, 1>(u, lane) : sdpa_tile<8, GPUOS_BF16, 1>(u, lane);
            }
            break;
        case GPUOS_OP_GEMV:
            if (bf) dout == GPUOS_F32 ? gemv_tile<GPUOS_BF16, GPUOS_F32>(u, lane) : gemv_tile<GPUOS_BF16, GPUOS_BF16>(u, lane);
            else dout == GPUOS_F32 ? gemv_tile<GPUOS_F32, GPUOS_F32>(u, lane) : gemv_tile<GPUOS_F32, GPUOS_BF16>(u, lane);
            break;
        case GPUOS_OP_COPY: copy_tile(u, lane); break;
        case GPUOS_OP_MATMUL:
            if (u.size <= 32u) dout == GPUOS_F32 ? matmul_tile<GPUOS_F32, 2, 8>(u, lane) : matmul_tile<GPUOS_BF16, 2, 8>(u, lane);
            else dout == GPUOS_F32 ? matmul_tile<GPUOS_F32, 4, 4>(u, lane) : matmul_tile<GPUOS_BF16, 4, 4>(u, lane);
            break;
        default: break;
    }
}

}  // namespace gpuos
