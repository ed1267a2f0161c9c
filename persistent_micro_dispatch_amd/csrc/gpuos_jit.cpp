// Compiled operator injection (host side).
//
// The pages inject an operator by compiling a curated template with its
// parameters substituted, loading the result, writing its address into the
// inactive slot of the operator table and flipping the version (digest
// page, section 3 Q2 "Dynamic Operator Table"; section 4, core technical
// barriers, template-based JIT).  Here the template is the element-wise
// loop of one work unit, laid out like the built-in element-wise bodies
// (4 KiB of each operand per unit, 16-byte device-scope loads issued one
// chunk ahead, write-through stores, an element per lane for the ragged
// tail), and the parameters are an element-wise program, emitted as
// straight-line fp32 code.  The resident executor calls the result through a
// function pointer.
//
// For a call through a pointer, the compiler sizes the calling kernel's
// registers for the largest non-kernel function of the kernel's own module,
// and the callee saves what it uses of the callee-saved registers on a
// stack in scratch memory.  The executor's module holds a never-called
// function that fixes that budget (gpuos_jit_budget); the code compiled
// here is accepted only if its probe kernel, which calls both bodies
// directly and so reports at least their usage, fits the budget.
//
// The compiler is the hipRTC of the ROCm installation the library was built
// with, loaded into a linker namespace of its own: a process that has
// loaded another copy of hipRTC and its compiler library (PyTorch ships
// one) would otherwise compile injected code with that copy's compiler,
// while the executor was compiled with this one.
#include "gpuos_jit.h"

#include <dlfcn.h>
#include <hip/hiprtc.h>

#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>
#include <vector>

#ifndef GPUOS_ROCM_LIB
#define GPUOS_ROCM_LIB "/opt/rocm/lib"
#endif

namespace gpuos {

bool expr_validate(const uint32_t* program, uint32_t n_words, uint32_t slot[PROG_WORDS], uint32_t* kflags) {
    if (!program || n_words == 0) return false;
    const uint32_t w0 = program[0];
    const uint32_t ni = w0 & 0xFFu, nk = (w0 >> 8) & 0xFFu;
    if ((w0 >> 16) != 0 || ni == 0 || ni > GPUOS_EXPR_MAX_INSTR || nk > GPUOS_EXPR_MAX_CONSTS ||
        n_words != 1 + ni + nk)
        return false;
    uint32_t kf = ni << 8;
    for (uint32_t i = 0; i < PROG_WORDS; ++i) slot[i] = 0;
    slot[0] = w0;
    for (uint32_t i = 0; i < ni; ++i) {
        const uint32_t w = program[1 + i];
        const uint32_t op = w & 0xFFu, d = (w >> 8) & 0xFu, s1 = (w >> 12) & 0xFu, s2 = (w >> 16) & 0xFu;
        const uint32_t k = (w >> 20) & 0xFFu;
        if (op == 0 || op >= GPUOS_X_COUNT || d > 3 || s1 > 3 || s2 > 3 || (w >> 28) != 0) return false;
        if (op == GPUOS_X_CONST && k >= nk) return false;
        if (op == GPUOS_X_LDB) kf |= EXPR_USES_B;
        slot[PROG_INSTR + i] = w;
    }
    for (uint32_t i = 0; i < nk; ++i) slot[PROG_CONST + i] = program[1 + ni + i];
    *kflags = kf;
    return true;
}

namespace {

// Fixed part of the template: helpers with the same arithmetic as the
// interpreter of element-wise programs in the executor.
const char* kPrelude = R"(#include <stdint.h>
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32v2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16v2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) uint32_t g_u32;
typedef __attribute__((address_space(1))) uint16_t g_u16;
#define SC1 16
static __device__ __forceinline__ __amdgpu_buffer_rsrc_t win(const void* p, uint32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}
static __device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, SC1);
}
static __device__ __forceinline__ void st16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, SC1);
}
static __device__ __forceinline__ uint32_t f2bf2(float lo, float hi) {
  const f32v2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16v2));
}
template <int ES> static __device__ __forceinline__ float lde(const uint8_t* p, uint32_t i) {
  if constexpr (ES == 4) return __uint_as_float(__hip_atomic_load((g_u32*)(p + 4u * i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  else return __uint_as_float((uint32_t)__hip_atomic_load((g_u16*)(p + 2u * i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) << 16);
}
template <int ES> static __device__ __forceinline__ void ste(uint8_t* p, uint32_t i, float v) {
  if constexpr (ES == 4) __hip_atomic_store((g_u32*)(p + 4u * i), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else __hip_atomic_store((g_u16*)(p + 2u * i), (uint16_t)(f2bf2(v, 0.0f) & 0xFFFFu), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
static __device__ __forceinline__ float tmax(float a, float b) {
  const float m = a < b ? b : a;
  const float z = __uint_as_float(__float_as_uint(a) & __float_as_uint(b));
  const float r = a == b ? z : m;
  return a != a ? a : (b != b ? b : r);
}
static __device__ __forceinline__ float tmin(float a, float b) {
  const float m = a < b ? a : b;
  const float z = __uint_as_float(__float_as_uint(a) | __float_as_uint(b));
  const float r = a == b ? z : m;
  return a != a ? a : (b != b ? b : r);
}
static __device__ __forceinline__ float xexp(float x) {
  const float t = x * 1.44269504f;
  const float r = fmaf(x, 1.44269504f, -t) + x * 1.9259629e-8f;
  const bool sub = t < -126.0f;
  const float p = __builtin_amdgcn_exp2f(sub ? t + 64.0f : t) * fmaf(r, 0.693147181f, 1.0f);
  return sub ? p * 5.42101086e-20f : p;
}
static __device__ __forceinline__ float xlog(float x) {
  const bool sub = x > 0.0f && x < 1.17549435e-38f;
  return __builtin_amdgcn_logf(sub ? x * 16777216.0f : x) * 0.693147181f - (sub ? 16.6355324f : 0.0f);
}
static __device__ __forceinline__ float xtanh(float x) {
  const float e = xexp(2.0f * fabsf(x));
  const float t = 1.0f - 2.0f / (e + 1.0f);
  return x != x ? x : copysignf(t, x);
}
)";

// The unit loop; USES_B and the tile size are substituted before it.
const char* kBody = R"(
template <int ES>
static __device__ __forceinline__ void body(const uint8_t* a, const uint8_t* b, uint8_t* o, uint64_t n,
                                            uint32_t tile, uint32_t lane) {
  constexpr uint32_t TILE = TILE_BYTES / ES, VE = 16 / ES, CH = TILE_BYTES / 16 / 64;
  const uint64_t start = (uint64_t)tile * TILE;
  if (start >= n) return;
  const uint32_t cnt = n - start < TILE ? (uint32_t)(n - start) : TILE;
  const uint8_t* A = a + start * ES;
  const uint8_t* B = (USES_B ? b : a) + start * ES;
  uint8_t* O = o + start * ES;
  const uint64_t al = (uint64_t)a | (uint64_t)o | (USES_B ? (uint64_t)b : 0ull);
  if ((al & 15ull) == 0) {
    const uint32_t full = cnt / VE;
    const __amdgpu_buffer_rsrc_t ra = win(A, full * 16u), rb = win(B, full * 16u), ro = win(O, full * 16u);
    const uint32_t rem = full * VE;
    const bool tl = rem + lane < cnt;
    float xt = 0.0f, yt = 0.0f;
    if (tl) {
      xt = lde<ES>(A, rem + lane);
      if (USES_B) yt = lde<ES>(B, rem + lane);
    }
    u32x4 na = ld16(ra, lane * 16u), nb = na;
    if (USES_B) nb = ld16(rb, lane * 16u);
#pragma unroll 1
    for (uint32_t c = 0; c < CH; ++c) {
      const u32x4 ca = na, cb = nb;
      na = ld16(ra, (lane + 64u * (c + 1u)) * 16u);  // past the tile: outside the window, zero
      if (USES_B) nb = ld16(rb, (lane + 64u * (c + 1u)) * 16u);
      float x[VE], y[VE], r[VE];
      const uint32_t wa[4] = {ca.x, ca.y, ca.z, ca.w}, wb[4] = {cb.x, cb.y, cb.z, cb.w};
#pragma unroll
      for (uint32_t e = 0; e < VE; ++e) {
        if constexpr (ES == 4) { x[e] = __uint_as_float(wa[e]); y[e] = __uint_as_float(wb[e]); }
        else {
          x[e] = __uint_as_float(e & 1u ? wa[e / 2] & 0xFFFF0000u : wa[e / 2] << 16);
          y[e] = __uint_as_float(e & 1u ? wb[e / 2] & 0xFFFF0000u : wb[e / 2] << 16);
        }
      }
#pragma unroll
      for (uint32_t e = 0; e < VE; ++e) r[e] = f(x[e], y[e]);
      u32x4 v;
      if constexpr (ES == 4) v = u32x4{__float_as_uint(r[0]), __float_as_uint(r[1]), __float_as_uint(r[2]), __float_as_uint(r[3])};
      else v = u32x4{f2bf2(r[0], r[1]), f2bf2(r[2], r[3]), f2bf2(r[4], r[5]), f2bf2(r[6], r[7])};
      st16(ro, (lane + 64u * c) * 16u, v);  // chunks past `full` are dropped
    }
    if (tl) ste<ES>(O, rem + lane, f(xt, yt));
  } else {
    for (uint32_t i = lane; i < cnt; i += 64u) ste<ES>(O, i, f(lde<ES>(A, i), USES_B ? lde<ES>(B, i) : 0.0f));
  }
}
typedef void (*gpuos_jit_fn)(const uint8_t*, const uint8_t*, uint8_t*, uint64_t, uint32_t, uint32_t);
extern "C" __device__ __attribute__((noinline)) void gpuos_jit_f32(const uint8_t* a, const uint8_t* b, uint8_t* o,
                                                                   uint64_t n, uint32_t tile, uint32_t lane) {
  body<4>(a, b, o, n, tile, lane);
}
extern "C" __device__ __attribute__((noinline)) void gpuos_jit_bf16(const uint8_t* a, const uint8_t* b, uint8_t* o,
                                                                    uint64_t n, uint32_t tile, uint32_t lane) {
  body<2>(a, b, o, n, tile, lane);
}
extern "C" __device__ gpuos_jit_fn gpuos_jit_f32_addr = gpuos_jit_f32;
extern "C" __device__ gpuos_jit_fn gpuos_jit_bf16_addr = gpuos_jit_bf16;
extern "C" __global__ void __launch_bounds__(64) gpuos_jit_probe(const uint8_t* a, const uint8_t* b, uint8_t* o, uint64_t n) {
  gpuos_jit_f32(a, b, o, n, blockIdx.x, threadIdx.x);
  gpuos_jit_bf16(a, b, o, n, blockIdx.x, threadIdx.x);
}
)";

std::string reg(uint32_t r) { return "r" + std::to_string(r); }

// One program instruction as an fp32 expression of the registers before it.
std::string instr_expr(uint32_t w, const uint32_t* consts) {
    const uint32_t op = w & 0xFFu, s1 = (w >> 12) & 3u, s2 = (w >> 16) & 3u, k = (w >> 20) & 0xFFu;
    const std::string x = reg(s1), y = reg(s2);
    char buf[64];
    switch (op) {
        case GPUOS_X_LDA: return "a";
        case GPUOS_X_LDB: return "b";
        case GPUOS_X_CONST: snprintf(buf, sizeof buf, "__uint_as_float(0x%08xu)", consts[k]); return buf;
        case GPUOS_X_MOV: return x;
        case GPUOS_X_ADD: return x + " + " + y;
        case GPUOS_X_SUB: return x + " - " + y;
        case GPUOS_X_MUL: return x + " * " + y;
        case GPUOS_X_DIV: return x + " / " + y;
        case GPUOS_X_MIN: return "tmin(" + x + ", " + y + ")";
        case GPUOS_X_MAX: return "tmax(" + x + ", " + y + ")";
        case GPUOS_X_NEG: return "__uint_as_float(__float_as_uint(" + x + ") ^ 0x80000000u)";
        case GPUOS_X_ABS: return "__uint_as_float(__float_as_uint(" + x + ") & 0x7FFFFFFFu)";
        case GPUOS_X_EXP: return "xexp(" + x + ")";
        case GPUOS_X_LOG: return "xlog(" + x + ")";
        case GPUOS_X_SQRT: return "sqrtf(" + x + ")";
        case GPUOS_X_TANH: return "xtanh(" + x + ")";
        case GPUOS_X_SIGMOID: return "1.0f / (1.0f + xexp(-" + x + "))";
        default: return x + " > 0.0f ? " + x + " : (" + x + " != " + x + " ? " + x + " : 0.0f)";  // RELU
    }
}

// Parse "Key: value" remarks of the probe kernel from the compiler's log.
bool probe_resources(const std::string& log, JitCode* out) {
    bool in = false, got_v = false, got_a = false, got_s = false, got_st = false, got_dyn = false;
    size_t pos = 0;
    while (pos < log.size()) {
        size_t end = log.find('\n', pos);
        if (end == std::string::npos) end = log.size();
        const std::string line = log.substr(pos, end - pos);
        pos = end + 1;
        const size_t r = line.find("remark:");
        if (r == std::string::npos) continue;
        std::string body = line.substr(r + 7);
        const size_t tag = body.find(" [-Rpass");
        if (tag != std::string::npos) body.resize(tag);
        const size_t b0 = body.find_first_not_of(' ');
        if (b0 == std::string::npos) continue;
        body = body.substr(b0);
        const size_t colon = body.find(':');
        if (colon == std::string::npos) continue;
        const std::string key = body.substr(0, colon);
        std::string val = body.substr(colon + 1);
        const size_t v0 = val.find_first_not_of(' ');
        val = v0 == std::string::npos ? "" : val.substr(v0);
        if (key == "Function Name") {
            in = val == "gpuos_jit_probe";
            continue;
        }
        if (!in) continue;
        char* e = nullptr;
        const unsigned long n = strtoul(val.c_str(), &e, 10);
        const bool num = e && e != val.c_str() && *e == '\0';
        if (key == "VGPRs" && num) { out->vgprs = (uint32_t)n; got_v = true; }
        else if (key == "AGPRs" && num) { out->agprs = (uint32_t)n; got_a = true; }
        else if (key == "TotalSGPRs" && num) { out->sgprs = (uint32_t)n; got_s = true; }
        else if (key == "ScratchSize [bytes/lane]" && num) { out->stack = (uint32_t)n; got_st = true; }
        else if (key == "Dynamic Stack") { out->dynamic_stack = val != "False"; got_dyn = true; }
    }
    return got_v && got_a && got_s && got_st && got_dyn;
}

// hipRTC entry points, from the copy in this library's ROCm installation
struct Rtc {
    hiprtcResult (*create)(hiprtcProgram*, const char*, const char*, int, const char**, const char**);
    hiprtcResult (*compile)(hiprtcProgram, int, const char**);
    hiprtcResult (*log_size)(hiprtcProgram, size_t*);
    hiprtcResult (*log)(hiprtcProgram, char*);
    hiprtcResult (*code_size)(hiprtcProgram, size_t*);
    hiprtcResult (*code)(hiprtcProgram, char*);
    hiprtcResult (*destroy)(hiprtcProgram*);
    bool ok = false;
};

const Rtc& rtc() {
    static Rtc r;
    static std::once_flag once;
    std::call_once(once, [] {
        const char* path = GPUOS_ROCM_LIB "/libhiprtc.so.7";
        void* h = dlmopen(LM_ID_NEWLM, path, RTLD_NOW | RTLD_LOCAL);
        if (!h) {
            fprintf(stderr, "gpuos: cannot load %s: %s\n", path, dlerror());
            return;
        }
        bool all = true;
        auto get = [&](auto& f, const char* name) {
            f = reinterpret_cast<std::remove_reference_t<decltype(f)>>(dlsym(h, name));
            all = all && f != nullptr;
        };
        get(r.create, "hiprtcCreateProgram");
        get(r.compile, "hiprtcCompileProgram");
        get(r.log_size, "hiprtcGetProgramLogSize");
        get(r.log, "hiprtcGetProgramLog");
        get(r.code_size, "hiprtcGetCodeSize");
        get(r.code, "hiprtcGetCode");
        get(r.destroy, "hiprtcDestroyProgram");
        r.ok = all;
    });
    return r;
}

double ms_since(std::chrono::steady_clock::time_point t0) {
    return std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
}

}  // namespace

std::string jit_source(const uint32_t slot[PROG_WORDS], uint32_t kflags) {
    const uint32_t ni = slot[0] & 0xFFu;
    std::string s = "// element-wise body compiled by gpuos_register_jit\n";
    s += kPrelude;
    s += "#define TILE_BYTES " + std::to_string(JIT_TILE_BYTES) + "u\n";
    s += std::string("#define USES_B ") + ((kflags & EXPR_USES_B) ? "true" : "false") + "\n";
    s += "static __device__ __forceinline__ float f(float a, float b) {\n";
    s += "  float r0 = 0.0f, r1 = 0.0f, r2 = 0.0f, r3 = 0.0f;\n";
    s += "  (void)a; (void)b;\n";
    for (uint32_t i = 0; i < ni; ++i) {
        const uint32_t w = slot[PROG_INSTR + i];
        s += "  { const float t = " + instr_expr(w, slot + PROG_CONST) + "; " + reg((w >> 8) & 3u) + " = t; }\n";
    }
    s += "  (void)r1; (void)r2; (void)r3;\n  return r0;\n}\n";
    s += kBody;
    return s;
}

int jit_build(const std::string& src, const std::string& arch, bool load, hipStream_t s, JitCode* out,
              std::string* log) {
    *out = JitCode{};
    const Rtc& R = rtc();
    if (!R.ok) return GPUOS_E_HIP;
    const auto t0 = std::chrono::steady_clock::now();
    hiprtcProgram prog = nullptr;
    if (R.create(&prog, src.c_str(), "gpuos_jit.hip", 0, nullptr, nullptr) != HIPRTC_SUCCESS) return GPUOS_E_HIP;
    const std::string a = "--offload-arch=" + arch;
    // no fused multiply-adds formed from * and +, correctly rounded / and
    // sqrt, subnormals kept: each program step rounds like the interpreter's
    const char* opts[] = {a.c_str(), "-O3", "-std=c++17", "-ffp-contract=off",
                          "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
                          "-Rpass-analysis=kernel-resource-usage"};
    const hiprtcResult cr = R.compile(prog, (int)(sizeof(opts) / sizeof(opts[0])), opts);
    size_t ls = 0;
    std::string lg;
    if (R.log_size(prog, &ls) == HIPRTC_SUCCESS && ls > 1) {
        lg.resize(ls);
        if (R.log(prog, &lg[0]) != HIPRTC_SUCCESS) lg.clear();
        while (!lg.empty() && lg.back() == '\0') lg.pop_back();
    }
    if (log) *log = lg;
    if (cr != HIPRTC_SUCCESS) {
        R.destroy(&prog);
        return GPUOS_E_HIP;
    }
    size_t cs = 0;
    std::vector<char> code;
    if (R.code_size(prog, &cs) != HIPRTC_SUCCESS || cs == 0) {
        R.destroy(&prog);
        return GPUOS_E_HIP;
    }
    code.resize(cs);
    const hiprtcResult gr = R.code(prog, code.data());
    R.destroy(&prog);
    if (gr != HIPRTC_SUCCESS) return GPUOS_E_HIP;
    if (const char* dump = getenv("GPUOS_JIT_DUMP")) {  // keep the code object for inspection
        if (FILE* f = fopen(dump, "wb")) {
            fwrite(code.data(), 1, cs, f);
            fclose(f);
        }
    }
    out->code_bytes = cs;
    out->compile_ms = ms_since(t0);
    if (!probe_resources(lg, out)) return GPUOS_E_HIP;
    if (out->vgprs > GPUOS_JIT_MAX_VGPRS || out->agprs > GPUOS_JIT_MAX_AGPRS || out->sgprs > GPUOS_JIT_MAX_SGPRS ||
        out->stack > GPUOS_JIT_MAX_STACK || out->dynamic_stack)
        return GPUOS_E_STATE;
    if (!load) return GPUOS_OK;
    const auto t1 = std::chrono::steady_clock::now();
    hipModule_t mod = nullptr;
    if (hipModuleLoadData(&mod, code.data()) != hipSuccess) return GPUOS_E_HIP;
    uint64_t addr[2] = {0, 0};
    const char* names[2] = {"gpuos_jit_f32_addr", "gpuos_jit_bf16_addr"};
    for (int i = 0; i < 2; ++i) {
        hipDeviceptr_t p = nullptr;
        size_t bytes = 0;
        if (hipModuleGetGlobal(&p, &bytes, mod, names[i]) != hipSuccess || bytes != 8 ||
            hipMemcpyAsync(&addr[i], p, 8, hipMemcpyDeviceToHost, s) != hipSuccess) {
            (void)hipModuleUnload(mod);
            return GPUOS_E_HIP;
        }
    }
    // the variables hold relocated code addresses; a value inside the
    // object's own size would be an offset the loader did not relocate
    if (hipStreamSynchronize(s) != hipSuccess || addr[0] < cs || addr[1] < cs) {
        (void)hipModuleUnload(mod);
        return GPUOS_E_HIP;
    }
    out->mod = mod;
    out->fn_f32 = addr[0];
    out->fn_bf16 = addr[1];
    out->load_ms = ms_since(t1);
    return GPUOS_OK;
}

}  // namespace gpuos
