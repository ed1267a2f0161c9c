// Compiled operator injection: the source template, its compilation with
// hipRTC and the loading of the result (host side).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "gpuos_internal.h"

namespace gpuos {

// Check an element-wise program (gpuos_register_expr format) and copy it
// into a program slot; *kflags gets EXPR_USES_B | n_instr << 8.
bool expr_validate(const uint32_t* program, uint32_t n_words, uint32_t slot[PROG_WORDS], uint32_t* kflags);

// The HIP source of the injected body for a validated program slot: two
// extern "C" device functions (fp32 and bf16 operands), a device variable
// holding each one's address, and a probe kernel that calls both (its
// resource report bounds theirs).
std::string jit_source(const uint32_t slot[PROG_WORDS], uint32_t kflags);

struct JitCode {
    hipModule_t mod = nullptr;
    uint64_t fn_f32 = 0, fn_bf16 = 0;  // device code addresses
    uint32_t vgprs = 0, agprs = 0, sgprs = 0, stack = 0;
    bool dynamic_stack = true;
    uint64_t code_bytes = 0;
    double compile_ms = 0.0, load_ms = 0.0;
};

// Compile `src` for `arch` (the device's full target name), read the probe
// kernel's resources from the compiler's report into *out and check them
// against the budget; if they fit and `load` is set, load the code object
// on the current device and resolve both addresses (copies through the
// non-blocking stream `s`).  Returns GPUOS_OK, GPUOS_E_HIP (compile, load
// or copy failed; the log goes to *log) or GPUOS_E_STATE (over budget).
int jit_build(const std::string& src, const std::string& arch, bool load, hipStream_t s, JitCode* out,
              std::string* log);

}  // namespace gpuos
