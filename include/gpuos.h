/*
 * gpuos.h -- C ABI of the MI355X persistent micro-op dispatcher.
 *
 * The operation (GPUOS digest page, sections 2 and 3 Q2): a host thread
 * writes small task descriptors into a lock-free ring in device-visible
 * memory (prepare -> acquire slot -> write -> commit with store-release);
 * a persistent executor kernel, launched once with one workgroup per
 * compute unit, polls the ring with load-acquire, claims work atomically,
 * looks the op up in a dual-slot, version-flipped operator table and runs
 * the micro-op as a device function instead of a kernel launch; then it
 * releases the slot.  Results equal running every micro-op in submission
 * order (the pages keep eager semantics).
 *
 * Conventions for every entry point:
 *  - Pointers named "device pointer" are HIP device addresses (for example
 *    a torch tensor's data_ptr()); the library never allocates, frees or
 *    copies them.  Other pointers are host pointers.
 *  - Every function returns GPUOS_OK (0) or a negative GPUOS_E_* code and
 *    never throws or aborts.
 *  - A context is driven by one producer thread at a time (calls into one
 *    context are serialised internally; producers on different threads are
 *    ordered only by that serialisation).
 *  - While a context is alive, do not call hipDeviceSynchronize (or
 *    torch.cuda.synchronize()) on its device: the executor kernel does not
 *    exit until gpuos_pause or gpuos_shutdown.  Use gpuos_sync instead.
 */
#ifndef GPUOS_H
#define GPUOS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GPUOS_ABI_VERSION 5

/* ---------------------------------------------------------------- errors */
#define GPUOS_OK 0
#define GPUOS_E_INVAL (-1)    /* bad argument, descriptor layout or shape */
#define GPUOS_E_FULL (-2)     /* not enough free ring slots (no BLOCK flag) */
#define GPUOS_E_NOOP (-3)     /* register_op: unknown kind or op_id out of range */
#define GPUOS_E_TIMEOUT (-4)  /* gpuos_sync / shutdown deadline passed */
#define GPUOS_E_DEVICE (-5)   /* a descriptor completed with a non-zero status */
#define GPUOS_E_HIP (-6)      /* a HIP runtime call failed */
#define GPUOS_E_STATE (-7)    /* call not valid in the context's state */

/* per-descriptor device status codes (see gpuos_sync's err_seq/err_status) */
#define GPUOS_ST_OK 0
#define GPUOS_ST_BAD_OP 1     /* op_id out of range or table entry empty */
#define GPUOS_ST_BAD_SHAPE 2  /* shape the op body does not support */
#define GPUOS_ST_SPIN 3       /* a dependency wait exceeded the spin limit */

/* -------------------------------------------------------- operator kinds */
/* Built-in operator bodies (digest page, section 3 Q2 "Operator library").
 * At init op_id k is bound to kind k for every built-in kind except EXPR;
 * op id 15 and the op ids from GPUOS_KIND_COUNT upward start empty and can be
 * bound with gpuos_register_op or gpuos_register_expr (user op ids are
 * GPUOS_OP_USER and above). */
enum gpuos_kind {
    GPUOS_OP_NOP = 0,        /* nothing; the analogue of a null kernel */
    GPUOS_OP_ADD = 1,        /* out[i] = a[i] + b[i], i < size */
    GPUOS_OP_MUL = 2,        /* out[i] = a[i] * b[i] */
    GPUOS_OP_RELU = 3,       /* out[i] = max(a[i], +0); NaN stays NaN */
    GPUOS_OP_GELU = 4,       /* tanh-approximation GELU */
    GPUOS_OP_SUM = 5,        /* [rows, h] -> [rows], along the last dim */
    GPUOS_OP_MAX = 6,
    GPUOS_OP_MIN = 7,
    GPUOS_OP_SOFTMAX = 8,    /* [rows, h] -> [rows, h] */
    GPUOS_OP_LAYERNORM = 9,  /* [rows, h] -> [rows, h], gamma/beta [h] */
    GPUOS_OP_ROPE = 10,      /* in place on q and k, [B, H, D] */
    GPUOS_OP_KV_APPEND = 11, /* K/V cache [B, H, C, D] row L_b-1 <- k/v [B, H, D] */
    GPUOS_OP_SDPA = 12,      /* single-query attention over keys [0, L_b) */
    GPUOS_OP_GEMV = 13,      /* y[N] = x[K] . W[K, N] (W row-major) */
    GPUOS_OP_COPY = 14,      /* byte copy of `size` bytes */
    GPUOS_OP_EXPR = 15,      /* element-wise program bound by gpuos_register_expr */
    GPUOS_OP_MATMUL = 16,    /* y[M, N] = x[M, K] . Wt[N, K]^T, M <= 64 (small matmul) */
    GPUOS_OP_JIT = 17,       /* element-wise program compiled at run time, bound by
                                gpuos_register_jit (GPUOS_INIT_JIT contexts only) */
    GPUOS_KIND_COUNT = 18,
    GPUOS_KIND_EMPTY = 0xFFFFFFFFu /* register_op: unbind an op id */
};
#define GPUOS_MAX_OPS 256
#define GPUOS_OP_USER 64

/* element types */
#define GPUOS_F32 0u
#define GPUOS_BF16 1u

/* descriptor flags: bits 0-3 input dtype, bits 4-7 output dtype */
#define GPUOS_FLAGS(in_dtype, out_dtype) ((uint32_t)(in_dtype) | ((uint32_t)(out_dtype) << 4))
#define GPUOS_F_ROPE_HALF (1u << 8)  /* RoPE pairs (x_i, x_{i+D/2}) instead of (x_2i, x_2i+1) */
#define GPUOS_F_SDPA_MASK (1u << 9)  /* SDPA adds an fp32 mask [B, C] (aux[2]) to the scaled scores */
#define GPUOS_F_KV_PAGED (1u << 10)  /* KV_APPEND / SDPA: caches are page pools with a block table */

/* ------------------------------------------------------------ descriptor */
/* One ring entry, 128 bytes (the pages give 64-128 B holding op_id,
 * input_a, input_b, output, size, flags plus dims).  The caller fills the
 * first 88 bytes and `param`; gpuos_submit fills seq, dep_delta, dep_range
 * and table_version.
 *
 * Operand meaning by kind (all pointers are device pointers):
 *   ADD, MUL        a, b, output: `size` elements of the input dtype.
 *   RELU, GELU      a, output: `size` elements.
 *   SUM/MAX/MIN     a = x [size rows, dim[0]]; output [size].
 *   SOFTMAX         a = x [size, dim[0]]; output [size, dim[0]].
 *   LAYERNORM       as SOFTMAX; aux[0] = gamma [dim[0]], aux[1] = beta;
 *                   param.f[0] = eps (0 -> the table entry's default).
 *   ROPE            a = q [size=B, dim[0]=H, dim[1]=D], b = k [B, Hk, D]
 *                   with Hk = dim[3] (0 -> H, at most H: fewer key heads
 *                   under grouped-query attention), rotated in place at
 *                   position lens[b]-1; param.f[4] = theta (0 -> table
 *                   default, 10000).
 *   KV_APPEND       a = k, b = v [B, H, D]; aux[0] = K cache, aux[1] = V cache
 *                   [B, H, dim[2]=C, D]; writes row lens[b]-1.
 *   SDPA            a = q [B, H, D]; aux[0] = K, aux[1] = V [B, Hkv, C, D]
 *                   with Hkv = dim[3] (0 -> H) dividing H: query head h
 *                   attends with key/value head h / (H / Hkv) (grouped-
 *                   query attention; Hkv = 1 is multi-query attention);
 *                   output [B, H, D] in the output dtype; keys [0, lens[b]);
 *                   param.f[4] = scale (0 -> 1/sqrt(D)).  D must be 64 or 128;
 *                   lens[b] up to 65535 (at most 64 splits of 1024 keys).
 *                   Attention masking (the pages' operator library lists it
 *                   with SDPA): with flag GPUOS_F_SDPA_MASK, aux[2] = an fp32
 *                   mask [B, C] added to the scaled score of key j in row b
 *                   (the same for every head; -inf removes the key; a row
 *                   with every key removed gives NaN).
 *   GEMV            a = x [dim[0]=K], b = W [K, dim[1]=N] row-major, output [N].
 *   MATMUL          a = x [size=M, dim[0]=K] row-major, b = Wt [dim[1]=N, K]
 *                   row-major (the [out, in] weight of a linear layer),
 *                   output y [M, N] = x . Wt^T; bf16 inputs, fp32
 *                   accumulation on the matrix cores, output in the output
 *                   dtype; 1 <= M <= 64, K a multiple of 32 (the pages'
 *                   "small matmuls", too small for a BLAS call).
 *   Paged caches (flag GPUOS_F_KV_PAGED on KV_APPEND and SDPA): the caches
 *                   are pools of P pages [P, Hkv, PS, D] (K in aux[0], V in
 *                   aux[1]; Hkv = the append's dim[0] heads, SDPA's dim[3])
 *                   and a block table [B, MP] of int32 page numbers maps
 *                   position j of batch row b to page table[b][j / PS], row
 *                   j % PS (the usual paged-attention layout).  size = B in
 *                   the low 32 bits and P in the high 32 bits; dim[2] = PS, a
 *                   power of two from 64 to 1024; param.u[5] = MP (lens[b] at
 *                   most MP * PS).  The table
 *                   is in aux[2] for KV_APPEND and in b for SDPA (whose
 *                   mask, with GPUOS_F_SDPA_MASK, stays in aux[2], [B, MP *
 *                   PS]).  A table entry outside [0, P) writes nothing (append)
 *                   or drops that page's keys (SDPA).  Hazard tracking takes
 *                   each pool as one range: an append orders with every
 *                   earlier attention that reads the pool, and so on.
 *   COPY            a -> output, `size` bytes.
 * Within one descriptor an output must coincide exactly with an input or
 * not overlap it.  B must be at most 8 (lens are inline). */
typedef struct gpuos_desc {
    uint32_t op_id;          /*   0 */
    uint32_t flags;          /*   4 */
    uint64_t seq;            /*   8  set by gpuos_submit */
    uint64_t input_a;        /*  16 */
    uint64_t input_b;        /*  24 */
    uint64_t output;         /*  32 */
    uint64_t size;           /*  40 */
    uint32_t dim[4];         /*  48 */
    uint64_t aux[3];         /*  64 */
    uint16_t dep_delta[6];   /*  88  set by gpuos_submit: wait for seq - delta (0 = none) */
    uint16_t dep_range;      /* 100  set by gpuos_submit: wait for all of [seq - range, seq) */
    uint16_t table_version;  /* 102  set by gpuos_submit */
    union {
        float f[6];
        uint32_t u[6];
        uint16_t lens[12];   /* lens[0..7] per batch row for ROPE/KV_APPEND/SDPA */
    } param;                 /* 104 */
} gpuos_desc;

#ifdef __cplusplus
static_assert(sizeof(gpuos_desc) == 128, "gpuos_desc must be 128 bytes");
#endif

/* ---------------------------------------------------------------- init */
#define GPUOS_INIT_LOOPBACK (1u << 0) /* test only: no GPU; a host thread plays the
                                         consumer, completes descriptors in a random
                                         dependency-respecting order and computes nothing */
#define GPUOS_INIT_TRACE (1u << 1)    /* record one gpuos_trace_rec per work unit */
#define GPUOS_INIT_JIT (1u << 2)      /* run the executor build that can call code injected
                                         with gpuos_register_jit (one unit per wave; its
                                         injected calls use a stack in scratch memory) */

typedef struct gpuos_init_params {
    int32_t device;             /* HIP device ordinal */
    uint32_t ring_entries;      /* power of two in [8, 32768]; 0 -> 4096 */
    uint32_t num_wgs;           /* executor workgroups, at most 4 per CU, and at least
                                   2 waves in all (one fetches); 0 -> one per CU */
    uint32_t waves_per_wg;      /* wave64s per workgroup, 1..4; 0 -> 4 */
    uint32_t backoff_max;       /* s_sleep cap of idle waits, 1..127; 0 -> 64 (the fetcher
                                   wave, whose polls go over PCIe, stops at 8) */
    uint32_t flags;             /* GPUOS_INIT_* */
    void* hip_stream;           /* optional hipStream_t for the executor (must be
                                   non-blocking); NULL -> the library creates one */
    uint64_t scratch_bytes;     /* device scratch for split ops; 0 -> 256 MiB */
    uint32_t unit_queue_log2;   /* log2 of unit-queue entries, 12..24; 0 -> 20 */
    uint32_t spin_limit_ms;     /* dependency-wait limit before ST_SPIN; 0 -> 20000 */
    uint32_t units_per_wave;    /* units a worker wave holds at once, 1 or 2; 0 -> 1.
                                   With 2 a ready unit overtakes one still waiting for
                                   its dependencies (helps streams of long bodies, such
                                   as decode attention), but each wave holds two claims
                                   (slower on long dependency chains of short ops) */
    uint32_t idle_exit_ms;      /* 0: the executor stays resident until gpuos_pause or
                                   gpuos_shutdown.  Else it leaves the GPU once no
                                   descriptor is committed and no call of this context
                                   (each one is a heartbeat) has come for this long, so
                                   that a host that stops (hangs, waits elsewhere)
                                   does not hold the CUs; the next submit, sync or
                                   query launches it again */
} gpuos_init_params;

/* Allocate the ring (fine-grained coherent host memory), the device tables
 * and counters, bind the built-in op ids and launch the executor once: it
 * stays resident, one workgroup per compute unit by default, until the host
 * stops it (digest page, section 3 Q2 "Persistent Kernel Executor": launched
 * once, never exits on its own, a small share of each SM/CU).
 * params may be NULL for defaults.  *out receives the context.  One live
 * context per device and process: a second one's resident executor could
 * not be placed beside the first one's.
 * Errors: E_INVAL (bad params), E_STATE (the device already has a live
 * context in this process), E_HIP (allocation or launch failed). */
int gpuos_init(const gpuos_init_params* params, void** out);

/* ------------------------------------------------------------- register */
/* Bind op_id to a built-in kind with constants (the pages' operator
 * injection: write the inactive table slot, then flip the version counter;
 * digest page, section 3 Q2 "Dynamic Operator Table").  consts (may be NULL)
 * points to `len` bytes: up to two floats, the kind's default parameter
 * (LAYERNORM eps, ROPE theta, SDPA scale).  Descriptors submitted after this
 * call returns use the new entry; earlier ones keep the old one.
 * Errors: E_NOOP (op_id >= GPUOS_MAX_OPS or unknown kind), E_INVAL, E_HIP. */
int gpuos_register_op(void* ctx, uint32_t op_id, uint32_t kind, const void* consts, uint32_t len);

/* Bind op_id to an element-wise program (kind EXPR).  The pages inject
 * operators as code compiled at run time from curated templates with
 * parameters substituted, written to the inactive table slot and enabled by
 * the version flip (digest page, section 3 Q2 "Dynamic Operator Table";
 * section 4, core technical barriers).  Here the curated template is an
 * element-wise register machine and the parameters are its program: the
 * resident executor interprets it, so a new operator is installed by the
 * same table write and flip as gpuos_register_op, with no compilation, code
 * loading or relaunch.
 *
 * A descriptor of such an op reads a[i] (and b[i] if the program uses it),
 * i < size elements of the input dtype, and writes out[i] in the same dtype
 * (out may coincide with a or b).  For each element the program runs on
 * four fp32 registers r0..r3 (initially 0) and r0 is the result, rounded to
 * the dtype (bf16: to nearest even).  Layout (32-bit words):
 *   word 0: n_instr | n_consts << 8 (1..32 instructions, 0..16 constants);
 *   words 1..n_instr: instructions, op | dst << 8 | src1 << 12 | src2 << 16
 *     | const index << 20 (register numbers 0..3);
 *   then n_consts fp32 constants (bit patterns).
 * Ops (fp32; + - * / and sqrt correctly rounded, min/max propagate NaN and
 * order -0 below +0, exp/log/tanh/sigmoid from the hardware's exp2/log2
 * with errors near 1e-7 relative, absolute where the result is near 0):
 *   GPUOS_X_LDA d = a[i]; GPUOS_X_LDB d = b[i]; GPUOS_X_CONST d = k[c];
 *   GPUOS_X_MOV d = s1; ADD, SUB, MUL, DIV, MIN, MAX d = s1 op s2;
 *   NEG, ABS, EXP, LOG, SQRT, TANH, SIGMOID (1/(1+e^-x)), RELU d = f(s1).
 * Descriptors submitted after this call returns use the program; earlier
 * ones keep what they were submitted under.
 * Errors: E_NOOP (op_id >= GPUOS_MAX_OPS), E_INVAL (malformed program),
 * E_HIP. */
enum gpuos_expr_op {
    GPUOS_X_LDA = 1, GPUOS_X_LDB = 2, GPUOS_X_CONST = 3, GPUOS_X_MOV = 4,
    GPUOS_X_ADD = 5, GPUOS_X_SUB = 6, GPUOS_X_MUL = 7, GPUOS_X_DIV = 8,
    GPUOS_X_MIN = 9, GPUOS_X_MAX = 10, GPUOS_X_NEG = 11, GPUOS_X_ABS = 12,
    GPUOS_X_EXP = 13, GPUOS_X_LOG = 14, GPUOS_X_SQRT = 15, GPUOS_X_TANH = 16,
    GPUOS_X_SIGMOID = 17, GPUOS_X_RELU = 18,
    GPUOS_X_COUNT = 19
};
#define GPUOS_EXPR_MAX_INSTR 32
#define GPUOS_EXPR_MAX_CONSTS 16
int gpuos_register_expr(void* ctx, uint32_t op_id, const uint32_t* program, uint32_t n_words);

/* Bind op_id to compiled code (kind JIT): the pages' operator injection as
 * they describe it, a curated template compiled at run time with its
 * parameters substituted, loaded, its address written into the inactive
 * table slot and enabled by the version flip while the executor keeps
 * running (digest page, section 3 Q2 "Dynamic Operator Table", steps 1-5;
 * section 4, core technical barriers, template-based JIT).  The template is
 * an element-wise loop over one work unit and the parameters are an
 * element-wise program in the gpuos_register_expr format, with the same
 * meaning: the program becomes straight-line fp32 code (hipRTC, gfx950,
 * no contraction of * and + into fused multiply-adds, no flush of
 * subnormals; exp/log/tanh/sigmoid evaluated as in the interpreter), one
 * function per dtype, loaded into this context's device.  The running
 * executor reaches it through a function pointer: the library refuses
 * code that needs more registers or stack than the executor reserves for
 * injected calls (GPUOS_JIT_MAX_VGPRS VGPRs, GPUOS_JIT_MAX_AGPRS AGPRs,
 * GPUOS_JIT_MAX_SGPRS SGPRs, no stack of its own).  Loaded code stays
 * loaded until gpuos_shutdown.  Compiling the same program again in one
 * context reuses the loaded code.
 * info (may be NULL) receives the timings and the code's resources.
 * Errors: E_NOOP (op_id >= GPUOS_MAX_OPS), E_INVAL (malformed program, or a
 * context made without GPUOS_INIT_JIT), E_STATE (the compiled code exceeds
 * the reserved budget), E_HIP (compile, load or copy failed; the compiler's
 * log goes to stderr). */
#define GPUOS_JIT_MAX_VGPRS 96u
#define GPUOS_JIT_MAX_AGPRS 32u
#define GPUOS_JIT_MAX_SGPRS 102u
#define GPUOS_JIT_MAX_STACK 0u
typedef struct gpuos_jit_info {
    double compile_ms;   /* hipRTC compile of the generated source (0 when reused) */
    double load_ms;      /* code-object load and address resolution */
    double flip_ms;      /* table write and version flip */
    uint32_t vgprs;      /* resources of the compiled body (upper bounds) */
    uint32_t agprs;
    uint32_t sgprs;
    uint32_t stack_bytes;
    uint64_t code_bytes; /* size of the code object */
    uint32_t reused;     /* 1 if an earlier identical program's code was reused */
    uint32_t pad;
} gpuos_jit_info;
int gpuos_register_jit(void* ctx, uint32_t op_id, const uint32_t* program, uint32_t n_words,
                       gpuos_jit_info* info);
/* The HIP source gpuos_register_jit compiles for `program` (NUL-terminated,
 * truncated to cap bytes); *len_out receives the full length.  Needs no
 * context or GPU.  Errors: E_INVAL (malformed program). */
int gpuos_jit_source(const uint32_t* program, uint32_t n_words, char* out, uint64_t cap, uint64_t* len_out);

/* --------------------------------------------------------------- submit */
#define GPUOS_SUBMIT_BLOCK (1u << 0)     /* wait for free slots instead of E_FULL */
#define GPUOS_SUBMIT_NOHAZARD (1u << 1)  /* caller guarantees no overlap with work in flight */
#define GPUOS_SUBMIT_SERIAL (1u << 2)    /* each descriptor waits for its predecessor */

/* Copy `count` descriptors into consecutive ring slots and commit them in
 * order (store-release of each slot's stamp): the host side of the ring
 * protocol, prepare descriptor -> acquire slot -> write -> commit with a
 * store-release (digest page, section 3 Q2 "Ring Buffer Communication
 * Channel").  Before writing, every
 * descriptor is checked and annotated with dependencies on earlier
 * descriptors whose byte ranges it reads or writes (read-after-write,
 * write-after-read, write-after-write), so results equal sequential
 * execution.  A descriptor waits for up to 62 earlier descriptors by
 * number (six in dep_delta, the rest in a side array owned by the library
 * and copied to device memory with the descriptor); with more it waits for
 * every descriptor from the oldest on (dep_range).  Annotation runs before
 * the wait for free slots, so it overlaps the device's work.  The caller's
 * array may be reused on return.  *first_seq
 * (may be NULL) receives the sequence number of descriptor 0; the others
 * follow consecutively.  All or nothing: on error no descriptor is
 * submitted.  Errors: E_INVAL (a descriptor fails validation),
 * E_FULL (fewer than count free slots and no BLOCK), E_DEVICE (the
 * executor reported an error while this call waited), E_STATE. */
int gpuos_submit(void* ctx, const gpuos_desc* descs, uint32_t count, uint32_t flags,
                 uint64_t* first_seq);

/* Producer loop in native code: submit descs[0..sum(bursts)) as n_bursts
 * consecutive gpuos_submit calls of burst_sizes[i] descriptors each (each
 * burst is committed as a group; a burst larger than the ring is committed
 * in ring-sized groups).  Stops at the first error and returns it; *n_done
 * (may be NULL) receives the number of descriptors submitted. */
int gpuos_submit_bursts(void* ctx, const gpuos_desc* descs, const uint32_t* burst_sizes, uint32_t n_bursts,
                        uint32_t flags, uint64_t* first_seq, uint64_t* n_done);

/* ----------------------------------------------------------------- sync */
#define GPUOS_SEQ_ALL 0xFFFFFFFFFFFFFFFFull

/* Wait until every descriptor with seq <= upto_seq (GPUOS_SEQ_ALL: every
 * submitted one) has completed, that is until the executor has released its
 * ring slot, the last device step after dispatch (digest page, section 3 Q2
 * "Ring Buffer Communication Channel", device side: poll -> claim ->
 * dispatch -> release slot).  timeout_ns < 0 waits forever.  Returns
 * E_DEVICE if any of them completed with a non-zero status (the first one's
 * seq and status go to *err_seq and *err_status, either may be NULL),
 * E_TIMEOUT if the deadline passed. */
int gpuos_sync(void* ctx, uint64_t upto_seq, int64_t timeout_ns, uint64_t* err_seq,
               uint32_t* err_status);

/* Non-blocking: 1 if seq has completed, 0 if not, negative on error. */
int gpuos_query(void* ctx, uint64_t seq);

/* ----------------------------------------------------- pause / shutdown */
/* Wait for all submitted work, then stop the executor kernel (it exits and
 * frees the compute units) while keeping the ring, tables and sequence
 * numbers.  The resident executor of the pages never exits (digest page,
 * section 3 Q2 "Persistent Kernel Executor"); pausing it is this library's
 * way to give every CU back between bursts of work.  The next gpuos_submit or gpuos_resume relaunches it. */
int gpuos_pause(void* ctx, int64_t timeout_ns);
int gpuos_resume(void* ctx);

/* Stop the executor (work already submitted is finished first) and free
 * every resource: the end of the executor's life that starts with
 * gpuos_init (digest page, section 3 Q2 "Persistent Kernel Executor").  The context pointer is invalid afterwards.  If the
 * executor does not exit within the timeout the device is told to abort
 * and E_TIMEOUT is returned after the context is freed as far as safe. */
int gpuos_shutdown(void* ctx);

/* ---------------------------------------------------------------- stats */
typedef struct gpuos_stats {
    uint64_t submitted;          /* descriptors submitted */
    uint64_t completed;          /* descriptors observed complete by the host */
    uint64_t full_rejections;    /* submits that returned E_FULL */
    uint64_t launches;           /* executor launches (init + resumes) */
    float last_launch_ms;        /* duration of the last finished executor launch
                                    (HIP events on the executor stream) */
    float total_launch_ms;       /* sum over finished launches */
    uint64_t units;              /* work units executed (device counter) */
    uint64_t fetch_batches;      /* ring batches the fetcher read (device counter) */
    uint64_t fetched;            /* descriptors fetched (device counter) */
    uint64_t dep_waits;          /* units that found a dependency not yet done */
    uint32_t num_wgs, waves_per_wg, ring_entries, cu_count;
    uint64_t next_seq;           /* sequence number the next submit will get */
    uint64_t deps_explicit;      /* explicit dependencies written (host) */
    uint64_t deps_range;         /* descriptors that fell back to a range dependency */
    uint64_t ns_submit;          /* host time spent inside gpuos_submit */
    uint64_t ns_blocked;         /*   of which waiting for free ring slots (BLOCK) */
    uint64_t ns_annotate;        /*   of which annotating and writing descriptors */
    uint64_t idle_exits;         /* executor launches that ended for lack of heartbeat */
} gpuos_stats;

/* Snapshot of the counters.  Device counters are added up when a launch
 * ends (gpuos_pause / gpuos_shutdown); while the executor runs, units and
 * dependency waits of still-running waves are not yet included. */
int gpuos_stats_get(void* ctx, gpuos_stats* out);

/* Test only (GPUOS_INIT_LOOPBACK contexts): copy up to max sequence
 * numbers in the order the loopback consumer completed them. */
int gpuos_loopback_order(void* ctx, uint64_t* out, uint64_t max, uint64_t* n_out);

/* Test only: copy the descriptor committed with sequence number seq, as the
 * executor reads it (seq, dependencies and table version filled in), into
 * *out (host memory), and its side dependency deltas -- 56 uint16 values,
 * each "wait for seq - delta", 0 = none; all 0 unless dep_delta[5] is set --
 * into extra (host memory, may be NULL).  The descriptor must still be in
 * its ring slot: seq in [next_seq - ring_entries, next_seq).  The ring is
 * ordinary host memory, so this is safe while the executor runs.
 * Errors: E_INVAL (null ctx or out), E_STATE (seq not in the ring). */
int gpuos_ring_peek(void* ctx, uint64_t seq, gpuos_desc* out, uint16_t* extra);

/* ---------------------------------------------------------------- trace */
/* One record per executed work unit (GPUOS_INIT_TRACE contexts).  Times are
 * the device's constant-rate wall clock (hipDeviceAttributeWallClockRate,
 * kHz); unit numbers restart at 0 with every executor launch. */
typedef struct gpuos_trace_rec {
    uint64_t seq;          /* descriptor */
    uint32_t tile;         /* unit within the descriptor */
    uint32_t hw;           /* XCC id << 16 | workgroup id */
    uint64_t t_claim;      /* unit claimed and published */
    uint64_t t_ready;      /* dependencies satisfied */
    uint64_t t_body;       /* op body finished */
    uint64_t t_done;       /* completion written (last unit: slot released) */
    uint64_t unit;         /* unit number within the launch */
    uint64_t pad;
} gpuos_trace_rec;

/* Copy the trace of the last finished launch (call after gpuos_pause):
 * up to max records into out (host memory); *n_out = records available. */
int gpuos_trace_read(void* ctx, gpuos_trace_rec* out, uint64_t max, uint64_t* n_out);

/* ------------------------------------------------- baselines (measurement) */
/* Eager baseline: run each descriptor as its own hipLaunchKernel (one or
 * more kernels per descriptor, same op bodies as the executor) on
 * hip_stream, in order, with no dependency tracking beyond stream order.
 * No persistent context is needed; scratch (device pointer, scratch_bytes)
 * is caller-provided working memory for split ops (>= gpuos_eager_scratch_bytes).
 * Asynchronous: returns after enqueueing.  Errors: E_INVAL, E_HIP. */
int gpuos_eager_submit(const gpuos_desc* descs, uint32_t count, void* hip_stream,
                       void* scratch, uint64_t scratch_bytes);
/* Scratch bytes gpuos_eager_submit needs for these descriptors. */
uint64_t gpuos_eager_scratch_bytes(const gpuos_desc* descs, uint32_t count);

/* gpuos_eager_submit without a workspace argument and without allocating,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The split
 * partials and counters of attention and vector-matrix descriptors live in a
 * file-scope device array of GPUOS_EAGER_STATIC_SCRATCH_BYTES (16 MiB) that
 * each GPU holds until the process ends; the call clears its counters with a
 * small kernel first (no memset, so it can be captured).  Descriptors are
 * those gpuos_eager_submit takes; all are checked before anything is
 * launched.  Every call on one GPU shares the array, so calls that overlap
 * on one GPU (on different streams, or from different threads) race: issue
 * them on one stream, or order them.  Asynchronous: returns after
 * enqueueing on hip_stream.  Errors: E_INVAL (a bad descriptor, or one whose
 * split partials need more than GPUOS_EAGER_STATIC_SCRATCH_BYTES -- see
 * gpuos_eager_scratch_bytes), E_HIP. */
#define GPUOS_EAGER_STATIC_SCRATCH_BYTES (16u << 20)
int gpuos_eager_submit_static(const gpuos_desc* descs, uint32_t count, void* hip_stream);

/* hipGraph baseline: capture the eager launches of `descs` into a graph
 * and instantiate it; *graph_exec receives an opaque handle. */
int gpuos_graph_build(const gpuos_desc* descs, uint32_t count, void* hip_stream, void* scratch,
                      uint64_t scratch_bytes, void** graph_exec);
int gpuos_graph_launch(void* graph_exec, void* hip_stream);
int gpuos_graph_destroy(void* graph_exec);

/* Null-kernel launch cost: launch an empty kernel n times on hip_stream;
 * *ns_per_launch_async = host time per back-to-back launch call,
 * *ns_launch_sync = mean time of launch + hipStreamSynchronize. */
int gpuos_null_launch_bench(void* hip_stream, uint32_t n, double* ns_per_launch_async,
                            double* ns_launch_sync);

/* Closed-loop per-op latency as a C caller sees it: for each of the count
 * descriptors in turn, gpuos_submit it alone (BLOCK) and gpuos_sync until it
 * has completed; out_us[i] (host memory, count doubles, owned by the caller)
 * receives the time from before the submit to the return of the sync, in
 * microseconds.  Stops at the first error and returns it (E_INVAL for a null
 * ctx, descs or out_us; E_TIMEOUT if one descriptor takes longer than 10 s;
 * any error of gpuos_submit or gpuos_sync).  What it measures is the
 * per-op latency of the GPUOS digest page, section 3 Q3 (results), latency
 * breakdown on H100. */
int gpuos_latency_bench(void* ctx, const gpuos_desc* descs, uint32_t count, double* out_us);

/* Achievable HBM bandwidth with the memory instructions the op bodies use
 * (device-scope 16-byte loads, write-through stores), one workgroup of four
 * waves per CU: mode 0 reads `bytes` at src (dst: device memory of at least
 * 4 KiB, written only in the unlikely case that the xor of the data equals a
 * fixed value), mode 1 copies `bytes` from src to dst (device memory, no
 * overlap).  bytes: a multiple of 16, 4 KiB to 1 GiB.  One untimed launch,
 * then `reps` launches between two events on hip_stream; *gbs = bytes moved
 * (read, or read + written) per second / 1e9.  Blocks until done; run it
 * while no executor is resident.  Errors: E_INVAL, E_HIP. */
int gpuos_hbm_probe(const void* src, void* dst, uint64_t bytes, uint32_t mode, uint32_t reps, void* hip_stream,
                    double* gbs);

/* gpuos_hbm_probe with the grid given: `workgroups` workgroups of four
 * waves (0: one per compute unit, as gpuos_hbm_probe does; at most 4096).
 * Each lane keeps 16 loads of 16 bytes in flight, 64 KiB per workgroup; with
 * one workgroup per CU, a sweep over the workgroup count gives achievable
 * bandwidth against the number of active CUs, and by Little's law the
 * latency and the bytes in flight per CU that a share of the peak needs
 * (the method of "The GPU Needs an Operating System", appendix A.3).
 * Errors: as gpuos_hbm_probe; E_INVAL for more than 4096 workgroups. */
int gpuos_hbm_probe_grid(const void* src, void* dst, uint64_t bytes, uint32_t mode, uint32_t reps,
                         uint32_t workgroups, void* hip_stream, double* gbs);

/* ABI version of the loaded library. */
int gpuos_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GPUOS_H */
