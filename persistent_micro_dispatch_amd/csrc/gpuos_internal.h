// Internal layouts shared by the host runtime and the device executor.
// Not part of the public ABI (include/gpuos.h is).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gpuos.h"

namespace gpuos {

// ---------------------------------------------------------------------------
// Device-side operator table: two slots of GPUOS_MAX_OPS entries.  A
// descriptor carries the table version it was submitted under and is
// resolved against slot (version & 1) (the pages' dual-slot table with a
// version counter flip; digest page, section 3 Q2 "Dynamic Operator Table").
// ---------------------------------------------------------------------------
struct alignas(32) TableEntry {
    uint32_t kind;     // gpuos_kind, or GPUOS_KIND_EMPTY
    uint32_t flags;    // EXPR: EXPR_USES_B | n_instr << 8
    float p0;          // kind's default parameter (eps / theta / scale), 0 = built-in
    float p1;          // reserved
    uint64_t fn;       // EXPR: device address of this slot's copy of the program
    uint64_t reserved;
};
static_assert(sizeof(TableEntry) == 32, "TableEntry is 32 bytes");

constexpr uint32_t KIND_BAD = 0xFEu;  // internal: descriptor rejected on the device

// Element-wise programs (kind EXPR) as the library stores them: one slot of
// PROG_WORDS 32-bit words per op id and table slot; word 0 = n_instr |
// n_consts << 8, instructions at PROG_INSTR, constants at PROG_CONST.
constexpr uint32_t PROG_WORDS = 64;
constexpr uint32_t PROG_INSTR = 1;
constexpr uint32_t PROG_CONST = 1 + GPUOS_EXPR_MAX_INSTR;
static_assert(PROG_CONST + GPUOS_EXPR_MAX_CONSTS <= PROG_WORDS, "program slot");
static_assert(PROG_WORDS <= 64, "one program word per lane");
constexpr uint32_t EXPR_USES_B = 1u;

// Per-slot metadata the fetcher writes next to the mirrored descriptor.
struct alignas(64) MirrorMeta {
    uint32_t kind;          // resolved body
    uint32_t status;        // GPUOS_ST_* decided at fetch time
    uint32_t ntiles;        // work units
    float p0;               // default parameter from the table entry
    uint64_t ubegin;        // first unit number (this launch's numbering)
    uint64_t scratch_v;     // virtual scratch offset (physical = v % scratch_bytes), or ~0
    uint64_t scratch_mark;  // scratch watermark before this descriptor's allocation
    uint64_t prog;          // EXPR: device address of the program
    uint64_t pad[2];
};
static_assert(sizeof(MirrorMeta) == 64, "MirrorMeta is 64 bytes");

// Control words in fine-grained host memory (host writes, device polls).
struct HostCtl {
    alignas(64) uint64_t stop;       // host -> device: finish and exit when idle
    alignas(64) uint64_t abort;      // host -> device: exit at once
    alignas(64) uint64_t dev_error;  // device -> host: sticky error code
    alignas(64) uint64_t heartbeat;  // host -> device: bumped by every call of the context
    alignas(64) uint64_t fetch_end;  // device -> host: first seq the fetcher did not take
    alignas(64) uint64_t idle_exit;  // device -> host: 1 if the launch ended for lack of heartbeat
};

// Control words in device memory (one 128-byte line each).
// Unit tickets are handed out by CLAIM_SHARDS_MAX counters, each on a
// cache line of its own: shard x owns the units whose queue index is
// x modulo the shard count, and its counter numbers them in queue order.
// One counter for all waves saturates under contention (the more waves
// claim, the fewer claims per second succeed).
constexpr uint32_t CLAIM_SHARDS_MAX = 8;
struct alignas(256) ClaimLine {
    uint64_t next;  // next ticket of this shard (workers fetch_add)
};
struct DevCtl {
    ClaimLine claim[CLAIM_SHARDS_MAX];
    alignas(128) uint64_t q_tail;    // units published by the fetcher
    alignas(128) uint64_t stop;      // fetcher -> workers
    alignas(128) uint64_t error;     // sticky device error
    alignas(128) uint64_t stat_units;
    uint64_t stat_dep_waits;
    uint64_t stat_batches;
    uint64_t stat_fetched;
};

// ---------------------------------------------------------------------------
// Executor protocol arithmetic, shared by the executor, the host runtime and
// the host-side model of the protocol that the CPU tests drive.
// ---------------------------------------------------------------------------
// Claim shards: workgroup b claims from shard b % shards, so every shard
// needs a worker wave (workgroup 0's first wave is the fetcher), and all of
// them must be resident at once, or a shard could wait for a workgroup that
// never starts.  One workgroup per compute unit at most guarantees that;
// otherwise one shared counter is used.
__host__ __device__ inline uint32_t claim_shards(uint32_t num_wgs, uint32_t waves_per_wg, uint32_t cu_count) {
    if (num_wgs > cu_count) return 1;
    const uint32_t worker_wgs = waves_per_wg > 1 ? num_wgs : num_wgs - 1;
    const uint32_t s = worker_wgs < CLAIM_SHARDS_MAX ? worker_wgs : CLAIM_SHARDS_MAX;
    return s ? s : 1;
}
__host__ __device__ inline uint32_t wg_shard(uint32_t block, uint32_t shards) { return block % shards; }
// the unit (queue position) that ticket t of a shard stands for: shard x
// owns the positions congruent to x modulo the shard count, in order
__host__ __device__ inline uint64_t ticket_unit(uint64_t ticket, uint32_t shards, uint32_t shard) {
    return ticket * shards + shard;
}
// a unit-queue entry: the descriptor's sequence number and the unit's index in it
constexpr uint32_t QE_TILE_BITS = 24;
static_assert((1ull << QE_TILE_BITS) >= (1ull << 22), "tile field holds MAX_TILES");
// units of a batch after which the fetcher publishes the prefix written so
// far (a large descriptor's first units start while the rest are queued)
constexpr uint64_t PUBLISH_STEP = 2048;
static_assert((PUBLISH_STEP & (PUBLISH_STEP - 1)) == 0 && PUBLISH_STEP % 64 == 0, "a power of two, whole windows");
__host__ __device__ inline uint64_t queue_entry(uint64_t seq, uint64_t tile) { return (seq << QE_TILE_BITS) | tile; }
__host__ __device__ inline uint64_t entry_seq(uint64_t e) { return e >> QE_TILE_BITS; }
__host__ __device__ inline uint32_t entry_tile(uint64_t e) { return (uint32_t)(e & ((1u << QE_TILE_BITS) - 1u)); }
// the fetcher may publish units up to position u_end only while the oldest
// incomplete descriptor's first unit (cw_units) is at most Q positions back:
// a position is reused only after the unit that held it has run
__host__ __device__ inline bool units_fit(uint64_t u_end, uint64_t cw_units, uint64_t Q) { return u_end - cw_units <= Q; }
__host__ __device__ inline bool scratch_fits(uint64_t sv_end, uint64_t cw_scr, uint64_t S) { return sv_end - cw_scr <= S; }
// gpuos_submit refuses a descriptor of more units than this (or more
// scratch than half the scratch ring): once every earlier descriptor has
// completed, any single descriptor then fits, so the fetcher always
// progresses
__host__ __device__ inline uint64_t max_units_per_descriptor(uint64_t Q) { return Q / 2; }

// Kernel arguments of the executor.
struct ExecArgs {
    const gpuos_desc* ring;   // host-mapped
    const uint64_t* depx;     // host-mapped: DEPX_WORDS words of extra dependency deltas per slot
    uint64_t* depd;           // device copy of depx for descriptors that use it
    uint64_t* stamp;          // host-mapped
    uint32_t* status;         // host-mapped
    HostCtl* hctl;            // host-mapped
    DevCtl* dctl;
    gpuos_desc* mirror;
    MirrorMeta* meta;
    uint64_t* done;
    uint32_t* tiles_done;
    uint64_t* queue;
    const TableEntry* table;  // [2][GPUOS_MAX_OPS]
    uint8_t* scratch;
    uint64_t scratch_bytes;
    gpuos_trace_rec* trace;     // null unless tracing
    uint64_t trace_cap;         // records (power of two)
    uint64_t start_seq;
    uint64_t spin_limit_ticks;  // in wall-clock ticks
    uint64_t idle_exit_ticks;   // 0, or leave after this long without heartbeat or work
    uint32_t mask;              // ring_entries - 1
    uint32_t qmask;             // unit-queue entries - 1
    uint32_t backoff_max;
    uint32_t shards;            // claim shards in use (1..CLAIM_SHARDS_MAX)
};

// ---------------------------------------------------------------------------
// Work plan of a descriptor: how many work units (tiles) it splits into and
// how much scratch it needs.  Shared by the fetcher (device), the eager
// launcher and host-side validation so that all three agree.
// ---------------------------------------------------------------------------
// Element-wise tiles, per operand.  Small and mid-sized ops take 4 KiB
// units, which spreads a dependency level over more waves; ops of at least
// EW_BIG_OP_BYTES per operand take units of 8 KiB, done as two 4 KiB tiles
// one after the other, which halves their claims (many big ops at once are
// bound by the rate of unit claims).
constexpr uint32_t EW_TILE_BYTES = 4096;
constexpr uint32_t EW_TILE_BYTES_BIG = 8192;
constexpr uint64_t EW_BIG_OP_BYTES = 131072;
#ifndef GPUOS_GELU_TILE
#define GPUOS_GELU_TILE 2048
#endif
// done[] words per ring slot: one per 128-byte line, so that waves polling
// different slots, and the store that completes one, do not share a line
// (element-wise stream +3% with one wave per workgroup, +8% with four).
#ifndef GPUOS_DONE_STRIDE
#define GPUOS_DONE_STRIDE 16
#endif
constexpr uint32_t DONE_STRIDE = GPUOS_DONE_STRIDE;
constexpr uint32_t EW_TILE_BYTES_GELU = GPUOS_GELU_TILE;  // GELU costs ~40 instructions per element: smaller units

__host__ __device__ constexpr bool ew_big(uint64_t size, uint32_t es) { return size * es >= EW_BIG_OP_BYTES; }
__host__ __device__ constexpr uint32_t ew_tile_bytes(uint32_t kind, bool big) {
    return kind == GPUOS_OP_GELU ? EW_TILE_BYTES_GELU : big ? EW_TILE_BYTES_BIG : EW_TILE_BYTES;
}
// programs longer than 8 instructions cost as much per element as GELU
__host__ __device__ constexpr uint32_t expr_tile_bytes(uint32_t kflags, bool big) {
    return ((kflags >> 8) & 0xFFu) > 8u ? EW_TILE_BYTES_GELU : big ? EW_TILE_BYTES_BIG : EW_TILE_BYTES;
}
constexpr uint32_t COPY_TILE_BYTES = 32768;
constexpr uint32_t JIT_TILE_BYTES = 4096;     // bytes of each operand per unit of an injected (JIT) body
constexpr uint32_t ROW_MAX_CACHED = 4096;  // rows up to this length stay in registers
#ifndef GPUOS_SDPA_KT
#define GPUOS_SDPA_KT 1024
#endif
constexpr uint32_t SDPA_KT = GPUOS_SDPA_KT;  // keys per SDPA unit (fewer for small attention ops)
#ifndef GPUOS_GEMV_KC
#define GPUOS_GEMV_KC 128
#endif
constexpr uint32_t GEMV_KC = GPUOS_GEMV_KC;  // rows of W per GEMV unit (a multiple of 64)
constexpr uint32_t MM_NB = 64;             // output columns per MATMUL unit above 32 rows (four 16-column tiles)
constexpr uint32_t MM_NB_SMALL = 128;      // ... at most 32 rows (eight tiles: x is re-read by half as many units)
constexpr uint32_t MM_KC = 1024;           // k per MATMUL unit
constexpr uint32_t MM_MAX_M = 64;          // rows of x (four 16-row tiles)
constexpr uint32_t MAX_B = 8;              // batch rows with inline lengths
constexpr uint64_t COUNTER_AREA = 4096;    // bytes of per-descriptor group counters
constexpr uint32_t MAX_TILES = 1u << 22;   // hard cap of units per descriptor
constexpr uint32_t DEPX_WORDS = 14;        // side words of extra dependency deltas per ring slot
constexpr uint32_t MAX_DEPS = 6 + 4 * DEPX_WORDS;  // explicit dependencies: 6 in the descriptor + 56 beside it
static_assert(MAX_DEPS <= 64, "one dependency per lane");

__host__ __device__ inline uint32_t dt_in(uint32_t flags) { return flags & 15u; }
__host__ __device__ inline uint32_t dt_out(uint32_t flags) { return (flags >> 4) & 15u; }
__host__ __device__ inline uint32_t esz(uint32_t dt) { return dt == GPUOS_F32 ? 4u : 2u; }
__host__ __device__ inline bool dt_ok(uint32_t dt) { return dt == GPUOS_F32 || dt == GPUOS_BF16; }
__host__ __device__ inline uint64_t cdiv(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

// The fields of a descriptor the plan depends on.
struct PlanIn {
    uint32_t kind, flags;
    uint32_t kflags;  // the table entry's flags (EXPR: EXPR_USES_B | n_instr << 8)
    uint64_t size;
    uint32_t dim[4];
    uint64_t lensw[2];  // lens[0..7] as packed 16-bit fields (descriptor bytes 104..120)
    uint32_t pu5;       // param.u[5] (paged caches: table row length MP)
    uint64_t a, b, out, aux0, aux1, aux2;
};

// lens[i] from the two packed words (kept packed: a dynamically indexed
// array would live in private memory on the GPU)
__host__ __device__ inline uint32_t lens_at(const uint64_t* w, uint32_t i) {
    const uint64_t word = i < 4u ? w[0] : w[1];
    return (uint32_t)((word >> (16u * (i & 3u))) & 0xFFFFu);
}

struct Plan {
    uint32_t status;      // GPUOS_ST_OK or GPUOS_ST_BAD_SHAPE
    uint32_t ntiles;
    uint64_t scratch;     // bytes (0 = none); counters occupy the first COUNTER_AREA
};

// A row-op unit covers as many consecutive rows as fit in 16 KiB of input
// (at least one, at most 16): claims are the executor's scarcest resource
// for short rows, so small rows are grouped.
__host__ __device__ inline uint32_t rows_per_unit(uint32_t h, uint32_t dt) {
    const uint64_t rb = (uint64_t)h * esz(dt);
    if (rb == 0 || rb >= 16384u) return 1u;
    const uint64_t g = 16384u / rb;
    return g > 16u ? 16u : (uint32_t)g;
}

// A RoPE unit is one batch row and the heads one wave-wide load of 64 x 16
// bytes covers, when a head's row of D elements divides 1 KiB; else one head.
__host__ __device__ inline uint32_t rope_heads_per_unit(uint32_t D, uint32_t dt) {
    const uint32_t rb = D * esz(dt);
    if (rb == 0 || rb % 16u != 0 || rb > 1024u || (1024u % rb) != 0) return 1u;
    return 1024u / rb;
}

// Keys per SDPA unit: SDPA_KT, halved (down to 64) while the op would give
// fewer than 256 units, as long as no row needs more than 64 splits.  A small
// attention op (one sequence, few heads) is latency-bound: more, shorter
// units finish sooner; a large one keeps long units, whose split merges
// then cost less.
__host__ __device__ inline uint32_t sdpa_keys_per_unit(uint32_t B, uint32_t H, const uint64_t* lensw) {
    uint32_t kt = SDPA_KT;
    while (kt > 64u) {
        const uint32_t h = kt / 2u;
        uint64_t units = 0;
        bool fits = true;
        for (uint32_t i = 0; i < B; ++i) {
            const uint32_t L = lens_at(lensw, i);
            units += (uint64_t)H * ((L + kt - 1u) / kt);
            fits = fits && (L + h - 1u) / h <= 64u;
        }
        if (units >= 256u || !fits) break;
        kt = h;
    }
    return kt;
}

// Paged caches (GPUOS_F_KV_PAGED): `size` carries the batch rows in its low
// 32 bits and the pool's page count in its high 32 bits; pages hold a power
// of two of positions, 64 to 1024, so that a page holds a whole number of an
// attention unit's chunks of keys (32 or 64) and a unit spans at most 16
// pages.
__host__ __device__ inline bool kv_paged(uint32_t flags) { return (flags & GPUOS_F_KV_PAGED) != 0u; }
__host__ __device__ inline uint64_t kv_rows(uint64_t size, uint32_t flags) {
    return kv_paged(flags) ? (size & 0xFFFFFFFFull) : size;
}
__host__ __device__ inline uint64_t kv_pages(uint64_t size) { return size >> 32; }
__host__ __device__ inline bool page_size_ok(uint32_t ps) { return ps >= 64u && ps <= 1024u && (ps & (ps - 1u)) == 0u; }

// Query heads per SDPA unit: under grouped-query attention the query heads
// of a group share their key/value rows, so with D = 128 and groups of a
// multiple of 4 heads a unit takes 4 of them and reads each key/value chunk
// once for all four.
__host__ __device__ inline uint32_t sdpa_heads_per_unit(uint32_t H, uint32_t Hkv, uint32_t D) {
    const uint32_t g = Hkv ? H / Hkv : 1u;
    return (D == 128u && g % 4u == 0u) ? 4u : 1u;
}

// output columns of a MATMUL unit: every unit reads all of x [M, K] beside
// its slice of the weights, so at few rows wider units read x fewer times
__host__ __device__ inline uint32_t mm_cols_per_unit(uint32_t M) { return M <= 32u ? MM_NB_SMALL : MM_NB; }

// a GEMV unit covers 16 lanes x 16 bytes of columns (four rows per load)
__host__ __device__ inline uint32_t gemv_cols_per_block(uint32_t dt) { return 16u * (16u / esz(dt)); }

__host__ __device__ inline Plan make_plan(const PlanIn& d) {
    Plan p{GPUOS_ST_OK, 1u, 0u};
    const uint32_t di = dt_in(d.flags), dout = dt_out(d.flags);
    auto bad = [&]() { p.status = GPUOS_ST_BAD_SHAPE; p.ntiles = 1; p.scratch = 0; return p; };
    if (d.kind != GPUOS_OP_NOP && d.kind != GPUOS_OP_COPY && (!dt_ok(di) || !dt_ok(dout))) return bad();
    switch (d.kind) {
        case GPUOS_OP_NOP:
            return p;
        case GPUOS_OP_ADD:
        case GPUOS_OP_MUL:
        case GPUOS_OP_RELU:
        case GPUOS_OP_GELU: {
            if (di != dout) return bad();
            if (d.size > 0 && (d.a == 0 || d.out == 0)) return bad();
            if ((d.kind == GPUOS_OP_ADD || d.kind == GPUOS_OP_MUL) && d.size > 0 && d.b == 0) return bad();
            uint64_t t = cdiv(d.size, ew_tile_bytes(d.kind, ew_big(d.size, esz(di))) / esz(di));
            if (t > MAX_TILES) return bad();
            p.ntiles = t ? (uint32_t)t : 1u;
            return p;
        }
        case GPUOS_OP_SUM:
        case GPUOS_OP_MAX:
        case GPUOS_OP_MIN:
        case GPUOS_OP_SOFTMAX:
        case GPUOS_OP_LAYERNORM: {
            if (di != dout || d.dim[0] == 0) return bad();
            if (d.size > MAX_TILES) return bad();
            if (d.size > 0 && (d.a == 0 || d.out == 0)) return bad();
            if (d.kind == GPUOS_OP_LAYERNORM && d.size > 0 && (d.aux0 == 0 || d.aux1 == 0)) return bad();
            p.ntiles = d.size ? (uint32_t)cdiv(d.size, rows_per_unit(d.dim[0], di)) : 1u;
            return p;
        }
        case GPUOS_OP_ROPE:
        case GPUOS_OP_KV_APPEND: {
            const bool paged = d.kind == GPUOS_OP_KV_APPEND && kv_paged(d.flags);
            const uint64_t B = paged ? kv_rows(d.size, d.flags) : d.size;
            const uint32_t H = d.dim[0], D = d.dim[1];
            // capacity: positions per row (paged: MP pages of PS positions)
            const uint64_t C = paged ? (uint64_t)d.pu5 * d.dim[2] : d.dim[2];
            if (B == 0 || B > MAX_B || H == 0 || D == 0 || di != dout) return bad();
            if (d.kind == GPUOS_OP_ROPE) {
                // k has dim[3] heads (0: H), at most H
                if ((D & 1u) || D > 256u || d.a == 0 || d.b == 0 || d.dim[3] > H) return bad();
            } else {
                if (C == 0 || d.a == 0 || d.b == 0 || d.aux0 == 0 || d.aux1 == 0) return bad();
                if (paged && (!page_size_ok(d.dim[2]) || kv_pages(d.size) == 0 || d.aux2 == 0)) return bad();
            }
            for (uint32_t i = 0; i < B; ++i) {
                if (lens_at(d.lensw, i) == 0) return bad();
                if (d.kind == GPUOS_OP_KV_APPEND && lens_at(d.lensw, i) > C) return bad();
            }
            if (d.kind == GPUOS_OP_ROPE) {
                const uint64_t t = B * cdiv(H, rope_heads_per_unit(D, di));
                if (t > MAX_TILES) return bad();
                p.ntiles = (uint32_t)t;
            } else {
                p.ntiles = (uint32_t)B;
            }
            return p;
        }
        case GPUOS_OP_SDPA: {
            const bool paged = kv_paged(d.flags);
            const uint64_t B = kv_rows(d.size, d.flags);
            const uint32_t H = d.dim[0], D = d.dim[1];
            const uint64_t C = paged ? (uint64_t)d.pu5 * d.dim[2] : d.dim[2];
            if (B == 0 || B > MAX_B || H == 0 || C == 0 || (D != 64u && D != 128u)) return bad();
            if (d.dim[3] != 0 && H % d.dim[3] != 0) return bad();  // key/value heads divide the query heads
            if (di != GPUOS_BF16) return bad();
            if (d.a == 0 || d.out == 0 || d.aux0 == 0 || d.aux1 == 0) return bad();
            if ((d.flags & GPUOS_F_SDPA_MASK) && d.aux2 == 0) return bad();
            if (paged && (!page_size_ok(d.dim[2]) || kv_pages(d.size) == 0 || d.b == 0)) return bad();
            const uint32_t kt = sdpa_keys_per_unit((uint32_t)B, H, d.lensw);
            uint64_t units = 0;
            bool split = false;
            for (uint32_t i = 0; i < B; ++i) {
                const uint32_t L = lens_at(d.lensw, i);
                if (L == 0 || L > C) return bad();
                uint64_t ns = cdiv(L, kt);
                if (ns > 64) return bad();  // the split merge reads one split per lane
                if (ns > 1) split = true;
                units += ns * H;
            }
            if (units > MAX_TILES || (uint64_t)B * H * 4 > COUNTER_AREA) return bad();
            // a unit covers sdpa_heads_per_unit query heads; partial records
            // and counters stay per head
            p.ntiles = (uint32_t)(units / sdpa_heads_per_unit(H, d.dim[3], D));
            if (split) p.scratch = COUNTER_AREA + units * (uint64_t)(D + 4) * 4u;
            return p;
        }
        case GPUOS_OP_GEMV: {
            const uint32_t K = d.dim[0], N = d.dim[1];
            if (K == 0 || N == 0 || d.a == 0 || d.b == 0 || d.out == 0) return bad();
            const uint64_t ncb = cdiv(N, gemv_cols_per_block(di));
            const uint64_t nks = cdiv(K, GEMV_KC);
            if (ncb * nks > MAX_TILES || ncb * 4 > COUNTER_AREA) return bad();
            p.ntiles = (uint32_t)(ncb * nks);
            if (nks > 1) p.scratch = COUNTER_AREA + nks * (uint64_t)N * 4u;
            return p;
        }
        case GPUOS_OP_MATMUL: {
            const uint64_t M = d.size;
            const uint32_t K = d.dim[0], N = d.dim[1];
            if (di != GPUOS_BF16 || M == 0 || M > MM_MAX_M || K == 0 || N == 0 || K % 32u != 0) return bad();
            if (d.a == 0 || d.b == 0 || d.out == 0) return bad();
            if ((uint64_t)MM_MAX_M * K * 2u >= (1ull << 31)) return bad();  // 32-bit buffer offsets
            if ((uint64_t)mm_cols_per_unit((uint32_t)M) * K * 2u >= (1ull << 31)) return bad();
            const uint64_t ncb = cdiv(N, mm_cols_per_unit((uint32_t)M)), nks = cdiv(K, MM_KC);
            if (ncb * nks > MAX_TILES || ncb * 4 > COUNTER_AREA) return bad();
            if (nks > 1 && nks * M * (uint64_t)N * 4u >= (1ull << 31)) return bad();  // partials in one window
            p.ntiles = (uint32_t)(ncb * nks);
            if (nks > 1) p.scratch = COUNTER_AREA + nks * M * (uint64_t)N * 4u;
            return p;
        }
        case GPUOS_OP_EXPR: {
            if (di != dout) return bad();
            if (d.size > 0 && (d.a == 0 || d.out == 0)) return bad();
            if ((d.kflags & EXPR_USES_B) && d.size > 0 && d.b == 0) return bad();
            uint64_t t = cdiv(d.size, expr_tile_bytes(d.kflags, ew_big(d.size, esz(di))) / esz(di));
            if (t > MAX_TILES) return bad();
            p.ntiles = t ? (uint32_t)t : 1u;
            return p;
        }
        case GPUOS_OP_JIT: {
            if (di != dout) return bad();
            if (d.size > 0 && (d.a == 0 || d.out == 0)) return bad();
            if ((d.kflags & EXPR_USES_B) && d.size > 0 && d.b == 0) return bad();
            uint64_t t = cdiv(d.size, JIT_TILE_BYTES / esz(di));
            if (t > MAX_TILES) return bad();
            p.ntiles = t ? (uint32_t)t : 1u;
            return p;
        }
        case GPUOS_OP_COPY: {
            if (d.size > 0 && (d.a == 0 || d.out == 0)) return bad();
            uint64_t t = cdiv(d.size, COPY_TILE_BYTES);
            if (t > MAX_TILES) return bad();
            p.ntiles = t ? (uint32_t)t : 1u;
            return p;
        }
        default:
            p.status = GPUOS_ST_BAD_OP;
            return p;
    }
}

}  // namespace gpuos
