// Persistent executor for gfx950 (GPUOS digest page, section 3 Q2,
// "Persistent Kernel Executor" and "Ring Buffer Communication Channel").
//
// Launched once; one workgroup per CU; every wave64 is independent.
//  - Wave 0 of workgroup 0 is the fetcher.  It polls the host ring (fine-
//    grained host memory, system-scope loads) 64 slots at a time, reads the
//    committed descriptors over PCIe in one batch, resolves op_id through
//    the dual-slot operator table at the descriptor's table version, splits
//    each descriptor into work units, and publishes them to a unit queue in
//    HBM with a release store of the queue tail.
//  - Every other wave is a worker.  It claims the next unit with one atomic
//    fetch-add, waits until the unit is published, waits for the
//    descriptor's dependencies (done[] counters), runs the op body, and
//    completes: the last unit of a descriptor writes done[slot] (agent
//    scope) and the slot's stamp in host memory (system scope), which
//    releases the ring slot.
// Idle waits back off exponentially with s_sleep.  Every wait loop checks
// the stop flag, so the grid drains when the host asks it to.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "gpuos_internal.h"
#include "gpuos_ops.h"

namespace gpuos {

__device__ __forceinline__ uint64_t ld_agent(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_sys(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void st_agent(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_sys(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ uint64_t rl64(uint64_t v, int l) {
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ void nap(uint32_t n) {
    for (uint32_t i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(1);
}

constexpr uint64_t STOP_DRAIN = 1, STOP_ABORT = 2;
constexpr uint32_t DEP_BACKOFF_MAX = 2;
#ifndef GPUOS_SHORT_FIRST
#define GPUOS_SHORT_FIRST 1
#endif
constexpr uint32_t PASS_MAX = 4;
#ifndef GPUOS_NEAR_UNITS
#define GPUOS_NEAR_UNITS 64
#endif
constexpr uint64_t NEAR_UNITS = GPUOS_NEAR_UNITS;
#ifndef GPUOS_FETCH_BACKOFF_MAX
#define GPUOS_FETCH_BACKOFF_MAX 8
#endif
constexpr uint32_t FETCH_BACKOFF_MAX = GPUOS_FETCH_BACKOFF_MAX;
constexpr uint64_t NO_SCRATCH = ~0ull;

// ------------------------------------------------------------------ worker
// A worker wave holds up to SLOTS claimed units and runs whichever of them
// has its dependencies satisfied, so a unit waiting on a long chain does not
// hold back a ready unit claimed after it.  Among ready units, one of a
// short body (anything but attention, vector-matrix products and copies)
// goes first, then the oldest; a ready long unit is passed over at most
// PASS_MAX times in a row.  Each claim shard hands out its units in queue
// order, so the executor always progresses: if the oldest unfinished unit
// is unclaimed, every unit its shard has handed out is older, hence
// finished, and a wave of that shard (every shard has one, and all waves
// are resident) claims it once a slot is free; if it is claimed, its holder
// finds it ready and runs it after at most PASS_MAX other units.  No wave
// waits on one unit alone.
// SLOTS is 1 or 2 (gpuos_init_params.units_per_wave): with one, a wave
// claims its next unit only after running the current one; two let a ready
// unit overtake one that waits, at the price of holding two claims.
constexpr uint32_t SL_FREE = 0, SL_CLAIMED = 1, SL_WAIT = 2;

template <uint32_t SLOTS, class T>
__device__ __forceinline__ T pick(const T* v, uint32_t r) {
    T x = v[0];
#pragma unroll
    for (uint32_t k = 1; k < SLOTS; ++k) x = r == k ? v[k] : x;
    return x;
}

// Bodies injected with gpuos_register_jit are called through this pointer
// type by the executor build that allows it (JIT = true).
typedef void (*jit_body_fn)(const uint8_t* a, const uint8_t* b, uint8_t* out, uint64_t n, uint32_t tile,
                            uint32_t lane);

// For a call through a pointer the compiler gives the calling kernel the
// registers of the largest non-kernel function in this module, which the
// callee may then use.  This function is never called; its clobbers fix
// that budget at GPUOS_JIT_MAX_VGPRS VGPRs (v0..v95), GPUOS_JIT_MAX_AGPRS
// AGPRs (a0..a31) and SGPRs up to s95 (GPUOS_JIT_MAX_SGPRS with the special
// registers), and gpuos_register_jit refuses injected code that reports
// more.
extern "C" __device__ __attribute__((noinline, used)) void gpuos_jit_budget(const uint8_t*, const uint8_t*, uint8_t*,
                                                                            uint64_t, uint32_t, uint32_t) {
    asm volatile("" ::: "v95", "a31", "s95");
}
static_assert(GPUOS_JIT_MAX_VGPRS == 96u && GPUOS_JIT_MAX_AGPRS == 32u && GPUOS_JIT_MAX_SGPRS == 102u,
              "budget clobbers above");
__device__ jit_body_fn gpuos_jit_budget_addr = gpuos_jit_budget;

template <uint32_t SLOTS, bool JIT>
__device__ __forceinline__ void worker_loop(const ExecArgs& A, uint32_t lane) {
    uint64_t jit_seen = 0;  // the injected body this wave called last
    DevCtl* C = A.dctl;
    uint64_t n_units = 0, n_depw = 0;
    const uint64_t N = (uint64_t)A.mask + 1;
    uint32_t state[SLOTS];
    uint64_t su[SLOTS], sseq[SLOTS], srlo[SLOTS], st0[SLOTS], tclaim[SLOTS];
    uint64_t sw[SLOTS];   // per lane: mirror words in lanes 0..15, meta words in 16..23
    uint32_t sdl[SLOTS];  // per lane: dependency delta (lanes 0..13), 0 = none
    uint32_t stile[SLOTS];
    uint32_t spass[SLOTS];  // times a ready unit was passed over in a row
    bool sdeps[SLOTS], swaited[SLOTS];
#pragma unroll
    for (uint32_t k = 0; k < SLOTS; ++k) {
        state[k] = SL_FREE;
        su[k] = sseq[k] = srlo[k] = st0[k] = tclaim[k] = 0;
        sw[k] = 0;
        sdl[k] = 0;
        stile[k] = 0;
        spass[k] = 0;
        sdeps[k] = swaited[k] = false;
    }
    bool stop_seen = false;
    uint32_t bo = 1;
    // this wave's claim shard: workgroups take the shards in turn, so that
    // (with workgroups placed on the XCDs in turn) each XCD claims from
    // counters of its own
    const uint32_t S = A.shards;
    const uint32_t shard = wg_shard(blockIdx.x, S);
    uint64_t* const claim_ctr = &C->claim[shard].next;
    for (;;) {
        // One dependency load per waiting slot and the queue tail, issued
        // together.  Claims come after the run below, so their atomic round
        // trip never delays a ready unit.
        uint64_t dv[SLOTS];
#pragma unroll
        for (uint32_t k = 0; k < SLOTS; ++k) {
            const bool need = state[k] == SL_WAIT && sdl[k] != 0;
            const uint64_t d = need ? sseq[k] - sdl[k] : 0;
            dv[k] = ld_agent(&A.done[(d & A.mask) * DONE_STRIDE]);
        }
        const uint64_t tail = ld_agent(&C->q_tail);
        const uint64_t now = wall_clock64();
        uint32_t r = SLOTS, rstatus = GPUOS_ST_OK;
        uint64_t rseq = ~0ull;
        bool rdy[SLOTS];
#pragma unroll
        for (uint32_t k = 0; k < SLOTS; ++k) {
            rdy[k] = false;
            if (state[k] != SL_WAIT) continue;
            bool ready = true;
            if (sdeps[k]) {
                const uint64_t d = sseq[k] - sdl[k];
                const bool ok = sdl[k] == 0 || dv[k] >= d;
                if (srlo[k] < sseq[k]) {
                    // range dependency: advance over up to 64 completed seqs per check
                    const uint64_t x = srlo[k] + lane;
                    const bool okr = x >= sseq[k] || ld_agent(&A.done[(x & A.mask) * DONE_STRIDE]) >= x;
                    const uint64_t bal = __ballot(okr);
                    srlo[k] += bal == ~0ull ? 64u : (uint64_t)(__ffsll((long long)~bal) - 1);
                }
                ready = __all(ok) && srlo[k] >= sseq[k];
            }
            uint32_t stat = GPUOS_ST_OK;
            if (!ready) {
                if (!swaited[k]) { swaited[k] = true; st0[k] = now; ++n_depw; }
                if (now - st0[k] > A.spin_limit_ticks) { ready = true; stat = GPUOS_ST_SPIN; }
            }
            // among ready units, those of short bodies go first, then the
            // oldest: a RoPE or KV append held beside an attention unit
            // would otherwise wait out that unit's whole body, and the
            // attention units of its layer, held by other waves, with it
            uint64_t key = sseq[k];
#if GPUOS_SHORT_FIRST
            if constexpr (SLOTS > 1) {
                const uint32_t kind = (uint32_t)rl64(sw[k], 16);
                const bool lng = kind == GPUOS_OP_SDPA || kind == GPUOS_OP_GEMV || kind == GPUOS_OP_COPY;
                if (lng && spass[k] < PASS_MAX) key |= 1ull << 63;
            }
#endif
            if (ready && key < rseq) { r = k; rseq = key; rstatus = stat; }
            rdy[k] = ready;
        }
#pragma unroll
        for (uint32_t k = 0; k < SLOTS; ++k)  // ready units passed over this time
            spass[k] = k == r ? 0u : spass[k] + ((r < SLOTS && rdy[k]) ? 1u : 0u);
        if (r < SLOTS) {
            const uint64_t w = pick<SLOTS>(sw, r);
            const uint64_t seq = pick<SLOTS>(sseq, r), u = pick<SLOTS>(su, r), t_claim = pick<SLOTS>(tclaim, r);
            const uint32_t tile = pick<SLOTS>(stile, r);
            const uint64_t slot = seq & A.mask;
            Unit U;
            const uint64_t w0 = rl64(w, 0), w6 = rl64(w, 6), w7 = rl64(w, 7);
            const uint64_t w13 = rl64(w, 13), w14 = rl64(w, 14), w15 = rl64(w, 15);
            const uint64_t m0 = rl64(w, 16), m1 = rl64(w, 17), m3 = rl64(w, 19), m5 = rl64(w, 21);
            U.seq = seq;
            U.flags = (uint32_t)(w0 >> 32);
            U.tile = tile;
            U.a = rl64(w, 2); U.b = rl64(w, 3); U.out = rl64(w, 4); U.size = rl64(w, 5);
            U.dim[0] = (uint32_t)w6; U.dim[1] = (uint32_t)(w6 >> 32);
            U.dim[2] = (uint32_t)w7; U.dim[3] = (uint32_t)(w7 >> 32);
            U.aux0 = rl64(w, 8); U.aux1 = rl64(w, 9); U.aux2 = rl64(w, 10);
            U.pf[0] = __uint_as_float((uint32_t)w13); U.pf[1] = __uint_as_float((uint32_t)(w13 >> 32));
            U.pf[2] = __uint_as_float((uint32_t)w14); U.pf[3] = __uint_as_float((uint32_t)(w14 >> 32));
            U.pf[4] = __uint_as_float((uint32_t)w15); U.pf[5] = __uint_as_float((uint32_t)(w15 >> 32));
            U.lensw[0] = w13;
            U.lensw[1] = w14;
            U.kind = (uint32_t)m0;
            uint32_t status = (uint32_t)(m0 >> 32);
            U.ntiles = (uint32_t)m1;
            U.p0 = __uint_as_float((uint32_t)(m1 >> 32));
            U.scratch = m3 == NO_SCRATCH ? nullptr : A.scratch + (m3 % A.scratch_bytes);
            U.prog = m5;
            if (rstatus != GPUOS_ST_OK) {
                status = rstatus;
                if (lane == 0) {
                    __hip_atomic_store(&C->error, (uint64_t)rstatus, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    st_sys(&A.hctl->dev_error, rstatus);
                }
            }
            asm volatile("" ::: "memory");  // op loads are device-coherent: no invalidation
            const uint64_t t_ready = A.trace ? wall_clock64() : 0;
            // The lane id goes through an empty asm so that the compiler
            // computes lane-derived addresses inside each body instead of
            // hoisting hundreds of them out of the persistent loop, where they
            // would hold registers for the kernel's whole life.
            uint32_t ln = lane;
            asm volatile("" : "+v"(ln));
            if constexpr (JIT) {
                if (status == GPUOS_ST_OK && U.kind == GPUOS_OP_JIT) {
                    // new code: an acquire first, so that nothing this XCD's
                    // caches hold from before the code was loaded is used
                    if (U.prog != jit_seen) {
                        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
                        jit_seen = U.prog;
                    }
                    ((jit_body_fn)U.prog)((const uint8_t*)U.a, (const uint8_t*)U.b, (uint8_t*)U.out, U.size, U.tile, ln);
                } else if (status == GPUOS_ST_OK && U.kind != KIND_BAD) {
                    run_unit(U, ln);
                }
            } else {
                if (status == GPUOS_ST_OK && U.kind != KIND_BAD) run_unit(U, ln);
            }
            ++n_units;
            const uint64_t t_body = A.trace ? wall_clock64() : 0;
            // completion: publish this unit's (write-through) outputs, count
            // it; the last unit of the descriptor marks it done and releases
            // the slot.  Every unit's outputs were acknowledged before its
            // count, so once done[] is visible all of them are.
            stores_done();
            bool last = true;
            if (U.ntiles > 1) {
                uint32_t prev = 0;
                if (lane == 0)
                    prev = __hip_atomic_fetch_add(&A.tiles_done[slot], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                prev = (uint32_t)__builtin_amdgcn_readlane((int)prev, 0);
                last = prev == U.ntiles - 1;
            }
            if (last) {
                if (lane == 0) {
                    st_agent(&A.done[slot * DONE_STRIDE], seq);
                    if (status != GPUOS_ST_OK) {
                        __hip_atomic_store(&A.status[slot], status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                        stores_done();  // the status reaches the host before the stamp
                    }
                    st_sys(&A.stamp[slot], seq + N);
                }
            }
            if (A.trace && lane == 0) {
                uint32_t xcc = 0;
                asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(xcc));
                gpuos_trace_rec* tr = &A.trace[u & (A.trace_cap - 1)];
                tr->seq = seq;
                tr->tile = tile;
                tr->hw = (xcc << 16) | (uint32_t)blockIdx.x;
                tr->t_claim = t_claim;
                tr->t_ready = t_ready;
                tr->t_body = t_body;
                tr->t_done = wall_clock64();
                tr->unit = u;
            }
#pragma unroll
            for (uint32_t k = 0; k < SLOTS; ++k)
                if (k == r) state[k] = SL_FREE;
            bo = 1;
        }
        // claim units for the free slots (queue order), then read the units
        // published by the tail seen above: their entry, mirror and meta
        // were made device-visible before that tail, so device-coherent
        // loads issued after it need no cache invalidation.  Claims continue
        // after the stop: units published before it must all run, and a
        // ticket past the final tail is simply never used.
#pragma unroll
        for (uint32_t k = 0; k < SLOTS; ++k) {
            if (state[k] != SL_FREE) continue;
            uint64_t c = 0;
            if (lane == 0) c = __hip_atomic_fetch_add(claim_ctr, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            su[k] = ticket_unit(rl64(c, 0), S, shard);
            state[k] = SL_CLAIMED;
        }
        asm volatile("" ::: "memory");
        bool any_wait = false, fresh = false;
#pragma unroll
        for (uint32_t k = 0; k < SLOTS; ++k) {
            if (state[k] == SL_CLAIMED && tail > su[k]) {
                const uint64_t ent = ld_agent(&A.queue[su[k] & A.qmask]);
                const uint64_t seq = entry_seq(ent);
                const uint64_t slot = seq & A.mask;
                uint64_t w = 0;
                if (lane < 16) w = ld_agent(&((const uint64_t*)&A.mirror[slot])[lane]);
                else if (lane < 24) w = ld_agent(&((const uint64_t*)&A.meta[slot])[lane - 16]);
                const uint64_t w11 = rl64(w, 11), w12 = rl64(w, 12);
                // dependencies: one explicit delta per lane (6 in the
                // descriptor, the rest in the side words copied to HBM when
                // the sixth is in use) and a contiguous range
                uint64_t xw = 0;
                if (((w12 >> 16) & 0xFFFFu) != 0 && lane >= 6 && lane < MAX_DEPS)
                    xw = ld_agent(&A.depd[slot * DEPX_WORDS + (lane - 6) / 4]);
                sdl[k] = lane < 4 ? (uint32_t)((w11 >> (16 * lane)) & 0xFFFFu)
                       : lane < 6 ? (uint32_t)((w12 >> (16 * (lane - 4))) & 0xFFFFu)
                       : lane < MAX_DEPS ? (uint32_t)((xw >> (16 * ((lane - 6) & 3u))) & 0xFFFFu) : 0u;
                srlo[k] = seq - ((w12 >> 32) & 0xFFFFu);
                sdeps[k] = w11 != 0 || (w12 & 0xFFFFFFFFFFFFull) != 0;
                swaited[k] = false;
                sw[k] = w;
                sseq[k] = seq;
                stile[k] = entry_tile(ent);
                tclaim[k] = A.trace ? wall_clock64() : 0;
                state[k] = SL_WAIT;
                fresh = true;
            }
            any_wait = any_wait || state[k] == SL_WAIT;
        }
        if (r < SLOTS || fresh) continue;  // something ran or was just published: no sleep
        // nothing ready.  Once the fetcher has stopped, the tail read above
        // (after the stop flag was seen) is final: every slot not waiting
        // holds a ticket beyond it, which will never be published, and the
        // wave leaves when it holds no published unit.
        if (stop_seen && !any_wait) break;
        const uint64_t stp = ld_agent(&C->stop);
        if (stp == STOP_ABORT) break;
        if (stp) { stop_seen = true; continue; }
        // dependency waits back off to at most DEP_BACKOFF_MAX x 64 clocks
        // (the awaited op is in flight).  A wave waiting for publication
        // whose ticket is among the next NEAR_UNITS units to be published
        // does the same (its unit is the next work to arrive); the others
        // back off up to backoff_max.
        bool near = false;
#pragma unroll
        for (uint32_t k = 0; k < SLOTS; ++k)
            near = near || (state[k] == SL_CLAIMED && su[k] - tail < NEAR_UNITS);
        const uint32_t cap = any_wait || near ? DEP_BACKOFF_MAX : A.backoff_max;
        nap(bo);
        bo = bo * 2 < cap ? bo * 2 : cap;
    }
    if (lane == 0) {
        __hip_atomic_fetch_add(&C->stat_units, n_units, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(&C->stat_dep_waits, n_depw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ----------------------------------------------------------------- fetcher
// OR over the wave (DPP within 16-lane groups, then the four groups)
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, DPP_XOR1, 0xF, 0xF, false);
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, DPP_XOR2, 0xF, 0xF, false);
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, DPP_HALF_MIRROR, 0xF, 0xF, false);
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, DPP_MIRROR, 0xF, 0xF, false);
    return (uint32_t)(__builtin_amdgcn_readlane((int)v, 0) | __builtin_amdgcn_readlane((int)v, 16) |
                      __builtin_amdgcn_readlane((int)v, 32) | __builtin_amdgcn_readlane((int)v, 48));
}

__device__ __forceinline__ void fetcher_loop(const ExecArgs& A, uint32_t lane, uint64_t* lds) {
    DevCtl* C = A.dctl;
    const uint64_t mask = A.mask;
    const uint64_t Q = (uint64_t)A.qmask + 1;
    const uint64_t S = A.scratch_bytes;
    const uint64_t* ringw = (const uint64_t*)A.ring;
    uint64_t* mirw = (uint64_t*)A.mirror;
    uint64_t f = A.start_seq, u_next = 0, sv_next = 0, cw = A.start_seq;
    uint32_t cur_ver = 0xFFFFFFFFu, bo = 1;
    uint64_t batches = 0, fetched = 0;
    uint64_t stop_code = STOP_DRAIN;
    // capacity watermarks (unit queue, scratch) as of the last look at
    // done[]: older than the true ones, hence conservative
    uint64_t cw_units = 0, cw_scr = 0;
    // the fetcher's idle polls go to host memory and cost the device's
    // memory system nothing, so its backoff stops early: a descriptor
    // committed to an idle ring is seen sooner
    const uint32_t fcap = A.backoff_max < FETCH_BACKOFF_MAX ? A.backoff_max : FETCH_BACKOFF_MAX;
    // idle exit: the heartbeat last seen, and when it (or work) last changed
    uint64_t hb_seen = 0, hb_t = wall_clock64();
    bool worked = false;
    // whether the last batch held a descriptor with extra-dependency side
    // words: then this batch's side words are read with its bodies
    bool xpre = false;
    for (;;) {
        // the stamps and the control words in one round trip over PCIe
        const uint64_t sl = f + lane;
        const uint64_t st = ld_sys(&A.stamp[sl & mask]);
        const uint64_t abt = ld_sys(&A.hctl->abort);
        const uint64_t stp = ld_sys(&A.hctl->stop);
        const uint64_t hb = A.idle_exit_ticks ? ld_sys(&A.hctl->heartbeat) : 0;
        const uint64_t rb = __ballot(st == sl + 1);
        uint32_t count = rb == ~0ull ? 64u : (uint32_t)(__ffsll((long long)~rb) - 1);
        if (count == 0) {
            if (abt) { stop_code = STOP_ABORT; break; }
            if (stp) {
                // the host commits before it sets stop: look once more
                if (ld_sys(&A.stamp[f & mask]) == f + 1) continue;
                break;
            }
            if (A.idle_exit_ticks) {
                const uint64_t now = wall_clock64();
                if (hb != hb_seen || worked) {
                    hb_seen = hb;
                    hb_t = now;
                    worked = false;
                } else if (now - hb_t > A.idle_exit_ticks) {
                    // no work and no call for the whole interval: look once
                    // more, then leave (the host relaunches from fetch_end)
                    if (ld_sys(&A.stamp[f & mask]) == f + 1) continue;
                    if (lane == 0) st_sys(&A.hctl->idle_exit, 1ull);
                    break;
                }
            }
            nap(bo);
            bo = bo * 2 < fcap ? bo * 2 : fcap;
            continue;
        }
        bo = 1;
        worked = true;
        // read the committed bodies (count x 16 words) in one go
        const uint32_t nw = count * 16u;
        uint64_t v[16];
#pragma unroll
        for (uint32_t k = 0; k < 16; ++k) {
            const uint32_t wi = lane + 64u * k;
            if (wi < nw) v[k] = ld_sys(&ringw[((f + (wi >> 4)) & mask) * 16u + (wi & 15u)]);
        }
        // In a stream of many-dependency descriptors the side words of the
        // whole batch come in the same round trip over PCIe as the bodies
        // (a few KB) instead of a second round trip after the bodies are
        // parsed; the host writes them before the stamp.  Word wi of the
        // batch goes to lane wi % 64, xv[wi / 64].
        const uint32_t nx = xpre ? count * DEPX_WORDS : 0u;
        uint64_t xv[DEPX_WORDS];
#pragma unroll
        for (uint32_t k = 0; k < DEPX_WORDS; ++k) {
            const uint32_t wi = lane + 64u * k;
            xv[k] = wi < nx ? ld_sys(&A.depx[((f + wi / DEPX_WORDS) & mask) * DEPX_WORDS + wi % DEPX_WORDS]) : 0ull;
        }
#pragma unroll
        for (uint32_t k = 0; k < 16; ++k) {
            const uint32_t wi = lane + 64u * k;
            if (wi < nw) lds[wi] = v[k];
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        __builtin_amdgcn_wave_barrier();
        // lane i parses descriptor i
        const bool act = lane < count;
        const uint64_t* dw = lds + (act ? lane : 0) * 16u;
        const uint64_t d0 = dw[0], d12 = dw[12];
        // a descriptor with more than six dependencies keeps the rest in
        // DEPX_WORDS side words of the host array: copy them to HBM for the
        // workers (the slot's previous descriptor has completed, so nobody
        // reads its copy any more)
        // (read on demand when they were not read with the bodies; copied to
        // HBM with the batch's other stores, after every load of the batch:
        // loads and stores retire in order, so a load behind these stores
        // would wait for their acknowledgements)
        const uint64_t xneed = __ballot(act && ((d12 >> 16) & 0xFFFFu) != 0);
        if (!xpre && act && ((xneed >> lane) & 1ull)) {
            const uint64_t sl = (f + lane) & mask;
#pragma unroll
            for (uint32_t k = 0; k < DEPX_WORDS; ++k) xv[k] = ld_sys(&A.depx[sl * DEPX_WORDS + k]);
        }
        const uint32_t op_id = (uint32_t)d0;
        const uint32_t ver = (uint32_t)(d12 >> 48);
        const uint32_t maxver = (uint32_t)__shfl((int)ver, (int)count - 1, 64);
        if (maxver != cur_ver) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");  // the host rewrote a table slot
            cur_ver = maxver;
        }
        PlanIn pin;
        pin.flags = (uint32_t)(d0 >> 32);
        pin.size = dw[5];
        pin.dim[0] = (uint32_t)dw[6]; pin.dim[1] = (uint32_t)(dw[6] >> 32);
        pin.dim[2] = (uint32_t)dw[7]; pin.dim[3] = (uint32_t)(dw[7] >> 32);
        pin.a = dw[2]; pin.b = dw[3]; pin.out = dw[4]; pin.aux0 = dw[8]; pin.aux1 = dw[9]; pin.aux2 = dw[10];
        pin.lensw[0] = dw[13];
        pin.lensw[1] = dw[14];
        pin.pu5 = (uint32_t)(dw[15] >> 32);
        uint32_t kind = KIND_BAD;
        float p0 = 0.0f;
        uint64_t prog = 0;
        pin.kflags = 0;
        if (op_id < GPUOS_MAX_OPS) {
            const TableEntry* te = &A.table[(ver & 1u) * GPUOS_MAX_OPS + op_id];
            kind = te->kind;
            p0 = te->p0;
            pin.kflags = te->flags;
            // an injected body has one entry per operand type
            prog = kind == GPUOS_OP_JIT && dt_in(pin.flags) == GPUOS_BF16 ? te->reserved : te->fn;
        }
        Plan pl;
        if (kind < GPUOS_KIND_COUNT) {
            pin.kind = kind;
            pl = make_plan(pin);
        } else {
            pl.status = GPUOS_ST_BAD_OP;
            pl.ntiles = 1;
            pl.scratch = 0;
        }
        if (pl.status != GPUOS_ST_OK) { kind = KIND_BAD; pl.ntiles = 1; pl.scratch = 0; }
        uint32_t nt = act ? max(pl.ntiles, 1u) : 0u;  // every plan has a unit
        // inclusive prefix of units over lanes
        uint64_t inc = nt;
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
            const uint64_t o = __shfl_up(inc, (unsigned)m, 64);
            if ((int)lane >= m) inc += o;
        }
        // scratch allocation in lane order (few descriptors need any); my_mark
        // is the watermark before descriptor i, my_end the one after it
        const uint64_t need = act ? ((pl.scratch + 255u) & ~255ull) : 0ull;
        uint64_t my_sv = NO_SCRATCH, my_mark = sv_next, sv = sv_next;
        uint64_t nm = __ballot(need > 0);
        while (nm) {
            const int j = __ffsll((long long)nm) - 1;
            nm &= nm - 1;
            const uint64_t nj = rl64(need, j);
            const uint64_t phys = sv % S;
            if (phys + nj > S) sv += S - phys;  // an allocation never wraps
            if ((int)lane == j) my_sv = sv;
            sv += nj;
            if ((int)lane > j) my_mark = sv;
        }
        const uint64_t sv_end_i = my_sv != NO_SCRATCH ? my_sv + need : my_mark;
        // capacity: units and scratch still held by incomplete descriptors.
        // The watermarks of the last look usually leave room for the whole
        // batch; done[] is read again only when they do not.
        uint32_t fit;
        for (bool fresh = false;; fresh = true) {
            if (fresh) {
                // advance the completion watermark cw
                for (;;) {
                    if (cw >= f) break;
                    const uint64_t x = cw + lane;
                    const bool ok = x >= f || ld_agent(&A.done[(x & mask) * DONE_STRIDE]) >= x;
                    const uint64_t bal = __ballot(ok);
                    if (bal == ~0ull) { cw = cw + 64 < f ? cw + 64 : f; continue; }
                    cw += (uint64_t)(__ffsll((long long)~bal) - 1);
                    break;
                }
                cw_units = cw < f ? A.meta[cw & mask].ubegin : u_next;
                cw_scr = cw < f ? A.meta[cw & mask].scratch_mark : sv_next;
            }
            const bool ok = !act || (units_fit(u_next + inc, cw_units, Q) && scratch_fits(sv_end_i, cw_scr, S));
            const uint64_t fb = __ballot(ok);
            fit = fb == ~0ull ? 64u : (uint32_t)(__ffsll((long long)~fb) - 1);
            if (fit > count) fit = count;
            if (fit == count || (fresh && fit > 0)) break;
            if (!fresh) continue;
            if (ld_sys(&A.hctl->abort)) { stop_code = STOP_ABORT; break; }
            nap(A.backoff_max);
        }
        if (fit == 0) break;  // abort while waiting for space
        count = fit;
        const bool keep = lane < count;
        const uint64_t T = rl64(inc, (int)count - 1);
        const uint64_t ubegin = u_next + inc - nt;
        // extra-dependency side words (batch layout when read with the
        // bodies, else lane i holds descriptor i's)
        if (xpre) {
#pragma unroll
            for (uint32_t k = 0; k < DEPX_WORDS; ++k) {
                const uint32_t wi = lane + 64u * k;
                if (wi < nx && ((xneed >> (wi / DEPX_WORDS)) & 1ull))
                    wst64(&A.depd[((f + wi / DEPX_WORDS) & mask) * DEPX_WORDS + wi % DEPX_WORDS], xv[k]);
            }
        } else if (act && ((xneed >> lane) & 1ull)) {
            const uint64_t sl = (f + lane) & mask;
#pragma unroll
            for (uint32_t k = 0; k < DEPX_WORDS; ++k) wst64(&A.depd[sl * DEPX_WORDS + k], xv[k]);
        }
        xpre = xneed != 0;
        // mirror bodies, meta, per-slot unit counters
#pragma unroll
        for (uint32_t k = 0; k < 16; ++k) {
            const uint32_t wi = lane + 64u * k;
            if (wi < count * 16u) wst64(&mirw[((f + (wi >> 4)) & mask) * 16u + (wi & 15u)], lds[wi]);
        }
        if (keep) {
            const uint64_t slot = (f + lane) & mask;
            uint64_t* mm = (uint64_t*)&A.meta[slot];  // MirrorMeta as 64-bit words
            wst64(mm + 0, (uint64_t)kind | ((uint64_t)pl.status << 32));
            wst64(mm + 1, (uint64_t)nt | ((uint64_t)__float_as_uint(p0) << 32));
            wst64(mm + 2, ubegin);
            wst64(mm + 3, my_sv);
            wst64(mm + 4, my_mark);
            wst64(mm + 5, prog);
            wst32(&A.tiles_done[slot], 0u);
        }
        // zero the group counters of descriptors that use scratch
        uint64_t zm = __ballot(keep && my_sv != NO_SCRATCH);
        while (zm) {
            const int j = __ffsll((long long)zm) - 1;
            zm &= zm - 1;
            const uint64_t svj = rl64(my_sv, j);
            const WBuf zb = wbuf(A.scratch + (svj % S));
#pragma unroll
            for (uint32_t k = 0; k < COUNTER_AREA / 16u / 64u; ++k)
                wst16(zb, (lane + 64u * k) * 16u, u32x4{0, 0, 0, 0});
        }
        // one queue entry per unit: its descriptor and index, 64 per store.
        // Descriptor j's units start at its exclusive prefix ustart; in each
        // window of 64 units the starts that fall inside form a mask M (OR
        // over the descriptor lanes); a unit's descriptor is the number of
        // starts at or below it (plus those before the window) minus one,
        // and its index counts from the highest such start.
        const uint64_t ustart = inc - nt;
        uint32_t jbase = 0;    // descriptors started before the window
        uint64_t cstart = 0;   // the start of the last of them
        for (uint64_t w0 = 0; w0 < T; w0 += 64u) {
            const uint64_t rel = ustart - w0;
            const bool here = nt > 0u && ustart >= w0 && rel < 64u;
            const uint32_t mlo = wave_or(here && rel < 32u ? 1u << rel : 0u);
            const uint32_t mhi = wave_or(here && rel >= 32u ? 1u << (rel - 32u) : 0u);
            const uint64_t M = (uint64_t)mlo | ((uint64_t)mhi << 32);
            const uint64_t below = M & (lane == 63u ? ~0ull : (2ull << lane) - 1ull);
            const uint32_t c = (uint32_t)__popcll(below);
            const uint32_t j = jbase + c - 1u;  // c = 0: the descriptor begun before the window
            const uint64_t st = c ? w0 + 63u - (uint64_t)__clzll(below) : cstart;
            const uint64_t wi = w0 + lane;
            if (wi < T) wst64(&A.queue[(u_next + wi) & A.qmask], queue_entry(f + j, wi - st));
            jbase += (uint32_t)__popcll(M);
            if (M) cstart = w0 + 63u - (uint64_t)__clzll(M);
            // a large batch is published in prefixes, so that workers start
            // on its first units while the rest of its entries are written
            // (the mirror, meta and counters written above are covered by
            // the first acknowledgement)
            if (((w0 + 64u) & (PUBLISH_STEP - 1u)) == 0 && w0 + 64u < T) {
                stores_done();
                if (lane == 0) st_agent(&C->q_tail, u_next + w0 + 64u);
            }
        }
        stores_done();  // entries, mirror, meta and counters are written through
        if (lane == 0) st_agent(&C->q_tail, u_next + T);
        f += count;
        u_next += T;
        sv_next = rl64(sv_end_i, (int)count - 1);
        ++batches;
        fetched += count;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (lane == 0) {
        st_sys(&A.hctl->fetch_end, f);
        st_agent(&C->stop, stop_code);
        __hip_atomic_fetch_add(&C->stat_batches, batches, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(&C->stat_fetched, fetched, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <uint32_t SLOTS, bool JIT = false>
__device__ __forceinline__ void executor_body(const ExecArgs& A, uint64_t* lds) {
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    // The host learns that the executor has finished from the launch's
    // completion event, which also makes every write of the kernel visible
    // to it: a wave leaves without a fence or a word in host memory (a
    // system-scope release and atomic per wave made an empty launch of 1,024
    // waves take about a millisecond).
    if (blockIdx.x == 0 && wave == 0) fetcher_loop(A, lane, lds);
    else worker_loop<SLOTS, JIT>(A, lane);
}

// one unit per worker wave
extern "C" __global__ void __launch_bounds__(256) gpuos_executor(ExecArgs A) {
    __shared__ uint64_t lds[64 * 16];
    executor_body<1>(A, lds);
}

// two units per worker wave
extern "C" __global__ void __launch_bounds__(256) gpuos_executor_s2(ExecArgs A) {
    __shared__ uint64_t lds[64 * 16];
    executor_body<2>(A, lds);
}

// one unit per worker wave, and calls into bodies injected with
// gpuos_register_jit (a stack in scratch memory for those calls)
extern "C" __global__ void __launch_bounds__(256) gpuos_executor_jit(ExecArgs A) {
    __shared__ uint64_t lds[64 * 16];
    executor_body<1, true>(A, lds);
}

// ------------------------------------------------------------ eager kernels
// One launch per descriptor; wave w of block x runs tile 4x + w.
extern "C" __global__ void __launch_bounds__(256) gpuos_eager_kernel(gpuos_desc d, uint32_t kind, uint32_t ntiles,
                                                                      uint8_t* scratch) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t tile = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (tile >= ntiles) return;
    Unit U;
    U.seq = 0;
    U.kind = kind;
    U.flags = d.flags;
    U.tile = tile;
    U.ntiles = ntiles;
    U.a = d.input_a; U.b = d.input_b; U.out = d.output; U.size = d.size;
    for (int i = 0; i < 4; ++i) U.dim[i] = d.dim[i];
    U.aux0 = d.aux[0]; U.aux1 = d.aux[1]; U.aux2 = d.aux[2];
    for (int i = 0; i < 6; ++i) U.pf[i] = d.param.f[i];
    U.lensw[0] = (uint64_t)d.param.u[0] | ((uint64_t)d.param.u[1] << 32);
    U.lensw[1] = (uint64_t)d.param.u[2] | ((uint64_t)d.param.u[3] << 32);
    U.p0 = 0.0f;
    U.scratch = scratch;
    U.prog = 0;
    run_unit(U, lane);
}

extern "C" __global__ void gpuos_null_kernel() {}

// ------------------------------------------------ eager launches, no allocation
// gpuos_eager_submit_static runs the eager launches with the split-op
// partials and counters in this file-scope array instead of a caller
// workspace (for callers that cannot allocate).  Host code never uses the
// array's name as an address: it takes each device's copy through
// hipGetSymbolAddress once, with that device current, and passes that.
namespace noalloc {
static __device__ __align__(256) uint8_t scratch[GPUOS_EAGER_STATIC_SCRATCH_BYTES];
constexpr int MAX_DEVICES = 64;
std::mutex mu;
uint8_t* dev_ptr[MAX_DEVICES];  // device address of `scratch` per device, once taken
}  // namespace noalloc

// zero n 16-byte words (the split counters, which must start at zero)
extern "C" __global__ void __launch_bounds__(256) gpuos_fill_zero_kernel(uint8_t* p, uint32_t n16) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n16) wst16(wbuf(p, n16 * 16u), i * 16u, u32x4{0, 0, 0, 0});
}

// device address of the static scratch on the current device (taken once per device)
hipError_t static_scratch(uint8_t** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= noalloc::MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(noalloc::mu);
    if (!noalloc::dev_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc::scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        noalloc::dev_ptr[dev] = (uint8_t*)p;
    }
    *out = noalloc::dev_ptr[dev];
    return hipSuccess;
}

hipError_t launch_fill_zero(uint8_t* p, uint32_t bytes, hipStream_t s) {
    const uint32_t n16 = bytes / 16u;
    hipLaunchKernelGGL(gpuos_fill_zero_kernel, dim3((n16 + 255u) / 256u), dim3(256), 0, s, p, n16);
    return hipGetLastError();
}

// ------------------------------------------------------------- HBM probe
// Achievable bandwidth with the memory instructions the op bodies use
// (device-scope 16-byte buffer loads, write-through stores): a grid-stride
// read (COPY = false; the xor of the data goes to sink only if it equals a
// magic value, so the loads cannot be dropped) or copy of n bytes, n a
// multiple of 16.  Each lane keeps PROBE_U loads in flight.
constexpr uint32_t PROBE_U = 16;
template <bool COPY>
__global__ void __launch_bounds__(256) gpuos_hbm_probe_kernel(const uint8_t* src, uint8_t* dst, uint32_t n) {
    const RBuf rs = rbuf(src, n);
    const WBuf wd = wbuf(dst, COPY ? n : 4096u);
    const uint64_t T = (uint64_t)gridDim.x * blockDim.x;
    const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t x = 0;
    for (uint64_t base = tid * 16u; base < n; base += T * 16u * PROBE_U) {
        u32x4 v[PROBE_U];
#pragma unroll
        for (uint32_t k = 0; k < PROBE_U; ++k) {
            const uint64_t off = base + (uint64_t)k * T * 16u;
            v[k] = rld16(rs, off < n ? (uint32_t)off : n);  // at n: outside the window, reads zero
        }
#pragma unroll
        for (uint32_t k = 0; k < PROBE_U; ++k) {
            const uint64_t off = base + (uint64_t)k * T * 16u;
            if constexpr (COPY) {
                if (off < n) wst16(wd, (uint32_t)off, v[k]);
            } else {
                x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
            }
        }
    }
    if constexpr (!COPY) {
        if (x == 0x9E3779B9u) wst16(wd, (uint32_t)(tid & 255u) * 16u, u32x4{x, x, x, x});
    }
}

// ------------------------------------------------------ host-side launchers
hipError_t launch_executor(const ExecArgs& a, uint32_t slots, bool jit, uint32_t grid, uint32_t block, hipStream_t s) {
    if (jit) hipLaunchKernelGGL(gpuos_executor_jit, dim3(grid), dim3(block), 0, s, a);
    else if (slots == 2) hipLaunchKernelGGL(gpuos_executor_s2, dim3(grid), dim3(block), 0, s, a);
    else hipLaunchKernelGGL(gpuos_executor, dim3(grid), dim3(block), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_eager(const gpuos_desc& d, uint32_t kind, uint32_t ntiles, uint8_t* scratch, hipStream_t s) {
    const uint32_t grid = (ntiles + 3u) / 4u;
    hipLaunchKernelGGL(gpuos_eager_kernel, dim3(grid), dim3(256), 0, s, d, kind, ntiles, scratch);
    return hipGetLastError();
}

hipError_t launch_hbm_probe(const void* src, void* dst, uint32_t n, bool copy, uint32_t grid, hipStream_t s) {
    if (copy)
        hipLaunchKernelGGL(gpuos_hbm_probe_kernel<true>, dim3(grid), dim3(256), 0, s, (const uint8_t*)src, (uint8_t*)dst, n);
    else
        hipLaunchKernelGGL(gpuos_hbm_probe_kernel<false>, dim3(grid), dim3(256), 0, s, (const uint8_t*)src, (uint8_t*)dst, n);
    return hipGetLastError();
}

hipError_t launch_null(hipStream_t s) {
    hipLaunchKernelGGL(gpuos_null_kernel, dim3(1), dim3(64), 0, s);
    return hipGetLastError();
}

}  // namespace gpuos
