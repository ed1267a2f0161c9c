// Host runtime of the persistent micro-op dispatcher (C ABI in gpuos.h).
//
// Submission follows the pages' producer protocol (GPUOS digest page,
// section 3 Q2 "Ring Buffer Communication Channel"): prepare descriptor ->
// acquire slot -> write -> commit with store-release.  Slot p of a ring of
// N entries is free for sequence number p when stamp[p % N] == p; the host
// writes the body and stores stamp = p + 1 (commit); the executor stores
// stamp = p + N when descriptor p has completed, which frees the slot for
// p + N (the slot is released after the op finishes).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <map>
#include <mutex>
#include <random>
#include <string>
#include <thread>
#include <vector>

#include "gpuos.h"
#include "gpuos_internal.h"
#include "gpuos_jit.h"
#include "hazard.h"

#if defined(__x86_64__)
#include <immintrin.h>
#define GPUOS_PAUSE() _mm_pause()
#else
#define GPUOS_PAUSE() std::this_thread::yield()
#endif

namespace gpuos {
hipError_t launch_executor(const ExecArgs& a, uint32_t slots, bool jit, uint32_t grid, uint32_t block, hipStream_t s);
hipError_t launch_eager(const gpuos_desc& d, uint32_t kind, uint32_t ntiles, uint8_t* scratch, hipStream_t s);
hipError_t launch_null(hipStream_t s);
hipError_t launch_hbm_probe(const void* src, void* dst, uint32_t n, bool copy, uint32_t grid, hipStream_t s);
hipError_t static_scratch(uint8_t** out);
hipError_t launch_fill_zero(uint8_t* p, uint32_t bytes, hipStream_t s);
}  // namespace gpuos

using namespace gpuos;

namespace {

inline uint64_t now_ns() {
    return (uint64_t)std::chrono::duration_cast<std::chrono::nanoseconds>(
               std::chrono::steady_clock::now().time_since_epoch())
        .count();
}

template <typename T>
inline T ld_acq(const T* p) { return __atomic_load_n(p, __ATOMIC_ACQUIRE); }
template <typename T>
inline void st_rel(T* p, T v) { __atomic_store_n(p, v, __ATOMIC_RELEASE); }

// --------------------------------------------------------------------------
// Operand byte ranges of a descriptor for hazard tracking.  A declared range
// may be larger than what the op touches (an extra wait, never a missing
// one: the op itself waits for every earlier conflict in the range, so a
// later op that waits for it is ordered after those too).  The KV caches
// are declared whole: an append writes one row per head, H rows C rows
// apart, and attention reads each head's first L rows; declaring the
// batch rows' whole span of each cache gives the same conflicts between
// the appends and attention ops of a decode stream, and keeps the tracker
// from cutting the cache into a new sliver of intervals at every step.
// --------------------------------------------------------------------------
int accesses(uint32_t kind, const gpuos_desc& d, Access* out) {
    int n = 0;
    auto add = [&](uint64_t p, uint64_t bytes, bool w) {
        if (p && bytes) out[n++] = Access{p, p + bytes, w};
    };
    const uint32_t di = dt_in(d.flags), dout = dt_out(d.flags);
    const uint64_t es = esz(di), eo = esz(dout);
    const uint64_t sz = d.size;
    const uint64_t lensw[2] = {(uint64_t)d.param.u[0] | ((uint64_t)d.param.u[1] << 32),
                               (uint64_t)d.param.u[2] | ((uint64_t)d.param.u[3] << 32)};
    switch (kind) {
        case GPUOS_OP_ADD:
        case GPUOS_OP_MUL:
            add(d.input_a, sz * es, false);
            add(d.input_b, sz * es, false);
            add(d.output, sz * eo, true);
            break;
        case GPUOS_OP_RELU:
        case GPUOS_OP_GELU:
            add(d.input_a, sz * es, false);
            add(d.output, sz * eo, true);
            break;
        case GPUOS_OP_SUM:
        case GPUOS_OP_MAX:
        case GPUOS_OP_MIN:
            add(d.input_a, sz * d.dim[0] * es, false);
            add(d.output, sz * eo, true);
            break;
        case GPUOS_OP_SOFTMAX:
            add(d.input_a, sz * d.dim[0] * es, false);
            add(d.output, sz * d.dim[0] * eo, true);
            break;
        case GPUOS_OP_LAYERNORM:
            add(d.input_a, sz * d.dim[0] * es, false);
            add(d.aux[0], (uint64_t)d.dim[0] * es, false);
            add(d.aux[1], (uint64_t)d.dim[0] * es, false);
            add(d.output, sz * d.dim[0] * eo, true);
            break;
        case GPUOS_OP_ROPE: {
            const uint64_t bq = sz * d.dim[0] * d.dim[1] * es;
            const uint64_t bk = sz * (d.dim[3] ? d.dim[3] : d.dim[0]) * d.dim[1] * es;
            add(d.input_a, bq, false);
            add(d.input_b, bk, false);
            add(d.input_a, bq, true);
            add(d.input_b, bk, true);
            break;
        }
        case GPUOS_OP_KV_APPEND: {
            const uint64_t H = d.dim[0], D = d.dim[1], C = d.dim[2];
            if (kv_paged(d.flags)) {  // whole pools: which pages are written is in device memory
                const uint64_t B = kv_rows(d.size, d.flags), pool = kv_pages(d.size) * H * C * D * es;
                add(d.input_a, B * H * D * es, false);
                add(d.input_b, B * H * D * es, false);
                add(d.aux[2], B * d.param.u[5] * 4ull, false);
                add(d.aux[0], pool, true);
                add(d.aux[1], pool, true);
                break;
            }
            add(d.input_a, sz * H * D * es, false);
            add(d.input_b, sz * H * D * es, false);
            add(d.aux[0], sz * H * C * D * es, true);  // batch rows 0..B-1 of each cache, whole
            add(d.aux[1], sz * H * C * D * es, true);
            break;
        }
        case GPUOS_OP_SDPA: {
            const uint64_t H = d.dim[0], D = d.dim[1], C = d.dim[2];
            const uint64_t Hkv = d.dim[3] ? d.dim[3] : H;
            if (kv_paged(d.flags)) {
                const uint64_t B = kv_rows(d.size, d.flags), pool = kv_pages(d.size) * Hkv * C * D * es;
                add(d.input_a, B * H * D * es, false);
                add(d.input_b, B * d.param.u[5] * 4ull, false);
                add(d.aux[0], pool, false);
                add(d.aux[1], pool, false);
                if (d.flags & GPUOS_F_SDPA_MASK) add(d.aux[2], B * d.param.u[5] * C * 4, false);
                add(d.output, B * H * D * eo, true);
                break;
            }
            add(d.input_a, sz * H * D * es, false);
            if (sz > 0 && sz <= MAX_B) {
                // from the first key of batch row 0 to the last key read in row B-1
                const uint64_t hi = (((sz - 1) * Hkv + Hkv - 1) * C + lens_at(lensw, (uint32_t)sz - 1)) * D * es;
                add(d.aux[0], hi, false);
                add(d.aux[1], hi, false);
                if (d.flags & GPUOS_F_SDPA_MASK) add(d.aux[2], sz * C * 4, false);
            }
            add(d.output, sz * H * D * eo, true);
            break;
        }
        case GPUOS_OP_GEMV:
            add(d.input_a, (uint64_t)d.dim[0] * es, false);
            add(d.input_b, (uint64_t)d.dim[0] * d.dim[1] * es, false);
            add(d.output, (uint64_t)d.dim[1] * eo, true);
            break;
        case GPUOS_OP_COPY:
            add(d.input_a, sz, false);
            add(d.output, sz, true);
            break;
        case GPUOS_OP_MATMUL:
            add(d.input_a, sz * d.dim[0] * es, false);
            add(d.input_b, (uint64_t)d.dim[1] * d.dim[0] * es, false);
            add(d.output, sz * d.dim[1] * eo, true);
            break;
        case GPUOS_OP_EXPR:  // b is counted as read whenever it is given
        case GPUOS_OP_JIT:
            add(d.input_a, sz * es, false);
            add(d.input_b, sz * es, false);
            add(d.output, sz * eo, true);
            break;
        default:
            break;
    }
    return n;
}

PlanIn plan_in(uint32_t kind, const gpuos_desc& d, uint32_t kflags = 0) {
    PlanIn p;
    p.kind = kind;
    p.kflags = kflags;
    p.flags = d.flags;
    p.size = d.size;
    for (int i = 0; i < 4; ++i) p.dim[i] = d.dim[i];
    p.lensw[0] = (uint64_t)d.param.u[0] | ((uint64_t)d.param.u[1] << 32);
    p.lensw[1] = (uint64_t)d.param.u[2] | ((uint64_t)d.param.u[3] << 32);
    p.pu5 = d.param.u[5];
    p.a = d.input_a;
    p.b = d.input_b;
    p.out = d.output;
    p.aux0 = d.aux[0];
    p.aux1 = d.aux[1];
    p.aux2 = d.aux[2];
    return p;
}

void* aligned_zalloc(size_t bytes) {
    void* p = nullptr;
    if (posix_memalign(&p, 4096, (bytes + 4095) & ~(size_t)4095) != 0) return nullptr;
    memset(p, 0, bytes);
    return p;
}

}  // namespace

// --------------------------------------------------------------------------
// Context
// --------------------------------------------------------------------------
struct gpuos_ctx {
    gpuos_init_params P{};
    bool loopback = false;
    uint32_t N = 0, mask = 0, Q = 0, cu_count = 0;
    // host-coherent ring memory
    gpuos_desc* ring = nullptr;
    uint64_t* depx = nullptr;  // [N][DEPX_WORDS]: dependency deltas 6..MAX_DEPS-1
    uint64_t* depd = nullptr;  // device copy, written by the fetcher
    std::vector<gpuos_desc> stage;     // annotated descriptors waiting for ring slots
    std::vector<uint64_t> stage_ex;    // their side dependency words
    bool hz_reset = false;             // tracker cleared after a failed blocking submit
    uint64_t* stamp = nullptr;
    uint32_t* status = nullptr;
    HostCtl* hctl = nullptr;
    // device memory
    DevCtl* dctl = nullptr;
    gpuos_desc* mirror = nullptr;
    MirrorMeta* meta = nullptr;
    uint64_t* done = nullptr;
    uint32_t* tiles_done = nullptr;
    uint64_t* queue = nullptr;
    TableEntry* table = nullptr;
    uint32_t* prog = nullptr;  // [2][GPUOS_MAX_OPS][PROG_WORDS] element-wise programs
    uint8_t* scratch = nullptr;
    gpuos_trace_rec* trace = nullptr;
    uint64_t trace_cap = 0;
    hipStream_t exec = nullptr, aux = nullptr;
    bool own_exec = false;
    hipEvent_t ev_start = nullptr, ev_stop = nullptr;
    uint64_t spin_ticks = 0;
    uint64_t idle_ticks = 0;   // idle exit after this many wall-clock ticks (0: never)
    uint64_t idle_exits = 0;
    // producer state
    std::mutex mu;
    uint64_t next_seq = 0;
    uint64_t wm = 0;  // every seq < wm observed complete
    HazardTracker hz;
    std::vector<uint64_t> deps;
    TableEntry shadow[2][GPUOS_MAX_OPS];
    uint32_t shadow_prog[2][GPUOS_MAX_OPS][PROG_WORDS];
    uint32_t version = 0;
    uint64_t flip_seq = 0;  // first seq submitted under the current version
    // errors
    struct Err { uint64_t seq; uint32_t st; };
    std::vector<Err> errors;
    // executor state
    bool running = false;
    uint64_t launches = 0;
    float last_ms = 0.f, total_ms = 0.f;
    // stats (device counters are accumulated here when a launch ends)
    uint64_t submitted = 0, completed = 0, full_rej = 0;
    uint64_t acc_units = 0, acc_depw = 0, acc_batches = 0, acc_fetched = 0;
    uint64_t deps_explicit = 0, deps_range = 0;
    uint64_t ns_submit = 0, ns_blocked = 0, ns_hazard = 0;  // host time inside gpuos_submit
    // injected code (gpuos_register_jit): the device's target name and every
    // code object loaded so far, by source (each stays loaded until shutdown)
    std::string arch;
    std::mutex jit_mu;
    std::map<std::string, JitCode> jit_code;
    bool holds_device = false;  // counted in g_live
    // loopback consumer
    std::thread lb_thread;
    std::atomic<bool> lb_stop{false};
    std::vector<uint64_t> lb_done;
    std::vector<uint64_t> lb_order;
    std::mutex lb_mu;
};

namespace {

// Devices with a live (GPU) context in this process.  A resident executor
// holds a share of every CU it runs on; a second one on the same device
// could not be placed beside a full-size first one and would wait forever,
// so gpuos_init refuses it.
std::mutex g_live_mu;
std::map<int, int> g_live;

void refresh_wm(gpuos_ctx* c) {
    const uint64_t N = c->N;
    while (c->wm < c->next_seq) {
        const uint64_t s = c->wm;
        const uint64_t st = ld_acq(&c->stamp[s & c->mask]);
        if (st < s + N) break;
        const uint32_t code = ld_acq(&c->status[s & c->mask]);
        if (code) c->errors.push_back({s, code});
        ++c->completed;
        ++c->wm;
    }
}

void executor_finished(gpuos_ctx* c);

// Every call of a context is a heartbeat: an executor with an idle-exit
// interval leaves the GPU only when none has come for that long.
void beat(gpuos_ctx* c) { __atomic_fetch_add(&c->hctl->heartbeat, 1ull, __ATOMIC_RELEASE); }

// A launch starts fetching where the previous one stopped: after a host
// stop that is every committed descriptor; after an idle exit the host may
// have committed more since the fetcher's last look.
int executor_launch(gpuos_ctx* c) {
    if (c->loopback || c->running) return GPUOS_OK;
    hipError_t e = hipMemsetAsync(c->dctl, 0, sizeof(DevCtl), c->exec);
    if (e != hipSuccess) return GPUOS_E_HIP;
    const uint64_t start = ld_acq(&c->hctl->fetch_end);
    st_rel(&c->hctl->stop, (uint64_t)0);
    st_rel(&c->hctl->abort, (uint64_t)0);
    st_rel(&c->hctl->idle_exit, (uint64_t)0);
    ExecArgs a{};
    a.ring = c->ring;
    a.depx = c->depx;
    a.depd = c->depd;
    a.stamp = c->stamp;
    a.status = c->status;
    a.hctl = c->hctl;
    a.dctl = c->dctl;
    a.mirror = c->mirror;
    a.meta = c->meta;
    a.done = c->done;
    a.tiles_done = c->tiles_done;
    a.queue = c->queue;
    a.table = c->table;
    a.scratch = c->scratch;
    a.scratch_bytes = c->P.scratch_bytes;
    a.trace = c->trace;
    a.trace_cap = c->trace_cap;
    a.start_seq = start;
    a.spin_limit_ticks = c->spin_ticks;
    a.idle_exit_ticks = c->idle_ticks;
    a.mask = c->mask;
    a.qmask = c->Q - 1;
    a.backoff_max = c->P.backoff_max;
    a.shards = claim_shards(c->P.num_wgs, c->P.waves_per_wg, c->cu_count);
    if (c->trace && hipMemsetAsync(c->trace, 0, c->trace_cap * sizeof(gpuos_trace_rec), c->exec) != hipSuccess)
        return GPUOS_E_HIP;
    if (hipEventRecord(c->ev_start, c->exec) != hipSuccess) return GPUOS_E_HIP;
    if (launch_executor(a, c->P.units_per_wave, (c->P.flags & GPUOS_INIT_JIT) != 0, c->P.num_wgs, 64u * c->P.waves_per_wg,
                        c->exec) != hipSuccess)
        return GPUOS_E_HIP;
    if (hipEventRecord(c->ev_stop, c->exec) != hipSuccess) return GPUOS_E_HIP;
    c->running = true;
    ++c->launches;
    return GPUOS_OK;
}

// Ask the executor to drain and exit; wait for its completion event.
int executor_stop(gpuos_ctx* c, int64_t timeout_ns) {
    if (c->loopback || !c->running) return GPUOS_OK;
    st_rel(&c->hctl->stop, (uint64_t)1);
    const uint64_t t0 = now_ns();
    bool aborted = false;
    for (;;) {
        hipError_t q = hipEventQuery(c->ev_stop);
        if (q == hipSuccess) break;
        if (q != hipErrorNotReady) return GPUOS_E_HIP;
        const uint64_t el = now_ns() - t0;
        if (!aborted && timeout_ns >= 0 && el > (uint64_t)timeout_ns) {
            st_rel(&c->hctl->abort, (uint64_t)1);
            aborted = true;
        }
        if (aborted && el > (uint64_t)timeout_ns + 5000000000ull) return GPUOS_E_TIMEOUT;
        // a drained executor leaves within tens of microseconds: yield at
        // first (a sleep can take several times what it asks for), sleep
        // once the wait has gone on
        if (el < 5000000ull) std::this_thread::yield();
        else std::this_thread::sleep_for(std::chrono::microseconds(20));
    }
    executor_finished(c);
    return aborted ? GPUOS_E_TIMEOUT : GPUOS_OK;
}

// The launch has ended: its duration and device counters.
void executor_finished(gpuos_ctx* c) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, c->ev_start, c->ev_stop) == hipSuccess) {
        c->last_ms = ms;
        c->total_ms += ms;
    }
    c->running = false;
    DevCtl d;
    if (hipMemcpyAsync(&d, c->dctl, sizeof(DevCtl), hipMemcpyDeviceToHost, c->aux) == hipSuccess &&
        hipStreamSynchronize(c->aux) == hipSuccess) {
        c->acc_units += d.stat_units;
        c->acc_depw += d.stat_dep_waits;
        c->acc_batches += d.stat_batches;
        c->acc_fetched += d.stat_fetched;
    }
}

// An executor with an idle-exit interval may have left by itself: account
// for the launch and, when descriptors are waiting (`pending`), launch again
// from where its fetcher stopped.  Caller holds c->mu.
int revive(gpuos_ctx* c, bool pending) {
    if (c->loopback || !c->idle_ticks) return GPUOS_OK;
    if (c->running) {
        if (hipEventQuery(c->ev_stop) != hipSuccess || !ld_acq(&c->hctl->idle_exit)) return GPUOS_OK;
        executor_finished(c);
        ++c->idle_exits;
    }
    return pending ? executor_launch(c) : GPUOS_OK;
}

// ---- loopback consumer (test only): completes descriptors in a random order
// that respects their dependency annotations, computing nothing.
void loopback_main(gpuos_ctx* c) {
    std::mt19937_64 rng(12345);
    const uint64_t N = c->N;
    uint64_t f = c->N;  // next seq to fetch
    struct Pend { uint64_t seq; gpuos_desc d; uint16_t ex[4 * DEPX_WORDS]; };
    std::vector<Pend> pend;
    auto is_done = [&](uint64_t s) { return c->lb_done[s & c->mask] >= s; };
    while (!c->lb_stop.load()) {
        bool progress = false;
        while (ld_acq(&c->stamp[f & c->mask]) == f + 1 && pend.size() < 256) {
            Pend pe;
            pe.seq = f;
            pe.d = c->ring[f & c->mask];
            memset(pe.ex, 0, sizeof(pe.ex));
            if (pe.d.dep_delta[5]) memcpy(pe.ex, &c->depx[DEPX_WORDS * (f & c->mask)], 8 * DEPX_WORDS);
            pend.push_back(pe);
            ++f;
            progress = true;
        }
        // runnable candidates
        std::vector<size_t> ready;
        for (size_t i = 0; i < pend.size(); ++i) {
            const gpuos_desc& d = pend[i].d;
            const uint64_t s = pend[i].seq;
            bool ok = true;
            for (int k = 0; k < 6 && ok; ++k)
                if (d.dep_delta[k]) ok = is_done(s - d.dep_delta[k]);
            const uint16_t* ex = pend[i].ex;
            for (uint32_t k = 0; k < 4 * DEPX_WORDS && ok; ++k)
                if (ex[k]) ok = is_done(s - ex[k]);
            for (uint64_t x = s - d.dep_range; x < s && ok; ++x) ok = is_done(x);
            if (ok) ready.push_back(i);
        }
        if (!ready.empty()) {
            const size_t pick = ready[rng() % ready.size()];
            const Pend p = pend[pick];
            pend.erase(pend.begin() + (long)pick);
            const uint32_t slot = (uint32_t)(p.seq & c->mask);
            // mirror the device's table lookup and shape check for the status
            uint32_t st = GPUOS_ST_OK;
            const uint32_t op = p.d.op_id;
            if (op >= GPUOS_MAX_OPS) st = GPUOS_ST_BAD_OP;
            else {
                std::lock_guard<std::mutex> g(c->lb_mu);
                const TableEntry& te = c->shadow[p.d.table_version & 1u][op];
                if (te.kind >= GPUOS_KIND_COUNT) st = GPUOS_ST_BAD_OP;
                else st = make_plan(plan_in(te.kind, p.d, te.flags)).status;
            }
            {
                std::lock_guard<std::mutex> g(c->lb_mu);
                c->lb_order.push_back(p.seq);
            }
            c->lb_done[slot] = p.seq;
            if (st) st_rel(&c->status[slot], st);
            st_rel(&c->stamp[slot], p.seq + N);
            progress = true;
        }
        if (!progress) std::this_thread::sleep_for(std::chrono::microseconds(5));
    }
}

int validate_params(gpuos_init_params& P) {
    if (P.ring_entries == 0) P.ring_entries = 4096;
    if (P.ring_entries < 8 || P.ring_entries > 32768 || (P.ring_entries & (P.ring_entries - 1))) return GPUOS_E_INVAL;
    if (P.waves_per_wg == 0) P.waves_per_wg = 4;
    if (P.waves_per_wg > 4) return GPUOS_E_INVAL;
    if (P.units_per_wave == 0) P.units_per_wave = 1;
    if (P.units_per_wave > 2) return GPUOS_E_INVAL;
    if ((P.flags & GPUOS_INIT_JIT) && P.units_per_wave != 1) return GPUOS_E_INVAL;  // one build: one unit per wave
    if (P.backoff_max == 0) P.backoff_max = 64;
    if (P.backoff_max > 127) return GPUOS_E_INVAL;
    if (P.scratch_bytes == 0) P.scratch_bytes = 256ull << 20;
    if (P.scratch_bytes < (1u << 20)) return GPUOS_E_INVAL;
    P.scratch_bytes = (P.scratch_bytes + 255) & ~255ull;
    if (P.unit_queue_log2 == 0) P.unit_queue_log2 = 20;
    if (P.unit_queue_log2 < 12 || P.unit_queue_log2 > 24) return GPUOS_E_INVAL;
    if (P.spin_limit_ms == 0) P.spin_limit_ms = 20000;
    return GPUOS_OK;
}

void free_ctx(gpuos_ctx* c) {
    if (c->loopback) {
        c->lb_stop = true;
        if (c->lb_thread.joinable()) c->lb_thread.join();
        free(c->ring);
        free(c->depx);
        free(c->stamp);
        free(c->status);
        free(c->hctl);
        delete c;
        return;
    }
    if (c->ring) (void)hipHostFree(c->ring);
    if (c->depx) (void)hipHostFree(c->depx);
    if (c->stamp) (void)hipHostFree(c->stamp);
    if (c->status) (void)hipHostFree(c->status);
    if (c->hctl) (void)hipHostFree(c->hctl);
    void* dev[] = {c->dctl, c->mirror, c->meta, c->done, c->tiles_done, c->depd, c->queue, c->table, c->prog, c->scratch,
                   c->trace};
    for (void* p : dev)
        if (p) (void)hipFree(p);
    if (c->ev_start) (void)hipEventDestroy(c->ev_start);
    if (c->ev_stop) (void)hipEventDestroy(c->ev_stop);
    if (c->aux) (void)hipStreamDestroy(c->aux);
    if (c->own_exec && c->exec) (void)hipStreamDestroy(c->exec);
    for (auto& kv : c->jit_code)  // the executor has exited: nothing runs this code any more
        if (kv.second.mod) (void)hipModuleUnload(kv.second.mod);
    if (c->holds_device) {
        std::lock_guard<std::mutex> lg(g_live_mu);
        --g_live[c->P.device];
    }
    delete c;
}

}  // namespace

// --------------------------------------------------------------------------
// C ABI
// --------------------------------------------------------------------------
extern "C" {

int gpuos_abi_version(void) { return GPUOS_ABI_VERSION; }

int gpuos_init(const gpuos_init_params* params, void** out) {
    if (!out) return GPUOS_E_INVAL;
    *out = nullptr;
    gpuos_init_params P{};
    if (params) P = *params;
    int rc = validate_params(P);
    if (rc) return rc;
    gpuos_ctx* c = new gpuos_ctx();
    c->P = P;
    c->N = P.ring_entries;
    c->mask = c->N - 1;
    c->Q = 1u << P.unit_queue_log2;
    c->loopback = (P.flags & GPUOS_INIT_LOOPBACK) != 0;
    c->next_seq = c->N;  // seqs start at N so that done[i] = i means "nothing done"
    c->wm = c->N;
    c->flip_seq = c->N;
    for (int v = 0; v < 2; ++v)
        for (uint32_t i = 0; i < GPUOS_MAX_OPS; ++i)
            c->shadow[v][i] = TableEntry{i < GPUOS_KIND_COUNT && i != GPUOS_OP_EXPR && i != GPUOS_OP_JIT ? i : (uint32_t)GPUOS_KIND_EMPTY,
                                         0, 0.f, 0.f, 0, 0};
    memset(c->shadow_prog, 0, sizeof(c->shadow_prog));
    const size_t N = c->N;
    if (c->loopback) {
        c->ring = (gpuos_desc*)aligned_zalloc(N * sizeof(gpuos_desc));
        c->depx = (uint64_t*)aligned_zalloc(N * 8 * DEPX_WORDS);
        c->stamp = (uint64_t*)aligned_zalloc(N * 8);
        c->status = (uint32_t*)aligned_zalloc(N * 4);
        c->hctl = (HostCtl*)aligned_zalloc(sizeof(HostCtl));
        if (!c->ring || !c->depx || !c->stamp || !c->status || !c->hctl) { free_ctx(c); return GPUOS_E_INVAL; }
        for (size_t i = 0; i < N; ++i) c->stamp[i] = N + i;
        c->lb_done.assign(N, 0);
        for (size_t i = 0; i < N; ++i) c->lb_done[i] = i;
        c->P.num_wgs = 1;
        c->lb_thread = std::thread(loopback_main, c);
        *out = c;
        return GPUOS_OK;
    }
    hipError_t e;
#define HIPCHK(x)                                      \
    do {                                               \
        e = (x);                                       \
        if (e != hipSuccess) { free_ctx(c); return GPUOS_E_HIP; } \
    } while (0)
    {
        std::lock_guard<std::mutex> lg(g_live_mu);
        if (g_live[P.device] > 0) {
            fprintf(stderr, "gpuos_init: device %d already has a live context in this process (its resident "
                            "executor would keep a second one from being placed)\n", P.device);
            free_ctx(c);
            return GPUOS_E_STATE;
        }
        ++g_live[P.device];
        c->holds_device = true;
    }
    HIPCHK(hipSetDevice(P.device));
    hipDeviceProp_t prop;
    HIPCHK(hipGetDeviceProperties(&prop, P.device));
    c->cu_count = (uint32_t)prop.multiProcessorCount;
    c->arch = prop.gcnArchName;
    if (c->P.num_wgs == 0) c->P.num_wgs = c->cu_count;
    // one fetcher wave plus at least one worker; every workgroup must be able
    // to be resident at once (at most four one-wave workgroups per CU)
    if ((uint64_t)c->P.num_wgs * c->P.waves_per_wg < 2 || c->P.num_wgs > 4 * c->cu_count) {
        free_ctx(c);
        return GPUOS_E_INVAL;
    }
    int wclk = 0;
    if (hipDeviceGetAttribute(&wclk, hipDeviceAttributeWallClockRate, P.device) != hipSuccess || wclk <= 0)
        wclk = 100000;  // kHz
    c->spin_ticks = (uint64_t)P.spin_limit_ms * (uint64_t)wclk;
    c->idle_ticks = (uint64_t)P.idle_exit_ms * (uint64_t)wclk;
    const unsigned hflags = hipHostMallocCoherent | hipHostMallocMapped;
    HIPCHK(hipHostMalloc((void**)&c->ring, N * sizeof(gpuos_desc), hflags));
    HIPCHK(hipHostMalloc((void**)&c->depx, N * 8 * DEPX_WORDS, hflags));
    HIPCHK(hipHostMalloc((void**)&c->stamp, N * 8, hflags));
    HIPCHK(hipHostMalloc((void**)&c->status, N * 4, hflags));
    HIPCHK(hipHostMalloc((void**)&c->hctl, sizeof(HostCtl), hflags));
    memset(c->ring, 0, N * sizeof(gpuos_desc));
    memset(c->depx, 0, N * 8 * DEPX_WORDS);
    memset(c->status, 0, N * 4);
    memset(c->hctl, 0, sizeof(HostCtl));
    c->hctl->fetch_end = c->next_seq;  // the first launch fetches from the first seq
    for (size_t i = 0; i < N; ++i) c->stamp[i] = N + i;
    HIPCHK(hipMalloc((void**)&c->dctl, sizeof(DevCtl)));
    HIPCHK(hipMalloc((void**)&c->mirror, N * sizeof(gpuos_desc)));
    HIPCHK(hipMalloc((void**)&c->meta, N * sizeof(MirrorMeta)));
    HIPCHK(hipMalloc((void**)&c->done, N * 8 * DONE_STRIDE));
    HIPCHK(hipMalloc((void**)&c->tiles_done, N * 4));
    HIPCHK(hipMalloc((void**)&c->depd, N * 8 * DEPX_WORDS));
    HIPCHK(hipMalloc((void**)&c->queue, (size_t)c->Q * 8));
    HIPCHK(hipMalloc((void**)&c->table, 2 * GPUOS_MAX_OPS * sizeof(TableEntry)));
    HIPCHK(hipMalloc((void**)&c->prog, sizeof(c->shadow_prog)));
    HIPCHK(hipMalloc((void**)&c->scratch, P.scratch_bytes));
    if (P.flags & GPUOS_INIT_TRACE) {
        c->trace_cap = 1u << 20;
        HIPCHK(hipMalloc((void**)&c->trace, c->trace_cap * sizeof(gpuos_trace_rec)));
    }
    HIPCHK(hipStreamCreateWithFlags(&c->aux, hipStreamNonBlocking));
    if (P.hip_stream) {
        c->exec = (hipStream_t)P.hip_stream;
        unsigned int fl = 0;
        HIPCHK(hipStreamGetFlags(c->exec, &fl));
        if (!(fl & hipStreamNonBlocking)) { free_ctx(c); return GPUOS_E_INVAL; }
    } else {
        HIPCHK(hipStreamCreateWithFlags(&c->exec, hipStreamNonBlocking));
        c->own_exec = true;
    }
    HIPCHK(hipEventCreate(&c->ev_start));
    HIPCHK(hipEventCreate(&c->ev_stop));
    {
        std::vector<uint64_t> d(N * DONE_STRIDE, 0);
        for (size_t i = 0; i < N; ++i) d[i * DONE_STRIDE] = i;
        HIPCHK(hipMemcpyAsync(c->done, d.data(), N * 8 * DONE_STRIDE, hipMemcpyHostToDevice, c->aux));
        HIPCHK(hipMemsetAsync(c->tiles_done, 0, N * 4, c->aux));
        HIPCHK(hipMemsetAsync(c->meta, 0, N * sizeof(MirrorMeta), c->aux));
        HIPCHK(hipMemsetAsync(c->scratch, 0, P.scratch_bytes, c->aux));
        HIPCHK(hipMemcpyAsync(c->table, c->shadow, sizeof(c->shadow), hipMemcpyHostToDevice, c->aux));
        HIPCHK(hipMemcpyAsync(c->prog, c->shadow_prog, sizeof(c->shadow_prog), hipMemcpyHostToDevice, c->aux));
        HIPCHK(hipStreamSynchronize(c->aux));
    }
#undef HIPCHK
    rc = executor_launch(c);
    if (rc) { free_ctx(c); return rc; }
    *out = c;
    return GPUOS_OK;
}

// Write entry `te` (and, for EXPR, its program) for op_id into the inactive
// table slot, then flip.  The inactive slot is first made a copy of the
// active one, programs included; every EXPR entry's program address is set
// to the copy in the new slot, so a slot's entries only ever point into
// that slot's program area.  Caller holds c->mu.
static int table_flip(gpuos_ctx* c, uint32_t op_id, TableEntry te, const uint32_t* prog) {
    // Grace period: the slot about to be rewritten was last used by version
    // (version - 1); every descriptor submitted before the current version's
    // flip must have completed (and so been resolved) first.
    const uint64_t t0 = now_ns();
    for (;;) {
        refresh_wm(c);
        if (c->wm >= c->flip_seq) break;
        beat(c);
        if (const int rr = revive(c, true)) return rr;
        if (now_ns() - t0 > 60000000000ull) return GPUOS_E_TIMEOUT;
        GPUOS_PAUSE();
    }
    const uint32_t nv = c->version + 1, slot = nv & 1u, old = c->version & 1u;
    {
        std::lock_guard<std::mutex> lg(c->lb_mu);
        memcpy(c->shadow[slot], c->shadow[old], sizeof(c->shadow[0]));
        memcpy(c->shadow_prog[slot], c->shadow_prog[old], sizeof(c->shadow_prog[0]));
        c->shadow[slot][op_id] = te;
        if (prog) memcpy(c->shadow_prog[slot][op_id], prog, sizeof(c->shadow_prog[0][0]));
        for (uint32_t i = 0; i < GPUOS_MAX_OPS; ++i)
            if (c->shadow[slot][i].kind == GPUOS_OP_EXPR)
                c->shadow[slot][i].fn = c->prog ? (uint64_t)(c->prog + ((size_t)slot * GPUOS_MAX_OPS + i) * PROG_WORDS) : 0;
    }
    if (!c->loopback) {
        if (hipMemcpyAsync(c->prog + (size_t)slot * GPUOS_MAX_OPS * PROG_WORDS, c->shadow_prog[slot],
                           sizeof(c->shadow_prog[0]), hipMemcpyHostToDevice, c->aux) != hipSuccess)
            return GPUOS_E_HIP;
        if (hipMemcpyAsync(c->table + (size_t)slot * GPUOS_MAX_OPS, c->shadow[slot], sizeof(c->shadow[0]),
                           hipMemcpyHostToDevice, c->aux) != hipSuccess)
            return GPUOS_E_HIP;
        if (hipStreamSynchronize(c->aux) != hipSuccess) return GPUOS_E_HIP;
    }
    // the flip: descriptors committed from now on carry the new version
    c->version = nv;
    c->flip_seq = c->next_seq;
    if (getenv("GPUOS_AUDIT"))
        fprintf(stderr, "gpuos: op %u -> kind %u (version %u, from seq %llu)\n", op_id, te.kind, nv,
                (unsigned long long)c->next_seq);
    return GPUOS_OK;
}

int gpuos_register_op(void* ctx, uint32_t op_id, uint32_t kind, const void* consts, uint32_t len) {
    gpuos_ctx* c = (gpuos_ctx*)ctx;
    if (!c) return GPUOS_E_INVAL;
    if (op_id >= GPUOS_MAX_OPS || (kind >= GPUOS_KIND_COUNT && kind != GPUOS_KIND_EMPTY)) return GPUOS_E_NOOP;
    if (kind == GPUOS_OP_EXPR || kind == GPUOS_OP_JIT) return GPUOS_E_INVAL;  // bound with register_expr / _jit
    if (len > 8 || (len && !consts)) return GPUOS_E_INVAL;
    std::lock_guard<std::mutex> g(c->mu);
    TableEntry te{kind, 0, 0.f, 0.f, 0, 0};
    if (len >= 4) memcpy(&te.p0, consts, 4);
    if (len >= 8) memcpy(&te.p1, (const char*)consts + 4, 4);
    return table_flip(c, op_id, te, nullptr);
}

int gpuos_register_expr(void* ctx, uint32_t op_id, const uint32_t* program, uint32_t n_words) {
    gpuos_ctx* c = (gpuos_ctx*)ctx;
    if (!c || !program || n_words == 0) return GPUOS_E_INVAL;
    if (op_id >= GPUOS_MAX_OPS) return GPUOS_E_NOOP;
    uint32_t slot[PROG_WORDS], kflags = 0;
    if (!expr_validate(program, n_words, slot, &kflags)) return GPUOS_E_INVAL;
    std::lock_guard<std::mutex> g(c->mu);
    TableEntry te{GPUOS_OP_EXPR, kflags, 0.f, 0.f, 0, 0};
    return table_flip(c, op_id, te, slot);
}

int gpuos_register_jit(void* ctx, uint32_t op_id, const uint32_t* program, uint32_t n_words, gpuos_jit_info* info) {
    gpuos_ctx* c = (gpuos_ctx*)ctx;
    if (info) memset(info, 0, sizeof(*info));
    if (!c || !program || n_words == 0) return GPUOS_E_INVAL;
    if (op_id >= GPUOS_MAX_OPS) return GPUOS_E_NOOP;
    uint32_t slot[PROG_WORDS], kflags = 0;
    if (!expr_validate(program, n_words, slot, &kflags)) return GPUOS_E_INVAL;
    if (!(c->P.flags & GPUOS_INIT_JIT)) return GPUOS_E_INVAL;
    const std::string src = jit_source(slot, kflags);
    JitCode jc;
    bool reused = false;
    {
        // compiled and loaded without the producer lock: submissions go on
        std::lock_guard<std::mutex> jg(c->jit_mu);
        auto it = c->jit_code.find(src);
        if (it != c->jit_code.end()) {
            jc = it->second;
            reused = true;
        } else {
            std::string log;
            // loopback contexts compile and check the code but load nothing
            const std::string arch = c->loopback ? std::string("gfx950") : c->arch;
            if (!c->loopback && hipSetDevice(c->P.device) != hipSuccess) return GPUOS_E_HIP;
            const int rc = jit_build(src, arch, !c->loopback, c->aux, &jc, &log);
            if (info) {
                info->compile_ms = jc.compile_ms;
                info->vgprs = jc.vgprs;
                info->agprs = jc.agprs;
                info->sgprs = jc.sgprs;
                info->stack_bytes = jc.stack;
                info->code_bytes = jc.code_bytes;
            }
            if (rc != GPUOS_OK) {
                if (rc == GPUOS_E_HIP && !log.empty()) fprintf(stderr, "gpuos_register_jit: compiler log:\n%s\n", log.c_str());
                return rc;
            }
            c->jit_code[src] = jc;
        }
    }
    if (info) {
        info->load_ms = reused ? 0.0 : jc.load_ms;
        info->vgprs = jc.vgprs;
        info->agprs = jc.agprs;
        info->sgprs = jc.sgprs;
        info->stack_bytes = jc.stack;
        info->code_bytes = jc.code_bytes;
        info->reused = reused ? 1u : 0u;
        if (!reused) info->compile_ms = jc.compile_ms;
    }
    std::lock_guard<std::mutex> g(c->mu);
    const uint64_t t0 = now_ns();
    TableEntry te{GPUOS_OP_JIT, kflags, 0.f, 0.f, jc.fn_f32, jc.fn_bf16};
    const int rc = table_flip(c, op_id, te, nullptr);
    if (info) info->flip_ms = (double)(now_ns() - t0) * 1e-6;
    return rc;
}

int gpuos_jit_source(const uint32_t* program, uint32_t n_words, char* out, uint64_t cap, uint64_t* len_out) {
    uint32_t slot[PROG_WORDS], kflags = 0;
    if (!expr_validate(program, n_words, slot, &kflags)) return GPUOS_E_INVAL;
    const std::string src = jit_source(slot, kflags);
    if (len_out) *len_out = src.size();
    if (out && cap) {
        const uint64_t n = std::min<uint64_t>(cap - 1, src.size());
        memcpy(out, src.data(), n);
        out[n] = '\0';
    }
    return GPUOS_OK;
}

int gpuos_submit(void* ctx, const gpuos_desc* descs, uint32_t count, uint32_t flags, uint64_t* first_seq) {
    gpuos_ctx* c = (gpuos_ctx*)ctx;
    if (!c || (count && !descs)) return GPUOS_E_INVAL;
    if (count > c->N) return GPUOS_E_INVAL;
    std::lock_guard<std::mutex> g(c->mu);
    if (first_seq) *first_seq = c->next_seq;
    if (count == 0) return GPUOS_OK;
    const uint64_t t_enter = now_ns();
    // resolve kinds and validate shapes before touching the ring
    uint32_t kinds_small[64];
    std::vector<uint32_t> kinds_big;
    uint32_t* kinds = kinds_small;
    if (count > 64) { kinds_big.resize(count); kinds = kinds_big.data(); }
    const TableEntry* tab = c->shadow[c->version & 1u];
    for (uint32_t i = 0; i < count; ++i) {
        const gpuos_desc& d = descs[i];
        uint32_t kind = d.op_id < GPUOS_MAX_OPS ? tab[d.op_id].kind : (uint32_t)GPUOS_KIND_EMPTY;
        if (kind < GPUOS_KIND_COUNT) {
            const Plan pl = make_plan(plan_in(kind, d, tab[d.op_id].flags));
            if (pl.status != GPUOS_ST_OK) return GPUOS_E_INVAL;
            if (pl.ntiles > max_units_per_descriptor(c->Q) || pl.scratch > c->P.scratch_bytes / 2) return GPUOS_E_INVAL;
        } else {
            kind = GPUOS_KIND_EMPTY;  // the device reports BAD_OP; nothing to order
        }
        kinds[i] = kind;
    }
    beat(c);
    if (const int rr = revive(c, false)) return rr;
    if (!c->running && !c->loopback) {
        int rc = executor_launch(c);
        if (rc) return rc;
    }
    const bool block = (flags & GPUOS_SUBMIT_BLOCK) != 0;
    // wait until seq `upto` is complete (spinning, then yielding)
    auto wait_wm = [&](uint64_t upto) -> int {
        uint32_t spins = 0;
        const uint64_t tb = now_ns();
        while (c->wm < upto) {
            if (c->hctl && ld_acq(&c->hctl->dev_error)) return GPUOS_E_DEVICE;
            if (++spins > 1000) {
                std::this_thread::yield();
                beat(c);
                if (const int rr = revive(c, true)) return rr;
            } else {
                GPUOS_PAUSE();
            }
            refresh_wm(c);
        }
        c->ns_blocked += now_ns() - tb;
        return GPUOS_OK;
    };
    refresh_wm(c);
    if (c->hz_reset) {
        // an earlier blocking submit failed after annotating and cleared the
        // tracker: nothing it knew about may still be in flight
        if (c->wm < c->next_seq) {
            if (!block) { ++c->full_rej; return GPUOS_E_FULL; }
            const int rc = wait_wm(c->next_seq);
            if (rc) return rc;
        }
        c->hz_reset = false;
    }
    // slots: seq s needs seq s - N complete
    const uint64_t need_wm = c->next_seq + count - c->N;
    if (c->wm < need_wm && !block) { ++c->full_rej; return GPUOS_E_FULL; }
    // Annotate before waiting for slots, so that this work overlaps the
    // device's.  Dependencies are computed against the watermark seen now;
    // an older watermark only adds waits on descriptors already complete.
    const uint64_t t_hz0 = now_ns();
    const uint64_t s0 = c->next_seq;
    if (c->stage.size() < count) {
        c->stage.resize(count);
        c->stage_ex.resize((size_t)count * DEPX_WORDS);
    }
    Access acc[2 * MAX_B + 4];
    for (uint32_t i = 0; i < count; ++i) {
        const uint64_t s = s0 + i;
        gpuos_desc& d = c->stage[i];
        d = descs[i];
        d.seq = s;
        d.table_version = (uint16_t)c->version;
        memset(d.dep_delta, 0, sizeof(d.dep_delta));
        d.dep_range = 0;
        c->deps.clear();
        uint64_t range_from = UINT64_MAX;
        if (!(flags & GPUOS_SUBMIT_NOHAZARD) && kinds[i] < GPUOS_KIND_COUNT) {
            const int n = accesses(kinds[i], d, acc);
            c->hz.analyze(s, acc, n, c->wm, c->deps, &range_from);
        }
        if ((flags & GPUOS_SUBMIT_SERIAL) && s - 1 >= c->wm) c->deps.push_back(s - 1);
        uint16_t* ex = (uint16_t*)&c->stage_ex[(size_t)i * DEPX_WORDS];
        if (!c->deps.empty() || range_from != UINT64_MAX) {
            std::sort(c->deps.begin(), c->deps.end());
            c->deps.erase(std::unique(c->deps.begin(), c->deps.end()), c->deps.end());
            if (range_from != UINT64_MAX && range_from < c->wm) range_from = c->wm;
            if (range_from != UINT64_MAX)  // the range covers every dep at or after it
                c->deps.erase(std::lower_bound(c->deps.begin(), c->deps.end(), range_from), c->deps.end());
            if (c->deps.size() > MAX_DEPS) {
                range_from = std::min<uint64_t>(range_from, c->deps.front());
                c->deps.clear();
            }
            for (size_t k = 0; k < c->deps.size(); ++k) {
                const uint16_t dl = (uint16_t)(s - c->deps[k]);
                if (k < 6) d.dep_delta[k] = dl;
                else ex[k - 6] = dl;
            }
            c->deps_explicit += c->deps.size();
            if (range_from != UINT64_MAX && range_from < s) {
                d.dep_range = (uint16_t)(s - range_from);
                ++c->deps_range;
            }
        }
        // the side words are read whenever dep_delta[5] is set, that is with
        // six dependencies or more: clear every one past the last in use, so
        // that none is left from an earlier descriptor at this stage index
        if (c->deps.size() >= 6)
            for (size_t k = c->deps.size() - 6; k < 4 * DEPX_WORDS; ++k) ex[k] = 0;
    }
    const uint64_t t_hz1 = now_ns();
    if (c->wm < need_wm) {
        const int rc = wait_wm(need_wm);
        if (rc) {
            // the tracker already holds accesses that will not be submitted
            c->hz.clear();
            c->hz_reset = true;
            return rc;
        }
    }
    for (uint32_t i = 0; i < count; ++i) {
        const uint32_t slot = (uint32_t)((s0 + i) & c->mask);
        const gpuos_desc& d = c->stage[i];
        if (d.dep_delta[5]) memcpy(&c->depx[DEPX_WORDS * slot], &c->stage_ex[(size_t)i * DEPX_WORDS], 8 * DEPX_WORDS);
        c->status[slot] = 0;
        memcpy(&c->ring[slot], &d, sizeof(gpuos_desc));
    }
    // commit in order (store-release of each stamp)
    for (uint32_t i = 0; i < count; ++i) {
        const uint64_t s = s0 + i;
        st_rel(&c->stamp[s & c->mask], s + 1);
    }
    c->next_seq += count;
    c->submitted += count;
    c->ns_hazard += t_hz1 - t_hz0;
    // an executor that left for lack of heartbeat just before this commit
    // became visible would not see it: launch again from its stopping point
    const int rr = revive(c, true);
    c->ns_submit += now_ns() - t_enter;
    return rr;
}

int gpuos_submit_bursts(void* ctx, const gpuos_desc* descs, const uint32_t* burst_sizes, uint32_t n_bursts,
                        uint32_t flags, uint64_t* first_seq, uint64_t* n_done) {
    if (!ctx || (n_bursts && (!descs || !burst_sizes))) return GPUOS_E_INVAL;
    uint64_t off = 0;
    int rc = GPUOS_OK;
    const uint32_t ring = ((gpuos_ctx*)ctx)->N;
    for (uint32_t i = 0; i < n_bursts && rc == GPUOS_OK; ++i) {
        // a burst larger than the ring is committed in ring-sized groups
        for (uint32_t done = 0; done < burst_sizes[i];) {
            const uint32_t n = std::min(burst_sizes[i] - done, ring);
            uint64_t f = 0;
            rc = gpuos_submit(ctx, descs + off, n, flags, &f);
            if (rc != GPUOS_OK) break;
            if (off == 0 && first_seq) *first_seq = f;
            off += n;
            done += n;
        }
    }
    if (n_done) *n_done = off;
    return rc;
}

int gpuos_query(void* ctx, uint64_t seq) {
    gpuos_ctx* c = (gpuos_ctx*)ctx;
    if (!c) return GPUOS_E_INVAL;
    std::lock_guard<std::mutex> g(c->mu);
    beat(c);
    refresh_wm(c);
    if (const int rr = revive(c, c->wm < c->next_seq)) return rr;
    return seq < c->wm ? 1 : 0;
}

int gpuos_sync(void* ctx, uint64_t upto, int64_t timeout_ns, uint64_t* err_seq, uint32_t* err_status) {
    gpuos_ctx* c = (gpuos_ctx*)ctx;
    if (!c) return GPUOS_E_INVAL;
    const uint64_t t0 = now_ns();
    uint32_t spins = 0;
    for (;;) {
        {
            std::lock_guard<std::mutex> g(c->mu);
            const uint64_t target = (upto == GPUOS_SEQ_ALL || upto >= c->next_seq) ? c->next_seq : upto + 1;
            refresh_wm(c);
            if (c->wm >= target) {
                for (size_t i = 0; i < c->errors.size(); ++i) {
                    if (c->errors[i].seq < target) {
                        if (err_seq) *err_seq = c->errors[i].seq;
                        if (err_status) *err_status = c->errors[i].st;
                        c->errors.erase(c->errors.begin() + (long)i);
                        return GPUOS_E_DEVICE;
                    }
                }
                return GPUOS_OK;
            }
            beat(c);
            if (const int rr = revive(c, true)) return rr;  // an idle exit: launched again
            if (!c->loopback && c->running && hipEventQuery(c->ev_stop) == hipSuccess) {
                // the executor exited with work outstanding
                return GPUOS_E_DEVICE;
            }
        }
        if (timeout_ns >= 0 && now_ns() - t0 > (uint64_t)timeout_ns) return GPUOS_E_TIMEOUT;
        if (++spins > 20000) std::this_thread::yield();
        else GPUOS_PAUSE();
    }
}

int gpuos_pause(void* ctx, int64_t timeout_ns) {
    gpuos_ctx* c = (gpuos_ctx*)ctx;
    if (!c) return GPUOS_E_INVAL;
    int rc = gpuos_sync(ctx, GPUOS_SEQ_ALL, timeout_ns, nullptr, nullptr);
    if (rc != GPUOS_OK && rc != GPUOS_E_DEVICE) return rc;
    std::lock_guard<std::mutex> g(c->mu);
    int rs = executor_stop(c, timeout_ns < 0 ? 10000000000ll : timeout_ns);
    return rs ? rs : rc;
}

int gpuos_resume(void* ctx) {
    gpuos_ctx* c = (gpuos_ctx*)ctx;
    if (!c) return GPUOS_E_INVAL;
    std::lock_guard<std::mutex> g(c->mu);
    return executor_launch(c);
}

int gpuos_shutdown(void* ctx) {
    gpuos_ctx* c = (gpuos_ctx*)ctx;
    if (!c) return GPUOS_E_INVAL;
    int rc = GPUOS_OK;
    {
        std::lock_guard<std::mutex> g(c->mu);
        rc = executor_stop(c, 10000000000ll);
    }
    if (rc == GPUOS_E_TIMEOUT && c->running) {
        // the kernel is still resident: freeing its memory would fault it
        return rc;
    }
    free_ctx(c);
    return rc;
}

int gpuos_stats_get(void* ctx, gpuos_stats* out) {
    gpuos_ctx* c = (gpuos_ctx*)ctx;
    if (!c || !out) return GPUOS_E_INVAL;
    std::lock_guard<std::mutex> g(c->mu);
    beat(c);
    refresh_wm(c);
    memset(out, 0, sizeof(*out));
    out->idle_exits = c->idle_exits;
    out->submitted = c->submitted;
    out->completed = c->completed;
    out->full_rejections = c->full_rej;
    out->launches = c->launches;
    out->last_launch_ms = c->last_ms;
    out->total_launch_ms = c->total_ms;
    out->num_wgs = c->P.num_wgs;
    out->waves_per_wg = c->P.waves_per_wg;
    out->ring_entries = c->N;
    out->cu_count = c->cu_count;
    out->next_seq = c->next_seq;
    out->deps_explicit = c->deps_explicit;
    out->deps_range = c->deps_range;
    out->ns_submit = c->ns_submit;
    out->ns_blocked = c->ns_blocked;
    out->ns_annotate = c->ns_hazard;
    if (!c->loopback) {
        out->units = c->acc_units;
        out->dep_waits = c->acc_depw;
        out->fetch_batches = c->acc_batches;
        out->fetched = c->acc_fetched;
        if (c->running) {  // add the live launch's counters (workers add theirs when they exit)
            DevCtl d;
            if (hipMemcpyAsync(&d, c->dctl, sizeof(DevCtl), hipMemcpyDeviceToHost, c->aux) != hipSuccess)
                return GPUOS_E_HIP;
            if (hipStreamSynchronize(c->aux) != hipSuccess) return GPUOS_E_HIP;
            out->units += d.stat_units;
            out->dep_waits += d.stat_dep_waits;
            out->fetch_batches += d.stat_batches;
            out->fetched += d.stat_fetched;
        }
    } else {
        std::lock_guard<std::mutex> lg(c->lb_mu);
        out->units = c->lb_order.size();
        out->fetched = c->lb_order.size();
    }
    return GPUOS_OK;
}

int gpuos_loopback_order(void* ctx, uint64_t* out, uint64_t max, uint64_t* n_out) {
    gpuos_ctx* c = (gpuos_ctx*)ctx;
    if (!c || !c->loopback) return GPUOS_E_STATE;
    std::lock_guard<std::mutex> g(c->lb_mu);
    const uint64_t n = std::min<uint64_t>(max, c->lb_order.size());
    if (out) memcpy(out, c->lb_order.data(), n * 8);
    if (n_out) *n_out = c->lb_order.size();
    return GPUOS_OK;
}

int gpuos_ring_peek(void* ctx, uint64_t seq, gpuos_desc* out, uint16_t* extra) {
    gpuos_ctx* c = (gpuos_ctx*)ctx;
    if (!c || !out) return GPUOS_E_INVAL;
    std::lock_guard<std::mutex> g(c->mu);
    if (seq >= c->next_seq || seq + c->N < c->next_seq) return GPUOS_E_STATE;
    const uint64_t slot = seq & c->mask;
    memcpy(out, &c->ring[slot], sizeof(gpuos_desc));
    if (extra) {
        if (out->dep_delta[5]) memcpy(extra, &c->depx[slot * DEPX_WORDS], 8 * DEPX_WORDS);
        else memset(extra, 0, 8 * DEPX_WORDS);
    }
    return GPUOS_OK;
}

int gpuos_trace_read(void* ctx, gpuos_trace_rec* out, uint64_t max, uint64_t* n_out) {
    gpuos_ctx* c = (gpuos_ctx*)ctx;
    if (!c) return GPUOS_E_INVAL;
    std::lock_guard<std::mutex> g(c->mu);
    if (!c->trace || c->running) return GPUOS_E_STATE;
    const uint64_t n = std::min<uint64_t>(max, c->trace_cap);
    if (n_out) *n_out = c->trace_cap;
    if (n && out) {
        if (hipMemcpyAsync(out, c->trace, n * sizeof(gpuos_trace_rec), hipMemcpyDeviceToHost, c->aux) != hipSuccess)
            return GPUOS_E_HIP;
        if (hipStreamSynchronize(c->aux) != hipSuccess) return GPUOS_E_HIP;
    }
    return GPUOS_OK;
}

// ------------------------------------------------------------ baselines
uint64_t gpuos_eager_scratch_bytes(const gpuos_desc* descs, uint32_t count) {
    uint64_t m = COUNTER_AREA;
    for (uint32_t i = 0; i < count; ++i) {
        const uint32_t kind = descs[i].op_id;
        if (kind >= GPUOS_KIND_COUNT || kind == GPUOS_OP_EXPR || kind == GPUOS_OP_JIT) continue;
        const Plan p = make_plan(plan_in(kind, descs[i]));
        m = std::max<uint64_t>(m, p.scratch);
    }
    return m;
}

int gpuos_eager_submit(const gpuos_desc* descs, uint32_t count, void* hip_stream, void* scratch,
                       uint64_t scratch_bytes) {
    if (count && !descs) return GPUOS_E_INVAL;
    hipStream_t s = (hipStream_t)hip_stream;
    for (uint32_t i = 0; i < count; ++i) {
        const gpuos_desc& d = descs[i];
        if (d.op_id >= GPUOS_KIND_COUNT || d.op_id == GPUOS_OP_EXPR || d.op_id == GPUOS_OP_JIT)
            return GPUOS_E_INVAL;  // no table here
        const Plan p = make_plan(plan_in(d.op_id, d));
        if (p.status != GPUOS_ST_OK) return GPUOS_E_INVAL;
        if (p.scratch > 0 && (!scratch || p.scratch > scratch_bytes)) return GPUOS_E_INVAL;
        if (d.op_id == GPUOS_OP_NOP) {
            if (launch_null(s) != hipSuccess) return GPUOS_E_HIP;
            continue;
        }
        if (launch_eager(d, d.op_id, p.ntiles, (uint8_t*)scratch, s) != hipSuccess) return GPUOS_E_HIP;
    }
    return GPUOS_OK;
}

int gpuos_eager_submit_static(const gpuos_desc* descs, uint32_t count, void* hip_stream) {
    if (count && !descs) return GPUOS_E_INVAL;
    // every descriptor is checked before anything is launched
    bool split = false;
    for (uint32_t i = 0; i < count; ++i) {
        const gpuos_desc& d = descs[i];
        if (d.op_id >= GPUOS_KIND_COUNT || d.op_id == GPUOS_OP_EXPR || d.op_id == GPUOS_OP_JIT) return GPUOS_E_INVAL;
        const Plan p = make_plan(plan_in(d.op_id, d));
        if (p.status != GPUOS_ST_OK || p.scratch > GPUOS_EAGER_STATIC_SCRATCH_BYTES) return GPUOS_E_INVAL;
        split = split || p.scratch > 0;
    }
    if (count == 0) return GPUOS_OK;
    uint8_t* scr = nullptr;
    if (static_scratch(&scr) != hipSuccess) return GPUOS_E_HIP;
    hipStream_t s = (hipStream_t)hip_stream;
    // the split counters start at zero (each merge leaves them at zero, but
    // an earlier call may have ended early): a fill kernel, which a graph
    // capture records as an ordinary kernel node
    if (split && launch_fill_zero(scr, (uint32_t)COUNTER_AREA, s) != hipSuccess) return GPUOS_E_HIP;
    for (uint32_t i = 0; i < count; ++i) {
        const gpuos_desc& d = descs[i];
        if (d.op_id == GPUOS_OP_NOP) {
            if (launch_null(s) != hipSuccess) return GPUOS_E_HIP;
            continue;
        }
        const Plan p = make_plan(plan_in(d.op_id, d));
        if (launch_eager(d, d.op_id, p.ntiles, scr, s) != hipSuccess) return GPUOS_E_HIP;
    }
    return GPUOS_OK;
}

int gpuos_graph_build(const gpuos_desc* descs, uint32_t count, void* hip_stream, void* scratch,
                      uint64_t scratch_bytes, void** graph_exec) {
    if (!graph_exec) return GPUOS_E_INVAL;
    *graph_exec = nullptr;
    hipStream_t s = (hipStream_t)hip_stream;
    if (hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) != hipSuccess) return GPUOS_E_HIP;
    int rc = gpuos_eager_submit(descs, count, hip_stream, scratch, scratch_bytes);
    hipGraph_t g = nullptr;
    hipError_t e = hipStreamEndCapture(s, &g);
    if (rc) { if (g) (void)hipGraphDestroy(g); return rc; }
    if (e != hipSuccess) return GPUOS_E_HIP;
    hipGraphExec_t ge = nullptr;
    e = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    if (e != hipSuccess) return GPUOS_E_HIP;
    *graph_exec = ge;
    return GPUOS_OK;
}

int gpuos_graph_launch(void* graph_exec, void* hip_stream) {
    if (!graph_exec) return GPUOS_E_INVAL;
    return hipGraphLaunch((hipGraphExec_t)graph_exec, (hipStream_t)hip_stream) == hipSuccess ? GPUOS_OK : GPUOS_E_HIP;
}

int gpuos_graph_destroy(void* graph_exec) {
    if (!graph_exec) return GPUOS_E_INVAL;
    return hipGraphExecDestroy((hipGraphExec_t)graph_exec) == hipSuccess ? GPUOS_OK : GPUOS_E_HIP;
}

int gpuos_null_launch_bench(void* hip_stream, uint32_t n, double* ns_async, double* ns_sync) {
    if (n == 0) return GPUOS_E_INVAL;
    hipStream_t s = (hipStream_t)hip_stream;
    if (launch_null(s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess) return GPUOS_E_HIP;
    uint64_t t0 = now_ns();
    for (uint32_t i = 0; i < n; ++i)
        if (launch_null(s) != hipSuccess) return GPUOS_E_HIP;
    uint64_t t1 = now_ns();
    if (hipStreamSynchronize(s) != hipSuccess) return GPUOS_E_HIP;
    if (ns_async) *ns_async = (double)(t1 - t0) / n;
    const uint32_t m = n < 2000 ? n : 2000;
    t0 = now_ns();
    for (uint32_t i = 0; i < m; ++i) {
        if (launch_null(s) != hipSuccess) return GPUOS_E_HIP;
        if (hipStreamSynchronize(s) != hipSuccess) return GPUOS_E_HIP;
    }
    t1 = now_ns();
    if (ns_sync) *ns_sync = (double)(t1 - t0) / m;
    return GPUOS_OK;
}

int gpuos_latency_bench(void* ctx, const gpuos_desc* descs, uint32_t count, double* out_us) {
    if (!ctx || (count && (!descs || !out_us))) return GPUOS_E_INVAL;
    for (uint32_t i = 0; i < count; ++i) {
        const uint64_t t0 = now_ns();
        uint64_t seq = 0;
        int rc = gpuos_submit(ctx, descs + i, 1, GPUOS_SUBMIT_BLOCK, &seq);
        if (rc != GPUOS_OK) return rc;
        rc = gpuos_sync(ctx, seq, 10'000'000'000ll, nullptr, nullptr);
        if (rc != GPUOS_OK) return rc;
        out_us[i] = (double)(now_ns() - t0) * 1e-3;
    }
    return GPUOS_OK;
}

int gpuos_hbm_probe_grid(const void* src, void* dst, uint64_t bytes, uint32_t mode, uint32_t reps,
                         uint32_t workgroups, void* hip_stream, double* gbs) {
    if (!src || !dst || bytes == 0 || (bytes & 15u) || bytes > (1ull << 30) || mode > 1 || reps == 0 ||
        workgroups > 4096)
        return GPUOS_E_INVAL;
    if (mode == 0 && bytes < 4096) return GPUOS_E_INVAL;
    hipStream_t s = (hipStream_t)hip_stream;
    uint32_t grid = workgroups;
    if (grid == 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            return GPUOS_E_HIP;
        grid = (uint32_t)cus;
    }
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess) return GPUOS_E_HIP;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return GPUOS_E_HIP;
    }
    int rc = GPUOS_OK;
    const bool copy = mode == 1;
    float ms = 0.0f;
    if (launch_hbm_probe(src, dst, (uint32_t)bytes, copy, grid, s) != hipSuccess ||
        hipEventRecord(e0, s) != hipSuccess) {
        rc = GPUOS_E_HIP;
    } else {
        for (uint32_t i = 0; i < reps && rc == GPUOS_OK; ++i)
            if (launch_hbm_probe(src, dst, (uint32_t)bytes, copy, grid, s) != hipSuccess) rc = GPUOS_E_HIP;
        if (rc == GPUOS_OK && (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                               hipEventElapsedTime(&ms, e0, e1) != hipSuccess))
            rc = GPUOS_E_HIP;
    }
    if (rc == GPUOS_OK && gbs) *gbs = ms > 0.0f ? (copy ? 2.0 : 1.0) * (double)bytes * reps / (ms * 1e-3) / 1e9 : 0.0;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return rc;
}

int gpuos_hbm_probe(const void* src, void* dst, uint64_t bytes, uint32_t mode, uint32_t reps, void* hip_stream,
                    double* gbs) {
    return gpuos_hbm_probe_grid(src, dst, bytes, mode, reps, 0, hip_stream, gbs);
}

}  // extern "C"
