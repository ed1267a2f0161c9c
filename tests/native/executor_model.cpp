// Host model of the executor's work-distribution protocol: one thread per
// wave, over bounds-checked arrays, using the executor's own index
// arithmetic (claim shards, ticket -> queue position, queue-entry encoding,
// queue capacity) from gpuos_internal.h.
//
// Modelled, as the executor does it (the lane-0 view of each wave):
//  - a host producer commits descriptors into a ring of N slots (stamp
//    protocol: slot free for seq s when stamp == s, committed with s + 1,
//    released by the executor with s + N);
//  - the fetcher (wave 0 of workgroup 0) reads up to 64 committed slots,
//    splits each descriptor into units, waits while the unit queue (Q
//    positions) would overrun the oldest incomplete descriptor, writes meta,
//    resets the slot's unit counter, writes one queue entry per unit and
//    publishes the queue tail; when the host asks it to stop it drains and
//    sets the device stop word;
//  - every other wave claims tickets from its workgroup's shard, holds up to
//    SLOTS claimed units, reads a unit's entry once the tail covers it,
//    waits for its dependencies (done[] of earlier descriptors), runs it,
//    counts it, and the last unit of a descriptor stores done[] and releases
//    the ring slot; a wave leaves once the stop is seen and it holds no
//    published unit.
// Checked: every array access in bounds (std::vector::at), every queue
// entry read is the one published for that position (not an older or newer
// one), the meta a worker reads belongs to the entry's descriptor, every
// unit runs exactly once, dependencies have completed before a unit runs,
// every descriptor completes, and every thread leaves (a watchdog reports a
// hang).  Prints "ok <config>" per configuration, or the first violation
// and exits with status 1.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <atomic>
#include <chrono>
#include <stdexcept>
#include <string>
#include <thread>
#include <vector>

#include "gpuos_internal.h"

constexpr uint64_t MODEL_PUBLISH_STEP = 32;
static_assert(gpuos::PUBLISH_STEP % MODEL_PUBLISH_STEP == 0, "the executor's step is a multiple of the model's");

using namespace gpuos;

namespace {

struct Body {
    uint32_t ntiles = 0;
    uint32_t ndeps = 0;
    uint16_t delta[4] = {0, 0, 0, 0};  // wait for seq - delta
};

struct Fail : std::runtime_error {
    using std::runtime_error::runtime_error;
};

struct Model {
    // configuration
    uint32_t num_wgs, waves, slots, S, N, Q;
    uint64_t M;  // descriptors
    uint64_t base;  // first sequence number
    // ring in "host memory"
    std::vector<std::atomic<uint64_t>> stamp;
    std::vector<Body> ring;
    std::atomic<uint64_t> hstop{0};
    // "device memory"
    std::vector<std::atomic<uint64_t>> done;
    std::vector<std::atomic<uint32_t>> tiles_done;
    std::vector<std::atomic<uint64_t>> queue, queue_tag;  // entry, and the position it was written for
    std::vector<std::atomic<uint64_t>> meta_ntiles, meta_ubegin, meta_seq;
    std::vector<Body> mirror;
    std::atomic<uint64_t> claim[CLAIM_SHARDS_MAX];
    std::atomic<uint64_t> q_tail{0}, dstop{0};
    // checking
    std::vector<std::atomic<uint32_t>> ran;  // per descriptor: units run
    std::vector<uint32_t> ntiles_of;         // per descriptor (host's copy)
    std::atomic<uint64_t> units_run{0};
    std::atomic<int> failed{0};
    std::string why;
    std::atomic<uint32_t> exited{0};

    Model(uint32_t wgs, uint32_t w, uint32_t sl, uint32_t n, uint32_t q, uint64_t m)
        : num_wgs(wgs), waves(w), slots(sl), N(n), Q(q), M(m), base(n),
          stamp(n), ring(n), done(n), tiles_done(n), queue(q), queue_tag(q), meta_ntiles(n), meta_ubegin(n),
          meta_seq(n), mirror(n), ran(m), ntiles_of(m) {
        S = claim_shards(num_wgs, waves, num_wgs);  // one workgroup per CU
        for (uint32_t i = 0; i < n; ++i) {
            stamp[i] = n + i;
            done[i] = i;
            tiles_done[i] = 0;
            meta_seq[i] = ~0ull;
        }
        for (uint32_t i = 0; i < q; ++i) queue_tag[i] = ~0ull;
        for (auto& c : claim) c = 0;
    }

    void fail(const std::string& w) {
        int z = 0;
        if (failed.compare_exchange_strong(z, 1)) why = w;
        throw Fail(w);
    }
};

uint64_t rnd_state = 0x9E3779B97F4A7C15ull;
uint64_t rnd() {  // SplitMix64 (the producer thread only)
    uint64_t z = (rnd_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

void producer(Model& m, bool stop_early) {
    const uint64_t mask = m.N - 1;
    for (uint64_t i = 0; i < m.M && !m.failed; ++i) {
        const uint64_t s = m.base + i;
        Body b;
        const uint64_t r = rnd() % 100;
        // unit counts the library accepts (at most max_units_per_descriptor)
        const uint64_t umax = max_units_per_descriptor(m.Q);
        b.ntiles = (uint32_t)std::min<uint64_t>(umax, r < 60 ? 1 + rnd() % 8 : r < 95 ? 1 + rnd() % 200 : 1 + rnd() % umax);
        b.ndeps = (uint32_t)(rnd() % 5);
        for (uint32_t k = 0; k < b.ndeps; ++k) {
            const uint64_t back = 1 + rnd() % std::min<uint64_t>(m.N - 1, 40);
            b.delta[k] = (uint16_t)(back <= i ? back : 0);
        }
        m.ntiles_of.at(i) = b.ntiles;
        while (m.stamp.at(s & mask).load(std::memory_order_acquire) != s) {
            if (m.failed) return;
            std::this_thread::yield();
        }
        m.ring.at(s & mask) = b;
        m.stamp.at(s & mask).store(s + 1, std::memory_order_release);
    }
    if (!stop_early) {  // a pause: wait for completion, then stop
        for (uint64_t i = 0; i < m.M && !m.failed; ++i) {
            const uint64_t s = m.base + i;
            while (m.stamp.at(s & mask).load(std::memory_order_acquire) < s + m.N && !m.failed)
                std::this_thread::yield();
        }
    }
    m.hstop.store(1, std::memory_order_release);  // (a shutdown stops with work in flight)
}

void fetcher(Model& m) {
    const uint64_t mask = m.N - 1;
    uint64_t f = m.base, u_next = 0, cw = m.base, cw_units = 0;
    for (;;) {
        uint32_t count = 0;
        while (count < 64 && m.stamp.at((f + count) & mask).load(std::memory_order_acquire) == f + count + 1) ++count;
        if (count == 0) {
            if (m.hstop.load(std::memory_order_acquire)) {
                if (m.stamp.at(f & mask).load(std::memory_order_acquire) == f + 1) continue;
                break;
            }
            if (m.failed) return;
            std::this_thread::yield();
            continue;
        }
        std::vector<uint64_t> inc(count);
        uint64_t acc = 0;
        for (uint32_t i = 0; i < count; ++i) {
            m.mirror.at((f + i) & mask) = m.ring.at((f + i) & mask);
            acc += m.mirror.at((f + i) & mask).ntiles;
            inc[i] = acc;
        }
        uint32_t fit = 0;
        for (bool fresh = false;; fresh = true) {
            if (fresh) {
                while (cw < f && m.done.at(cw & mask).load(std::memory_order_acquire) >= cw) ++cw;
                cw_units = cw < f ? m.meta_ubegin.at(cw & mask).load(std::memory_order_acquire) : u_next;
            }
            fit = 0;
            while (fit < count && units_fit(u_next + inc[fit], cw_units, m.Q)) ++fit;
            if (fit == count || (fresh && fit > 0)) break;
            if (!fresh) continue;
            if (m.failed) return;
            std::this_thread::yield();
        }
        for (uint32_t i = 0; i < fit; ++i) {
            const uint64_t slot = (f + i) & mask;
            const uint64_t nt = m.mirror.at(slot).ntiles;
            m.meta_ntiles.at(slot).store(nt, std::memory_order_relaxed);
            m.meta_ubegin.at(slot).store(u_next + inc[i] - nt, std::memory_order_relaxed);
            m.meta_seq.at(slot).store(f + i, std::memory_order_relaxed);
            m.tiles_done.at(slot).store(0, std::memory_order_relaxed);
        }
        const uint64_t T = inc[fit - 1];
        uint32_t j = 0;
        for (uint64_t wi = 0; wi < T; ++wi) {
            while (inc[j] <= wi) ++j;
            const uint64_t first = j ? inc[j - 1] : 0;
            const uint64_t pos = (u_next + wi) & (m.Q - 1);
            m.queue.at(pos).store(queue_entry(f + j, wi - first), std::memory_order_relaxed);
            m.queue_tag.at(pos).store(u_next + wi, std::memory_order_relaxed);
            // a large batch is published in prefixes, as the executor's
            // fetcher does every PUBLISH_STEP units; the model uses 32 so
            // that its small queues see prefixes too
            if ((wi + 1) % MODEL_PUBLISH_STEP == 0 && wi + 1 < T)
                m.q_tail.store(u_next + wi + 1, std::memory_order_release);
        }
        m.q_tail.store(u_next + T, std::memory_order_release);
        f += fit;
        u_next += T;
    }
    m.dstop.store(1, std::memory_order_release);
}

void worker(Model& m, uint32_t block) {
    const uint64_t mask = m.N - 1;
    const uint32_t shard = wg_shard(block, m.S);
    enum { FREE, CLAIMED, WAIT };
    int state[2] = {FREE, FREE};
    uint64_t su[2] = {0, 0}, seq[2] = {0, 0};
    uint32_t tile[2] = {0, 0};
    Body body[2];
    bool stop_seen = false;
    for (;;) {
        const uint64_t tail = m.q_tail.load(std::memory_order_acquire);
        int r = -1;
        for (uint32_t k = 0; k < m.slots; ++k) {
            if (state[k] != WAIT) continue;
            bool ready = true;
            for (uint32_t d = 0; d < body[k].ndeps; ++d)
                if (body[k].delta[d]) {
                    const uint64_t ds = seq[k] - body[k].delta[d];
                    ready = ready && m.done.at(ds & mask).load(std::memory_order_acquire) >= ds;
                }
            if (ready && (r < 0 || seq[k] < seq[r])) r = (int)k;
        }
        if (r >= 0) {
            const uint64_t s = seq[r], slot = s & mask;
            for (uint32_t d = 0; d < body[r].ndeps; ++d)
                if (body[r].delta[d] && m.stamp.at((s - body[r].delta[d]) & mask).load() < s - body[r].delta[d] + m.N &&
                    m.done.at((s - body[r].delta[d]) & mask).load() < s - body[r].delta[d])
                    m.fail("a unit ran before its dependency completed");
            if (m.ran.at(s - m.base).fetch_add(1) >= m.ntiles_of.at(s - m.base)) m.fail("a descriptor ran too many units");
            m.units_run.fetch_add(1);
            const uint32_t nt = (uint32_t)m.meta_ntiles.at(slot).load(std::memory_order_acquire);
            const uint32_t prev = m.tiles_done.at(slot).fetch_add(1, std::memory_order_acq_rel);
            if (prev + 1 > nt) m.fail("unit counter overran the descriptor's units");
            if (prev + 1 == nt) {
                m.done.at(slot).store(s, std::memory_order_release);
                m.stamp.at(slot).store(s + m.N, std::memory_order_release);
            }
            state[r] = FREE;
        }
        for (uint32_t k = 0; k < m.slots; ++k) {
            if (state[k] != FREE) continue;
            su[k] = ticket_unit(m.claim[shard].fetch_add(1, std::memory_order_relaxed), m.S, shard);
            state[k] = CLAIMED;
        }
        bool any_wait = false, fresh = false;
        for (uint32_t k = 0; k < m.slots; ++k) {
            if (state[k] == CLAIMED && tail > su[k]) {
                const uint64_t pos = su[k] & (m.Q - 1);
                const uint64_t ent = m.queue.at(pos).load(std::memory_order_relaxed);
                if (m.queue_tag.at(pos).load(std::memory_order_relaxed) != su[k])
                    m.fail("queue position " + std::to_string(pos) + " holds another unit than the claimed one");
                seq[k] = entry_seq(ent);
                tile[k] = entry_tile(ent);
                const uint64_t slot = seq[k] & mask;
                if (m.meta_seq.at(slot).load(std::memory_order_relaxed) != seq[k]) m.fail("meta of another descriptor");
                if (tile[k] >= m.meta_ntiles.at(slot).load()) m.fail("unit index beyond the descriptor's units");
                body[k] = m.mirror.at(slot);
                state[k] = WAIT;
                fresh = true;
            }
            any_wait = any_wait || state[k] == WAIT;
        }
        if (r >= 0 || fresh) continue;
        if (stop_seen && !any_wait) break;
        if (m.dstop.load(std::memory_order_acquire)) {
            stop_seen = true;
            continue;
        }
        if (m.failed) return;
        std::this_thread::yield();
    }
}

int run(uint32_t wgs, uint32_t waves, uint32_t slots, uint32_t N, uint32_t Q, uint64_t M, bool stop_early,
        uint64_t seed) {
    rnd_state = seed;
    Model m(wgs, waves, slots, N, Q, M);
    std::vector<std::thread> th;
    auto guard = [&m](auto fn) {
        return [&m, fn]() {
            try {
                fn();
            } catch (const Fail&) {
            } catch (const std::out_of_range& e) {
                int z = 0;
                if (m.failed.compare_exchange_strong(z, 1)) m.why = std::string("out of bounds: ") + e.what();
            }
            m.exited.fetch_add(1);
        };
    };
    th.emplace_back(guard([&] { producer(m, stop_early); }));
    th.emplace_back(guard([&] { fetcher(m); }));
    uint32_t nworkers = 0;
    for (uint32_t b = 0; b < wgs; ++b)
        for (uint32_t w = 0; w < waves; ++w) {
            if (b == 0 && w == 0) continue;  // the fetcher
            th.emplace_back(guard([&m, b] { worker(m, b); }));
            ++nworkers;
        }
    const auto t0 = std::chrono::steady_clock::now();
    while (m.exited.load() < th.size()) {
        if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(15)) {
            int z = 0;
            if (m.failed.compare_exchange_strong(z, 1)) m.why = "hang: threads did not leave";
            // let the spinning threads see `failed` and leave
            std::this_thread::sleep_for(std::chrono::seconds(2));
            break;
        }
        std::this_thread::sleep_for(std::chrono::milliseconds(2));
    }
    for (auto& t : th)
        if (t.joinable()) t.join();
    char cfg[160];
    snprintf(cfg, sizeof cfg, "wgs=%u waves=%u slots=%u shards=%u ring=%u queue=%u descriptors=%llu stop=%s",
             wgs, waves, slots, m.S, N, Q, (unsigned long long)M, stop_early ? "early" : "after");
    if (!m.failed) {
        uint64_t total = 0;
        for (uint64_t i = 0; i < M; ++i) {
            total += m.ntiles_of[i];
            if (m.ran[i] != m.ntiles_of[i]) { m.failed = 1; m.why = "descriptor " + std::to_string(i) + " ran "
                                              + std::to_string(m.ran[i].load()) + " of its units"; break; }
            const uint64_t s = m.base + i;
            if (i + m.N >= M && m.stamp[s & (N - 1)] != s + N) { m.failed = 1; m.why = "slot not released"; break; }
        }
        if (!m.failed && m.units_run != total) { m.failed = 1; m.why = "unit count"; }
    }
    if (m.failed) {
        printf("FAIL %s: %s\n", cfg, m.why.c_str());
        return 1;
    }
    printf("ok %s\n", cfg);
    return 0;
}

}  // namespace

int main(int argc, char** argv) {
    setvbuf(stdout, nullptr, _IOLBF, 0);
    const uint64_t M = argc > 1 ? strtoull(argv[1], nullptr, 10) : 3000;
    struct C { uint32_t wgs, waves, slots, N, Q; };
    const C cfgs[] = {{2, 1, 1, 8, 4096}, {3, 1, 1, 64, 4096}, {3, 1, 2, 8, 4096}, {9, 1, 2, 64, 4096},
                      {9, 1, 1, 512, 4096}, {5, 2, 1, 64, 8192}, {8, 1, 1, 64, 4096}, {8, 2, 2, 8, 4096},
                      {12, 4, 2, 64, 4096}, {16, 2, 2, 512, 4096}, {10, 1, 2, 128, 4096}, {4, 4, 1, 32, 4096},
                      // more worker workgroups than claim shards: shards served by two workgroups
                      {20, 1, 1, 64, 4096}, {24, 2, 2, 64, 256},
                      // small unit queues: the fetcher keeps waiting for capacity
                      {2, 1, 1, 64, 64}, {3, 1, 2, 64, 128}, {9, 1, 2, 128, 256}, {12, 4, 2, 64, 64}};
    int rc = 0;
    uint64_t seed = 1;
    for (const C& c : cfgs)
        for (int early = 0; early < 2; ++early)
            rc |= run(c.wgs, c.waves, c.slots, c.N, c.Q, M, early != 0, seed++);
    return rc;
}
