// Host-side ordering of concurrently executed descriptors.
//
// The pages keep eager (sequential) semantics while many device waves claim
// descriptors independently, but give no ordering mechanism.  The reading
// taken here: the producer annotates each descriptor with the earlier
// descriptors it conflicts with -- read-after-write, write-after-read and
// write-after-write on byte ranges -- and the executor waits for those to
// complete before running it.  Descriptors without conflicts run
// concurrently.
//
// Data structure.  Byte intervals are kept in clusters: a cluster covers a
// contiguous span that accesses have touched (in practice one tensor) and
// holds a small sorted vector of disjoint intervals, each with its last
// writer and the readers since that write.  An access costs one map lookup
// to find its cluster plus a few edits of a short vector; clusters are
// created or merged only when an access reaches memory not seen before.
//  - A read never splits an interval: the reader is recorded on every
//    interval it overlaps, whole, so intervals are created only by writes
//    (which coalesce what they cover) and by reads of untouched bytes.  A
//    later write to the part that was not read then waits for that reader
//    too: an extra wait, never a missing one.
//  - A writer's dependency on the interval's previous writer is dropped when
//    the interval has a live reader: every reader waited for that writer.
//  - An interval keeps up to MAXR readers; beyond that it keeps the oldest
//    overflowed reader, and a writer then depends on the whole range from it
//    (reported through `range_from`).
//  - Clusters are found through a small direct-mapped cache keyed by the
//    access's start address, else the map; a merge invalidates the cache.
//  - A cluster that holds more than SPLIT_AT live intervals (a long-lived
//    buffer written piece by piece, such as an output arena) is split in two
//    at an interval boundary, so that inserting an interval never moves more
//    than a few dozen of them.
// Sequence numbers below the host's completion watermark are known complete
// and are never returned.
#pragma once
#include <stdint.h>

#include <algorithm>
#include <deque>
#include <iterator>
#include <map>
#include <vector>

namespace gpuos {

struct Access {
    uint64_t lo, hi;  // byte range [lo, hi)
    bool write;
};

class HazardTracker {
public:
    static constexpr int MAXR = 30;
    static constexpr size_t SPLIT_AT = 96;

    // Appends to `deps` every live seq (>= floor) that `seq` must wait for
    // and lowers *range_from to the first seq of a range that must be waited
    // for entirely (left untouched if none); then records the accesses.
    void analyze(uint64_t seq, const Access* acc, int n, uint64_t floor, std::vector<uint64_t>& deps,
                 uint64_t* range_from) {
        // resolve each access's cluster once (a merge invalidates earlier
        // ones: resolve again until no merge happens)
        Cluster* cp[24];
        if (n > 24) n = 24;
        for (int round = 0; round < 4; ++round) {
            const uint64_t m0 = merges_;
            for (int i = 0; i < n; ++i) cp[i] = acc[i].hi > acc[i].lo ? &cluster_for(acc[i].lo, acc[i].hi) : nullptr;
            if (merges_ == m0) break;
        }
        bool distinct = true;
        for (int i = 0; i < n && distinct; ++i)
            for (int j = 0; j < i; ++j)
                if (cp[i] && cp[i] == cp[j]) { distinct = false; break; }
        if (distinct) {
            // no two accesses share a cluster: each can be collected and
            // recorded in one pass without seeing the others
            for (int i = 0; i < n; ++i) {
                if (!cp[i]) continue;
                collect(*cp[i], acc[i], floor, deps, range_from);
                if (acc[i].write) record_write(*cp[i], acc[i].lo, acc[i].hi, seq);
                else record_read(*cp[i], acc[i].lo, acc[i].hi, seq, floor);
                if (cp[i]->regs.size() > cp[i]->prune_at) prune(*cp[i], floor);
            }
        } else {
            for (int i = 0; i < n; ++i)
                if (cp[i]) collect(*cp[i], acc[i], floor, deps, range_from);
            for (int pass = 0; pass < 2; ++pass) {
                for (int i = 0; i < n; ++i) {
                    if (!cp[i] || acc[i].write != (pass == 1)) continue;
                    if (acc[i].write) record_write(*cp[i], acc[i].lo, acc[i].hi, seq);
                    else record_read(*cp[i], acc[i].lo, acc[i].hi, seq, floor);
                    if (cp[i]->regs.size() > cp[i]->prune_at) prune(*cp[i], floor);
                }
            }
        }
        // split large clusters only now: the pointers in cp stay valid above
        for (int i = 0; i < n; ++i)
            if (cp[i] && cp[i]->regs.size() > SPLIT_AT) split(*cp[i], floor);
    }

    void clear() {
        cl_.clear();
        store_.clear();
        free_.clear();
        std::fill(hits_.begin(), hits_.end(), Hit{});
    }
    size_t size() const {
        size_t n = 0;
        for (auto& kv : cl_) n += kv.second->regs.size();
        return n;
    }
    size_t clusters() const { return cl_.size(); }

private:
    struct Region {
        uint64_t lo, hi;
        uint64_t writer;    // 0 = none
        uint64_t overflow;  // 0 = none; else the oldest reader not kept inline
        uint32_t nr;
        uint64_t readers[MAXR];
    };
    struct Cluster {
        uint64_t lo = 0, hi = 0;  // lo is also the map key
        std::vector<Region> regs;  // sorted by lo, disjoint, inside [key, hi)
        size_t prune_at = 64;
        bool alive = false;
    };
    // Clusters live in a pool and are recycled, never freed, so a pointer to
    // one always points to some cluster object; cl_ maps live ones by start.
    std::map<uint64_t, Cluster*> cl_;
    std::deque<Cluster> store_;
    std::vector<Cluster*> free_;
    uint64_t merges_ = 0;
    // A direct-mapped cache from an access's start address to its cluster,
    // checked against the cluster's current span (merges retire clusters,
    // splits shrink them, recycling reuses them).
    struct Hit {
        uint64_t lo = 0;
        Cluster* c = nullptr;
    };
    static constexpr size_t NHIT = 4096;  // 2^12: the hash below keeps 12 bits
    std::vector<Hit> hits_ = std::vector<Hit>(NHIT);

    Cluster* alloc_cluster() {
        Cluster* c;
        if (!free_.empty()) {
            c = free_.back();
            free_.pop_back();
        } else {
            store_.emplace_back();
            c = &store_.back();
        }
        c->alive = true;
        c->prune_at = 64;
        return c;
    }
    void retire(Cluster* c) {
        c->alive = false;
        c->lo = c->hi = 0;
        c->regs.clear();
        free_.push_back(c);
    }

    static Region make(uint64_t lo, uint64_t hi, uint64_t writer) {
        Region r;
        r.lo = lo;
        r.hi = hi;
        r.writer = writer;
        r.overflow = 0;
        r.nr = 0;
        return r;
    }

    // The cluster containing [lo, hi), created, extended or merged as needed.
    Cluster& cluster_for(uint64_t lo, uint64_t hi) {
        Hit& h = hits_[(lo * 0x9E3779B97F4A7C15ull) >> 52];  // Fibonacci hash to 12 bits
        if (h.c && h.lo == lo && h.c->alive && h.c->lo <= lo && h.c->hi >= hi) return *h.c;
        auto it = cl_.upper_bound(lo);
        if (it != cl_.begin()) {
            auto p = std::prev(it);
            if (p->second->hi > lo) it = p;
        }
        if (it != cl_.end() && it->first <= lo && it->second->hi >= hi) {  // common case
            h.lo = lo;
            h.c = it->second;
            return *it->second;
        }
        // collect every cluster overlapping [lo, hi)
        ++merges_;
        auto first = it;
        uint64_t nlo = lo, nhi = hi;
        size_t k = 0;
        for (auto j = it; j != cl_.end() && j->first < hi; ++j, ++k) {
            nlo = std::min(nlo, j->first);
            nhi = std::max(nhi, j->second->hi);
        }
        std::vector<Region> regs;
        auto j = first;
        for (size_t q = 0; q < k; ++q) {
            regs.insert(regs.end(), j->second->regs.begin(), j->second->regs.end());
            retire(j->second);
            j = cl_.erase(j);
        }
        Cluster* m = alloc_cluster();
        m->lo = nlo;
        m->hi = nhi;
        m->regs = std::move(regs);
        m->prune_at = std::max<size_t>(64, 2 * m->regs.size());
        cl_.emplace_hint(j, nlo, m);
        return *m;
    }

    // index of the first region with hi > x
    static size_t first_after(const std::vector<Region>& v, uint64_t x) {
        size_t a = 0, b = v.size();
        while (a < b) {
            const size_t m = (a + b) >> 1;
            if (v[m].hi > x) b = m; else a = m + 1;
        }
        return a;
    }

    // readers are appended in sequence order, so the array is sorted and the
    // completed ones form a prefix
    static void prune_readers(Region& r, uint64_t floor) {
        if (r.overflow && r.overflow < floor) r.overflow = 0;
        if (r.nr == 0 || r.readers[0] >= floor) return;
        uint32_t k = 1;
        while (k < r.nr && r.readers[k] < floor) ++k;
        std::copy(r.readers + k, r.readers + r.nr, r.readers);
        r.nr -= k;
    }

    void collect(Cluster& c, const Access& a, uint64_t floor, std::vector<uint64_t>& deps, uint64_t* range_from) {
        for (size_t i = first_after(c.regs, a.lo); i < c.regs.size() && c.regs[i].lo < a.hi; ++i) {
            Region& r = c.regs[i];
            prune_readers(r, floor);
            const bool live_w = r.writer >= floor && r.writer != 0;
            if (!a.write || (r.nr == 0 && !r.overflow)) {
                if (live_w) deps.push_back(r.writer);
                continue;
            }
            for (uint32_t k = 0; k < r.nr; ++k) deps.push_back(r.readers[k]);
            if (r.overflow && r.overflow < *range_from) *range_from = r.overflow;
        }
    }

    static void record_write(Cluster& c, uint64_t lo, uint64_t hi, uint64_t seq) {
        auto& v = c.regs;
        const size_t i0 = first_after(v, lo);
        size_t i1 = i0;
        while (i1 < v.size() && v[i1].lo < hi) ++i1;
        if (i1 == i0 + 1 && v[i0].lo == lo && v[i0].hi == hi) {  // exact match: reuse
            v[i0].writer = seq;
            v[i0].nr = 0;
            v[i0].overflow = 0;
            return;
        }
        Region parts[3];
        int np = 0;
        if (i1 > i0 && v[i0].lo < lo) { parts[np] = v[i0]; parts[np].hi = lo; ++np; }
        parts[np++] = make(lo, hi, seq);
        if (i1 > i0 && v[i1 - 1].hi > hi) { parts[np] = v[i1 - 1]; parts[np].lo = hi; ++np; }
        const size_t old = i1 - i0;
        if ((size_t)np <= old) {
            std::copy(parts, parts + np, v.begin() + (long)i0);
            v.erase(v.begin() + (long)(i0 + np), v.begin() + (long)i1);
        } else {
            std::copy(parts, parts + old, v.begin() + (long)i0);
            v.insert(v.begin() + (long)(i0 + old), parts + old, parts + np);
        }
    }

    static void add_reader(Region& r, uint64_t seq) {
        if (r.nr < MAXR) {
            r.readers[r.nr++] = seq;
            return;
        }
        const uint64_t oldest = r.readers[0];
        if (!r.overflow || oldest < r.overflow) r.overflow = oldest;
        std::copy(r.readers + 1, r.readers + MAXR, r.readers);
        r.readers[MAXR - 1] = seq;
    }

    static void record_read(Cluster& c, uint64_t lo, uint64_t hi, uint64_t seq, uint64_t floor) {
        auto& v = c.regs;
        size_t i = first_after(v, lo);
        uint64_t cur = lo;
        while (cur < hi) {
            if (i == v.size() || v[i].lo > cur) {
                // gap [cur, next start or hi): an interval with no writer
                const uint64_t end = (i == v.size() || v[i].lo > hi) ? hi : v[i].lo;
                Region g = make(cur, end, 0);
                g.nr = 1;
                g.readers[0] = seq;
                v.insert(v.begin() + (long)i, g);
                ++i;
                cur = end;
                continue;
            }
            prune_readers(v[i], floor);
            add_reader(v[i], seq);
            cur = v[i].hi;
            ++i;
        }
    }

    // Prune, and if the cluster is still large move its upper half into a
    // cluster of its own (pool entries do not move, so other Cluster
    // pointers stay valid).
    void split(Cluster& c, uint64_t floor) {
        prune(c, floor);
        if (c.regs.size() <= SPLIT_AT) return;
        const size_t mid = c.regs.size() / 2;
        Cluster* up = alloc_cluster();  // the pool is a deque: c stays valid
        up->lo = c.regs[mid].lo;
        up->hi = c.hi;
        up->regs.assign(c.regs.begin() + (long)mid, c.regs.end());
        up->prune_at = std::max<size_t>(64, 2 * up->regs.size());
        c.regs.resize(mid);
        c.hi = up->lo;
        c.prune_at = std::max<size_t>(64, 2 * c.regs.size());
        cl_.emplace(up->lo, up);
    }

    // drop intervals that carry no live information
    static void prune(Cluster& c, uint64_t floor) {
        auto& v = c.regs;
        size_t k = 0;
        for (size_t i = 0; i < v.size(); ++i) {
            prune_readers(v[i], floor);
            const bool live = (v[i].writer >= floor && v[i].writer != 0) || v[i].nr || v[i].overflow;
            if (live) v[k++] = v[i];
        }
        v.resize(k);
        c.prune_at = std::max<size_t>(64, 2 * v.size());
    }
};

}  // namespace gpuos
