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
// contiguous span that accesses have touched (in practice one tensor, or one
// arena) and holds a small sorted vector of disjoint intervals, each with
// its last writer and the readers since that write.  An access costs one
// cluster lookup plus a few edits of a short vector; clusters are created,
// extended or merged only when an access reaches memory not seen before.
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
//  - Readers are kept as the low 32 bits of their sequence numbers (a live
//    one is at most a ring's length older than the descriptor being
//    annotated, so the full number is the largest one not above it with
//    those bits) and are dropped from the front by advancing a start index,
//    so an interval is 160 bytes and nothing is shifted when readers retire.
//  - Clusters are found through a small direct-mapped cache keyed by the
//    access's start address, else by binary search in a sorted array of
//    cluster starts.  An access that reaches past one cluster's span, and
//    touches no other, extends that cluster in place; only an access that
//    touches several clusters merges them (moving the intervals of the later
//    ones into the first).
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
#include <vector>

namespace gpuos {

struct Access {
    uint64_t lo, hi;  // byte range [lo, hi)
    bool write;
};

class HazardTracker {
public:
    static constexpr uint32_t MAXR = 30;
    static constexpr size_t SPLIT_AT = 96;

    // Appends to `deps` every live seq (>= floor) that `seq` must wait for
    // and lowers *range_from to the first seq of a range that must be waited
    // for entirely (left untouched if none); then records the accesses.
    void analyze(uint64_t seq, const Access* acc, int n, uint64_t floor, std::vector<uint64_t>& deps,
                 uint64_t* range_from) {
        cur_ = seq;
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
                if (acc[i].write) {
                    collect(*cp[i], acc[i], floor, deps, range_from);
                    record_write(*cp[i], acc[i].lo, acc[i].hi, seq);
                } else {
                    read_pass(*cp[i], acc[i].lo, acc[i].hi, seq, floor, deps);
                }
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
        idx_.clear();
        store_.clear();
        free_.clear();
        std::fill(hits_.begin(), hits_.end(), Hit{});
    }
    size_t size() const {
        size_t n = 0;
        for (const Entry& e : idx_) n += e.c->regs.size();
        return n;
    }
    size_t clusters() const { return idx_.size(); }

private:
    struct Region {
        uint64_t lo, hi;
        uint64_t writer;    // 0 = none
        uint64_t overflow;  // 0 = none; else the oldest reader not kept
        uint16_t r0, nr;    // the kept readers are rd[r0 .. nr), in sequence order
        uint32_t rd[MAXR];  // low 32 bits of the readers' sequence numbers
    };
    struct Cluster {
        uint64_t lo = 0, hi = 0;
        std::vector<Region> regs;  // sorted by lo, disjoint, inside [lo, hi)
        size_t prune_at = 64;
        bool alive = false;
    };
    // Clusters live in a pool and are recycled, never freed, so a pointer to
    // one always points to some cluster object; idx_ lists the live ones,
    // sorted by start.
    struct Entry {
        uint64_t lo;
        Cluster* c;
    };
    std::vector<Entry> idx_;
    std::deque<Cluster> store_;
    std::vector<Cluster*> free_;
    uint64_t merges_ = 0;
    uint64_t cur_ = 0;  // the sequence number being annotated
    // A direct-mapped cache from an access's start address to its cluster,
    // checked against the cluster's current span (merges retire clusters,
    // splits shrink them, recycling reuses them).
    struct Hit {
        uint64_t lo = 0;
        Cluster* c = nullptr;
    };
    static constexpr size_t NHIT = 4096;  // 2^12: the hash below keeps 12 bits
    std::vector<Hit> hits_ = std::vector<Hit>(NHIT);

    // full sequence number of a kept reader: the largest one not above the
    // descriptor being annotated that has these low 32 bits
    uint64_t widen(uint32_t r) const { return cur_ - (uint32_t)((uint32_t)cur_ - r); }

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
        r.r0 = r.nr = 0;
        return r;
    }

    // index of the first cluster starting above x
    size_t idx_upper(uint64_t x) const {
        size_t a = 0, b = idx_.size();
        while (a < b) {
            const size_t m = (a + b) >> 1;
            if (idx_[m].lo > x) b = m; else a = m + 1;
        }
        return a;
    }

    // The cluster containing [lo, hi), created, extended or merged as needed.
    Cluster& cluster_for(uint64_t lo, uint64_t hi) {
        Hit& h = hits_[(lo * 0x9E3779B97F4A7C15ull) >> 52];  // Fibonacci hash to 12 bits
        if (h.c && h.lo == lo && h.c->alive && h.c->lo <= lo && h.c->hi >= hi) return *h.c;
        // clusters overlapping [lo, hi): idx_[first, last)
        const size_t p = idx_upper(lo);
        size_t first = p;
        if (p > 0 && idx_[p - 1].c->hi > lo) first = p - 1;
        size_t last = first;
        while (last < idx_.size() && idx_[last].lo < hi) ++last;
        Cluster* c;
        if (last == first) {  // untouched memory: a new cluster
            c = alloc_cluster();
            c->lo = lo;
            c->hi = hi;
            idx_.insert(idx_.begin() + (long)first, Entry{lo, c});
        } else {
            c = idx_[first].c;
            if (last > first + 1) {
                // several clusters: move the later ones' intervals into the
                // first (all are sorted and lie above it)
                ++merges_;
                for (size_t q = first + 1; q < last; ++q) {
                    Cluster* o = idx_[q].c;
                    c->regs.insert(c->regs.end(), o->regs.begin(), o->regs.end());
                    c->hi = std::max(c->hi, o->hi);
                    retire(o);
                }
                idx_.erase(idx_.begin() + (long)(first + 1), idx_.begin() + (long)last);
                c->prune_at = std::max<size_t>(64, 2 * c->regs.size());
            }
            // extend in place (no other cluster overlaps [lo, hi) now)
            if (lo < c->lo) {
                c->lo = lo;
                idx_[first].lo = lo;
            }
            if (hi > c->hi) c->hi = hi;
        }
        h.lo = lo;
        h.c = c;
        return *c;
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

    // readers are appended in sequence order, so the completed ones (below
    // the watermark) form a prefix of the kept ones
    void prune_readers(Region& r, uint64_t floor) const {
        if (r.overflow && r.overflow < floor) r.overflow = 0;
        while (r.r0 < r.nr && widen(r.rd[r.r0]) < floor) ++r.r0;
        if (r.r0 == r.nr) r.r0 = r.nr = 0;
    }

    void collect(Cluster& c, const Access& a, uint64_t floor, std::vector<uint64_t>& deps, uint64_t* range_from) {
        for (size_t i = first_after(c.regs, a.lo); i < c.regs.size() && c.regs[i].lo < a.hi; ++i) {
            Region& r = c.regs[i];
            prune_readers(r, floor);
            const bool live_w = r.writer >= floor && r.writer != 0;
            if (!a.write || (r.r0 == r.nr && !r.overflow)) {
                if (live_w) deps.push_back(r.writer);
                continue;
            }
            for (uint32_t k = r.r0; k < r.nr; ++k) deps.push_back(widen(r.rd[k]));
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
            v[i0].r0 = v[i0].nr = 0;
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

    void add_reader(Region& r, uint64_t seq) const {
        if (r.nr == MAXR) {
            if (r.r0 > 0) {  // room at the front: move the kept readers down
                std::copy(r.rd + r.r0, r.rd + r.nr, r.rd);
                r.nr = (uint16_t)(r.nr - r.r0);
                r.r0 = 0;
            } else {
                const uint64_t oldest = widen(r.rd[0]);
                if (!r.overflow || oldest < r.overflow) r.overflow = oldest;
                std::copy(r.rd + 1, r.rd + MAXR, r.rd);
                r.nr = MAXR - 1;
            }
        }
        r.rd[r.nr++] = (uint32_t)seq;
    }

    void record_read(Cluster& c, uint64_t lo, uint64_t hi, uint64_t seq, uint64_t floor) const {
        auto& v = c.regs;
        size_t i = first_after(v, lo);
        uint64_t cur = lo;
        while (cur < hi) {
            if (i == v.size() || v[i].lo > cur) {
                // gap [cur, next start or hi): an interval with no writer
                const uint64_t end = (i == v.size() || v[i].lo > hi) ? hi : v[i].lo;
                Region g = make(cur, end, 0);
                g.nr = 1;
                g.rd[0] = (uint32_t)seq;
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

    // collect and record_read of one read in a single pass: each interval it
    // overlaps yields its live writer and gets the reader; gaps become
    // intervals with no writer
    void read_pass(Cluster& c, uint64_t lo, uint64_t hi, uint64_t seq, uint64_t floor,
                   std::vector<uint64_t>& deps) const {
        auto& v = c.regs;
        size_t i = first_after(v, lo);
        uint64_t cur = lo;
        while (cur < hi) {
            if (i == v.size() || v[i].lo > cur) {
                const uint64_t end = (i == v.size() || v[i].lo > hi) ? hi : v[i].lo;
                Region g = make(cur, end, 0);
                g.nr = 1;
                g.rd[0] = (uint32_t)seq;
                v.insert(v.begin() + (long)i, g);
                ++i;
                cur = end;
                continue;
            }
            Region& r = v[i];
            if (r.writer >= floor && r.writer != 0) deps.push_back(r.writer);
            prune_readers(r, floor);
            add_reader(r, seq);
            cur = r.hi;
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
        idx_.insert(idx_.begin() + (long)idx_upper(c.lo), Entry{up->lo, up});
    }

    // drop intervals that carry no live information
    void prune(Cluster& c, uint64_t floor) const {
        auto& v = c.regs;
        size_t k = 0;
        for (size_t i = 0; i < v.size(); ++i) {
            prune_readers(v[i], floor);
            const bool live = (v[i].writer >= floor && v[i].writer != 0) || v[i].nr > v[i].r0 || v[i].overflow;
            if (live) v[k++] = v[i];
        }
        v.resize(k);
        c.prune_at = std::max<size_t>(64, 2 * v.size());
    }
};

}  // namespace gpuos
