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
// Data structure.  Memory that accesses have touched is kept in clusters: a
// cluster covers a contiguous span (in practice one tensor, or one arena).
// It holds
//  - the writes as a sorted vector of disjoint intervals, each with its last
//    writer (a write coalesces what it covers, so every byte has exactly the
//    last writer a later access must order after), and
//  - the reads as a log in sequence order (byte range and sequence number),
//    appended to in O(1): reads never conflict with reads, so a read is not
//    spread over the write intervals.
// A read waits for the live writers of the intervals it overlaps.  A write
// waits for those too and for every live logged read it overlaps; a logged
// read that lies inside the write's range is then dropped from the log, since
// any later access that conflicts with it overlaps the write, which waited
// for it.  Reads below the watermark leave from the front of the log.
//  - Clusters are found through a small direct-mapped cache keyed by the
//    access's start address, else by binary search in a sorted array of
//    cluster starts.  An access that reaches past one cluster's span, and
//    touches no other, extends that cluster in place; one that touches
//    several merges them (intervals concatenated, logs merged by sequence).
//  - A cluster whose write intervals or read log grow past SPLIT_AT live
//    entries (a long-lived buffer written piece by piece, such as an output
//    arena) is split in two at an interval boundary; logged reads that
//    straddle the cut go to both halves.
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
    static constexpr size_t SPLIT_AT = 96;

    // Appends to `deps` every live seq (>= floor) that `seq` must wait for;
    // then records the accesses.  `range_from` is for trackers that return a
    // whole range of earlier descriptors to wait for; this one returns
    // explicit dependencies only and leaves it untouched.
    void analyze(uint64_t seq, const Access* acc, int n, uint64_t floor, std::vector<uint64_t>& deps,
                 uint64_t* range_from) {
        (void)range_from;
        floor_ = floor;
        Cluster* cp[24];
        if (n > 24) n = 24;
        // resolve each access's cluster (a merge retires clusters found
        // earlier: resolve again until no merge happens)
        for (int round = 0; round < 4; ++round) {
            const uint64_t m0 = merges_;
            for (int i = 0; i < n; ++i) cp[i] = acc[i].hi > acc[i].lo ? &cluster_for(acc[i].lo, acc[i].hi) : nullptr;
            if (merges_ == m0) break;
        }
        // every access is checked before any is recorded, so that a
        // descriptor never waits for itself
        for (int i = 0; i < n; ++i) {
            if (!cp[i]) continue;
            prune_reads(*cp[i]);
            writers(*cp[i], acc[i].lo, acc[i].hi, deps);
            if (acc[i].write) readers(*cp[i], acc[i].lo, acc[i].hi, deps);
        }
        for (int i = 0; i < n; ++i) {
            if (!cp[i]) continue;
            Cluster& c = *cp[i];
            if (acc[i].write) {
                record_write(c, acc[i].lo, acc[i].hi, seq);
                if (c.w.size() > c.prune_at) prune_writes(c);
            } else {
                push_read(c, Ent{acc[i].lo, acc[i].hi, seq});
            }
        }
        // split large clusters only now: the pointers in cp stay valid above
        for (int i = 0; i < n; ++i)
            if (cp[i] && (cp[i]->w.size() > SPLIT_AT || cp[i]->rlive() > cp[i]->rsplit_at)) split(*cp[i]);
    }

    void clear() {
        idx_.clear();
        store_.clear();
        free_.clear();
        std::fill(hits_.begin(), hits_.end(), Hit{});
    }
    // write intervals plus live logged reads over all clusters (diagnostics)
    size_t size() const {
        size_t n = 0;
        for (const Entry& e : idx_) n += e.c->w.size() + e.c->rlive();
        return n;
    }
    size_t clusters() const { return idx_.size(); }

private:
    struct Region {
        uint64_t lo, hi;
        uint64_t writer;  // 0 = none
    };
    static constexpr uint64_t DEAD_LO = UINT64_MAX;  // a dropped read overlaps nothing
    struct Ent {
        uint64_t lo, hi, seq;
    };
    struct Cluster {
        uint64_t lo = 0, hi = 0;
        std::vector<Region> w;  // sorted by lo, disjoint, inside [lo, hi)
        std::vector<Ent> r;     // reads in sequence order; [rhead, size) may be live
        size_t rhead = 0, rdead = 0;
        size_t prune_at = 64, rsplit_at = SPLIT_AT;
        bool alive = false;
        size_t rlive() const { return r.size() - rhead - rdead; }
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
    uint64_t floor_ = 0;
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
        c->rsplit_at = SPLIT_AT;
        return c;
    }
    void retire(Cluster* c) {
        c->alive = false;
        c->lo = c->hi = 0;
        c->w.clear();
        c->r.clear();
        c->rhead = c->rdead = 0;
        free_.push_back(c);
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

    // the live reads of c's log, merged by sequence number with those of o
    void merge_reads(Cluster& c, Cluster& o) {
        prune_reads(c);
        prune_reads(o);
        std::vector<Ent> out;
        out.reserve(c.rlive() + o.rlive());
        size_t i = c.rhead, j = o.rhead;
        while (i < c.r.size() || j < o.r.size()) {
            const bool take_c = j == o.r.size() || (i < c.r.size() && c.r[i].seq <= o.r[j].seq);
            const Ent& t = take_c ? c.r[i++] : o.r[j++];
            if (t.lo != DEAD_LO) out.push_back(t);
        }
        c.r.swap(out);
        c.rhead = c.rdead = 0;
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
                // first (all are sorted and lie above it) and merge the logs
                ++merges_;
                for (size_t q = first + 1; q < last; ++q) {
                    Cluster* o = idx_[q].c;
                    c->w.insert(c->w.end(), o->w.begin(), o->w.end());
                    if (o->rlive()) merge_reads(*c, *o);
                    c->hi = std::max(c->hi, o->hi);
                    retire(o);
                }
                idx_.erase(idx_.begin() + (long)(first + 1), idx_.begin() + (long)last);
                c->prune_at = std::max<size_t>(64, 2 * c->w.size());
                c->rsplit_at = std::max(SPLIT_AT, 2 * c->rlive());
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

    // index of the first interval with hi > x
    static size_t first_after(const std::vector<Region>& v, uint64_t x) {
        size_t a = 0, b = v.size();
        while (a < b) {
            const size_t m = (a + b) >> 1;
            if (v[m].hi > x) b = m; else a = m + 1;
        }
        return a;
    }

    void prune_reads(Cluster& c) const {
        while (c.rhead < c.r.size() && c.r[c.rhead].seq < floor_) {
            if (c.r[c.rhead].lo == DEAD_LO) --c.rdead;
            ++c.rhead;
        }
        if (c.rhead == c.r.size()) {
            c.r.clear();
            c.rhead = c.rdead = 0;
        }
    }
    void compact_reads(Cluster& c) const {
        size_t k = 0;
        for (size_t i = c.rhead; i < c.r.size(); ++i)
            if (c.r[i].lo != DEAD_LO) c.r[k++] = c.r[i];
        c.r.resize(k);
        c.rhead = c.rdead = 0;
    }
    void push_read(Cluster& c, const Ent& x) const {
        if (c.rhead + c.rdead > 16 && 2 * (c.rhead + c.rdead) > c.r.size()) compact_reads(c);
        c.r.push_back(x);
    }

    // the live writers of the intervals overlapping [lo, hi)
    void writers(const Cluster& c, uint64_t lo, uint64_t hi, std::vector<uint64_t>& deps) const {
        for (size_t i = first_after(c.w, lo); i < c.w.size() && c.w[i].lo < hi; ++i)
            if (c.w[i].writer >= floor_ && c.w[i].writer != 0) deps.push_back(c.w[i].writer);
    }
    // the live logged reads overlapping [lo, hi) (a write); those inside it
    // are dropped: the write orders every later conflicting access after them
    void readers(Cluster& c, uint64_t lo, uint64_t hi, std::vector<uint64_t>& deps) const {
        for (size_t i = c.rhead; i < c.r.size(); ++i) {
            Ent& x = c.r[i];
            if (x.lo >= hi || x.hi <= lo) continue;  // also every dropped read
            deps.push_back(x.seq);
            if (x.lo >= lo && x.hi <= hi) {
                x.lo = DEAD_LO;
                x.hi = 0;
                ++c.rdead;
            }
        }
    }

    static void record_write(Cluster& c, uint64_t lo, uint64_t hi, uint64_t seq) {
        auto& v = c.w;
        const size_t i0 = first_after(v, lo);
        size_t i1 = i0;
        while (i1 < v.size() && v[i1].lo < hi) ++i1;
        if (i1 == i0 + 1 && v[i0].lo == lo && v[i0].hi == hi) {  // exact match: reuse
            v[i0].writer = seq;
            return;
        }
        Region parts[3];
        int np = 0;
        if (i1 > i0 && v[i0].lo < lo) { parts[np] = v[i0]; parts[np].hi = lo; ++np; }
        parts[np++] = Region{lo, hi, seq};
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

    // drop write intervals whose writer is complete
    void prune_writes(Cluster& c) const {
        auto& v = c.w;
        size_t k = 0;
        for (size_t i = 0; i < v.size(); ++i)
            if (v[i].writer >= floor_ && v[i].writer != 0) v[k++] = v[i];
        v.resize(k);
        c.prune_at = std::max<size_t>(64, 2 * v.size());
    }

    // Prune, and if the cluster is still large move its upper half (by the
    // write intervals, else by the logged reads' starts) into a cluster of
    // its own (pool entries do not move, so other Cluster pointers stay
    // valid).
    void split(Cluster& c) {
        prune_writes(c);
        prune_reads(c);
        compact_reads(c);
        const bool by_w = c.w.size() > SPLIT_AT;
        if (!by_w && c.rlive() <= c.rsplit_at) return;
        uint64_t cut;
        if (by_w) {
            cut = c.w[c.w.size() / 2].lo;
        } else {
            std::vector<uint64_t> starts;
            starts.reserve(c.r.size());
            for (const Ent& x : c.r) starts.push_back(x.lo);
            std::nth_element(starts.begin(), starts.begin() + (long)(starts.size() / 2), starts.end());
            cut = starts[starts.size() / 2];
            size_t below = 0, above = 0;
            for (const Ent& x : c.r) { below += x.lo < cut; above += x.hi > cut; }
            if (cut <= c.lo || 4 * below > 3 * c.r.size() || 4 * above > 3 * c.r.size()) {
                c.rsplit_at = 2 * c.r.size();  // reads of one range: no useful cut
                return;
            }
            // the cut must not fall inside a write interval
            const size_t i = first_after(c.w, cut);
            if (i < c.w.size() && c.w[i].lo < cut) cut = c.w[i].lo > c.lo ? c.w[i].lo : c.w[i].hi;
            if (cut <= c.lo || cut >= c.hi) {
                c.rsplit_at = 2 * c.r.size();
                return;
            }
        }
        Cluster* up = alloc_cluster();  // the pool is a deque: c stays valid
        up->lo = cut;
        up->hi = c.hi;
        const size_t wi = first_after(c.w, cut);  // every interval from wi on starts at or above cut
        up->w.assign(c.w.begin() + (long)wi, c.w.end());
        c.w.resize(wi);
        size_t k = 0;
        for (const Ent& x : c.r) {
            if (x.hi > cut) up->r.push_back(Ent{std::max(x.lo, cut), x.hi, x.seq});
            if (x.lo < cut) c.r[k++] = Ent{x.lo, std::min(x.hi, cut), x.seq};
        }
        c.r.resize(k);
        c.hi = cut;
        c.prune_at = std::max<size_t>(64, 2 * c.w.size());
        up->prune_at = std::max<size_t>(64, 2 * up->w.size());
        c.rsplit_at = std::max(SPLIT_AT, 2 * c.rlive());
        up->rsplit_at = std::max(SPLIT_AT, 2 * up->rlive());
        idx_.insert(idx_.begin() + (long)idx_upper(c.lo), Entry{up->lo, up});
    }
};

}  // namespace gpuos
