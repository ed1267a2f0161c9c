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
// The tracker keeps a map of disjoint byte intervals, each with its last
// writer and the readers since that write.  Sequence numbers below the
// host's completion watermark are known complete and are never returned.
#pragma once
#include <stdint.h>

#include <algorithm>
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
    // Appends to `deps` every live seq (>= floor) that `seq` must wait for,
    // then records the accesses of `seq`.  Reads are recorded before writes,
    // so an operand that is both read and written ends with `seq` as writer.
    void analyze(uint64_t seq, const Access* acc, int n, uint64_t floor, std::vector<uint64_t>& deps) {
        for (int i = 0; i < n; ++i) {
            if (acc[i].hi <= acc[i].lo) continue;
            collect(acc[i], floor, deps);
        }
        std::sort(deps.begin(), deps.end());
        deps.erase(std::unique(deps.begin(), deps.end()), deps.end());
        for (int pass = 0; pass < 2; ++pass) {
            for (int i = 0; i < n; ++i) {
                if (acc[i].hi <= acc[i].lo || acc[i].write != (pass == 1)) continue;
                if (acc[i].write) record_write(acc[i].lo, acc[i].hi, seq);
                else record_read(acc[i].lo, acc[i].hi, seq, floor);
            }
        }
        if (m_.size() > prune_at_) prune(floor);
    }

    void clear() { m_.clear(); }
    size_t size() const { return m_.size(); }

private:
    struct Region {
        uint64_t hi;
        uint64_t writer;                // 0 = none
        std::vector<uint64_t> readers;  // since the last write
    };
    using Map = std::map<uint64_t, Region>;
    Map m_;
    size_t prune_at_ = 1u << 16;

    Map::iterator first_overlap(uint64_t lo) {
        auto it = m_.upper_bound(lo);
        if (it != m_.begin()) {
            auto p = std::prev(it);
            if (p->second.hi > lo) return p;
        }
        return it;
    }

    void collect(const Access& a, uint64_t floor, std::vector<uint64_t>& deps) {
        for (auto it = first_overlap(a.lo); it != m_.end() && it->first < a.hi; ++it) {
            const Region& r = it->second;
            if (r.writer >= floor && r.writer != 0) deps.push_back(r.writer);
            if (a.write)
                for (uint64_t s : r.readers)
                    if (s >= floor) deps.push_back(s);
        }
    }

    // make x a region boundary
    void split_at(uint64_t x) {
        auto it = m_.upper_bound(x);
        if (it == m_.begin()) return;
        auto p = std::prev(it);
        if (p->first < x && x < p->second.hi) {
            Region tail = p->second;
            p->second.hi = x;
            m_.emplace_hint(it, x, std::move(tail));
        }
    }

    void record_write(uint64_t lo, uint64_t hi, uint64_t seq) {
        split_at(lo);
        split_at(hi);
        auto it = m_.lower_bound(lo);
        while (it != m_.end() && it->first < hi) it = m_.erase(it);
        m_.emplace_hint(it, lo, Region{hi, seq, {}});
    }

    void record_read(uint64_t lo, uint64_t hi, uint64_t seq, uint64_t floor) {
        split_at(lo);
        split_at(hi);
        uint64_t cur = lo;
        auto it = m_.lower_bound(lo);
        while (cur < hi) {
            if (it == m_.end() || it->first > cur) {
                // gap [cur, next start or hi): a region with no writer
                const uint64_t end = (it == m_.end() || it->first > hi) ? hi : it->first;
                it = m_.emplace_hint(it, cur, Region{end, 0, {seq}});
                ++it;
                cur = end;
                continue;
            }
            Region& r = it->second;
            auto& rd = r.readers;
            rd.erase(std::remove_if(rd.begin(), rd.end(), [&](uint64_t s) { return s < floor; }), rd.end());
            rd.push_back(seq);
            cur = r.hi;
            ++it;
        }
    }

    // drop intervals that carry no live information
    void prune(uint64_t floor) {
        for (auto it = m_.begin(); it != m_.end();) {
            Region& r = it->second;
            bool live = r.writer >= floor && r.writer != 0;
            for (uint64_t s : r.readers) live |= s >= floor;
            it = live ? std::next(it) : m_.erase(it);
        }
        prune_at_ = std::max<size_t>(1u << 16, 2 * m_.size());
    }
};

}  // namespace gpuos
