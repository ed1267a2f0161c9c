// Brute-force check of the host's hazard tracker (csrc/hazard.h).
//
// Random descriptor streams of byte-range accesses: prefixes and arbitrary
// sub-ranges of a few dozen "tensors", accesses spanning neighbouring
// tensors (cluster merges), long-lived arenas written piece by piece
// (cluster splits), hot tensors read by many descriptors (more than the 62
// dependencies a descriptor carries),
// and a completion process that retires descriptors in a random order
// allowed by their dependencies, so the watermark passed to the tracker
// moves the way the library's does.
//
// For every descriptor j the checker keeps the raw accesses of all live
// earlier descriptors and requires: every live i < j whose accesses
// conflict with j's (overlap, at least one of the two a write) is reached
// from j through the returned dependencies -- explicit ones and the range
// [range_from, j) -- directly or transitively (waiting for k, which waited
// for i, also orders j after i).  Dependencies must be live and older than j.
// Prints "ok <descriptors> <deps>" or the first violation, exit status 1.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <set>
#include <vector>

#include "hazard.h"

using namespace gpuos;

static uint64_t st = 0x243F6A8885A308D3ull;
static uint64_t rnd() {  // SplitMix64
    uint64_t z = (st += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static uint64_t below(uint64_t n) { return rnd() % n; }

struct Desc {
    std::vector<Access> acc;
    std::vector<uint64_t> deps;
    uint64_t range_from = UINT64_MAX;
    bool done = false;
};

static bool conflict(const Desc& a, const Desc& b) {
    for (const Access& x : a.acc)
        for (const Access& y : b.acc)
            if ((x.write || y.write) && x.lo < y.hi && y.lo < x.hi) return true;
    return false;
}

int run(uint64_t seed, int n_desc, int mode) {
    st = seed;
    HazardTracker hz;
    std::vector<Desc> D(n_desc);
    const uint64_t BASE = 1ull << 40, T = 1 << 20;  // tensors 1 MiB apart
    const int NT = 24;
    uint64_t arena = 0;
    uint64_t floor = 0;  // every seq < floor is done
    std::vector<uint64_t> deps;
    uint64_t total_deps = 0;
    for (int j = 0; j < n_desc; ++j) {
        Desc& d = D[j];
        const int na = 1 + (int)below(3);
        for (int k = 0; k < na; ++k) {
            const uint64_t t = below(mode == 2 ? 4 : NT), kind = below(10);
            uint64_t lo, hi;
            if (kind < 4) {            // prefix of a tensor
                lo = BASE + t * T;
                hi = lo + 64 + below(T - 64);
            } else if (kind < 7) {     // arbitrary sub-range
                lo = BASE + t * T + below(T);
                hi = lo + 1 + below(BASE + (t + 1) * T - lo);
            } else if (kind < 8) {     // spans into the next tensor (merges)
                lo = BASE + t * T + T - 1 - below(T / 2);
                hi = lo + T / 2 + below(T);
            } else {                   // a rotating arena far away (splits)
                const uint64_t sz = 256 + below(8192);
                if (arena + sz > (64u << 20)) arena = 0;
                lo = (1ull << 44) + arena;
                hi = lo + sz;
                arena += sz;
            }
            const bool w = mode == 1 ? below(8) == 0 : below(3) == 0;  // mode 1: mostly reads (overflow)
            d.acc.push_back(Access{lo, hi, w});
        }
        deps.clear();
        hz.analyze((uint64_t)j + 1, d.acc.data(), (int)d.acc.size(), floor + 1, deps, &d.range_from);
        // seqs are j + 1 (0 means "none" to the tracker); convert back to indices
        for (uint64_t s : deps) {
            if (s < floor + 1 || s >= (uint64_t)j + 1) {
                printf("seed %llu: descriptor %d got dependency %llu outside [%llu, %d)\n",
                       (unsigned long long)seed, j, (unsigned long long)s, (unsigned long long)floor + 1, j + 1);
                return 1;
            }
            d.deps.push_back(s - 1);
        }
        if (d.range_from != UINT64_MAX) d.range_from -= 1;
        total_deps += d.deps.size();
        // reachability from j over live descriptors
        std::vector<char> seen(j, 0);
        std::vector<int> stack;
        auto push = [&](uint64_t i) {
            if (i >= floor && i < (uint64_t)j && !seen[i]) { seen[i] = 1; stack.push_back((int)i); }
        };
        auto expand = [&](const Desc& x, uint64_t self) {
            for (uint64_t i : x.deps) push(i);
            if (x.range_from != UINT64_MAX)
                for (uint64_t i = std::max<uint64_t>(x.range_from, floor); i < self; ++i) push(i);
        };
        expand(d, j);
        while (!stack.empty()) {
            const int k = stack.back();
            stack.pop_back();
            expand(D[k], k);
        }
        for (uint64_t i = floor; i < (uint64_t)j; ++i) {
            if (D[i].done || seen[i] || !conflict(D[i], d)) continue;
            printf("seed %llu mode %d: descriptor %d conflicts with live %llu but does not wait for it\n",
                   (unsigned long long)seed, mode, j, (unsigned long long)i);
            return 1;
        }
        // complete a random subset of the descriptors whose dependencies are done
        const int tries = (int)below(4);
        for (int t = 0; t < tries; ++t) {
            const uint64_t lo = floor, span = (uint64_t)j + 1 - floor;
            if (span == 0) break;
            const uint64_t i = lo + below(std::min<uint64_t>(span, 64));
            Desc& x = D[i];
            if (x.done) continue;
            bool ok = true;
            for (uint64_t k : x.deps) ok = ok && (k < floor || D[k].done);
            if (x.range_from != UINT64_MAX)
                for (uint64_t k = std::max<uint64_t>(x.range_from, floor); k < i && ok; ++k) ok = D[k].done;
            if (ok) x.done = true;
        }
        while (floor <= (uint64_t)j && D[floor].done) ++floor;
    }
    printf("ok %d %llu\n", n_desc, (unsigned long long)total_deps);
    return 0;
}

int main(int argc, char** argv) {
    const int n = argc > 1 ? atoi(argv[1]) : 4000;
    for (uint64_t seed = 1; seed <= 6; ++seed)
        for (int mode = 0; mode < 3; ++mode)
            if (run(seed * 1000 + mode, n, mode)) return 1;
    return 0;
}
