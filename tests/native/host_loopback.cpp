// The host library's protocol code (gpuos_host.cpp) driven through the C ABI
// on a loopback context, for sanitizer builds on the CPU: a producer thread
// submits bursts of descriptors with overlapping byte ranges and rebinds
// op ids while a second thread polls sync, query and stats, and the
// library's loopback consumer completes descriptors in a random order their
// dependencies allow.  The device-side launchers are stubs (a loopback
// context never launches anything).  Exit status 0 = every descriptor
// completed, in an order that respects its dependencies.
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

#include "gpuos.h"
#include "gpuos_internal.h"

namespace gpuos {
hipError_t launch_executor(const ExecArgs&, uint32_t, bool, uint32_t, uint32_t, hipStream_t) { abort(); }
hipError_t launch_eager(const gpuos_desc&, uint32_t, uint32_t, uint8_t*, hipStream_t) { abort(); }
hipError_t launch_null(hipStream_t) { abort(); }
hipError_t launch_hbm_probe(const void*, void*, uint32_t, bool, uint32_t, hipStream_t) { abort(); }
hipError_t static_scratch(uint8_t**) { abort(); }
hipError_t launch_fill_zero(uint8_t*, uint32_t, hipStream_t) { abort(); }
}  // namespace gpuos

int main(int argc, char** argv) {
    const uint32_t n = argc > 1 ? (uint32_t)atoi(argv[1]) : 20000;
    gpuos_init_params P{};
    P.flags = GPUOS_INIT_LOOPBACK;
    P.ring_entries = 64;
    void* ctx = nullptr;
    if (gpuos_init(&P, &ctx) != GPUOS_OK) return 2;
    // descriptors over 16 fake tensors of 64 KiB: add/mul/relu of prefixes,
    // some in place, and op ids rebound between built-in kinds
    std::vector<gpuos_desc> d(n);
    std::vector<uint64_t> lo(3 * (size_t)n), hi(3 * (size_t)n);
    uint64_t s = 12345;
    auto rnd = [&]() { s ^= s << 13; s ^= s >> 7; s ^= s << 17; return s; };
    const uint64_t base = 1ull << 40;
    for (uint32_t i = 0; i < n; ++i) {
        memset(&d[i], 0, sizeof(gpuos_desc));
        const uint32_t op = 1 + (uint32_t)(rnd() % 3);
        d[i].op_id = i % 7 == 0 ? 100u : op;   // op id 100 is rebound while the stream runs
        d[i].flags = GPUOS_F32;
        d[i].size = 1 + rnd() % 16384;
        d[i].input_a = base + (rnd() % 16) * 65536;
        d[i].input_b = base + (rnd() % 16) * 65536;
        d[i].output = rnd() % 10 == 0 ? d[i].input_a : base + (rnd() % 16) * 65536;
    }
    if (gpuos_register_op(ctx, 100, GPUOS_OP_ADD, nullptr, 0) != GPUOS_OK) return 3;
    std::atomic<bool> done{false};
    std::atomic<int> bad{0};
    std::thread poller([&] {
        while (!done.load()) {
            gpuos_stats st;
            if (gpuos_stats_get(ctx, &st) != GPUOS_OK) bad = 1;
            (void)gpuos_query(ctx, st.next_seq ? st.next_seq - 1 : 0);
            uint64_t es = 0;
            uint32_t ec = 0;
            const int rc = gpuos_sync(ctx, GPUOS_SEQ_ALL, 1000000, &es, &ec);
            if (rc != GPUOS_OK && rc != GPUOS_E_TIMEOUT) bad = 2;
        }
    });
    uint64_t first = 0;
    for (uint32_t i = 0; i < n;) {
        const uint32_t burst = 1 + (uint32_t)(rnd() % 48);
        const uint32_t cnt = burst < n - i ? burst : n - i;
        uint64_t f = 0;
        if (gpuos_submit(ctx, &d[i], cnt, GPUOS_SUBMIT_BLOCK, &f) != GPUOS_OK) { bad = 3; break; }
        if (i == 0) first = f;
        if (rnd() % 64 == 0) {
            const uint32_t kinds[3] = {GPUOS_OP_ADD, GPUOS_OP_MUL, GPUOS_OP_RELU};
            if (gpuos_register_op(ctx, 100, kinds[rnd() % 3], nullptr, 0) != GPUOS_OK) bad = 4;
        }
        i += cnt;
    }
    if (gpuos_sync(ctx, GPUOS_SEQ_ALL, 60000000000ll, nullptr, nullptr) != GPUOS_OK) bad = 5;
    done = true;
    poller.join();
    // the completion order respects every conflict between two descriptors
    uint64_t total = 0;
    gpuos_loopback_order(ctx, nullptr, 0, &total);
    std::vector<uint64_t> order(total);
    gpuos_loopback_order(ctx, order.data(), total, &total);
    if (total != n) bad = 6;
    std::vector<uint32_t> pos(n);
    for (uint32_t k = 0; k < total; ++k) pos[order[k] - first] = k;
    // last writer / readers since, per fake tensor, at tensor granularity
    // (prefixes of one tensor always overlap)
    for (uint32_t j = 0; j < n && !bad; ++j)
        for (uint32_t i = j > 256 ? j - 256 : 0; i < j; ++i) {
            // b is read by add and mul; op id 100 may be bound to ReLU, so
            // its b is left out of the check (a weaker check, never a wrong one)
            auto reads_b = [&](uint32_t k) { return d[k].op_id == GPUOS_OP_ADD || d[k].op_id == GPUOS_OP_MUL; };
            const bool conflict = d[i].output == d[j].input_a || (reads_b(j) && d[i].output == d[j].input_b) ||
                                  d[i].output == d[j].output || d[j].output == d[i].input_a ||
                                  (reads_b(i) && d[j].output == d[i].input_b);
            if (conflict && pos[i] > pos[j]) { bad = 7; fprintf(stderr, "order: %u after %u\n", i, j); break; }
        }
    if (gpuos_shutdown(ctx) != GPUOS_OK) bad = 8;
    printf("%s %u descriptors\n", bad ? "FAIL" : "ok", n);
    return bad;
}
