// ring_model.cpp -- host-thread model of a producer -> chain handoff of chunk
// records through a ring with per-slot flags, the protocol a fused prefill
// would use between workgroups (test infrastructure; no GPU).
//
// Threads stand for workgroups.  Producers write the record of chunk c into
// ring slot c % R and publish it by storing c + 1 into the slot's "ready"
// word; every consumer of the sequence (one per value tile) waits for that
// value, reads the record, then bumps the slot's "done" count; a producer
// reuses a slot only once all consumers are done with its previous chunk.
//
// Two properties are checked:
//   1. Visibility: publication is a release store, observation an acquire
//      load of the same word (on the GPU: device-scope atomics, or an
//      L1-bypassing load inside one XCD's L2).  A "stale" mode models the
//      failure in which a poll is served by a private copy of the line that
//      never sees the producer's store (a non-coherent cache).
//   2. Bounded total time: every wait polls both its word and a shared abort
//      word.  The first wait that exceeds its bound sets abort (recording
//      which wait failed); every later wait sees abort and returns at once;
//      every thread then exits normally.  So a broken protocol ends within
//      about one bound, not one bound per wait (2048 chunk steps x several
//      waits each would otherwise add up to minutes).
//
// A third mode, stale_no_abort, drops the abort word: each wait is bounded on
// its own and a timed-out wait is skipped, as in a kernel whose every wait
// has a limit but nothing stops the rest.  Its run time grows as (waits) x
// (bound): the mechanism by which individually bounded waits can outlast any
// fixed time limit.
//
// Usage: ring_model MODE CHUNKS TILES PRODUCERS RING BOUND_MS
//   MODE normal | stale | missing_producer | stale_no_abort
// Prints "ok", or "aborted <who>", and the elapsed milliseconds; exit 0 when
// the outcome is the expected one for the mode (records verified in normal
// mode; abort within 3 bounds in the stale and missing modes; at least
// CHUNKS / 2 bounds without the abort word).
#include <atomic>
#include <chrono>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

namespace {

using Clock = std::chrono::steady_clock;
constexpr int kWords = 64;   // record payload (a stand-in for the 72 KB record)

struct Slot {
    std::atomic<int64_t> ready{0};   // c + 1 once chunk c's record is in the slot
    std::atomic<int64_t> done{0};    // consumers finished with the slot's current chunk
    int64_t payload[kWords];
};

struct Shared {
    std::vector<Slot> ring;
    std::atomic<int> abort{0};       // 0, or 1 + the id of the first wait that timed out
    std::atomic<int64_t> checked{0};
    std::atomic<int64_t> bad{0};
    int64_t chunks;
    int tiles;
    Clock::duration bound;
    bool stale;
    bool use_abort = true;
    explicit Shared(int r) : ring(r) {}
};

int64_t record_word(int64_t c, int w) { return c * 1000003 + w * 7919 + 11; }

// Polls `get()` until `want(value)` holds; gives up at the bound or as soon as
// another wait has aborted.  Returns false if the handoff failed.
template <class Get, class Want>
bool bounded_wait(Shared &sh, int who, Get get, Want want) {
    const auto t0 = Clock::now();
    for (uint64_t spin = 0;; ++spin) {
        if (sh.use_abort && sh.abort.load(std::memory_order_acquire)) return false;
        if (want(get())) return true;
        if ((spin & 255) == 0 && Clock::now() - t0 > sh.bound) {
            int expected = 0;
            if (sh.use_abort)
                sh.abort.compare_exchange_strong(expected, 1 + who, std::memory_order_acq_rel);
            return false;
        }
        std::this_thread::yield();
    }
}

void producer(Shared &sh, int id, int n_producers) {
    const int R = (int)sh.ring.size();
    for (int64_t c = id; c < sh.chunks; c += n_producers) {
        Slot &s = sh.ring[c % R];
        // The slot's previous chunk (c - R) must have been read by every tile.
        // `done` counts reads of this slot over all the chunks it has held:
        // chunks s, s + R, ..., c - R, i.e. (c - R) / R + 1 of them.
        if (c >= R) {
            const int64_t held = (c - R) / R + 1;
            if (!bounded_wait(sh, 1000 + id,
                              [&] { return s.done.load(std::memory_order_acquire); },
                              [&](int64_t d) { return d >= held * sh.tiles; }) &&
                sh.use_abort)
                return;
        }
        for (int w = 0; w < kWords; ++w) s.payload[w] = record_word(c, w);
        s.ready.store(c + 1, std::memory_order_release);   // publish
    }
}

void consumer(Shared &sh, int tile) {
    const int R = (int)sh.ring.size();
    int64_t sum = 0;
    for (int64_t c = 0; c < sh.chunks; ++c) {
        Slot &s = sh.ring[c % R];
        // A stale poll reads a private copy of the flag cached before any
        // publication (its initial value), as a cache line that is never
        // invalidated would: it never sees the producer's store.
        const int64_t stale_copy = 0;
        const bool ok = bounded_wait(
            sh, tile,
            [&] { return sh.stale ? stale_copy : s.ready.load(std::memory_order_acquire); },
            [&](int64_t r) { return r == c + 1; });
        if (!ok) {
            if (sh.use_abort) return;
            s.done.fetch_add(1, std::memory_order_acq_rel);   // skip this chunk and go on
            continue;
        }
        for (int w = 0; w < kWords; ++w) {
            const int64_t x = s.payload[w];
            if (x != record_word(c, w)) sh.bad.fetch_add(1, std::memory_order_relaxed);
            sum += x;
        }
        sh.checked.fetch_add(1, std::memory_order_relaxed);
        // Release the slot for chunk c + R (c's record was read above).
        s.done.fetch_add(1, std::memory_order_acq_rel);
    }
    (void)sum;
}

}  // namespace

int main(int argc, char **argv) {
    if (argc != 7) {
        std::fprintf(stderr, "usage: %s MODE CHUNKS TILES PRODUCERS RING BOUND_MS\n", argv[0]);
        return 2;
    }
    const char *mode = argv[1];
    const int64_t chunks = std::atoll(argv[2]);
    const int tiles = std::atoi(argv[3]);
    int producers = std::atoi(argv[4]);
    const int ring = std::atoi(argv[5]);
    const int bound_ms = std::atoi(argv[6]);
    const bool no_abort = std::strcmp(mode, "stale_no_abort") == 0;
    const bool stale = std::strcmp(mode, "stale") == 0 || no_abort;
    const bool missing = std::strcmp(mode, "missing_producer") == 0;
    if (missing) producers = 0;   // a role that no workgroup took

    Shared sh(ring);
    sh.chunks = chunks;
    sh.tiles = tiles;
    sh.bound = std::chrono::milliseconds(bound_ms);
    sh.stale = stale;
    sh.use_abort = !no_abort;

    const auto t0 = Clock::now();
    std::vector<std::thread> th;
    for (int p = 0; p < producers; ++p) th.emplace_back(producer, std::ref(sh), p, producers);
    for (int t = 0; t < tiles; ++t) th.emplace_back(consumer, std::ref(sh), t);
    for (auto &t : th) t.join();
    const double ms =
        std::chrono::duration<double, std::milli>(Clock::now() - t0).count();

    const int ab = sh.abort.load();
    if (ab) std::printf("aborted %d\n", ab - 1);
    else std::printf("ok\n");
    std::printf("elapsed_ms %.1f checked %lld bad %lld\n", ms, (long long)sh.checked.load(),
                (long long)sh.bad.load());
    // Without the abort word skipped handoffs let slots be reused under a
    // reader, so only the time is judged there.
    if (no_abort) return ms >= 0.5 * (double)chunks * bound_ms ? 0 : 1;
    if (sh.bad.load() != 0) return 1;                 // a record read before it was complete
    if (!stale && !missing)
        return (ab == 0 && sh.checked.load() == chunks * tiles) ? 0 : 1;
    return (ab != 0 && ms < 3.0 * bound_ms + 1000.0) ? 0 : 1;   // ended within ~one bound
}
