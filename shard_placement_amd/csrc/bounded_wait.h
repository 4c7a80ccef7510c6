// bounded_wait.h -- host-side waits with a deadline.
//
// The copy-engine calls wait for two things on the host: the caller's stream
// (so earlier kernels are done with the buffers) and the completion signal
// their copies share.  Either could in principle never finish (a hung
// kernel, a lost copy); a wait here gives up at a deadline instead of
// blocking its thread forever, and the call then reports a runtime failure.
//
// Header-only and free of HIP and ROCr types, so that the waiting logic can
// be built and tested on a host without a GPU: `done()` says whether the
// awaited thing has finished, `block(ns)` waits for it for up to about ns
// nanoseconds (it may return early, spuriously, or a little late).
#pragma once

#include <chrono>
#include <cstdint>

namespace tide {

// Wait until done() is true or timeout_ns have passed on the steady clock.
// block() is handed the time left, capped at slice_ns, so the deadline is
// re-checked at least every slice.  Returns true when done() held (checked
// once more at the deadline), false on timeout.
template <class Done, class Block>
bool wait_until(Done done, Block block, uint64_t timeout_ns, uint64_t slice_ns = 10000000) {
    using clock = std::chrono::steady_clock;
    const auto t0 = clock::now();
    for (;;) {
        if (done()) return true;
        const uint64_t spent = (uint64_t)std::chrono::duration_cast<std::chrono::nanoseconds>(
                                   clock::now() - t0)
                                   .count();
        if (spent >= timeout_ns) return done();
        uint64_t left = timeout_ns - spent;
        block(left < slice_ns ? left : slice_ns);
    }
}

// How long a copy-engine call waits for its copies: a fixed 10 s plus one
// second per GB moved (the engines move tens to hundreds of GB/s, so this
// only trips when the copies have stopped making progress).
inline uint64_t copy_timeout_ns(uint64_t bytes) {
    return 10000000000ull + bytes;  // 1 ns per byte = 1 s per GB
}

// How long a copy-engine call waits for the caller's stream to drain.
constexpr uint64_t kStreamTimeoutNs = 60000000000ull;  // 60 s

}  // namespace tide
