"""The deadline logic of the copy-engine calls' host waits
(shard_placement_amd/csrc/bounded_wait.h), built with g++ into a host-only
test library with fake completion sources: no GPU and no ROCr involved."""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "shard_placement_amd", "csrc")

SRC = r'''
#include <atomic>
#include <thread>
#include "bounded_wait.h"

extern "C" {
// done() turns true after `after` polls (never if after < 0); block() sleeps
// min(ns, sleep_cap_ns) (0: returns at once, as a spurious wake-up would).
int wait_case(long long after, unsigned long long timeout_ns, unsigned long long sleep_cap_ns,
              long long* polls, long long* blocks, unsigned long long* max_block_ns) {
    long long n = 0, b = 0;
    unsigned long long mx = 0;
    bool ok = tide::wait_until(
        [&] { ++n; return after >= 0 && n > after; },
        [&](unsigned long long ns) {
            ++b;
            if (ns > mx) mx = ns;
            unsigned long long s = ns < sleep_cap_ns ? ns : sleep_cap_ns;
            if (s) std::this_thread::sleep_for(std::chrono::nanoseconds(s));
        },
        timeout_ns, 2000000ull);
    *polls = n; *blocks = b; *max_block_ns = mx;
    return ok ? 1 : 0;
}
unsigned long long copy_timeout(unsigned long long bytes) { return tide::copy_timeout_ns(bytes); }
unsigned long long stream_timeout() { return tide::kStreamTimeoutNs; }
}
'''


@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    d = tmp_path_factory.mktemp("bw")
    src = d / "bw.cpp"
    so = d / "libbw.so"
    src.write_text(SRC)
    subprocess.run(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-Wall", "-Wextra", "-Werror",
                    "-I" + HDR, str(src), "-o", str(so)], check=True)
    L = ctypes.CDLL(str(so))
    u64, i64 = ctypes.c_ulonglong, ctypes.c_longlong
    L.wait_case.argtypes = [i64, u64, u64, ctypes.POINTER(i64), ctypes.POINTER(i64),
                            ctypes.POINTER(u64)]
    L.wait_case.restype = ctypes.c_int
    L.copy_timeout.argtypes = [u64]
    L.copy_timeout.restype = u64
    L.stream_timeout.restype = u64
    return L


def _run(L, after, timeout_ns, sleep_cap_ns):
    polls, blocks, mx = ctypes.c_longlong(), ctypes.c_longlong(), ctypes.c_ulonglong()
    t0 = time.perf_counter()
    ok = L.wait_case(after, timeout_ns, sleep_cap_ns, ctypes.byref(polls), ctypes.byref(blocks),
                     ctypes.byref(mx))
    return ok, time.perf_counter() - t0, polls.value, blocks.value, mx.value


def test_returns_when_done(lib):
    ok, dt, polls, blocks, _ = _run(lib, 5, 10 ** 9, 1000)
    assert ok == 1 and polls == 6 and blocks == 5 and dt < 0.5


def test_already_done_does_not_block(lib):
    ok, _, polls, blocks, _ = _run(lib, 0, 10 ** 9, 10 ** 6)
    assert ok == 1 and polls == 1 and blocks == 0


def test_gives_up_at_the_deadline(lib):
    ok, dt, _, blocks, mx = _run(lib, -1, 50 * 10 ** 6, 10 ** 9)
    assert ok == 0
    assert 0.045 <= dt < 1.0
    assert mx <= 2 * 10 ** 6       # each block gets at most one slice
    assert blocks >= 20


def test_spurious_wakeups_still_end_at_the_deadline(lib):
    # block() returns at once every time: the loop spins on the clock
    ok, dt, polls, _, _ = _run(lib, -1, 20 * 10 ** 6, 0)
    assert ok == 0 and 0.019 <= dt < 1.0 and polls > 1


def test_done_at_the_last_check_counts(lib):
    # a 1 ns deadline has passed by the second poll, which is the first to
    # see the work done: that is success, and nothing blocked
    ok, _, polls, blocks, _ = _run(lib, 1, 1, 10 ** 6)
    assert (ok, polls, blocks) == (1, 2, 0)
    ok, _, polls, blocks, _ = _run(lib, 2, 1, 10 ** 6)
    assert (ok, polls, blocks) == (0, 2, 0)


def test_timeouts(lib):
    assert lib.stream_timeout() == 60 * 10 ** 9
    assert lib.copy_timeout(0) == 10 * 10 ** 9
    assert lib.copy_timeout(110 * 10 ** 9) == 120 * 10 ** 9
