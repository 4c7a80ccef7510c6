"""Host-side parts of the interference probe (CPU)."""
import gc

from shard_placement_amd import probe


def test_timed_regions_pause_the_garbage_collector():
    assert gc.isenabled()
    with probe._no_gc():
        assert not gc.isenabled()
    assert gc.isenabled()
    try:
        with probe._no_gc():
            raise KeyError("x")
    except KeyError:
        pass
    assert gc.isenabled()
    gc.disable()
    try:
        with probe._no_gc():
            assert not gc.isenabled()
        assert not gc.isenabled()  # left as the caller had it
    finally:
        gc.enable()


def test_standalone_probe_needs_a_gpu():
    import pytest
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    with pytest.raises(SystemExit, match="needs a GPU"):
        probe.main(["--workload", "1"])


def test_timed_regions_freeze_the_heap():
    """Inside the window a collection has (almost) nothing to walk; the heap
    is unfrozen again on exit."""
    junk = [[i] for i in range(1000)]  # tracked containers
    before = gc.get_freeze_count()
    with probe._no_gc():
        assert gc.get_freeze_count() >= len(junk)
        assert len(gc.get_objects()) < 1000
    assert gc.get_freeze_count() == before
    assert len(junk) == 1000


def test_side_thread_collects_and_reports():
    import time

    s = probe._Side("collect")
    time.sleep(0.1)
    s.stop()
    r = s.report()
    assert r["mode"] == "collect" and r["calls"] >= 1 and r["collections"] >= 1
    assert r["tracked_objects"] > 0
    s = probe._Side("none")
    s.stop()
    assert s.report()["calls"] == 0


def test_hold_lock_side_thread_stalls_this_thread():
    """The hold-lock side thread keeps the interpreter lock through its
    30 ms sleeps: this thread, ticking every millisecond, sees gaps of about
    that length (a Python busy loop would give the lock up every switch
    interval)."""
    import time

    s = probe._Side("hold-lock")
    ticks = []
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.2:
        ticks.append(time.perf_counter())
        time.sleep(0.001)
    s.stop()
    gaps = [b - a for a, b in zip(ticks, ticks[1:])]
    assert max(gaps) >= 0.025
    r = s.report()
    assert r["mode"] == "hold-lock" and r["calls"] >= 1
