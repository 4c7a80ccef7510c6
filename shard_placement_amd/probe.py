"""Interference probe: how much the reduce-scatter slows a concurrent GEMM.

The paper measures a 69% slowdown of a concurrent GEMM (one that would fit
in one wave of thread blocks on its own) caused by the default NCCL
reduce-scatter, and reports that TIDE lowers that interference roughly
tenfold (Abstract of "The Endgame of
FSDP Communication", weekinpapers.com; kongchang.com article, sections "The
Root of FSDP2 Communication Overhead" and "Performance").  This probe times a
bf16 GEMM (torch.matmul -> hipBLASLt) alone, then beside a train of
reduce-scatter launches on another stream, under several ways of confining
the reduce-scatter: all CUs with one short-lived workgroup per tile, a capped
grid of persistent workgroups, a CU-masked stream, and the launch size (a
call cut into launches of about launch_mib MiB each).  The GEMM shape is
chosen so that its grid is at most one workgroup per CU (checked with the
rocprofv3 kernel trace).  It is a measurement: nothing here is parity.
"""
from __future__ import annotations

import contextlib
import gc
from typing import Dict, List, Optional, Sequence, Tuple

import torch

from . import api

# A mode: (name, plan, max_workgroups, CU-mask width); 0 = unlimited / all.
Mode = Tuple[str, "api.Plan", int, int]


def _median(xs: List[float]) -> Optional[float]:
    if not xs:
        return None
    xs = sorted(xs)
    return xs[len(xs) // 2]


@contextlib.contextmanager
def _no_gc():
    """The heap frozen and the collector paused while timing.

    A full collection walks every tracked Python object (about 170 K in a
    process holding torch and this package: 18-35 ms of one core) and keeps
    the interpreter lock for the whole walk, so the thread that issues GPU
    work stops for that long.  The GPU runs out of queued work and idles,
    and kernels issued after an idle stretch of 10 ms or more run slower
    for a while (the single-wave GEMM: a median of 219-225 us against 201-206
    right after other work, up to +25% ten to twenty GEMMs in; see
    gemm_after_idle).  Measured on the R = 64 layer with a side thread acting
    every 20 ms during the probe: collections, or a 30 ms sleep that keeps
    the lock and touches no memory, stretched the GEMM from 0.20-0.21 to up
    to 0.24-0.25 ms, alone or beside the reduce-scatter depending on where
    the stall fell (readings -7..+22% instead of +3..5%); after gc.freeze()
    the collections take 0.02 ms and the reading is the quiet one.  So the
    heap is frozen here (any collection in the window has almost nothing to
    walk), and the collector is also paused, as Python's timeit does; both
    are restored on exit."""
    was = gc.isenabled()
    gc.collect()
    gc.freeze()
    gc.disable()
    try:
        yield
    finally:
        gc.unfreeze()
        if was:
            gc.enable()


class DealtRS:
    """A mode's reduce-scatter with its launches dealt over the probe's
    stream and ``extra`` streams in turn (tide_rs_bf16_to_fp32_streams)."""

    def __init__(self, plan, extra):
        self.plan, self.extra, self.info = plan, list(extra), plan.info

    def rs(self, max_workgroups: int = 0, stream=None) -> None:
        self.plan.rs_streams(self.extra, max_workgroups=max_workgroups, stream=stream)


def _new_stream():
    """The stream the GEMM trains run on (its own, so that it gets a
    hardware queue apart from the reduce-scatter's)."""
    return torch.cuda.Stream()


def _gemm_train(a, b, c, stream, n):
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    with torch.cuda.stream(stream):
        for e0, e1 in evs:
            e0.record(stream)
            torch.matmul(a, b, out=c)
            e1.record(stream)
    return evs


def run(modes: Sequence[Mode], rs_bytes: int, iters: int = 40, M: int = 4096, N: int = 4096,
        K: int = 8192, quiet_gc: bool = True) -> Dict:
    """Time the GEMM alone, then, per mode, alone again and beside the
    mode's reduce-scatter (the slowdown is against the mode's own alone
    time).  The
    reduce-scatter always runs on a CU-masked stream, which HIP backs with a
    hardware queue of its own (with the full mask when the mode has none):
    two streams that share a hardware queue run one after the other, which
    would hide any interference.  Each mode's record says how many GEMMs
    overlapped a reduce-scatter call's own span (gemms_overlapping_rs,
    ran_concurrently), from events around every call.  The heap is frozen
    and the garbage collector paused meanwhile (quiet_gc=False leaves both
    alone)."""
    if not quiet_gc:
        return _run(modes, rs_bytes, iters, M, N, K)
    with _no_gc():
        return _run(modes, rs_bytes, iters, M, N, K)


def _run(modes, rs_bytes, iters, M, N, K) -> Dict:
    dev = torch.device("cuda")
    n_all = torch.cuda.get_device_properties(dev).multi_processor_count
    a = torch.randn(M, K, device=dev, dtype=torch.bfloat16)
    b = torch.randn(K, N, device=dev, dtype=torch.bfloat16)
    c = torch.empty(M, N, device=dev, dtype=torch.bfloat16)
    gemm_stream = _new_stream()
    for _ in range(5):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    alone = _gemm_train(a, b, c, gemm_stream, iters)
    torch.cuda.synchronize()
    t0 = _median([e0.elapsed_time(e1) for e0, e1 in alone])
    out = {"gemm": "bf16 [%d,%d]x[%d,%d] torch.matmul" % (M, K, K, N),
           "gemm_tflops_alone": round(2.0 * M * N * K / (t0 * 1e-3) / 1e12, 1),
           "t_gemm_alone_ms": round(t0, 4), "cus": n_all, "modes": []}
    for name, plan, max_wg, n_cu in modes:
        rs_stream = api.tide_stream_create_cu_limited(n_cu or n_all)
        try:
            plan.rs(max_workgroups=max_wg, stream=rs_stream)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(rs_stream)
            for _ in range(3):
                plan.rs(max_workgroups=max_wg, stream=rs_stream)
            e1.record(rs_stream)
            torch.cuda.synchronize()
            rs_alone = e0.elapsed_time(e1) / 3
            # the GEMM alone again, right before this mode (clocks drift
            # over a sweep; each mode is compared with its own baseline)
            own = _gemm_train(a, b, c, gemm_stream, iters)
            torch.cuda.synchronize()
            t0m = _median([e0.elapsed_time(e1) for e0, e1 in own])
            # concurrent: enough reduce-scatters to cover the GEMM train twice
            n_rs = max(2, int(2.0 * iters * t0m / rs_alone) + 2)
            # the GEMM train is queued right after the first reduce-scatter
            # call, so that its queue holds work while the reduce-scatter
            # runs however long the host takes to issue the rest
            # an event before and after every call marks the calls' own spans
            calls = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                     for _ in range(n_rs)]
            r0 = calls[0][0]
            for k, (c0, c1) in enumerate(calls):
                c0.record(rs_stream)
                plan.rs(max_workgroups=max_wg, stream=rs_stream)
                c1.record(rs_stream)
                if k == 0:
                    gemm_stream.wait_event(r0)
                    conc = _gemm_train(a, b, c, gemm_stream, iters)
            torch.cuda.synchronize()
            window = r0.elapsed_time(calls[-1][1])
            inside = [e1.elapsed_time(e2) for e1, e2 in conc
                      if r0.elapsed_time(e1) >= 0.0 and r0.elapsed_time(e2) <= window]
            t1 = _median(inside)
            rs_conc = window / n_rs
            # did the two trains run side by side?  Streams that share a
            # hardware queue run one after the other: then every GEMM falls
            # between the end of one call and the start of the next
            spans = [(r0.elapsed_time(c0), r0.elapsed_time(c1)) for c0, c1 in calls]
            gemms = [(r0.elapsed_time(e1), r0.elapsed_time(e2)) for e1, e2 in conc]
            overlapping = sum(1 for g0, g1 in gemms
                              if any(min(g1, s1) - max(g0, s0) > 0.1 * (g1 - g0) for s0, s1 in spans))
            info = plan.info
            out["modes"].append({
                "mode": name, "max_workgroups": max_wg or None, "cu_mask": n_cu or None,
                "tiles_per_launch": int(info.rs_launch_tiles),
                "lds_per_workgroup": int(info.rs_lds_bytes),
                "launches_per_rs": -(-int(info.rs_tiles) // max(1, int(info.rs_launch_tiles))),
                "rs_alone_ms": round(rs_alone, 4),
                "rs_alone_gbps": round(rs_bytes / (rs_alone * 1e-3) / 1e9, 1),
                "rs_concurrent_gbps": round(rs_bytes / (rs_conc * 1e-3) / 1e9, 1),
                "t_gemm_alone_ms": round(t0m, 4),
                "t_gemm_concurrent_ms": round(t1, 4) if t1 else None,
                "gemm_inside": len(inside),
                "gemms_overlapping_rs": overlapping,
                "ran_concurrently": bool(overlapping > 0),
                # no GEMM inside the window: it waited for the whole train
                "gemm_slowdown_pct": round(100.0 * (t1 / t0m - 1.0), 2) if t1 else "starved",
            })
        finally:
            torch.cuda.synchronize()
            api.tide_stream_destroy(rs_stream)
    return out


def gemm_during(host_call, expect_ms: float, M: int = 4096, N: int = 4096, K: int = 8192) -> Dict:
    with _no_gc():
        return _gemm_during(host_call, expect_ms, M, N, K)


def _gemm_during(host_call, expect_ms, M, N, K) -> Dict:
    """Median time of the single-wave GEMM alone (trains before and after,
    pooled), and while ``host_call`` (a host-synchronous call that keeps the
    DMA engines busy for about expect_ms, e.g. copy-engine staging) runs: a
    GEMM train of about half that length is queued on its own stream just
    before the call."""
    dev = torch.device("cuda")
    a = torch.randn(M, K, device=dev, dtype=torch.bfloat16)
    b = torch.randn(K, N, device=dev, dtype=torch.bfloat16)
    c = torch.empty(M, N, device=dev, dtype=torch.bfloat16)
    s = _new_stream()
    for _ in range(5):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    alone = _gemm_train(a, b, c, s, 30)
    torch.cuda.synchronize()
    t0 = _median([e0.elapsed_time(e1) for e0, e1 in alone])
    n = max(4, min(400, int(0.5 * expect_ms / t0)))
    conc = _gemm_train(a, b, c, s, n)
    host_call()
    torch.cuda.synchronize()
    t1 = _median([e0.elapsed_time(e1) for e0, e1 in conc])
    after = _gemm_train(a, b, c, s, 30)
    torch.cuda.synchronize()
    t0 = _median([e0.elapsed_time(e1) for e0, e1 in alone + after])
    return {"gemm_alone_ms": round(t0, 4), "gemm_during_staging_ms": round(t1, 4),
            "gemm_during_staging": n,
            "gemm_slowdown_during_staging_pct": round(100.0 * (t1 / t0 - 1.0), 2)}


def gemm_after_idle(idle_ms: Sequence[float] = (0, 2, 10, 30, 100, 300), n: int = 60,
                    rounds: int = 2, M: int = 4096, N: int = 4096, K: int = 8192) -> List[Dict]:
    """The single-wave GEMM train issued after the GPU sat idle (nothing
    queued, the host asleep) for idle_ms: the median per-GEMM time and the
    mean of each group of five by position in the train, in microseconds."""
    import time

    dev = torch.device("cuda")
    a = torch.randn(M, K, device=dev, dtype=torch.bfloat16)
    b = torch.randn(K, N, device=dev, dtype=torch.bfloat16)
    c = torch.empty(M, N, device=dev, dtype=torch.bfloat16)
    s = _new_stream()
    out = []
    with _no_gc():
        for _ in range(2):
            _gemm_train(a, b, c, s, n)
            torch.cuda.synchronize()
        for _ in range(rounds):
            for idle in idle_ms:
                torch.cuda.synchronize()
                time.sleep(idle / 1e3)
                evs = _gemm_train(a, b, c, s, n)
                torch.cuda.synchronize()
                t = [1e3 * e0.elapsed_time(e1) for e0, e1 in evs]
                out.append({"idle_ms": idle, "median_us": round(_median(t), 1),
                            "us_by_position_of_5": [round(sum(t[i:i + 5]) / len(t[i:i + 5]), 1)
                                                    for i in range(0, len(t), 5)]})
    return out


def main(argv=None) -> int:
    """Standalone probe: set up one layer (reduce-scatter buffers only) and
    run the default-launch probe ``--reps`` times in this process; prints
    one JSON line {"workload": ..., "probe": {...}} with every repetition.
    With --after-idle: only the GEMM trains after idle stretches
    (gemm_after_idle), one JSON line per train."""
    import argparse
    import json

    from . import configs, harness

    ap = argparse.ArgumentParser(description=main.__doc__)
    ap.add_argument("--workload", default="5", help="workload key or name")
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--iters", type=int, default=40)
    ap.add_argument("--side", default="none",
                    choices=("none", "collect", "collect-frozen", "trim", "hold-lock"),
                    help="a side thread acting every 20 ms during the probe: a full garbage "
                         "collection, the same after gc.freeze(), malloc_trim(0), or a 30 ms "
                         "sleep that keeps the interpreter lock")
    ap.add_argument("--after-idle", action="store_true",
                    help="time GEMM trains issued after the GPU idled 0-300 ms instead")
    a = ap.parse_args(argv)
    if not torch.cuda.is_available():
        raise SystemExit("the probe needs a GPU")
    if a.after_idle:
        for rec in gemm_after_idle():
            print(json.dumps(rec), flush=True)
        return 0
    w = configs.get(a.workload)
    st = harness.setup(w, with_ag=False)
    torch.cuda.synchronize()
    side = _Side(a.side)
    res = None
    for _ in range(a.reps):
        r = run([("default launches", st.plan, 0, 0)], harness.rs_bytes(w), iters=a.iters,
                 quiet_gc=a.side == "none")
        if res is None:
            res = r
        else:
            res["modes"] += r["modes"]
    side.stop()
    print(json.dumps({"workload": w.name, "R": w.R, "side": side.report(), "probe": res}),
          flush=True)
    return 0


class _Side:
    """A thread that, every 20 ms until stopped, runs a full garbage
    collection ("collect"), the same after freezing the heap once
    ("collect-frozen"), glibc's malloc_trim(0) ("trim"), or a 30 ms usleep
    called through ctypes.PyDLL, which keeps the interpreter lock for the
    whole call and touches no memory ("hold-lock": a collection also keeps
    the lock for its whole walk, while a Python-level busy loop would give it
    up every switch interval); collections are logged through gc.callbacks."""

    def __init__(self, mode: str):
        import ctypes
        import threading
        import time

        self.mode, self.took, self.log = mode, [], []
        self._t0 = 0.0
        gc.callbacks.append(self._cb)
        if mode == "collect-frozen":
            gc.collect()
            gc.freeze()
        self._stop = threading.Event()
        libc = ctypes.CDLL("libc.so.6") if mode == "trim" else None
        # PyDLL: the call runs with the interpreter lock held
        locked = ctypes.PyDLL("libc.so.6") if mode == "hold-lock" else None

        def loop():
            while not self._stop.is_set():
                time.sleep(0.02)
                t = time.perf_counter()
                if mode in ("collect", "collect-frozen"):
                    gc.collect()
                elif mode == "trim":
                    libc.malloc_trim(0)
                elif mode == "hold-lock":
                    locked.usleep(30000)
                self.took.append(time.perf_counter() - t)
        self._th = threading.Thread(target=loop, daemon=True)
        if mode != "none":
            self._th.start()

    def _cb(self, phase, info):
        import time

        if phase == "start":
            self._t0 = time.perf_counter()
        else:
            self.log.append((info["generation"], info["collected"], time.perf_counter() - self._t0))

    def stop(self):
        self._stop.set()
        if self._th.is_alive():
            self._th.join()
        gc.callbacks.remove(self._cb)
        if self.mode == "collect-frozen":
            gc.unfreeze()

    def report(self) -> Dict:
        return {"mode": self.mode, "calls": len(self.took),
                "call_ms_mean": round(1e3 * sum(self.took) / max(1, len(self.took)), 3),
                "collections": len(self.log),
                "objects_freed": sum(c for _, c, _ in self.log),
                "tracked_objects": len(gc.get_objects())}


if __name__ == "__main__":
    raise SystemExit(main())
