"""Two-phase reduce-scatter pipeline, emulated on one GPU.

The pages' reduce-scatter runs as a two-phase pipeline: an intra-node phase
reduces each chunk, a network phase delivers the partial results to their
owners, the phases overlap chunk by chunk, and the reduce-scatter's buffer
stays nearly constant as the job grows (Abstract of "The Endgame of FSDP
Communication", weekinpapers.com; "Performance" of the kongchang.com
article).  Here phase 1 is the fixed-order reduction of a chunk of tiles
into a slot of a ring of staging chunks (``tide_rs_tiles_to_stage``) and
phase 2, the stand-in for the network, moves a slot's results into the
shard arenas (``tide_rs_stage_to_shards``).  The library issues the chunk
loop itself (``tide_pipeline_run``): the phases run on two streams with
their own hardware queues; an event per ring slot orders phase 2 after
phase 1, and phase 1 of chunk i after phase 2 of chunk i - depth (the slot
it reuses).  The staging memory is depth * chunk_tiles * tile floats,
whatever the layer.
"""
from __future__ import annotations

import torch

from . import api


class TwoPhase:
    """phase2: "cu" moves each chunk with a kernel; "sdma" with
    stream-ordered copy-engine copies.  phase2_cus confines the phase-2
    kernel to that many compute units (0: all), which caps its bandwidth
    the way a network link would; phase 1 then runs on the other CUs."""

    def __init__(self, plan: "api.Plan", chunk_tiles: int, depth: int = 2, phase2: str = "cu",
                 phase2_cus: int = 0):
        if chunk_tiles < 1 or depth < 1:
            raise ValueError("chunk_tiles and depth must be >= 1")
        if phase2 not in ("cu", "sdma"):
            raise ValueError("phase2 must be 'cu' or 'sdma'")
        self.phase2 = phase2
        self.plan = plan
        self.T = int(plan.info.rs_tile_elems)
        self.n = int(plan.info.rs_tiles)
        self.chunk = min(int(chunk_tiles), max(1, self.n))
        self.depth = int(depth)
        dev = plan.d_blob.device
        slots = min(self.depth, self.chunks())
        self.ring = torch.empty(max(1, slots), self.chunk * self.T, dtype=torch.float32,
                                device=dev)
        with torch.cuda.device(dev):
            self.handle = api.tide_pipeline_create(self.depth, phase2_cus)

    @property
    def staging_bytes(self) -> int:
        return self.ring.numel() * 4

    def chunks(self) -> int:
        return -(-self.n // self.chunk)

    def run(self) -> None:
        """The whole reduce-scatter through the pipeline, ordered after the
        current stream's earlier work and before its later work.  Issue
        back-to-back calls from a stream other than the null stream (torch's
        default): the pipeline's CU-masked streams are blocking streams, and
        with work pending on the null stream they measured up to 20% slower."""
        if self.handle is None:
            raise RuntimeError("pipeline closed")
        api.tide_pipeline_run(self.handle, self.plan.blob, self.plan.d_blob, self.chunk,
                              self.ring, 1 if self.phase2 == "sdma" else 0)

    def close(self) -> None:
        """Wait for the pipeline's streams and release them (idempotent)."""
        if self.handle is None:
            return
        api.tide_pipeline_destroy(self.handle)
        self.handle = None

    def __enter__(self) -> "TwoPhase":
        return self

    def __exit__(self, *exc) -> None:
        self.close()


class Prequeued:
    """Tells a host-bound call from a device-bound one: the call timed as
    usual and with all of its work queued before the device starts on it,
    a spin kernel (a bounded count, torch.cuda._sleep) holding the stream
    while the host issues the call.  A call slower than its pre-queued self
    waits for the host; the host's issue time alone cannot tell, since a
    host blocked on a full queue also issues as slowly as the device runs.
    Both timings run on a stream of this object's own: behind a spin on the
    null stream, which synchronises with every blocking stream, the
    pre-queued call measured 10-70% slower than it runs."""

    def __init__(self):
        import time

        self._time = time.perf_counter
        self.stream = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.stream(self.stream):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(10 ** 6)
            e0.record()
            torch.cuda._sleep(10 ** 7)
            e1.record()
        torch.cuda.synchronize()
        self.units_per_ms = 1e7 / e0.elapsed_time(e1)

    def compare(self, fn):
        """{plain_ms, host_issue_ms, prequeued_ms} of fn (which issues its
        work on the current stream); prequeued_ms is None when the host took
        most of the spin (2 * issue time + 10 ms) to issue the call, so that
        the device may have started before the host finished."""
        torch.cuda.synchronize()
        with torch.cuda.stream(self.stream):
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record()
            h0 = self._time()
            fn()
            host = (self._time() - h0) * 1e3
            a1.record()
            torch.cuda.synchronize()
            gate = 2.0 * host + 10.0
            torch.cuda._sleep(int(gate * self.units_per_ms))
            b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            b0.record()
            h0 = self._time()
            fn()
            issued = (self._time() - h0) * 1e3
            b1.record()
            torch.cuda.synchronize()
        pre = None if issued > 0.8 * gate else b0.elapsed_time(b1)
        return {"plain_ms": a0.elapsed_time(a1), "host_issue_ms": host, "prequeued_ms": pre}


def main(argv=None) -> int:
    """Standalone pipelined runs on one layer, one phase-2 engine and a few
    chunk sizes, for kernel traces: prints one JSON line per configuration
    with the event time of a pipelined call (best of --reps), the host time
    to issue it, the call on a stream of its own timed as usual and queued
    before the device starts (see Prequeued), and its bits against the
    in-place reduce-scatter."""
    import argparse
    import json
    import time

    from . import configs, harness

    ap = argparse.ArgumentParser(description=main.__doc__)
    ap.add_argument("--workload", default="2")
    ap.add_argument("--phase2", default="cu", choices=("cu", "sdma"))
    ap.add_argument("--phase2-cus", type=int, default=0)
    ap.add_argument("--chunk-launches", default="1,4", help="chunk sizes in launches of the plan")
    ap.add_argument("--depth", type=int, default=2)
    ap.add_argument("--reps", type=int, default=2)
    ap.add_argument("--no-prequeued", action="store_true",
                    help="skip the own-stream and pre-queued timings (a kernel trace then holds "
                         "1 + reps pipelined calls per chunk size)")
    a = ap.parse_args(argv)
    if not torch.cuda.is_available():
        raise SystemExit("the pipeline needs a GPU")
    w = configs.get(a.workload)
    st = harness.setup(w, with_ag=False, guard=0)
    st.plan.rs()
    torch.cuda.synchronize()
    ref = [o.view(torch.int32).clone() for o in st.out]
    L = int(st.plan.info.rs_launch_tiles) or int(st.plan.info.rs_tiles)
    pq = None if a.no_prequeued else Prequeued()
    for mult in (float(x) for x in a.chunk_launches.split(",")):
        chunk = max(1, int(L * mult))
        with TwoPhase(st.plan, chunk, a.depth, a.phase2, a.phase2_cus) as tp:
            tp.run()
            torch.cuda.synchronize()
            best, host = None, None
            for _ in range(a.reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                h0 = time.perf_counter()
                tp.run()
                h1 = time.perf_counter()
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1)
                if best is None or ms < best:
                    best, host = ms, (h1 - h0) * 1e3
            cmp = pq.compare(tp.run) if pq else None
        same = all(torch.equal(r, o.view(torch.int32)) for r, o in zip(ref, st.out))
        rec = {"workload": w.name, "phase2": a.phase2, "phase2_cus": a.phase2_cus,
               "chunk_tiles": chunk, "depth": a.depth, "ms": round(best, 3),
               "host_issue_ms": round(host, 3), "same_bits": same}
        if cmp:
            pre = cmp["prequeued_ms"]
            rec.update({"own_stream_ms": round(cmp["plain_ms"], 3),
                        "own_stream_prequeued_ms": None if pre is None else round(pre, 3),
                        "host_bound": None if pre is None else bool(cmp["plain_ms"] > 1.1 * pre)})
        print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
