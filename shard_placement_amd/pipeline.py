"""Two-phase reduce-scatter pipeline, emulated on one GPU.

The pages' reduce-scatter runs as a two-phase pipeline: an intra-node phase
reduces each chunk, a network phase delivers the partial results to their
owners, the phases overlap chunk by chunk, and the reduce-scatter's buffer
stays nearly constant as the job grows (Abstract of "The Endgame of FSDP
Communication", weekinpapers.com; "Performance" of the kongchang.com
article).  Here phase 1 is the fixed-order reduction of a chunk of tiles
into a slot of a ring of staging chunks (``tide_rs_tiles_to_stage``) and
phase 2, the stand-in for the network, moves a slot's results into the
shard arenas (``tide_rs_stage_to_shards``).  The phases run on two streams
with their own hardware queues; an event per chunk orders phase 2 after
phase 1, and phase 1 of chunk i waits for phase 2 of chunk i - depth (the
ring slot it reuses).  The staging memory is depth * chunk_tiles * tile
floats, whatever the layer.
"""
from __future__ import annotations

import torch

from . import api


class TwoPhase:
    """phase2: "cu" moves each chunk with a kernel; "sdma" with
    stream-ordered copy-engine copies.  phase2_cus confines the phase-2
    kernel to that many compute units (0: all), which caps its bandwidth
    the way a network link would."""

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
        self.chunk = int(chunk_tiles)
        self.depth = int(depth)
        dev = plan.d_blob.device
        self.ring = torch.empty(self.depth, self.chunk * self.T, dtype=torch.float32, device=dev)
        n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
        # two streams with hardware queues of their own (streams that share a
        # queue run one after the other)
        self.s1 = api.tide_stream_create_cu_limited(n_cu)
        self.s2 = api.tide_stream_create_cu_limited(phase2_cus or n_cu)

    @property
    def staging_bytes(self) -> int:
        return self.ring.numel() * 4

    def chunks(self) -> int:
        return -(-self.n // self.chunk)

    def run(self) -> None:
        """The whole reduce-scatter through the pipeline, ordered after the
        current stream's earlier work and before its later work."""
        cur = torch.cuda.current_stream()
        start = torch.cuda.Event()
        start.record(cur)
        self.s1.wait_event(start)
        self.s2.wait_event(start)
        drained = []
        for i in range(self.chunks()):
            b = i * self.chunk
            cnt = min(self.chunk, self.n - b)
            slot = self.ring[i % self.depth]
            if i >= self.depth:
                self.s1.wait_event(drained[i - self.depth])
            api.tide_rs_tiles_to_stage(self.plan.blob, self.plan.d_blob, b, cnt, slot,
                                       stream=self.s1)
            produced = torch.cuda.Event()
            produced.record(self.s1)
            self.s2.wait_event(produced)
            if self.phase2 == "cu":
                api.tide_rs_stage_to_shards(self.plan.blob, self.plan.d_blob, b, cnt, slot,
                                            stream=self.s2)
            else:
                api.tide_rs_stage_to_shards_sdma(self.plan.blob, b, cnt, slot, stream=self.s2)
            ev = torch.cuda.Event()
            ev.record(self.s2)
            drained.append(ev)
        cur.wait_stream(self.s1)
        cur.wait_stream(self.s2)

    def close(self) -> None:
        """Wait for the device and release the two streams (idempotent)."""
        if self.s1 is None:
            return
        torch.cuda.synchronize()
        api.tide_stream_destroy(self.s1)
        api.tide_stream_destroy(self.s2)
        self.s1 = self.s2 = None

    def __enter__(self) -> "TwoPhase":
        return self

    def __exit__(self, *exc) -> None:
        self.close()
