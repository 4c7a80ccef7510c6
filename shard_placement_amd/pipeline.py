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
        current stream's earlier work and before its later work."""
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
