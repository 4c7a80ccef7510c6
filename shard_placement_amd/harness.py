"""Device-side set-up of a workload: seeded gradients, shard arenas, the
gathered buffer and the full tensors, and the plan that ties them together.

Used by bench.py, the GPU tests and the smoke check.  It allocates with torch
(device memory is PyTorch's job here) and draws inputs with ``synth``; all
data-path work is done by the library through ``api``.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import torch

from . import api, configs, synth

F32_NAN_BITS = -1  # 0xFFFFFFFF as int32: a NaN pre-fill that shows unwritten words
BF16_SENTINEL = -1  # 0xFFFF as int16


@dataclass
class Setup:
    w: configs.Workload
    device: torch.device
    arenas: List[torch.Tensor]                 # per rank: flat bf16 gradient arena
    grads: List[List[torch.Tensor]]            # per rank, per param: views
    out: List[torch.Tensor]                    # per rank: fp32 arena (S floats, view)
    out_alloc: List[torch.Tensor]              # what holds the arenas (incl. guard bands)
    gathered: Optional[torch.Tensor] = None    # rank-major bf16 slots (R*S)
    full: Optional[List[torch.Tensor]] = None  # per param: bf16 full tensor
    full_arena: Optional[torch.Tensor] = None
    vacated: Optional[List[torch.Tensor]] = None  # Slot-Reuse: per-rank gathered buffers
    plan: Optional[api.Plan] = None
    S: int = 0
    guard: int = 0

    def free(self):
        for name in ("arenas", "grads", "out", "out_alloc", "gathered", "full", "full_arena",
                     "vacated", "plan"):
            setattr(self, name, None)


def rs_bytes(w: configs.Workload) -> int:
    """Algorithmic bytes of one reduce-scatter: R*N*2 read + N*4 written."""
    n = w.numel()
    return w.R * n * 2 + n * 4


def ag_bytes(w: configs.Workload) -> int:
    """Algorithmic bytes of one placement: N*2 read + N*2 written."""
    n = w.numel()
    return 4 * n


ROW_QUANTUM_BYTES = 2 << 20  # packed rank rows start on 2 MiB boundaries


def _rank_rows(R: int, n: int, dtype, device, packed: bool) -> List[torch.Tensor]:
    """R flat buffers of n elements: views of one allocation whose rows start
    every round_up(n, 2 MiB) bytes (packed), or R allocations of their own."""
    if not packed:
        return [torch.empty(n, dtype=dtype, device=device) for _ in range(R)]
    q = ROW_QUANTUM_BYTES // torch.empty(0, dtype=dtype).element_size()
    stride = -(-n // q) * q if n else 0
    whole = torch.empty(R * stride, dtype=dtype, device=device)
    return [whole[r * stride: r * stride + n] for r in range(R)]


def setup(w: configs.Workload, device="cuda", with_rs=True, with_ag=True, guard: int = 256,
          slot_reuse: Optional[bool] = None, same_for_all: bool = False, align: int = 1,
          rs_tile: int = 0, ag_tile: int = 0, flags: int = -1, gen_device=None,
          launch_mib: int = 0, rank_layout: str = "packed") -> Setup:
    """Allocate and fill one workload.  Output arenas carry `guard` NaN-filled
    floats on each side (canaries).  With Slot-Reuse, rank r's fp32 arena is
    placed at byte 0 of rank r's own vacated gathered buffer (2*R*S bytes,
    R >= 2) and no other output memory is allocated.

    rank_layout: "packed" carves the R ranks' gradient arenas (and the
    per-rank output arenas / vacated gathered buffers) out of one allocation
    each, one row per rank on 2 MiB boundaries; "separate" allocates every
    rank's arena on its own.  The
    library takes any pointers either way; on MI355X the packed layout reads
    4-8% faster at R = 16..32 (fewer distinct allocations for the R source
    streams to walk)."""
    if rank_layout not in ("packed", "separate"):
        raise ValueError("rank_layout must be 'packed' or 'separate'")
    packed = rank_layout == "packed"
    device = torch.device(device)
    gen_device = torch.device(gen_device) if gen_device is not None else device
    slot_reuse = w.slot_reuse if slot_reuse is None else slot_reuse
    _, _, _, S = api.tide_desc_geometry(w.shapes, w.R, align)
    st = Setup(w=w, device=device, arenas=[], grads=[], out=[], out_alloc=[], S=S, guard=guard)
    if with_rs:
        n = synth.arena_numel(w.shapes)
        rows = _rank_rows(w.R, n, torch.bfloat16, device, packed)
        for q in range(w.R):
            a = rows[q] if gen_device == device else torch.empty(n, dtype=torch.bfloat16,
                                                                  device=gen_device)
            synth.fill_normal_(a, synth.SEED_STRIDE * w.key + (0 if same_for_all else q), w.sigma)
            if a is not rows[q]:
                rows[q].copy_(a)
                a = rows[q]
            st.arenas.append(a)
            st.grads.append(synth.views(a, w.shapes))
        if slot_reuse:
            if w.R < 2:
                raise ValueError("Slot-Reuse needs R >= 2 (an fp32 arena is twice a bf16 slot)")
            st.vacated = []
            rows = _rank_rows(w.R, w.R * S + 2 * guard, torch.bfloat16, device, packed)
            for r in range(w.R):
                buf = rows[r]
                buf.view(torch.int16).fill_(BF16_SENTINEL)
                st.vacated.append(buf)
                st.out_alloc.append(buf)
                st.out.append(buf[: 2 * S].view(torch.float32) if S else
                              torch.empty(0, dtype=torch.float32, device=device))
        else:
            rows = _rank_rows(w.R, S + 2 * guard, torch.float32, device, packed)
            for r in range(w.R):
                buf = rows[r]
                buf.view(torch.int32).fill_(F32_NAN_BITS)
                st.out_alloc.append(buf)
                st.out.append(buf[guard:guard + S])
    if with_ag:
        if st.vacated is not None:
            # rank 0's own gathered buffer: placed first, then vacated and
            # reused for rank 0's fp32 arena
            st.gathered = st.vacated[0][: w.R * S]
            synth.fill_normal_(st.gathered, synth.SEED_STRIDE * w.key + synth.GATHERED_SEED_OFFSET,
                               w.sigma)
        else:
            st.gathered = torch.empty(w.R * S, dtype=torch.bfloat16, device=gen_device)
            synth.fill_normal_(st.gathered, synth.SEED_STRIDE * w.key + synth.GATHERED_SEED_OFFSET,
                               w.sigma)
            if st.gathered.device != device:
                st.gathered = st.gathered.to(device)
        n = synth.arena_numel(w.shapes)
        st.full_arena = torch.empty(n + 2 * guard, dtype=torch.bfloat16, device=device)
        st.full_arena.view(torch.int16).fill_(BF16_SENTINEL)
        st.full = synth.views(st.full_arena[guard:guard + n], w.shapes)
    st.plan = api.Plan(w.shapes, w.R,
                       grads=st.grads if with_rs else None, out=st.out if with_rs else None,
                       gathered=st.gathered, full=st.full, align=align, rs_tile=rs_tile,
                       ag_tile=ag_tile, flags=flags, launch_mib=launch_mib)
    return st


def stage_buffers(st: Setup, slot_stride: int = 0, rank_layout: str = "packed",
                  offset: int = 0) -> List[torch.Tensor]:
    """R staging buffers for the copy-engine-staged reduce-scatter, each R
    slots of slot_stride (default S) bf16 elements, filled with the 0xFFFF
    sentinel; ``offset`` elements into their allocation (to test unaligned
    slots)."""
    w = st.w
    stride = slot_stride or st.S
    n = w.R * stride
    rows = _rank_rows(w.R, n + offset, torch.bfloat16, st.device, rank_layout == "packed")
    out = []
    for r in range(w.R):
        rows[r].view(torch.int16).fill_(BF16_SENTINEL)
        out.append(rows[r][offset:offset + n])
    return out


class BlockReader:
    """Reads one workload's reduce-scatter inputs and results back to the
    host in blocks of consecutive flat indices of one parameter, through
    pinned buffers, so that a whole layer can be checked on the CPU with
    bounded host memory.

    The caller supplies the shard geometry (chunk numel m[p] and arena
    offset off[p] of every param) that says where the results of a flat
    index lie: rank j // m[p], element off[p] + j % m[p] of its arena.
    Two buffer sets alternate: the copies of block k + 1 run while the
    caller works on block k.  Each block holds the R ranks' bf16 bits
    (uint16) and the result words (uint32) for flat indices [a, b); the
    arrays handed out stay valid until the next block is requested."""

    def __init__(self, st: Setup, m, off, block_bytes: int = 512 << 20):
        self.st = st
        self.m = [int(x) for x in m]
        self.off = [int(x) for x in off]
        R = st.w.R
        self.block = max(1 << 16, block_bytes // (2 * R) // 4096 * 4096)
        self.g = [torch.empty((R, self.block), dtype=torch.int16, pin_memory=True) for _ in range(2)]
        self.o = [torch.empty(self.block, dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self.stream = torch.cuda.Stream(device=st.device)
        self.copy_s = 0.0  # host time spent waiting for copies

    def _issue(self, k: int, p: int, a: int, b: int):
        st, R = self.st, self.st.w.R
        mp, L = self.m[p], b - a
        ev = torch.cuda.Event()
        self.stream.wait_stream(torch.cuda.current_stream(st.device))
        with torch.cuda.stream(self.stream):
            for q in range(R):
                src = st.grads[q][p].reshape(-1)[a:b].view(torch.int16)
                self.g[k][q, :L].copy_(src, non_blocking=True)
            pos = 0
            for r in range(a // mp, (b - 1) // mp + 1):
                lo, hi = max(a, r * mp), min(b, (r + 1) * mp)
                base = self.off[p] - r * mp
                src = st.out[r][base + lo: base + hi].view(torch.int32)
                self.o[k][pos:pos + hi - lo].copy_(src, non_blocking=True)
                pos += hi - lo
            ev.record(self.stream)
        return ev

    def blocks(self, p: int):
        """Yield (a, b, grads, out): grads a list of R uint16 arrays of b - a
        elements, out a uint32 array of b - a result words."""
        import time

        import numpy as np

        shp = self.st.w.shapes[p]
        n = 1
        for d in shp:
            n *= int(d)
        if n == 0 or self.m[p] == 0:
            return
        spans = [(a, min(n, a + self.block)) for a in range(0, n, self.block)]
        pending = self._issue(0, p, *spans[0])
        try:
            for i, (a, b) in enumerate(spans):
                k = i & 1
                t0 = time.perf_counter()
                pending.synchronize()
                self.copy_s += time.perf_counter() - t0
                if i + 1 < len(spans):
                    pending = self._issue(k ^ 1, p, *spans[i + 1])
                L = b - a
                g = [self.g[k][q, :L].numpy().view(np.uint16) for q in range(self.st.w.R)]
                yield a, b, g, self.o[k][:L].numpy().view(np.uint32)
        finally:
            # a caller that stops early (an exception, a break) must not free
            # the pinned buffers under a copy that is still writing them
            pending.synchronize()
