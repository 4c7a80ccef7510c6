"""Device-side set-up of a workload: seeded gradients, shard arenas, the
gathered buffer and the full tensors, and the plan that ties them together.

Used by bench.py, the GPU tests and the smoke check.  It allocates with torch
(device memory is PyTorch's job here) and draws inputs with ``synth``; all
data-path work is done by the library through ``api``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
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


def setup(w: configs.Workload, device="cuda", with_rs=True, with_ag=True, guard: int = 256,
          slot_reuse: Optional[bool] = None, same_for_all: bool = False, align: int = 1,
          rs_tile: int = 0, ag_tile: int = 0, flags: int = -1, gen_device=None,
          launch_mib: int = 0) -> Setup:
    """Allocate and fill one workload.  Output arenas carry `guard` NaN-filled
    floats on each side (canaries).  With Slot-Reuse, rank r's fp32 arena is
    placed at byte 0 of rank r's own vacated gathered buffer (2*R*S bytes,
    R >= 2) and no other output memory is allocated."""
    device = torch.device(device)
    gen_device = torch.device(gen_device) if gen_device is not None else device
    slot_reuse = w.slot_reuse if slot_reuse is None else slot_reuse
    _, _, _, S = api.tide_desc_geometry(w.shapes, w.R, align)
    st = Setup(w=w, device=device, arenas=[], grads=[], out=[], out_alloc=[], S=S, guard=guard)
    if with_rs:
        n = synth.arena_numel(w.shapes)
        for q in range(w.R):
            a = torch.empty(n, dtype=torch.bfloat16, device=gen_device)
            synth.fill_normal_(a, synth.SEED_STRIDE * w.key + (0 if same_for_all else q), w.sigma)
            if a.device != device:
                a = a.to(device)
            st.arenas.append(a)
            st.grads.append(synth.views(a, w.shapes))
        if slot_reuse:
            if w.R < 2:
                raise ValueError("Slot-Reuse needs R >= 2 (an fp32 arena is twice a bf16 slot)")
            st.vacated = []
            for r in range(w.R):
                buf = torch.empty(w.R * S + 2 * guard, dtype=torch.bfloat16, device=device)
                buf.view(torch.int16).fill_(BF16_SENTINEL)
                st.vacated.append(buf)
                st.out_alloc.append(buf)
                st.out.append(buf[: 2 * S].view(torch.float32) if S else
                              torch.empty(0, dtype=torch.float32, device=device))
        else:
            for r in range(w.R):
                buf = torch.empty(S + 2 * guard, dtype=torch.float32, device=device)
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
