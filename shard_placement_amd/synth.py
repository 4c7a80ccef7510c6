"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module draws numbers and lays them out; it holds none of the method's
arithmetic (no reduction, no shard or offset rule).  Every rank's gradients
live in one contiguous bf16 arena of the rank, and the per-parameter tensors
are views into it (tight packing, registration order), as FSDP2 stores
gradients as per-parameter tensors.

Recipe: rank q of workload k draws from a generator seeded 1000*k + q; values
are float32 N(0, 1) scaled by sigma and rounded to bf16 (round to nearest
even, torch's conversion).  Large workloads are drawn on the GPU in chunks;
the tiny one on the CPU.
"""
from __future__ import annotations

from typing import List, Sequence

import torch

SEED_STRIDE = 1000
GATHERED_SEED_OFFSET = 999
CHUNK = 1 << 26  # elements drawn per torch.randn call


def numel(shape: Sequence[int]) -> int:
    n = 1
    for d in shape:
        n *= int(d)
    return n


def views(arena: torch.Tensor, shapes: Sequence[Sequence[int]]) -> List[torch.Tensor]:
    """Split a flat arena into contiguous per-parameter views, in order."""
    out, pos = [], 0
    for shp in shapes:
        n = numel(shp)
        out.append(arena[pos:pos + n].view(tuple(int(d) for d in shp)))
        pos += n
    return out


def arena_numel(shapes) -> int:
    return sum(numel(s) for s in shapes)


def fill_normal_(buf: torch.Tensor, seed: int, sigma: float) -> torch.Tensor:
    """Fill a flat bf16 tensor with RNE(N(0,1) * sigma), seeded."""
    gen = torch.Generator(device=buf.device)
    gen.manual_seed(int(seed))
    flat = buf.view(-1)
    for start in range(0, flat.numel(), CHUNK):
        stop = min(flat.numel(), start + CHUNK)
        tmp = torch.randn(stop - start, generator=gen, dtype=torch.float32,
                          device=buf.device)
        if sigma != 1.0:
            tmp.mul_(sigma)
        flat[start:stop].copy_(tmp)  # float32 -> bf16, round to nearest even
    return buf


def integer_grid_(buf: torch.Tensor, seed: int, kmax: int = 127, scale_log2: int = -10) -> torch.Tensor:
    """Fill with k * 2**scale_log2, k uniform in [-kmax, kmax] (exact in bf16)."""
    gen = torch.Generator(device=buf.device)
    gen.manual_seed(int(seed))
    k = torch.randint(-kmax, kmax + 1, (buf.numel(),), generator=gen,
                      dtype=torch.int32, device=buf.device)
    buf.view(-1).copy_(k.to(torch.float32) * (2.0 ** scale_log2))
    return buf


def bits_(buf: torch.Tensor, seed: int) -> torch.Tensor:
    """Fill a bf16 tensor with uniformly random 16-bit patterns (NaN payloads,
    infinities, subnormals and -0 included)."""
    gen = torch.Generator(device=buf.device)
    gen.manual_seed(int(seed))
    v = torch.randint(0, 1 << 16, (buf.numel(),), generator=gen, dtype=torch.int32,
                      device=buf.device)
    buf.view(-1).view(torch.int16).copy_(v.to(torch.int16))
    return buf


# Special bf16 bit patterns for edge-value tests.
SPECIAL_BF16 = {
    "+0": 0x0000, "-0": 0x8000, "min_sub": 0x0001, "max_sub": 0x007F,
    "-min_sub": 0x8001, "min_norm": 0x0080, "one": 0x3F80, "-one": 0xBF80,
    "max": 0x7F7F, "-max": 0xFF7F, "+inf": 0x7F80, "-inf": 0xFF80,
    "qnan": 0x7FC0,
}
