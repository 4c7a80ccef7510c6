"""One-GPU analog of stock FSDP2's layout conversion, kept beside the fused
path for comparison.

The pages put 6.4% of a Llama-3.1-70B training step into layout conversion:
packing each rank's gradients into a flat, rank-major fp32 buffer before the
reduce-scatter, and copying the all-gather output back out into parameter
storage (Abstract and "The Root of FSDP2 Communication Overhead" of "The
Endgame of FSDP Communication", weekinpapers.com / kongchang.com).  This
module does those steps the way stock FSDP2 does them, with PyTorch's own
operators on the GPU, for the same R simulated ranks:

* reduce-scatter: for every rank, ``torch._chunk_cat`` casts its bf16
  gradients to fp32 and packs them, dim-0 chunk r of every parameter into
  row r of an [R, S] buffer (zero-padded, the same slot layout as the fused
  path); the rows are then summed over ranks in rank order with
  ``add_``.  Row r of the sum is rank r's fp32 shard arena.
* placement: ``torch.split_with_sizes_copy`` copies the [R, S] gathered
  buffer into padded [R, m_p] views of per-parameter buffers; the parameter
  is the first dim0 rows of its buffer.

The adds are element-wise fp32 in rank order 0..R-1, starting from rank 0's
value, so the result is bit-identical to the fused kernel's fixed order.
Nothing here is part of the fused path, and nothing here is the oracle.
"""
from __future__ import annotations

from typing import List

import torch

from . import configs


def _rows(shape):
    """(dim0, row numel) of a parameter; a 0-d parameter is one row of one."""
    if len(shape) == 0:
        return 1, 1
    c = 1
    for d in shape[1:]:
        c *= int(d)
    return int(shape[0]), c


def rs_traffic(w: configs.Workload, S: int) -> int:
    """HBM bytes the stock analog moves for one reduce-scatter: per rank a
    pack (N*2 read, R*S*4 written), then R-1 in-place adds of R*S floats
    (two reads, one write each)."""
    n = w.numel()
    return w.R * (n * 2 + w.R * S * 4) + (w.R - 1) * 3 * w.R * S * 4


class StockPath:
    """Stock-FSDP2-style buffers over given gradients (grads[q][p], bf16)
    and a gathered buffer (bf16, R*S), tight packing only.  Runs wherever
    the tensors are (the comparison is made on the GPU)."""

    def __init__(self, w: configs.Workload, S: int, grads=None, gathered=None, device=None):
        self.w = w
        self.R = w.R
        self.S = S
        live = []
        for p, shape in enumerate(w.shapes):
            d0, c = _rows(shape)
            if d0 * c:
                live.append((p, d0, c))
        self.live = live
        dev = device
        self.g2d: List[List[torch.Tensor]] = []
        if grads:
            for q in range(self.R):
                self.g2d.append([grads[q][p].reshape(d0, c) for p, d0, c in live])
            self.acc = torch.empty(self.R, self.S, dtype=torch.float32, device=dev)
            self.flat = torch.empty(self.R, self.S, dtype=torch.float32, device=dev)
        self.gathered = gathered
        if gathered is not None:
            self.sizes = []
            self.unsharded = []
            self.ag_out = []
            for p, d0, c in live:
                s = -(-d0 // self.R)
                buf = torch.empty(self.R * s * c, dtype=torch.bfloat16, device=dev)
                self.unsharded.append((p, buf[: d0 * c]))
                self.ag_out.append(buf.view(self.R, s * c))
                self.sizes.append(s * c)

    @classmethod
    def from_setup(cls, st) -> "StockPath":
        """Over the buffers of a ``harness.Setup``."""
        return cls(st.w, st.S, st.grads or None, st.gathered, st.device)

    def rs(self) -> None:
        """Pack every rank (cast + chunk + pad into [R, S] fp32) and add the
        packed buffers in rank order into ``acc``."""
        for q in range(self.R):
            dst = self.acc if q == 0 else self.flat
            torch._chunk_cat(self.g2d[q], dim=0, num_chunks=self.R, out=dst)
            if q:
                self.acc.add_(self.flat)

    def pack(self) -> None:
        """The layout-conversion part of ``rs`` alone: every rank's cast and
        pack, no adds."""
        for q in range(self.R):
            torch._chunk_cat(self.g2d[q], dim=0, num_chunks=self.R, out=self.flat)

    def ag(self) -> None:
        """Copy the gathered [R, S] buffer out into padded per-parameter
        buffers."""
        torch.split_with_sizes_copy(self.gathered.view(self.R, self.S), self.sizes, dim=1,
                                    out=self.ag_out)

    def same_rs_bits(self, out: List[torch.Tensor]) -> bool:
        """Row r of ``acc`` against the fused path's rank-r arena, bit for bit."""
        return all(torch.equal(self.acc[r].view(torch.int32), out[r][: self.S].view(torch.int32))
                   for r in range(self.R))

    def same_ag_bits(self, full: List[torch.Tensor]) -> bool:
        return all(torch.equal(t.view(torch.int16), full[p].reshape(-1).view(torch.int16))
                   for p, t in self.unsharded)
