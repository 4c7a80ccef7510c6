"""Python binding of libtide: argument marshalling only.

Functions carry the C ABI's names (include/tide.h) and pass torch tensors'
device addresses and the current HIP stream straight through; every step of
the data path runs in the library's HIP kernels (or, for
``tide_ag_place_sdma``, on the DMA engines).  ``Plan`` bundles one layer's
descriptor table (host blob + its device copy) with the tensors it points
at, so that they outlive it.

Operations (Abstract of "The Endgame of FSDP Communication",
weekinpapers.com): the reduce-scatter reads R ranks' per-parameter bf16
gradients in place and writes each rank's fp32 dim-0 shards; the placement
writes a rank-major bf16 gathered buffer into per-parameter tensors.
"""
from __future__ import annotations

import ctypes
from typing import Sequence, Tuple

import numpy as np
import torch

from . import _lib
from ._lib import TideError, TideOpts, TidePlanInfo, TideShape, check

ORDERS = {"fixed": 0, "tree": 1}


def _shapes(shapes: Sequence[Sequence[int]]):
    arr = (TideShape * max(1, len(shapes)))()
    for i, shp in enumerate(shapes):
        shp = tuple(int(x) for x in shp)
        if len(shp) == 0:
            arr[i].dim0, arr[i].row_numel = 1, 1
        else:
            c = 1
            for d in shp[1:]:
                c *= d
            arr[i].dim0, arr[i].row_numel = shp[0], c
    return arr


def _opts(align: int = 1, rs_tile: int = 0, ag_tile: int = 0, flags: int = -1,
          launch_mib: int = 0) -> TideOpts:
    return TideOpts(int(align), int(rs_tile), int(ag_tile), int(flags), int(launch_mib))


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


def tide_desc_geometry(shapes, R: int, align: int = 1) -> Tuple[np.ndarray, np.ndarray, np.ndarray, int]:
    """(chunk rows, shard numel, offsets, slot numel S) from the library."""
    L = _lib.lib()
    P = len(shapes)
    s = np.zeros(max(1, P), np.int64)
    m = np.zeros(max(1, P), np.int64)
    off = np.zeros(max(1, P), np.int64)
    S = ctypes.c_int64(0)
    i64p = ctypes.POINTER(ctypes.c_int64)
    o = _opts(align)
    check(L.tide_desc_geometry(_shapes(shapes), P, int(R), ctypes.byref(o),
                               s.ctypes.data_as(i64p), m.ctypes.data_as(i64p),
                               off.ctypes.data_as(i64p), ctypes.byref(S)), "tide_desc_geometry")
    return s[:P], m[:P], off[:P], int(S.value)


def tide_desc_size(shapes, R: int, align: int = 1, rs_tile: int = 0, ag_tile: int = 0,
                   flags: int = -1, launch_mib: int = 0) -> int:
    n = ctypes.c_size_t(0)
    o = _opts(align, rs_tile, ag_tile, flags, launch_mib)
    check(_lib.lib().tide_desc_size(_shapes(shapes), len(shapes), int(R), ctypes.byref(o),
                                    ctypes.byref(n)), "tide_desc_size")
    return int(n.value)


def tide_desc_build(shapes, R: int, grad_ptrs=None, out_ptrs=None, gathered_ptr=None,
                    full_ptrs=None, align: int = 1, rs_tile: int = 0, ag_tile: int = 0,
                    flags: int = -1, launch_mib: int = 0) -> Tuple[np.ndarray, TidePlanInfo]:
    """Build a host plan blob from raw device addresses (ints).  grad_ptrs is
    rank-major [R*P]; out_ptrs [R]; full_ptrs [P].  Returns (blob, info)."""
    L = _lib.lib()
    P = len(shapes)
    size = tide_desc_size(shapes, R, align, rs_tile, ag_tile, flags, launch_mib)
    blob = np.zeros(size, np.uint8)
    vp = ctypes.c_void_p

    def arr(ptrs, n):
        if ptrs is None:
            return None
        a = (vp * max(1, n))()
        for i, x in enumerate(ptrs):
            a[i] = int(x) if x else None
        return a

    info = TidePlanInfo()
    o = _opts(align, rs_tile, ag_tile, flags, launch_mib)
    st = L.tide_desc_build(_shapes(shapes), P, int(R), ctypes.byref(o), arr(grad_ptrs, R * P),
                           arr(out_ptrs, R), vp(int(gathered_ptr)) if gathered_ptr else None,
                           arr(full_ptrs, P), blob.ctypes.data, blob.nbytes, ctypes.byref(info))
    check(st, "tide_desc_build")
    return blob, info


def tide_plan_rank_tiles(h_plan: np.ndarray, r: int) -> Tuple[int, int]:
    """(tile_begin, tile_count) of output rank r's reduce-scatter tiles."""
    b, c = ctypes.c_int64(0), ctypes.c_int64(0)
    check(_lib.lib().tide_plan_rank_tiles(h_plan.ctypes.data, int(r), ctypes.byref(b), ctypes.byref(c)),
          "tide_plan_rank_tiles")
    return int(b.value), int(c.value)


def tide_rs_bf16_to_fp32(h_plan: np.ndarray, d_plan: torch.Tensor, order: int = 0,
                         max_workgroups: int = 0, stream=None) -> None:
    check(_lib.lib().tide_rs_bf16_to_fp32(h_plan.ctypes.data, d_plan.data_ptr(), int(order),
                                          int(max_workgroups), _stream(stream)),
          "tide_rs_bf16_to_fp32")


def tide_rs_bf16_to_fp32_tiles(h_plan: np.ndarray, d_plan: torch.Tensor, order: int,
                               tile_begin: int, tile_count: int, max_workgroups: int = 0,
                               stream=None) -> None:
    check(_lib.lib().tide_rs_bf16_to_fp32_tiles(h_plan.ctypes.data, d_plan.data_ptr(), int(order),
                                                int(tile_begin), int(tile_count),
                                                int(max_workgroups), _stream(stream)),
          "tide_rs_bf16_to_fp32_tiles")


def tide_rs_bf16_to_fp32_streams(h_plan: np.ndarray, d_plan: torch.Tensor, streams,
                                 order: int = 0, max_workgroups: int = 0) -> None:
    """The reduce-scatter's launches dealt over ``streams`` in turn (the
    caller orders the streams against its other work)."""
    arr = (ctypes.c_void_p * len(streams))(*[int(s.cuda_stream) for s in streams])
    check(_lib.lib().tide_rs_bf16_to_fp32_streams(h_plan.ctypes.data, d_plan.data_ptr(), int(order),
                                                  int(max_workgroups), arr, len(streams)),
          "tide_rs_bf16_to_fp32_streams")


def tide_rs_bf16_to_fp32_census(h_plan: np.ndarray, d_plan: torch.Tensor, census: torch.Tensor,
                                order: int = 0, max_workgroups: int = 0, stream=None) -> None:
    if census.dtype != torch.int32 or census.device.type != "cuda" or not census.is_contiguous():
        raise TideError(-6, "census must be a contiguous int32 GPU tensor")
    check(_lib.lib().tide_rs_bf16_to_fp32_census(h_plan.ctypes.data, d_plan.data_ptr(), int(order),
                                                 int(max_workgroups), census.data_ptr(),
                                                 census.numel(), _stream(stream)),
          "tide_rs_bf16_to_fp32_census")


def tide_rs_bf16_to_fp32_trace(h_plan: np.ndarray, d_plan: torch.Tensor, census: torch.Tensor,
                               stamps: torch.Tensor, order: int = 0, max_workgroups: int = 0,
                               stream=None) -> None:
    """The census call that also records each tile's start and end on the
    GPU's real-time counter (stamps: int64, two per tile)."""
    if census.dtype != torch.int32 or census.device.type != "cuda" or not census.is_contiguous():
        raise TideError(-6, "census must be a contiguous int32 GPU tensor")
    if stamps.dtype != torch.int64 or stamps.device.type != "cuda" or not stamps.is_contiguous():
        raise TideError(-6, "stamps must be a contiguous int64 GPU tensor")
    n = min(census.numel(), stamps.numel() // 2)
    check(_lib.lib().tide_rs_bf16_to_fp32_trace(h_plan.ctypes.data, d_plan.data_ptr(), int(order),
                                                int(max_workgroups), census.data_ptr(),
                                                stamps.data_ptr(), n, _stream(stream)),
          "tide_rs_bf16_to_fp32_trace")


def tide_ag_place(h_plan: np.ndarray, d_plan: torch.Tensor, max_workgroups: int = 0,
                  stream=None) -> None:
    check(_lib.lib().tide_ag_place(h_plan.ctypes.data, d_plan.data_ptr(), int(max_workgroups),
                                   _stream(stream)), "tide_ag_place")


def tide_ag_place_sdma(h_plan: np.ndarray, engine_only: bool = True, stream=None) -> None:
    check(_lib.lib().tide_ag_place_sdma(h_plan.ctypes.data, 1 if engine_only else 0,
                                        _stream(stream)), "tide_ag_place_sdma")


def tide_ag_place_sdma_streams(h_plan: np.ndarray, streams) -> None:
    arr = (ctypes.c_void_p * len(streams))(*[int(s.cuda_stream) for s in streams])
    check(_lib.lib().tide_ag_place_sdma_streams(h_plan.ctypes.data, arr, len(streams)),
          "tide_ag_place_sdma_streams")


def tide_ag_place_dma(h_plan: np.ndarray, stream=None) -> None:
    """Placement on the DMA engines (ROCr engine-pinned copies); returns
    when the copies are done."""
    check(_lib.lib().tide_ag_place_dma(h_plan.ctypes.data, _stream(stream)), "tide_ag_place_dma")


def tide_dma_engine_count() -> int:
    n = ctypes.c_int32(0)
    check(_lib.lib().tide_dma_engine_count(ctypes.byref(n)), "tide_dma_engine_count")
    return int(n.value)


def tide_rs_stage_dma(h_plan: np.ndarray, h_stage: np.ndarray, slot_stride: int,
                      stream=None) -> None:
    """Phase 1 of the copy-engine-staged reduce-scatter; h_stage: uint64
    array of R device addresses.  Returns when the copies are done."""
    check(_lib.lib().tide_rs_stage_dma(h_plan.ctypes.data, h_stage.ctypes.data, int(slot_stride),
                                       _stream(stream)), "tide_rs_stage_dma")


def tide_rs_fold_staged(h_plan: np.ndarray, d_plan: torch.Tensor, order: int,
                        h_stage: np.ndarray, d_stage: torch.Tensor, slot_stride: int,
                        max_workgroups: int = 0, stream=None) -> None:
    """Phase 2: fold the staged slots into the fp32 arenas (asynchronous)."""
    check(_lib.lib().tide_rs_fold_staged(h_plan.ctypes.data, d_plan.data_ptr(), int(order),
                                         h_stage.ctypes.data, d_stage.data_ptr(),
                                         int(slot_stride), int(max_workgroups), _stream(stream)),
          "tide_rs_fold_staged")


def tide_rs_tiles_to_stage(h_plan: np.ndarray, d_plan: torch.Tensor, tile_begin: int,
                           tile_count: int, stage: torch.Tensor, max_workgroups: int = 0,
                           stream=None) -> None:
    """Pipeline phase 1: reduce tiles [tile_begin, +tile_count) into the
    dense fp32 staging chunk ``stage``."""
    _require(stage, torch.float32, "stage")
    check(_lib.lib().tide_rs_tiles_to_stage(h_plan.ctypes.data, d_plan.data_ptr(), int(tile_begin),
                                            int(tile_count), stage.data_ptr(), stage.numel(),
                                            int(max_workgroups), _stream(stream)),
          "tide_rs_tiles_to_stage")


def tide_rs_stage_to_shards(h_plan: np.ndarray, d_plan: torch.Tensor, tile_begin: int,
                            tile_count: int, stage: torch.Tensor, max_workgroups: int = 0,
                            stream=None) -> None:
    """Pipeline phase 2: move a staging chunk's results into the arenas."""
    _require(stage, torch.float32, "stage")
    check(_lib.lib().tide_rs_stage_to_shards(h_plan.ctypes.data, d_plan.data_ptr(), int(tile_begin),
                                             int(tile_count), stage.data_ptr(), stage.numel(),
                                             int(max_workgroups), _stream(stream)),
          "tide_rs_stage_to_shards")


def tide_rs_stage_to_shards_sdma(h_plan: np.ndarray, tile_begin: int, tile_count: int,
                                 stage: torch.Tensor, stream=None) -> None:
    """Pipeline phase 2 on the copy engines (stream-ordered copies)."""
    _require(stage, torch.float32, "stage")
    check(_lib.lib().tide_rs_stage_to_shards_sdma(h_plan.ctypes.data, int(tile_begin),
                                                  int(tile_count), stage.data_ptr(), stage.numel(),
                                                  _stream(stream)),
          "tide_rs_stage_to_shards_sdma")


def tide_rs_two_phase_noalloc(h_plan: np.ndarray, d_plan: torch.Tensor, tile_begin: int,
                              tile_count: int, max_workgroups: int = 0, stream=None) -> None:
    """Both pipeline phases over tiles [tile_begin, +tile_count) through the
    library's own staging array (no allocation by anyone; at most
    TIDE_SCRATCH_BYTES of staging per call)."""
    check(_lib.lib().tide_rs_two_phase_noalloc(h_plan.ctypes.data, d_plan.data_ptr(),
                                               int(tile_begin), int(tile_count),
                                               int(max_workgroups), _stream(stream)),
          "tide_rs_two_phase_noalloc")


def tide_stream_create_cu_limited(n_cu: int) -> torch.cuda.ExternalStream:
    """A torch stream wrapping a HIP stream confined to the first n_cu CUs.
    Release it with tide_stream_destroy."""
    h = ctypes.c_void_p(0)
    check(_lib.lib().tide_stream_create_cu_limited(int(n_cu), ctypes.byref(h)),
          "tide_stream_create_cu_limited")
    return torch.cuda.ExternalStream(int(h.value))


def tide_stream_create_cu_range(first_cu: int, n_cu: int) -> torch.cuda.ExternalStream:
    """A torch stream wrapping a HIP stream confined to CU mask bits
    [first_cu, first_cu + n_cu).  Release it with tide_stream_destroy."""
    h = ctypes.c_void_p(0)
    check(_lib.lib().tide_stream_create_cu_range(int(first_cu), int(n_cu), ctypes.byref(h)),
          "tide_stream_create_cu_range")
    return torch.cuda.ExternalStream(int(h.value))


def tide_pipeline_create(depth: int, phase2_cus: int = 0) -> int:
    """Handle of a two-phase pipeline object (two streams, per-slot events)
    on the current device; release it with tide_pipeline_destroy."""
    h = ctypes.c_void_p(0)
    check(_lib.lib().tide_pipeline_create(int(depth), int(phase2_cus), ctypes.byref(h)),
          "tide_pipeline_create")
    return int(h.value)


def tide_pipeline_run(handle: int, h_plan: np.ndarray, d_plan: torch.Tensor, chunk_tiles: int,
                      ring: torch.Tensor, phase2: int = 0, stream=None) -> None:
    """The whole reduce-scatter through the pipeline, ordered on ``stream``
    (default: the current stream)."""
    _require(ring, torch.float32, "ring")
    check(_lib.lib().tide_pipeline_run(ctypes.c_void_p(handle), h_plan.ctypes.data,
                                       d_plan.data_ptr(), int(chunk_tiles), ring.data_ptr(),
                                       ring.numel(), int(phase2), _stream(stream)),
          "tide_pipeline_run")


def tide_pipeline_destroy(handle: int) -> None:
    check(_lib.lib().tide_pipeline_destroy(ctypes.c_void_p(handle)), "tide_pipeline_destroy")


def tide_stream_destroy(stream) -> None:
    check(_lib.lib().tide_stream_destroy(ctypes.c_void_p(int(stream.cuda_stream))),
          "tide_stream_destroy")


def _require(t: torch.Tensor, dtype, what: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % what)
    if t.dtype != dtype:
        raise TideError(-6, "%s has dtype %s, expected %s" % (what, t.dtype, dtype))
    if t.device.type != "cuda":
        raise TideError(-6, "%s is on %s, expected a GPU tensor" % (what, t.device))
    if not t.is_contiguous():
        raise TideError(-6, "%s is not contiguous" % what)


class Plan:
    """One layer's descriptor table.

    grads:    R lists of P bf16 tensors (rank q's per-parameter gradients);
    out:      R fp32 tensors of >= S elements (each rank's shard arena);
    gathered: one bf16 tensor of >= R*S elements (rank-major slots);
    full:     P bf16 tensors (the per-parameter full tensors).
    Either pair may be omitted.  Shapes come from ``shapes`` (torch-style).
    """

    def __init__(self, shapes, R: int, grads=None, out=None, gathered=None, full=None,
                 align: int = 1, rs_tile: int = 0, ag_tile: int = 0, flags: int = -1,
                 launch_mib: int = 0):
        self.shapes = [tuple(int(d) for d in s) for s in shapes]
        self.R = int(R)
        self.P = len(self.shapes)
        _, self.m, self.off, self.S = tide_desc_geometry(self.shapes, self.R, align)
        numels = [int(np.prod(s)) if len(s) else 1 for s in self.shapes]
        device = None
        grad_ptrs = out_ptrs = full_ptrs = None
        gptr = None
        if grads is not None:
            if out is None or len(grads) != self.R or len(out) != self.R:
                raise TideError(-1, "need R gradient lists and R output arenas")
            grad_ptrs = []
            for q, gl in enumerate(grads):
                if len(gl) != self.P:
                    raise TideError(-1, "rank %d has %d gradients, expected %d" % (q, len(gl), self.P))
                for p, g in enumerate(gl):
                    _require(g, torch.bfloat16, "grads[%d][%d]" % (q, p))
                    if g.numel() != numels[p]:
                        raise TideError(-1, "grads[%d][%d] has %d elements, expected %d"
                                        % (q, p, g.numel(), numels[p]))
                    grad_ptrs.append(g.data_ptr() if g.numel() else 0)
                    device = g.device
            out_ptrs = []
            for r, o in enumerate(out):
                _require(o, torch.float32, "out[%d]" % r)
                if o.numel() < self.S:
                    raise TideError(-1, "out[%d] holds %d floats, need S=%d" % (r, o.numel(), self.S))
                out_ptrs.append(o.data_ptr())
                device = o.device
        if gathered is not None:
            if full is None or len(full) != self.P:
                raise TideError(-1, "need P full tensors with the gathered buffer")
            _require(gathered, torch.bfloat16, "gathered")
            if gathered.numel() < self.R * self.S:
                raise TideError(-1, "gathered holds %d elements, need R*S=%d"
                                % (gathered.numel(), self.R * self.S))
            gptr = gathered.data_ptr()
            full_ptrs = []
            for p, f in enumerate(full):
                _require(f, torch.bfloat16, "full[%d]" % p)
                if f.numel() != numels[p]:
                    raise TideError(-1, "full[%d] has %d elements, expected %d" % (p, f.numel(), numels[p]))
                full_ptrs.append(f.data_ptr() if f.numel() else 0)
            device = gathered.device
        if device is None:
            raise TideError(-1, "a plan needs gradients or a gathered buffer")
        self.blob, self.info = tide_desc_build(self.shapes, self.R, grad_ptrs, out_ptrs, gptr,
                                               full_ptrs, align, rs_tile, ag_tile, flags,
                                               launch_mib)
        used = int(self.info.blob_bytes)
        self.blob = self.blob[:used].copy()
        self.d_blob = torch.from_numpy(self.blob).to(device)
        self._keep = (grads, out, gathered, full)

    def rs(self, order: str = "fixed", max_workgroups: int = 0, stream=None) -> None:
        tide_rs_bf16_to_fp32(self.blob, self.d_blob, ORDERS[order], max_workgroups, stream)

    def rs_streams(self, streams, order: str = "fixed", max_workgroups: int = 0,
                   stream=None) -> None:
        """The reduce-scatter with its launches dealt over ``stream`` (default:
        the current stream) and the extra ``streams`` in turn, ordered after
        ``stream``'s earlier work and before its later work (events)."""
        main = stream if stream is not None else torch.cuda.current_stream()
        start = torch.cuda.Event()
        start.record(main)
        for s in streams:
            s.wait_event(start)
        tide_rs_bf16_to_fp32_streams(self.blob, self.d_blob, [main] + list(streams),
                                     ORDERS[order], max_workgroups)
        for s in streams:
            done = torch.cuda.Event()
            done.record(s)
            main.wait_event(done)

    def rs_chunked(self, chunk_tiles: int, order: str = "fixed", max_workgroups: int = 0,
                   stream=None) -> int:
        """The reduce-scatter as ceil(rs_tiles / chunk_tiles) launches of at
        most chunk_tiles tiles each; returns the number of launches."""
        n = int(self.info.rs_tiles)
        launches = 0
        for b in range(0, n, chunk_tiles):
            tide_rs_bf16_to_fp32_tiles(self.blob, self.d_blob, ORDERS[order], b,
                                       min(chunk_tiles, n - b), max_workgroups, stream)
            launches += 1
        return launches

    def rs_rank(self, r: int, order: str = "fixed", max_workgroups: int = 0, stream=None) -> None:
        """Only output rank r's shards (one contiguous tile range)."""
        b, c = tide_plan_rank_tiles(self.blob, r)
        if c:
            tide_rs_bf16_to_fp32_tiles(self.blob, self.d_blob, ORDERS[order], b, c, max_workgroups,
                                       stream)

    def rs_census(self, order: str = "fixed", max_workgroups: int = 0, stream=None) -> torch.Tensor:
        """The reduce-scatter, returning for every tile the packed id of the
        compute unit that processed it (int32 GPU tensor)."""
        census = torch.full((max(1, int(self.info.rs_tiles)),), -1, dtype=torch.int32,
                            device=self.d_blob.device)
        tide_rs_bf16_to_fp32_census(self.blob, self.d_blob, census, ORDERS[order],
                                    max_workgroups, stream)
        return census

    def rs_trace(self, order: str = "fixed", max_workgroups: int = 0, stream=None):
        """The reduce-scatter, returning (census, stamps): per tile the packed
        compute-unit id (int32) and its start and end ticks on the GPU's
        real-time counter (int64 [tiles, 2]); GPU tensors."""
        n = max(1, int(self.info.rs_tiles))
        census = torch.full((n,), -1, dtype=torch.int32, device=self.d_blob.device)
        stamps = torch.zeros((n, 2), dtype=torch.int64, device=self.d_blob.device)
        tide_rs_bf16_to_fp32_trace(self.blob, self.d_blob, census, stamps, ORDERS[order],
                                   max_workgroups, stream)
        return census, stamps

    def ag(self, max_workgroups: int = 0, stream=None) -> None:
        tide_ag_place(self.blob, self.d_blob, max_workgroups, stream)

    def ag_sdma(self, engine_only: bool = True, stream=None) -> None:
        tide_ag_place_sdma(self.blob, engine_only, stream)

    def ag_sdma_streams(self, streams) -> None:
        """Engine-only placement spread over several streams.  The caller
        orders them against other work (e.g. with events)."""
        tide_ag_place_sdma_streams(self.blob, streams)

    def ag_dma(self, stream=None) -> None:
        """Placement on the DMA engines through ROCr (host-synchronous)."""
        tide_ag_place_dma(self.blob, stream)

    def shard(self, out_arena: torch.Tensor, p: int) -> torch.Tensor:
        """View of param p's shard in one rank's fp32 arena, shaped [s, rest...]."""
        shp = self.shapes[p]
        s = int(self.m[p]) // (int(np.prod(shp[1:])) if len(shp) > 1 else 1) if int(self.m[p]) else 0
        v = out_arena[int(self.off[p]):int(self.off[p]) + int(self.m[p])]
        return v.view((s,) + tuple(shp[1:])) if len(shp) else v


class StagedRS:
    """Copy-engine-staged reduce-scatter over a plan: ``stage`` holds R bf16
    tensors (rank r's staging buffer of R slots of ``slot_stride`` elements,
    e.g. the rank's vacated gathered buffer with slot_stride = S).
    ``stage_dma()`` moves every rank's slices into the slots on the DMA
    engines (host-synchronous); ``fold()`` reduces the slots into the plan's
    fp32 arenas on the compute units (asynchronous)."""

    def __init__(self, plan: Plan, stage, slot_stride: int = 0):
        if len(stage) != plan.R:
            raise TideError(-1, "need R staging buffers")
        self.plan = plan
        self.slot_stride = int(slot_stride) if slot_stride else int(plan.S)
        for r, t in enumerate(stage):
            _require(t, torch.bfloat16, "stage[%d]" % r)
            if t.numel() < plan.R * self.slot_stride:
                raise TideError(-1, "stage[%d] holds %d elements, need R*slot_stride=%d"
                                % (r, t.numel(), plan.R * self.slot_stride))
        self.stage = list(stage)
        self.h_stage = np.array([t.data_ptr() for t in stage], dtype=np.uint64)
        self.d_stage = torch.from_numpy(self.h_stage.view(np.int64).copy()).to(stage[0].device)

    def stage_dma(self, stream=None) -> None:
        tide_rs_stage_dma(self.plan.blob, self.h_stage, self.slot_stride, stream)

    def fold(self, order: str = "fixed", max_workgroups: int = 0, stream=None) -> None:
        tide_rs_fold_staged(self.plan.blob, self.plan.d_blob, ORDERS[order], self.h_stage,
                            self.d_stage, self.slot_stride, max_workgroups, stream)
