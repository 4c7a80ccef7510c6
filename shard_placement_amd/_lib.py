"""ctypes loader for libtide.so (the C ABI declared in include/tide.h).

The library is built in-tree by ``shard_placement_amd.build`` (hipcc,
gfx950).  Loading fails loudly when it is missing: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtide.so")

TIDE_OK = 0
STATUS_NAMES = {0: "TIDE_OK", -1: "TIDE_EINVAL", -2: "TIDE_EALIGN", -3: "TIDE_EOVERLAP",
                -4: "TIDE_ENOSPACE", -5: "TIDE_EHIP", -6: "TIDE_EUNSUPPORTED",
                -7: "TIDE_EPLAN"}
FLAG_NT_LOADS = 1
FLAG_NT_STORES = 2
SCRATCH_BYTES = 32 << 20  # TIDE_SCRATCH_BYTES: staging array of the allocation-free call

# Every symbol include/tide.h declares.
EXPORTS = ("tide_abi_version", "tide_status_str", "tide_desc_size", "tide_desc_geometry",
           "tide_desc_build", "tide_plan_query", "tide_rs_bf16_to_fp32", "tide_ag_place",
           "tide_ag_place_sdma", "tide_stream_create_cu_limited", "tide_stream_destroy",
           "tide_rs_bf16_to_fp32_tiles", "tide_ag_place_sdma_streams",
           "tide_rs_bf16_to_fp32_census", "tide_ag_place_dma", "tide_dma_engine_count",
           "tide_rs_stage_dma", "tide_rs_fold_staged", "tide_rs_tiles_to_stage",
           "tide_rs_stage_to_shards", "tide_rs_stage_to_shards_sdma", "tide_plan_rank_tiles",
           "tide_stream_create_cu_range", "tide_pipeline_create", "tide_pipeline_run",
           "tide_pipeline_destroy", "tide_rs_two_phase_noalloc", "tide_rs_bf16_to_fp32_trace",
           "tide_rs_bf16_to_fp32_streams")


class TideShape(ctypes.Structure):
    _fields_ = [("dim0", ctypes.c_int64), ("row_numel", ctypes.c_int64)]


class TideOpts(ctypes.Structure):
    _fields_ = [("align_elems", ctypes.c_int64), ("rs_tile_elems", ctypes.c_int32),
                ("ag_tile_elems", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("launch_mib", ctypes.c_int32)]


class TidePlanInfo(ctypes.Structure):
    _fields_ = [("R", ctypes.c_int32), ("P", ctypes.c_int32),
                ("slot_numel", ctypes.c_int64), ("numel", ctypes.c_int64),
                ("padded_numel", ctypes.c_int64), ("rs_tiles", ctypes.c_int64),
                ("ag_tiles", ctypes.c_int64), ("rs_tile_elems", ctypes.c_int32),
                ("ag_tile_elems", ctypes.c_int32), ("blob_bytes", ctypes.c_int64),
                ("rs_launch_tiles", ctypes.c_int64), ("ag_launch_tiles", ctypes.c_int64),
                ("rs_lds_bytes", ctypes.c_int64)]


class TideError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = "%s: %s (%s)" % (what, STATUS_NAMES.get(status, str(status)),
                               _status_text(status))
        super().__init__(msg)


_lib = None


def _status_text(status: int) -> str:
    try:
        return lib().tide_status_str(status).decode()
    except Exception:  # the library itself failed to load
        return "?"


def lib():
    """Load libtide.so or raise: the product path has no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libtide.so is not built (%s); run __graft_entry__.build() "
                           "or python -m shard_placement_amd.build" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    i64p = ctypes.POINTER(ctypes.c_int64)
    L.tide_abi_version.argtypes = []
    L.tide_abi_version.restype = i32
    L.tide_status_str.argtypes = [i32]
    L.tide_status_str.restype = ctypes.c_char_p
    L.tide_desc_size.argtypes = [ctypes.POINTER(TideShape), i32, i32,
                                 ctypes.POINTER(TideOpts), ctypes.POINTER(ctypes.c_size_t)]
    L.tide_desc_geometry.argtypes = [ctypes.POINTER(TideShape), i32, i32,
                                     ctypes.POINTER(TideOpts), i64p, i64p, i64p, i64p]
    L.tide_desc_build.argtypes = [ctypes.POINTER(TideShape), i32, i32, ctypes.POINTER(TideOpts),
                                  ctypes.POINTER(vp), ctypes.POINTER(vp), vp,
                                  ctypes.POINTER(vp), vp, ctypes.c_size_t,
                                  ctypes.POINTER(TidePlanInfo)]
    L.tide_plan_query.argtypes = [vp, ctypes.POINTER(TidePlanInfo)]
    L.tide_plan_rank_tiles.argtypes = [vp, i32, i64p, i64p]
    L.tide_rs_bf16_to_fp32.argtypes = [vp, vp, i32, i32, vp]
    L.tide_rs_bf16_to_fp32_tiles.argtypes = [vp, vp, i32, i64, i64, i32, vp]
    L.tide_ag_place.argtypes = [vp, vp, i32, vp]
    L.tide_ag_place_sdma.argtypes = [vp, i32, vp]
    L.tide_stream_create_cu_limited.argtypes = [i32, ctypes.POINTER(vp)]
    L.tide_stream_destroy.argtypes = [vp]
    L.tide_ag_place_sdma_streams.argtypes = [vp, ctypes.POINTER(vp), i32]
    L.tide_rs_bf16_to_fp32_census.argtypes = [vp, vp, i32, i32, vp, i64, vp]
    L.tide_ag_place_dma.argtypes = [vp, vp]
    L.tide_dma_engine_count.argtypes = [ctypes.POINTER(i32)]
    L.tide_rs_stage_dma.argtypes = [vp, vp, i64, vp]
    L.tide_rs_fold_staged.argtypes = [vp, vp, i32, vp, vp, i64, i32, vp]
    L.tide_rs_tiles_to_stage.argtypes = [vp, vp, i64, i64, vp, i64, i32, vp]
    L.tide_rs_stage_to_shards.argtypes = [vp, vp, i64, i64, vp, i64, i32, vp]
    L.tide_rs_stage_to_shards_sdma.argtypes = [vp, i64, i64, vp, i64, vp]
    L.tide_stream_create_cu_range.argtypes = [i32, i32, ctypes.POINTER(vp)]
    L.tide_pipeline_create.argtypes = [i32, i32, ctypes.POINTER(vp)]
    L.tide_pipeline_run.argtypes = [vp, vp, vp, i64, vp, i64, i32, vp]
    L.tide_pipeline_destroy.argtypes = [vp]
    L.tide_rs_two_phase_noalloc.argtypes = [vp, vp, i64, i64, i32, vp]
    L.tide_rs_bf16_to_fp32_trace.argtypes = [vp, vp, i32, i32, vp, vp, i64, vp]
    L.tide_rs_bf16_to_fp32_streams.argtypes = [vp, vp, i32, i32, ctypes.POINTER(vp), i32]
    for name in ("tide_desc_size", "tide_desc_geometry", "tide_desc_build", "tide_plan_query",
                 "tide_rs_bf16_to_fp32", "tide_ag_place", "tide_ag_place_sdma",
                 "tide_stream_create_cu_limited", "tide_stream_destroy",
                 "tide_rs_bf16_to_fp32_tiles", "tide_ag_place_sdma_streams",
                 "tide_rs_bf16_to_fp32_census", "tide_ag_place_dma", "tide_dma_engine_count",
                 "tide_rs_stage_dma", "tide_rs_fold_staged", "tide_rs_tiles_to_stage",
                 "tide_rs_stage_to_shards", "tide_rs_stage_to_shards_sdma", "tide_plan_rank_tiles",
                 "tide_stream_create_cu_range", "tide_pipeline_create", "tide_pipeline_run",
                 "tide_pipeline_destroy", "tide_rs_two_phase_noalloc",
                 "tide_rs_bf16_to_fp32_trace", "tide_rs_bf16_to_fp32_streams"):
        getattr(L, name).restype = ctypes.c_int
    if L.tide_abi_version() != 2:
        raise RuntimeError("libtide ABI version %d, expected 2" % L.tide_abi_version())
    _lib = L
    return L


def check(status: int, what: str) -> None:
    if status != TIDE_OK:
        raise TideError(status, what)
