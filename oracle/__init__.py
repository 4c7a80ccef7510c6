"""CPU oracle for TIDE's node-local reduce-scatter and all-gather placement.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package; the product path never
does.  It shares no code with the HIP library.  The arithmetic lives in
``tide_oracle.c`` (plain loops, fixed rank order, IEEE binary32); this module
only marshals numpy arrays into it.  The readings it takes where the pages are
silent are listed at the top of ``tide_oracle.c``.

Functions follow the problem statement of the paper's Abstract ("The Endgame
of FSDP Communication", weekinpapers.com): per-parameter bf16 gradients of R
ranks reduced into per-rank fp32 dim-0 shards, and a rank-major bf16 gathered
buffer placed into per-parameter tensors.  All arrays are numpy, host memory.
bf16 values travel as their raw uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tide_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libtide_oracle.so")
_lib = None

ORDERS = {"fixed": 0, "tree": 1}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no flag that reassociates or flushes)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
           "-fopenmp", "-shared", "-fPIC", "-Wall", "-Wextra", _SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64p = ctypes.POINTER(ctypes.c_int64)
    vpp = ctypes.POINTER(ctypes.c_void_p)
    lib.oracle_layout.argtypes = [ctypes.c_int32, i64p, i64p, ctypes.c_int32,
                                  ctypes.c_int64, i64p, i64p, i64p, i64p]
    lib.oracle_rs.argtypes = [ctypes.c_int32, i64p, i64p, ctypes.c_int32,
                              ctypes.c_int64, ctypes.c_int32, vpp, vpp]
    lib.oracle_ag.argtypes = [ctypes.c_int32, i64p, i64p, ctypes.c_int32,
                              ctypes.c_int64, ctypes.c_void_p, vpp]
    lib.oracle_fold_points.argtypes = [ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int64, ctypes.c_void_p,
                                       ctypes.c_void_p]
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = None
    for name in ("oracle_layout", "oracle_rs", "oracle_ag",
                 "oracle_fold_points", "oracle_max_threads", "oracle_version"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _dims(shapes: Sequence[Sequence[int]]) -> Tuple[np.ndarray, np.ndarray]:
    """Flatten each shape to (dim0, row numel); a 0-d shape is one row."""
    d0, c = [], []
    for shp in shapes:
        shp = tuple(int(x) for x in shp)
        if len(shp) == 0:
            d0.append(1)
            c.append(1)
        else:
            d0.append(shp[0])
            c.append(int(np.prod(shp[1:], dtype=np.int64)) if len(shp) > 1 else 1)
    return np.asarray(d0, dtype=np.int64), np.asarray(c, dtype=np.int64)


def _i64(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError("%s failed with oracle status %d" % (what, rc))


def layout(shapes, R: int, align: int = 1):
    """Return (s, m, off, S): chunk rows, shard numel and arena offset per
    param, and the slot numel."""
    lib = _load()
    d0, c = _dims(shapes)
    P = len(d0)
    s = np.zeros(P, np.int64)
    m = np.zeros(P, np.int64)
    off = np.zeros(P, np.int64)
    S = np.zeros(1, np.int64)
    _check(lib.oracle_layout(P, _i64(d0), _i64(c), R, align, _i64(s), _i64(m),
                             _i64(off), _i64(S)), "oracle_layout")
    return s, m, off, int(S[0])


def rs(shapes, R: int, grads: Sequence[Sequence[np.ndarray]], align: int = 1,
       order: str = "fixed", out: List[np.ndarray] = None) -> List[np.ndarray]:
    """Reduce-scatter.  grads[q][p] is rank q's param p as uint16 bf16 bits
    (contiguous, d0*c elements).  Returns R float32 arenas of S elements; if
    ``out`` is given it is written in place (gaps keep their content)."""
    lib = _load()
    d0, c = _dims(shapes)
    P = len(d0)
    _, _, _, S = layout(shapes, R, align)
    if len(grads) != R:
        raise ValueError("need R rank lists")
    keep = []
    ptrs = (ctypes.c_void_p * max(1, R * P))()
    for q in range(R):
        if len(grads[q]) != P:
            raise ValueError("rank %d has %d params, expected %d" % (q, len(grads[q]), P))
        for p in range(P):
            a = np.ascontiguousarray(grads[q][p]).view(np.uint16).reshape(-1)
            if a.size != d0[p] * c[p]:
                raise ValueError("rank %d param %d has %d elements" % (q, p, a.size))
            keep.append(a)
            ptrs[q * P + p] = a.ctypes.data
    if out is None:
        out = [np.zeros(S, np.float32) for _ in range(R)]
    optrs = (ctypes.c_void_p * R)()
    for r in range(R):
        if out[r].dtype != np.float32 or out[r].size < S or not out[r].flags.c_contiguous:
            raise ValueError("out[%d] must be contiguous float32 of >= S elements" % r)
        optrs[r] = out[r].ctypes.data
    _check(lib.oracle_rs(P, _i64(d0), _i64(c), R, align, ORDERS[order], ptrs, optrs),
           "oracle_rs")
    return out


def fold_points(vals: np.ndarray, order: str = "fixed") -> np.ndarray:
    """vals: uint16 [K, R] (one row per element, ranks in order).  Returns the
    float32 fold of every row."""
    lib = _load()
    v = np.ascontiguousarray(vals).view(np.uint16)
    if v.ndim != 2:
        raise ValueError("vals must be [K, R]")
    K, R = v.shape
    out = np.empty(K, np.float32)
    _check(lib.oracle_fold_points(R, ORDERS[order], K, v.ctypes.data,
                                  out.ctypes.data), "oracle_fold_points")
    return out


def ag(shapes, R: int, gathered: np.ndarray, align: int = 1,
       out: List[np.ndarray] = None) -> List[np.ndarray]:
    """All-gather placement.  gathered: uint16 [R*S] rank-major slots.
    Returns P uint16 arrays of d0*c elements (or writes ``out`` in place)."""
    lib = _load()
    d0, c = _dims(shapes)
    P = len(d0)
    _, _, _, S = layout(shapes, R, align)
    g = np.ascontiguousarray(gathered).view(np.uint16).reshape(-1)
    if g.size < R * S:
        raise ValueError("gathered buffer holds %d elements, need %d" % (g.size, R * S))
    if out is None:
        out = [np.zeros(int(d0[p] * c[p]), np.uint16) for p in range(P)]
    fptrs = (ctypes.c_void_p * max(1, P))()
    for p in range(P):
        if out[p].dtype != np.uint16 or out[p].size != d0[p] * c[p] or not out[p].flags.c_contiguous:
            raise ValueError("out[%d] must be contiguous uint16 of d0*c elements" % p)
        fptrs[p] = out[p].ctypes.data
    _check(lib.oracle_ag(P, _i64(d0), _i64(c), R, align, g.ctypes.data, fptrs),
           "oracle_ag")
    return out


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())
