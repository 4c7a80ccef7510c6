"""CPU tests of the C-ABI library: it loads, exports every symbol the header
declares, and its host logic (geometry, plan builder, validation) is right.
No compute call is made: plans are built from made-up device addresses and
the launch entry points are only exercised on arguments they reject before
touching the GPU.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from shard_placement_amd import _lib, api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# mirror of the plan blob layout (shard_placement_amd/csrc/plan_format.h)
HDR = np.dtype([("magic", "<u4"), ("version", "<u4"), ("R", "<i4"), ("P", "<i4"),
                ("align", "<i8"), ("S", "<i8"), ("N", "<i8"), ("Npad", "<i8"),
                ("rs_tile", "<i4"), ("ag_tile", "<i4"), ("n_rs", "<i8"), ("n_ag", "<i8"),
                ("off_params", "<u8"), ("off_gptr", "<u8"), ("off_obase", "<u8"),
                ("off_full", "<u8"), ("off_rs", "<u8"), ("off_ag", "<u8"),
                ("gathered", "<u8"), ("bytes", "<u8"), ("has_rs", "<i4"), ("has_ag", "<i4"),
                ("flags", "<u4"), ("reserved", "<u4"), ("rs_launch", "<i8"), ("ag_launch", "<i8"),
                ("rs_launch_tree", "<i8")])
RS_TILE = np.dtype([("j0", "<i8"), ("o0", "<i8"), ("p", "<i4"), ("r", "<i4"),
                    ("len", "<i4"), ("kind", "<i4")])
AG_TILE = np.dtype([("src", "<i8"), ("dst", "<i8"), ("p", "<i4"), ("len", "<i4"),
                    ("kind", "<i4"), ("reserved", "<i4")])
PARAM = np.dtype([("d0", "<i8"), ("c", "<i8"), ("s", "<i8"), ("m", "<i8"), ("n", "<i8"),
                  ("off", "<i8")])


def decode(blob):
    h = np.frombuffer(blob[:HDR.itemsize].tobytes(), HDR)[0]

    def sec(off, n, dt):
        off, n = int(h[off]), int(n)
        return np.frombuffer(blob[off:off + np.dtype(dt).itemsize * n].tobytes(), dt)

    rs = sec("off_rs", h["n_rs"], RS_TILE)
    ag = sec("off_ag", h["n_ag"], AG_TILE)
    ps = sec("off_params", h["P"], PARAM)
    gp = sec("off_gptr", int(h["P"]) * int(h["R"]), "<u8")
    return h, ps, gp, rs, ag


def test_header_is_plain_c(tmp_path):
    """include/tide.h compiles on its own as C99 and as C++11, warnings as
    errors: a C ABI with no HIP, torch or C++ types in its signatures."""
    import shutil
    import subprocess

    for cc, std, ext in (("gcc", "-std=c99", "c"), ("g++", "-std=c++11", "cpp")):
        if shutil.which(cc) is None:
            pytest.skip("%s not available" % cc)
        src = tmp_path / ("use_header." + ext)
        src.write_text('#include "tide.h"\nint main(void) { return (int)TIDE_OK; }\n')
        subprocess.run([cc, std, "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                        "-I" + os.path.join(ROOT, "include"), str(src)], check=True)


def test_library_loads_and_exports_header_symbols():
    with open(os.path.join(ROOT, "include", "tide.h")) as fh:
        hdr = fh.read()
    declared = set(re.findall(r"^\s*(?:tide_status|const char \*|int32_t)\s*\**\s*(tide_\w+)\s*\(",
                              hdr, re.M))
    assert declared == set(_lib.EXPORTS), declared ^ set(_lib.EXPORTS)
    L = _lib.lib()
    for name in declared:
        assert hasattr(L, name)
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value
    assert L.tide_abi_version() == 2
    assert L.tide_status_str(-3).decode().startswith("an output range overlaps")


SHAPES = [(37, 16), (64, 64), (5,), (), (0, 3), (1001, 8), (6, 5), (3, 0)]


@pytest.mark.parametrize("R", [1, 2, 3, 4, 8, 17, 64])
@pytest.mark.parametrize("align", [1, 8])
def test_geometry_agrees_with_oracle(orc, R, align):
    s, m, off, S = api.tide_desc_geometry(SHAPES, R, align)
    os_, om, ooff, oS = orc.layout(SHAPES, R, align)
    assert list(s) == list(os_) and list(m) == list(om) and list(off) == list(ooff) and S == oS


def _fake_ptrs(shapes, R, S, base=1 << 40, grad_misalign=0, out_misalign=0):
    """Disjoint made-up device addresses: per rank one gradient arena and one
    output arena, a gathered buffer and full tensors."""
    numels = [int(np.prod(s)) if len(s) else 1 for s in shapes]
    pos = base
    grads, outs, full = [], [], []
    for q in range(R):
        p0 = pos + grad_misalign
        for n in numels:
            grads.append(p0 if n else 0)
            p0 += 2 * n
        pos += ((2 * sum(numels) + grad_misalign + 4095) // 4096 + 1) * 4096
    for r in range(R):
        outs.append(pos + out_misalign)
        pos += ((4 * S + 4095) // 4096 + 1) * 4096
    gathered = pos
    pos += ((2 * R * S + 4095) // 4096 + 1) * 4096
    for n in numels:
        full.append(pos if n else 0)
        pos += ((2 * n + 4095) // 4096 + 1) * 4096
    return grads, outs, gathered, full


def _check_rs_tiles(shapes, R, blob, gptrs):
    h, ps, gp, rs, _ = decode(blob)
    assert h["magic"] == 0x45444954 and h["has_rs"] == 1
    covered = {}
    for t in rs:
        p, r = int(t["p"]), int(t["r"])
        d = ps[p]
        assert r * d["m"] <= t["j0"] and t["j0"] + t["len"] <= (r + 1) * d["m"]
        assert t["o0"] == d["off"] + t["j0"] - r * d["m"]
        if t["kind"] == 2:
            assert t["j0"] >= d["n"]
        else:
            assert t["j0"] + t["len"] <= d["n"]
        if t["kind"] == 0:
            assert t["len"] % 8 == 0
            for q in range(R):
                assert (int(gp[p * R + q]) + 2 * int(t["j0"])) % 16 == 0
        assert 0 < t["len"] <= h["rs_tile"]
        covered.setdefault(p, []).append((int(t["j0"]), int(t["j0"] + t["len"])))
    for p, d in enumerate(ps):
        runs = sorted(covered.get(p, []))
        total = R * int(d["m"])
        pos = 0
        for a, b in runs:
            assert a == pos, (p, a, pos)
            pos = b
        assert pos == total
    # pointer table is param-major
    P = len(shapes)
    for q in range(R):
        for p in range(P):
            assert int(gp[p * R + q]) == int(gptrs[q * P + p])


@pytest.mark.parametrize("R", [1, 3, 4, 8, 64])
@pytest.mark.parametrize("mis", [(0, 0), (2, 4), (6, 8), (14, 12)])
def test_rs_tiles_partition_every_shard(R, mis):
    _, _, _, S = api.tide_desc_geometry(SHAPES, R)
    g, o, ga, f = _fake_ptrs(SHAPES, R, S, grad_misalign=mis[0], out_misalign=mis[1])
    blob, info = api.tide_desc_build(SHAPES, R, g, o, None, None, rs_tile=2048)
    assert info.rs_tiles > 0 and info.ag_tiles == 0
    assert info.blob_bytes <= api.tide_desc_size(SHAPES, R, rs_tile=2048)
    _check_rs_tiles(SHAPES, R, blob, g)


def test_rs_vector_tiles_dominate_when_aligned():
    shapes = [(1024, 8192), (8192,)]
    R = 8
    _, _, _, S = api.tide_desc_geometry(shapes, R)
    g, o, _, _ = _fake_ptrs(shapes, R, S)
    blob, info = api.tide_desc_build(shapes, R, g, o)
    _, _, _, rs, _ = decode(blob)
    assert set(rs["kind"].tolist()) == {0}
    assert info.rs_tile_elems == 2048
    assert int(rs["len"].sum()) == R * S


def test_rs_mixed_phases_fall_back_to_scalar():
    shapes = [(40, 8)]
    R = 2
    _, _, _, S = api.tide_desc_geometry(shapes, R)
    g, o, _, _ = _fake_ptrs(shapes, R, S)
    g[1] += 2  # rank 1's gradient two bytes off rank 0's phase
    blob, _ = api.tide_desc_build(shapes, R, g, o)
    _, _, _, rs, _ = decode(blob)
    assert set(rs["kind"].tolist()) == {1}


@pytest.mark.parametrize("R", [1, 2, 4, 17])
@pytest.mark.parametrize("gmis", [0, 2, 4, 6])
def test_ag_tiles_cover_valid_rows_only(R, gmis):
    _, m, off, S = api.tide_desc_geometry(SHAPES, R)
    _, _, ga, f = _fake_ptrs(SHAPES, R, S)
    blob, info = api.tide_desc_build(SHAPES, R, None, None, ga + gmis, f, ag_tile=2048)
    h, ps, _, _, ag = decode(blob)
    assert h["has_rs"] == 0 and h["has_ag"] == 1 and info.rs_tiles == 0
    shifted = 0
    for p, d in enumerate(ps):
        tiles = sorted((int(t["dst"]), int(t["src"]), int(t["len"]), int(t["kind"]))
                       for t in ag if t["p"] == p)
        pos = 0
        for dst, src, ln, kind in tiles:
            assert dst == pos
            r = dst // int(d["m"])
            assert src == r * S + int(d["off"]) + (dst - r * int(d["m"]))
            if kind == 0:
                assert (ga + gmis + 2 * src) % 16 == 0 and (f[p] + 2 * dst) % 16 == 0 and ln % 8 == 0
            if kind == 1:
                assert (ga + gmis + 2 * src) % 4 == 0 and (f[p] + 2 * dst) % 4 == 0 and ln % 2 == 0
            # never crosses into the rank's padding rows
            valid = min(max(int(d["d0"]) - r * int(d["s"]), 0), int(d["s"])) * int(d["c"])
            assert dst + ln <= r * int(d["m"]) + valid
            if kind == 3:
                # realigning copy: aligned destination, a source in another
                # 16-byte phase, whole vectors (it reads only its own elements)
                assert (f[p] + 2 * dst) % 16 == 0 and ln % 8 == 0
                assert (ga + gmis + 2 * src) % 16 != 0
                shifted += 1
            pos = dst + ln
        assert pos == int(d["n"])


def _status(fn, *a):
    try:
        fn(*a)
    except _lib.TideError as e:
        return e.status
    return 0


def test_validation_errors():
    R = 4
    _, _, _, S = api.tide_desc_geometry(SHAPES, R)
    g, o, ga, f = _fake_ptrs(SHAPES, R, S)
    b = api.tide_desc_build
    assert _status(b, SHAPES, 0, g, o, None, None) == -1          # R < 1
    assert _status(api.tide_desc_geometry, SHAPES, 4097) == -1    # R above the limit
    assert _status(api.tide_desc_geometry, SHAPES, 4096) == 0     # the limit itself
    assert _status(b, SHAPES, R, g, None, None, None) == -1       # grads without outputs
    assert _status(b, SHAPES, R, g, o, ga, None) == -1            # gathered without full
    g2 = list(g); g2[0] = 0
    assert _status(b, SHAPES, R, g2, o, None, None) == -1         # NULL gradient
    g2 = list(g); g2[1] += 1
    assert _status(b, SHAPES, R, g2, o, None, None) == -2         # odd bf16 address
    o2 = list(o); o2[0] += 2
    assert _status(b, SHAPES, R, g, o2, None, None) == -2         # misaligned fp32 arena
    o2 = list(o); o2[1] = o2[0]
    assert _status(b, SHAPES, R, g, o2, None, None) == -3         # two ranks share an arena
    o2 = list(o); o2[2] = g[5]
    assert _status(b, SHAPES, R, g, o2, None, None) == -3         # output over a gradient
    f2 = list(f); f2[0] = ga + 64
    assert _status(b, SHAPES, R, None, None, ga, f2) == -3        # full over the gathered buffer
    # Slot-Reuse: outputs inside the gathered buffer are allowed
    o3 = [ga + 4 * S * r for r in range(R)]
    assert _status(b, SHAPES, R, g, o3, ga, f) == 0
    # identical ranks may alias one gradient tensor
    g4 = g[:len(SHAPES)] * R
    assert _status(b, SHAPES, R, g4, o, None, None) == 0
    assert _status(b, [(-1, 2)], R, [1 << 40] * R, o, None, None) == -1
    assert _status(b, SHAPES, R, g, o, None, None, 1, 1000) == -1  # tile not a multiple of 2048


def test_enospace_reports_needed_size():
    R = 4
    _, _, _, S = api.tide_desc_geometry(SHAPES, R)
    g, o, _, _ = _fake_ptrs(SHAPES, R, S)
    L = _lib.lib()
    shp = api._shapes(SHAPES)
    info = _lib.TidePlanInfo()
    opts = api._opts()
    vp = ctypes.c_void_p
    garr = (vp * len(g))(*[x or None for x in g])
    oarr = (vp * R)(*o)
    buf = np.zeros(64, np.uint8)
    st = L.tide_desc_build(shp, len(SHAPES), R, ctypes.byref(opts), garr, oarr, None, None,
                           buf.ctypes.data, buf.nbytes, ctypes.byref(info))
    assert st == -4 and info.blob_bytes > 64


def test_launches_reject_before_touching_the_gpu():
    R = 4
    _, _, _, S = api.tide_desc_geometry(SHAPES, R)
    g, o, ga, f = _fake_ptrs(SHAPES, R, S)
    L = _lib.lib()
    blob, _ = api.tide_desc_build(SHAPES, R, g, o, None, None)
    fake_dev = ctypes.c_void_p(1 << 44)
    assert L.tide_rs_bf16_to_fp32(blob.ctypes.data, fake_dev, 2, 0, None) == -1   # bad order
    assert L.tide_rs_bf16_to_fp32(blob.ctypes.data, fake_dev, 0, -1, None) == -1  # bad grid cap
    assert L.tide_rs_bf16_to_fp32(blob.ctypes.data, ctypes.c_void_p((1 << 44) + 8), 0, 0, None) == -2
    assert L.tide_ag_place(blob.ctypes.data, fake_dev, 0, None) == -6             # no AG pointers
    assert L.tide_ag_place_sdma(blob.ctypes.data, 1, None) == -6
    junk = np.zeros(4096, np.uint8)
    assert L.tide_rs_bf16_to_fp32(junk.ctypes.data, fake_dev, 0, 0, None) == -7
    assert L.tide_ag_place(junk.ctypes.data, fake_dev, 0, None) == -7
    info = _lib.TidePlanInfo()
    assert L.tide_plan_query(junk.ctypes.data, ctypes.byref(info)) == -7
    assert L.tide_plan_query(blob.ctypes.data, ctypes.byref(info)) == 0
    assert info.R == R and info.slot_numel == S
    # a blob of another format version (here the previous one, without the
    # tree-order launch size) is refused, not misread
    old = blob.copy()
    hv = np.frombuffer(old[:HDR.itemsize].tobytes(), HDR)[0]
    assert hv["version"] == 2
    old[4:8] = np.frombuffer(np.uint32(1).tobytes(), np.uint8)
    assert L.tide_plan_query(old.ctypes.data, ctypes.byref(info)) == -7
    assert L.tide_rs_bf16_to_fp32(old.ctypes.data, fake_dev, 0, 0, None) == -7
    n_rs = int(np.frombuffer(blob[:HDR.itemsize].tobytes(), HDR)[0]["n_rs"])
    T = L.tide_rs_bf16_to_fp32_tiles
    assert T(blob.ctypes.data, fake_dev, 0, 0, n_rs + 1, 0, None) == -1          # past the end
    assert T(blob.ctypes.data, fake_dev, 0, n_rs, 1, 0, None) == -1
    assert T(blob.ctypes.data, fake_dev, 0, -1, 1, 0, None) == -1
    assert T(blob.ctypes.data, fake_dev, 0, 0, -1, 0, None) == -1
    assert T(blob.ctypes.data, fake_dev, 0, n_rs, 0, 0, None) == 0              # empty range
    ag_blob, _ = api.tide_desc_build(SHAPES, R, None, None, ga, f)
    assert L.tide_rs_bf16_to_fp32(ag_blob.ctypes.data, fake_dev, 0, 0, None) == -6


def test_launch_granularity():
    shapes = [(8192, 1024), (100, 7)]
    R = 8
    _, _, _, S = api.tide_desc_geometry(shapes, R)
    g, o, ga, f = _fake_ptrs(shapes, R, S)
    _, info = api.tide_desc_build(shapes, R, g, o, ga, f)
    per_tile = info.rs_tile_elems * (2 * R + 4)
    # library defaults: 160 MiB for the reduce-scatter (at R = 8, 4096 tiles:
    # no rounding), 256 MiB for the placement
    assert (160 << 20) // per_tile >= 1024
    assert info.rs_launch_tiles == min(info.rs_tiles, (160 << 20) // per_tile)
    # 16 workgroups per CU: no LDS reservation (the kernels' own 8 KB)
    assert info.rs_lds_bytes == 8192
    assert info.ag_launch_tiles == min(info.ag_tiles, (256 << 20) // (info.ag_tile_elems * 4))
    _, big = api.tide_desc_build(shapes, R, g, o, ga, f, launch_mib=256)
    assert big.rs_launch_tiles == min(big.rs_tiles, (256 << 20) // per_tile)
    assert big.ag_launch_tiles == min(big.ag_tiles, (256 << 20) // (big.ag_tile_elems * 4))
    # below 4 workgroups per CU a default launch is rounded down to whole
    # workgroups per CU (multiples of 256 tiles), at least 512 tiles: at
    # R = 64 a 160 MiB launch would hold ~620 tiles -> 512; at R = 128,
    # ~315 -> 512; an explicit launch size is not rounded
    shapes64 = [(8192, 8192)]
    for R64, want in ((64, 512), (128, 512)):
        _, _, _, S64 = api.tide_desc_geometry(shapes64, R64)
        g64, o64, _, _ = _fake_ptrs(shapes64, R64, S64)
        _, i64 = api.tide_desc_build(shapes64, R64, g64, o64, None, None)
        per64 = i64.rs_tile_elems * (2 * R64 + 4)
        assert (160 << 20) // per64 < 1024
        assert i64.rs_launch_tiles == min(i64.rs_tiles, want)
        # 2 workgroups per CU: each holds 64 KB of LDS
        assert i64.rs_lds_bytes == 64 * 1024
        _, x64 = api.tide_desc_build(shapes64, R64, g64, o64, None, None, launch_mib=160)
        assert x64.rs_launch_tiles == min(x64.rs_tiles, (160 << 20) // per64)
        assert x64.rs_lds_bytes == 8192
    # R = 40: ~975 tiles -> 768 (3 per CU): rounded, not reserved
    _, _, _, S40 = api.tide_desc_geometry(shapes64, 40)
    g40, o40, _, _ = _fake_ptrs(shapes64, 40, S40)
    _, i40 = api.tide_desc_build(shapes64, 40, g40, o40, None, None)
    assert (160 << 20) // (i40.rs_tile_elems * (2 * 40 + 4)) == 975
    assert i40.rs_launch_tiles == 768 and i40.rs_lds_bytes == 8192
    # R a multiple of 8, 4 to 8.x workgroups per CU: rounded to the nearest
    # whole number per CU, at most 7.  R = 32: ~1204 tiles, 4.7 per CU ->
    # 1280; R = 24: ~1613, 6.3 -> 1536; R = 16: ~2275, 8.9 -> 1792; other R
    # keep the byte target (R = 20: ~1906, 7.4 per CU; R = 18: 2048);
    # explicit sizes: not rounded
    for Rr, want in ((32, 1280), (24, 1536), (16, 1792), (20, (160 << 20) // (2048 * 44)),
                     (18, (160 << 20) // (2048 * 40))):
        _, _, _, Sr = api.tide_desc_geometry(shapes64, Rr)
        gr, orr, _, _ = _fake_ptrs(shapes64, Rr, Sr)
        blob_r, ir = api.tide_desc_build(shapes64, Rr, gr, orr, None, None)
        assert ir.rs_tile_elems == 2048
        assert ir.rs_launch_tiles == min(ir.rs_tiles, want), (Rr, ir.rs_launch_tiles)
        # the tree-order launches: whole rounds of 4 per CU for R a multiple
        # of 8 (R = 32: 1024, R = 24: 1024, R = 16: 2048), else the byte target
        hr = decode(blob_r)[0]
        assert hr["rs_launch"] == ir.rs_launch_tiles
        target = (160 << 20) // (2048 * (2 * Rr + 4))
        want_tree = target // 1024 * 1024 if Rr % 8 == 0 else target
        assert hr["rs_launch_tree"] == min(ir.rs_tiles, want_tree), (Rr, hr["rs_launch_tree"])
        assert ir.rs_lds_bytes == 8192
        _, xr = api.tide_desc_build(shapes64, Rr, gr, orr, None, None, launch_mib=160)
        assert xr.rs_launch_tiles == min(xr.rs_tiles, (160 << 20) // (2048 * (2 * Rr + 4)))
    # a layer of at most 512 tiles is one launch of at most 2 workgroups per
    # CU: reserved too; the host blob carries it and tide_plan_query reads it
    for Rs in (4, 17):
        _, _, _, Ss = api.tide_desc_geometry([(64, 64)], Rs)
        gs, os_, _, _ = _fake_ptrs([(64, 64)], Rs, Ss)
        blob, tiny = api.tide_desc_build([(64, 64)], Rs, gs, os_, None, None)
        assert tiny.rs_launch_tiles == tiny.rs_tiles <= 512 and tiny.rs_lds_bytes == 64 * 1024
        q = _lib.TidePlanInfo()
        assert _lib.lib().tide_plan_query(blob.ctypes.data, ctypes.byref(q)) == 0
        assert q.rs_lds_bytes == 64 * 1024 and q.rs_launch_tiles == tiny.rs_launch_tiles
    _, one = api.tide_desc_build(shapes, R, g, o, ga, f, launch_mib=-1)
    assert one.rs_launch_tiles == one.rs_tiles and one.ag_launch_tiles == one.ag_tiles
    _, small = api.tide_desc_build(shapes, R, g, o, ga, f, launch_mib=1)
    assert small.rs_launch_tiles == max(1, (1 << 20) // per_tile)
    assert _status(api.tide_desc_build, shapes, R, g, o, ga, f, 1, 0, 0, -1, -2) == -1


@pytest.mark.parametrize("gmis", [2, 4, 6, 10, 14])
def test_ag_realigning_tiles_for_shifted_slots(gmis):
    """Slots 16-byte-misaligned against aligned full tensors get realigning
    tiles for everything but an element-wise head and tail of fewer than 8
    elements per run."""
    shapes = [(4096, 8)]
    R = 2
    _, _, _, S = api.tide_desc_geometry(shapes, R)
    _, _, ga, f = _fake_ptrs(shapes, R, S)
    blob, _ = api.tide_desc_build(shapes, R, None, None, ga + gmis, f)
    _, ps, _, _, ag = decode(blob)
    kinds = ag["kind"].tolist()
    assert 3 in kinds
    for t in ag:
        if t["kind"] != 3:
            assert t["kind"] == 2 and t["len"] < 8


def test_staging_validation_before_touching_the_gpu():
    """The copy-engine-staged reduce-scatter and the copy-engine placement
    reject bad staging buffers and plans on the host, before any GPU call."""
    R = 4
    _, _, _, S = api.tide_desc_geometry(SHAPES, R)
    g, o, ga, f = _fake_ptrs(SHAPES, R, S)
    L = _lib.lib()
    blob, _ = api.tide_desc_build(SHAPES, R, g, o, None, None)
    fake_dev = ctypes.c_void_p(1 << 44)
    span = ((2 * R * S + 4095) // 4096 + 1) * 4096
    good = np.array([(1 << 45) + r * span for r in range(R)], dtype=np.uint64)

    def fold(stage, stride=S, order=0, max_wg=0, d_stage=1 << 46, plan=blob):
        arr = stage.ctypes.data if stage is not None else None
        return L.tide_rs_fold_staged(plan.ctypes.data, fake_dev, order, arr, ctypes.c_void_p(d_stage),
                                     stride, max_wg, None)

    def stage_dma(stage, stride=S, plan=blob):
        arr = stage.ctypes.data if stage is not None else None
        return L.tide_rs_stage_dma(plan.ctypes.data, arr, stride, None)

    for call in (fold, stage_dma):
        assert call(good, stride=S - 1) == -1                     # slots shorter than S
        assert call(None) == -1                                   # no staging array
        bad = good.copy(); bad[2] = 0
        assert call(bad) == -1                                    # NULL staging buffer
        bad = good.copy(); bad[1] += 1
        assert call(bad) == -2                                    # odd bf16 address
        bad = good.copy(); bad[3] = bad[2] + 2 * S
        assert call(bad) == -3                                    # two ranks' buffers overlap
        bad = good.copy(); bad[0] = g[1] - 2
        assert call(bad) == -3                                    # over a gradient tensor
        bad = good.copy(); bad[0] = o[2] + 8
        assert call(bad) == -3                                    # over an output arena
    assert fold(good, order=2) == -1
    assert fold(good, max_wg=-1) == -1
    assert fold(good, d_stage=(1 << 46) + 4) == -2                # misaligned device array
    ag_blob, _ = api.tide_desc_build(SHAPES, R, None, None, ga, f)
    assert fold(good, plan=ag_blob) == -6 and stage_dma(good, plan=ag_blob) == -6
    junk = np.zeros(4096, np.uint8)
    assert fold(good, plan=junk) == -7 and stage_dma(good, plan=junk) == -7
    assert L.tide_ag_place_dma(blob.ctypes.data, None) == -6     # no placement pointers
    assert L.tide_ag_place_dma(junk.ctypes.data, None) == -7


def test_pipeline_phases_validate_before_touching_the_gpu():
    R = 4
    _, _, _, S = api.tide_desc_geometry(SHAPES, R)
    g, o, ga, f = _fake_ptrs(SHAPES, R, S)
    L = _lib.lib()
    blob, info = api.tide_desc_build(SHAPES, R, g, o, None, None)
    n = int(info.rs_tiles)
    T = int(info.rs_tile_elems)
    fake_dev = ctypes.c_void_p(1 << 44)
    stage = 1 << 45
    for fn in (L.tide_rs_tiles_to_stage, L.tide_rs_stage_to_shards):
        def call(b=0, cnt=n, st=stage, elems=n * T, mw=0, plan=blob):
            return fn(plan.ctypes.data, fake_dev, b, cnt, ctypes.c_void_p(st) if st else None, elems,
                      mw, None)
        assert call(b=-1) == -1 and call(cnt=n + 1) == -1 and call(b=n, cnt=1) == -1
        assert call(st=0) == -1                                   # no staging chunk
        assert call(st=stage + 4) == -2                           # not 16-byte aligned
        assert call(elems=n * T - 1) == -1                        # chunk too small
        assert call(st=o[1]) == -3                                # over an output arena
        assert call(st=(g[1] // 16) * 16) == -3                   # over a gradient tensor
        assert call(mw=-1) == -1
        ag_blob, _ = api.tide_desc_build(SHAPES, R, None, None, ga, f)
        assert call(plan=ag_blob) == -6
        assert call(plan=np.zeros(4096, np.uint8)) == -7
        assert call(cnt=0, elems=0) == 0                          # empty range: nothing to do
    D = L.tide_rs_stage_to_shards_sdma

    def dcall(b=0, cnt=n, st=stage, elems=n * T, plan=blob):
        return D(plan.ctypes.data, b, cnt, ctypes.c_void_p(st) if st else None, elems, None)
    assert dcall(b=-1) == -1 and dcall(cnt=n + 1) == -1 and dcall(st=0) == -1
    assert dcall(st=stage + 4) == -2 and dcall(elems=n * T - 1) == -1 and dcall(st=o[1]) == -3
    assert dcall(plan=np.zeros(4096, np.uint8)) == -7 and dcall(cnt=0, elems=0) == 0
    assert L.tide_rs_tiles_to_stage(blob.ctypes.data, None, 0, n, ctypes.c_void_p(stage), n * T, 0,
                                    None) == -1                   # no device plan


@pytest.mark.parametrize("R", [1, 3, 8, 17, 64])
def test_rank_tile_ranges_partition_the_plan(R):
    """Rank r's tiles are one contiguous range, the ranges follow each other
    in rank order and cover every tile; validation on the host."""
    _, _, _, S = api.tide_desc_geometry(SHAPES, R)
    g, o, ga, f = _fake_ptrs(SHAPES, R, S)
    blob, info = api.tide_desc_build(SHAPES, R, g, o, ga, f, rs_tile=2048)
    _, _, _, rs, _ = decode(blob)
    pos = 0
    for r in range(R):
        b, c = api.tide_plan_rank_tiles(blob, r)
        assert b == pos
        assert all(int(t["r"]) == r for t in rs[b:b + c])
        pos = b + c
    assert pos == int(info.rs_tiles)
    L = _lib.lib()
    b, c = ctypes.c_int64(), ctypes.c_int64()
    assert L.tide_plan_rank_tiles(blob.ctypes.data, R, ctypes.byref(b), ctypes.byref(c)) == -1
    assert L.tide_plan_rank_tiles(blob.ctypes.data, -1, ctypes.byref(b), ctypes.byref(c)) == -1
    ag_blob, _ = api.tide_desc_build(SHAPES, R, None, None, ga, f)
    assert L.tide_plan_rank_tiles(ag_blob.ctypes.data, 0, ctypes.byref(b), ctypes.byref(c)) == -6
    assert L.tide_plan_rank_tiles(np.zeros(4096, np.uint8).ctypes.data, 0, ctypes.byref(b),
                                  ctypes.byref(c)) == -7


def test_stream_calls_validate_before_touching_the_gpu():
    L = _lib.lib()
    out = ctypes.c_void_p(0)
    assert L.tide_stream_create_cu_limited(0, ctypes.byref(out)) == -1
    assert L.tide_stream_create_cu_limited(-3, ctypes.byref(out)) == -1
    assert L.tide_stream_create_cu_limited(8, None) == -1
    assert L.tide_stream_create_cu_range(-1, 8, ctypes.byref(out)) == -1
    assert L.tide_stream_create_cu_range(0, 0, ctypes.byref(out)) == -1
    assert L.tide_stream_create_cu_range(0, 8, None) == -1
    assert L.tide_stream_destroy(None) == -1
    assert L.tide_dma_engine_count(None) == -1
    # the pipeline object: argument checks come before any device query
    assert L.tide_pipeline_create(0, 0, ctypes.byref(out)) == -1
    assert L.tide_pipeline_create(65, 0, ctypes.byref(out)) == -1
    assert L.tide_pipeline_create(2, -1, ctypes.byref(out)) == -1
    assert L.tide_pipeline_create(2, 0, None) == -1
    fake = ctypes.c_void_p(1 << 44)
    assert L.tide_pipeline_run(None, None, fake, 4, fake, 1 << 20, 0, None) == -1
    assert L.tide_pipeline_destroy(None) == -1


def test_empty_layer_issues_nothing():
    """A layer with no params: the plan has no tiles, and both calls return
    OK without touching the device (so they run here, with no GPU)."""
    R = 4
    outs = [(5 + r) << 40 for r in range(R)]
    blob, info = api.tide_desc_build([], R, [], outs, None, None)
    assert int(info.rs_tiles) == 0 and int(info.ag_tiles) == 0
    L = _lib.lib()
    fake = ctypes.c_void_p(1 << 44)
    assert L.tide_rs_bf16_to_fp32(blob.ctypes.data, fake, 0, 0, None) == 0
    assert L.tide_rs_bf16_to_fp32(blob.ctypes.data, fake, 1, 0, None) == 0
    b, c = ctypes.c_int64(-1), ctypes.c_int64(-1)
    assert L.tide_plan_rank_tiles(blob.ctypes.data, R - 1, ctypes.byref(b), ctypes.byref(c)) == 0
    assert c.value == 0


def test_missing_library_fails_loudly(tmp_path):
    """With the library absent the binding raises: there is no fallback path
    (checked in a fresh interpreter so the loaded library stays untouched)."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import shard_placement_amd._lib as L\n"
            "L.LIB_PATH = %r\n"
            "from shard_placement_amd import api\n"
            "try:\n"
            "    api.tide_desc_geometry([(4, 4)], 2)\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n"
            "    sys.exit(0)\n"
            "sys.exit(1)\n") % (ROOT, str(tmp_path / "libtide.so"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "not built" in r.stdout, r.stdout + r.stderr


def test_product_path_never_touches_the_oracle():
    """The package and its native sources neither import, include nor load
    the oracle; bench.py imports it only inside its cpu_baseline leg."""
    import ast
    pkg = os.path.join(ROOT, "shard_placement_amd")
    for name in os.listdir(pkg):
        path = os.path.join(pkg, name)
        if name.endswith(".py"):
            tree = ast.parse(open(path).read())
            for node in ast.walk(tree):
                if isinstance(node, ast.Import):
                    assert all(a.name.split(".")[0] != "oracle" for a in node.names), name
                if isinstance(node, ast.ImportFrom):
                    assert (node.module or "").split(".")[0] != "oracle", name
    for name in os.listdir(os.path.join(pkg, "csrc")):
        text = open(os.path.join(pkg, "csrc", name)).read()
        assert "tide_oracle" not in text and "oracle/" not in text, name
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    users = set()
    for fn in ast.walk(tree):
        if isinstance(fn, ast.FunctionDef):
            for node in ast.walk(fn):
                if isinstance(node, ast.Import) and any(a.name == "oracle" for a in node.names):
                    users.add(fn.name)
    top = [n for n in tree.body if isinstance(n, (ast.Import, ast.ImportFrom))]
    assert all(not (isinstance(n, ast.Import) and any(a.name == "oracle" for a in n.names)) for n in top)
    assert users == {"cpu_baseline"}, users
    # and the other way round: the oracle uses none of the library's code
    src = open(os.path.join(ROOT, "oracle", "tide_oracle.c")).read()
    assert "tide.h" not in src and "plan_format" not in src
    tree = ast.parse(open(os.path.join(ROOT, "oracle", "__init__.py")).read())
    for node in ast.walk(tree):
        if isinstance(node, (ast.Import, ast.ImportFrom)):
            mods = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module or ""]
            assert all(not m.startswith("shard_placement_amd") for m in mods)


def test_noalloc_two_phase_validates_before_touching_the_gpu():
    """The allocation-free two-phase call checks its plan, tile range and
    the size of its staging array on the host, before any HIP call; an
    empty range is a no-op."""
    L = _lib.lib()
    with open(os.path.join(ROOT, "include", "tide.h")) as fh:
        m = re.search(r"#define TIDE_SCRATCH_BYTES \((\d+)u << (\d+)\)", fh.read())
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.SCRATCH_BYTES
    shapes = [(8192, 4096), (5,)]
    R = 2
    _, _, _, S = api.tide_desc_geometry(shapes, R)
    g, o, ga, f = _fake_ptrs(shapes, R, S)
    blob, info = api.tide_desc_build(shapes, R, g, o, None, None, rs_tile=2048)
    n, T = int(info.rs_tiles), int(info.rs_tile_elems)
    cap = _lib.SCRATCH_BYTES // (4 * T)
    assert n > cap
    fake_dev = ctypes.c_void_p(1 << 44)
    F = L.tide_rs_two_phase_noalloc

    def call(b=0, cnt=1, mw=0, plan=blob, dev=fake_dev):
        return F(plan.ctypes.data if plan is not None else None, dev, b, cnt, mw, None)
    assert call(plan=None) == -1 and call(dev=None) == -1
    assert call(plan=np.zeros(4096, np.uint8)) == -7
    ag_blob, _ = api.tide_desc_build(shapes, R, None, None, ga, f)
    assert call(plan=ag_blob) == -6
    assert call(b=-1) == -1 and call(cnt=-1) == -1 and call(mw=-1) == -1
    assert call(b=n, cnt=1) == -1 and call(b=n - 1, cnt=2) == -1
    assert call(cnt=cap + 1) == -4                      # more than the array holds
    assert call(b=n - cap - 1, cnt=cap + 1) == -4
    assert call(dev=ctypes.c_void_p((1 << 44) + 8)) == -2
    assert call(cnt=0) == 0 and call(b=n, cnt=0) == 0   # nothing to do


def test_streams_variant_validates_before_touching_the_gpu():
    R = 4
    _, _, _, S = api.tide_desc_geometry(SHAPES, R)
    g, o, ga, f = _fake_ptrs(SHAPES, R, S)
    L = _lib.lib()
    blob, _ = api.tide_desc_build(SHAPES, R, g, o, None, None)
    fake_dev = ctypes.c_void_p(1 << 44)
    vp = ctypes.c_void_p
    two = (vp * 2)(1 << 20, 2 << 20)                                   # made-up handles
    F = L.tide_rs_bf16_to_fp32_streams
    assert F(blob.ctypes.data, fake_dev, 0, 0, (vp * 2)(None, 2 << 20), 2) == -1  # null stream
    assert F(blob.ctypes.data, fake_dev, 0, 0, (vp * 2)(1 << 20, None), 2) == -1
    assert F(blob.ctypes.data, fake_dev, 0, 0, None, 1) == -1          # no stream array
    assert F(blob.ctypes.data, fake_dev, 0, 0, two, 0) == -1           # no stream
    assert F(blob.ctypes.data, fake_dev, 0, 0, two, 65) == -1          # too many
    assert F(blob.ctypes.data, fake_dev, 2, 0, two, 2) == -1           # bad order
    assert F(blob.ctypes.data, ctypes.c_void_p((1 << 44) + 8), 0, 0, two, 2) == -2
    assert F(np.zeros(4096, np.uint8).ctypes.data, fake_dev, 0, 0, two, 2) == -7
    ag_blob, _ = api.tide_desc_build(SHAPES, R, None, None, ga, f)
    assert F(ag_blob.ctypes.data, fake_dev, 0, 0, two, 2) == -6


def test_bench_refuses_several_gpus_and_needs_one():
    """bench.py measures one GPU: --gpus above 1 exits with a message that
    says so, and without a visible GPU it fails instead of falling back to
    anything on the host."""
    import subprocess
    import sys

    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    import torch

    if not torch.cuda.is_available():
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "1",
                            "--warmup", "0"], capture_output=True, text=True, timeout=300)
        assert r.returncode != 0
        assert "no GPU" in r.stderr
        assert not r.stdout.strip().startswith("{")
