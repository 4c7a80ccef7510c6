"""Helpers for the GPU parity tests: read device results back and compare
them with the CPU oracle (bit for bit) or with properties that hold at any
size.  Imports the oracle; test infrastructure only."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle

NAN32 = 0xFFFFFFFF
SENT16 = 0xFFFF


def say(*a):
    """Name the case before a GPU step, flushed, so a crash still names it."""
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().reshape(-1).contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bits32(t: torch.Tensor) -> np.ndarray:
    return t.detach().reshape(-1).contiguous().view(torch.int32).cpu().numpy().view(np.uint32)


def numel(shp) -> int:
    n = 1
    for d in shp:
        n *= int(d)
    return n


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str, nan_as_class=False):
    """Bit-exact comparison of uint32 (fp32) or uint16 arrays.  With
    nan_as_class, any NaN matches any NaN (payloads may differ by ISA)."""
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if nan_as_class and got.dtype == np.uint32:
        gf, wf = got.view(np.float32), want.view(np.float32)
        both_nan = np.isnan(gf) & np.isnan(wf)
        bad = (got != want) & ~both_nan
    else:
        bad = got != want
    if bad.any():
        i = np.flatnonzero(bad)
        raise AssertionError("%s: %d of %d words differ; first at %d: got %s want %s"
                             % (what, i.size, got.size, i[0], hex(int(got[i[0]])), hex(int(want[i[0]]))))


def grads_np(st, p=None):
    """Rank-major nested list of uint16 arrays read back from the device."""
    P = st.w.P
    ps = range(P) if p is None else [p]
    return [[bits16(st.grads[q][pp]) for pp in ps] for q in range(st.w.R)]


def check_rs_full(st, order="fixed", nan_as_class=False):
    """Whole-arena comparison with the oracle (small workloads): shards,
    alignment gaps (untouched NaN pre-fill) and guard bands."""
    w = st.w
    want = [np.full(st.S, np.nan, np.float32) for _ in range(w.R)]
    for a in want:
        a.view(np.uint32)[:] = NAN32
    oracle.rs(w.shapes, w.R, grads_np(st), align=_align_of(st), order=order, out=want)
    for r in range(w.R):
        assert_bits_equal(bits32(st.out[r]), want[r].view(np.uint32), "rank %d arena" % r,
                          nan_as_class)
        check_out_guards(st, r)


def _align_of(st) -> int:
    hdr = st.plan.blob[:32].view(np.int64)
    return int(hdr[2])  # PlanHeader.align (bytes 16..23)


def check_out_guards(st, r):
    g = st.guard
    if st.vacated is not None:
        tail = bits16(st.vacated[r][2 * st.S:])
        if r == 0 and st.gathered is not None:
            return  # rank 0's slot also holds the gathered data
        assert np.all(tail == SENT16), "rank %d: vacated buffer written beyond the arena" % r
        return
    if g:
        a = bits32(st.out_alloc[r])
        assert np.all(a[:g] == NAN32) and np.all(a[g + st.S:] == NAN32), \
            "rank %d: guard band written" % r


def check_rs_sampled(st, order="fixed", per_shard=64, edge=16, seed=0):
    """Bit-exact oracle comparison on sampled elements of every (param, rank)
    shard: its first and last `edge` elements plus `per_shard` random ones.
    The R source values of each sampled element are gathered on the device,
    folded by the oracle one element at a time, and compared with the
    device's shard element; padding samples must be +0.0."""
    w = st.w
    R = w.R
    _, m, off, _ = oracle.layout(w.shapes, R, _align_of(st))
    rng = np.random.default_rng(seed)
    dev = st.out[0].device
    checked = 0
    for p, shp in enumerate(w.shapes):
        mp, n = int(m[p]), numel(shp)
        if mp == 0:
            continue
        rr, ii = [], []
        for r in range(R):
            cand = np.unique(np.concatenate([np.arange(min(edge, mp)),
                                             np.arange(max(0, mp - edge), mp),
                                             rng.integers(0, mp, per_shard)]))
            rr.append(np.full(cand.size, r))
            ii.append(cand)
        rr = np.concatenate(rr)
        ii = np.concatenate(ii)
        j = rr.astype(np.int64) * mp + ii
        valid = j < n
        got = np.empty(j.size, np.uint32)
        for r in range(R):
            sel = np.flatnonzero(rr == r)
            idx = torch.from_numpy(int(off[p]) + ii[sel]).to(dev)
            got[sel] = bits32(st.out[r][idx])
        want = np.zeros(j.size, np.uint32)
        if valid.any():
            jv = torch.from_numpy(j[valid]).to(dev)
            vals = torch.stack([st.grads[q][p].reshape(-1)[jv] for q in range(R)], dim=1)
            v = bits16(vals).reshape(-1, R)
            want[valid] = oracle.fold_points(v, order).view(np.uint32)
        assert_bits_equal(got, want, "%s param %d sampled" % (w.name, p))
        checked += j.size
    return checked


def check_rs_points(st, p, flat, order="fixed"):
    """Bit-exact oracle comparison at given flat element indices of param p
    (each in the shard of rank j // m at element j % m); returns the count."""
    w = st.w
    R = w.R
    _, m, off, _ = oracle.layout(w.shapes, R, _align_of(st))
    mp, n = int(m[p]), numel(w.shapes[p])
    j = np.unique(np.asarray(flat, np.int64))
    assert mp > 0 and j.size and j.min() >= 0 and j.max() < n
    dev = st.out[0].device
    rr, ii = j // mp, j % mp
    got = np.empty(j.size, np.uint32)
    for r in np.unique(rr):
        sel = np.flatnonzero(rr == r)
        got[sel] = bits32(st.out[int(r)][torch.from_numpy(int(off[p]) + ii[sel]).to(dev)])
    jv = torch.from_numpy(j).to(dev)
    vals = torch.stack([st.grads[q][p].reshape(-1)[jv] for q in range(R)], dim=1)
    want = oracle.fold_points(bits16(vals).reshape(-1, R), order).view(np.uint32)
    assert_bits_equal(got, want, "%s param %d points" % (w.name, p))
    return j.size


def check_rs_bound_all(st, order="fixed"):
    """Every element of every shard, at any size: within the summation error
    bound of the exact sum (gamma_{R-1} for rank order, gamma_{ceil log2 R}
    for the tree), computed in fp64 on the device; padding exactly +0.0."""
    w = st.w
    R = w.R
    _, m, off, _ = oracle.layout(w.shapes, R, _align_of(st))
    u = 2.0 ** -24
    k = (R - 1) if order == "fixed" else max(1, math.ceil(math.log2(R))) if R > 1 else 0
    gamma = k * u / (1 - k * u)
    for p, shp in enumerate(w.shapes):
        mp, n = int(m[p]), numel(shp)
        if mp == 0:
            continue
        flat = torch.cat([st.out[r][int(off[p]):int(off[p]) + mp] for r in range(R)])
        pad = flat[n:]
        assert torch.all(pad.view(torch.int32) == 0), "%s param %d: padding not +0.0" % (w.name, p)
        CH = 1 << 25
        for a in range(0, n, CH):
            b = min(n, a + CH)
            exact = torch.zeros(b - a, dtype=torch.float64, device=flat.device)
            absum = torch.zeros_like(exact)
            for q in range(R):
                g = st.grads[q][p].reshape(-1)[a:b].to(torch.float64)
                exact += g
                absum += g.abs()
            err = (flat[a:b].to(torch.float64) - exact).abs()
            bad = err > gamma * absum * (1 + 1e-9) + 0.0
            if order == "tree":
                bad |= err > 1e-6 * absum
            assert not bool(bad.any()), "%s param %d: %d elements outside the bound" % (
                w.name, p, int(bad.sum()))


def check_ag_full(st):
    """Whole placement compared with the oracle: every full tensor bit for
    bit, guard bands of the full arena untouched."""
    w = st.w
    g = bits16(st.gathered)
    want = [np.full(numel(s), SENT16, np.uint16) for s in w.shapes]
    oracle.ag(w.shapes, w.R, g, align=_align_of(st), out=want)
    for p in range(w.P):
        assert_bits_equal(bits16(st.full[p]), want[p], "%s full[%d]" % (w.name, p))
    guard = st.guard
    if guard:
        fa = bits16(st.full_arena)
        assert np.all(fa[:guard] == SENT16) and np.all(fa[-guard:] == SENT16), "AG guard band written"


def check_rs_whole(st, order="fixed", block_bytes=512 << 20):
    """Every element of every shard of the layer against the oracle, bit for
    bit, with bounded host memory: each param is read back in blocks of
    consecutive flat indices (all R ranks' values of those indices and the
    result words the arenas hold for them), and the oracle reduces each
    block as a 1-D problem of its own (the sum of an element does not
    depend on where the shard boundaries fall, so the concatenated shards of
    that sub-problem are the block's expected results).  Padding words are
    checked for +0.0 on the device.  Returns the number of elements."""
    from shard_placement_amd import harness

    w = st.w
    R = w.R
    _, m, off, _ = oracle.layout(w.shapes, R, _align_of(st))
    reader = harness.BlockReader(st, m, off, block_bytes)
    total = 0
    for p, shp in enumerate(w.shapes):
        n, mp = numel(shp), int(m[p])
        say("whole-layer oracle check", w.name, "param", p, shp, order)
        for a, b, g, got in reader.blocks(p):
            L = b - a
            arenas = oracle.rs([(L,)], R, [[gq] for gq in g], order=order)
            s = -(-L // R)
            want = np.concatenate([x[:s] for x in arenas])[:L]
            assert_bits_equal(got, want.view(np.uint32),
                              "%s param %d flat [%d, %d)" % (w.name, p, a, b))
            total += L
        for r in range(R):
            lo = max(0, n - r * mp)
            if lo < mp:
                pad = st.out[r][int(off[p]) + lo:int(off[p]) + mp]
                assert bool(torch.all(pad.view(torch.int32) == 0)), \
                    "%s param %d rank %d: padding not +0.0" % (w.name, p, r)
    say("whole-layer oracle check done", w.name, total, "elements; copies waited %.1f s"
        % reader.copy_s)
    return total
