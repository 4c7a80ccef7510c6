"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test checks the oracle against something fixed from outside it: hand-
derived IEEE results (tests/golden), exact integer arithmetic, closed forms,
error bounds of recursive and pairwise summation, torch's own dim-0 chunking
(the shard rule) and concatenation (the arena / slot layout), and a pure-
Python brute force on tiny inputs.  A dropped rank, a wrong start value, a
wrong order, a floor instead of a ceil, a wrong offset or slot stride each
fails at least one of them.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from shard_placement_amd import configs, synth
from tests.brute import rs_brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U = 2.0 ** -24  # unit roundoff of binary32


def _bits16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16).reshape(-1)


def _f32_bits(a) -> np.ndarray:
    return np.asarray(a, np.float32).view(np.uint32)


def _widen(bits16: np.ndarray) -> np.ndarray:
    return (bits16.astype(np.uint32) << 16).view(np.float32)


def _draw(shapes, R, gen_fn):
    """grads[q][p] as uint16 arrays, drawn rank by rank with torch (CPU)."""
    grads = []
    for q in range(R):
        arena = torch.empty(synth.arena_numel(shapes), dtype=torch.bfloat16)
        gen_fn(arena, q)
        grads.append([_bits16(v) for v in synth.views(arena, shapes)])
    return grads


def _chunk_shards(full: torch.Tensor, R: int):
    """Shard rule from torch: dim-0 chunks of ceil(d0/R) rows (torch.chunk),
    the missing rows zero-padded, missing chunks all zero (FSDP2's
    convention for a rank without rows)."""
    if full.dim() == 0:
        full = full.reshape(1)
    d0 = full.shape[0]
    s = -(-d0 // R)
    chunks = list(torch.chunk(full, R, dim=0)) if d0 > 0 else []
    out = []
    for r in range(R):
        ch = chunks[r] if r < len(chunks) else full[0:0]
        pad = [0, 0] * (full.dim() - 1) + [0, s - ch.shape[0]]
        out.append(F.pad(ch, pad).reshape(-1))
    return out


# ---------------------------------------------------------------- golden
def _golden_rows():
    rows = []
    with open(os.path.join(GOLDEN, "order_discriminators.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, inputs, fixed, tree = line.split()
            vals = [int(x, 16) for x in inputs.split(",")]
            rows.append((name, vals, fixed, tree))
    return rows


@pytest.mark.parametrize("row", _golden_rows(), ids=lambda r: r[0])
def test_hand_derived_order_and_ieee(orc, row):
    name, vals, fixed, tree = row
    v = np.asarray([vals], np.uint16)
    for order, want in (("fixed", fixed), ("tree", tree)):
        got = orc.fold_points(v, order)[0]
        if want == "nan":
            assert math.isnan(got), (name, order)
        else:
            assert int(_f32_bits(got)) == int(want, 16), (name, order, hex(int(_f32_bits(got))))
    # the same element through the full reduce-scatter entry point
    R = len(vals)
    grads = [[np.asarray([vals[q]], np.uint16)] for q in range(R)]
    for order, want in (("fixed", fixed), ("tree", tree)):
        out = orc.rs([(1,)], R, grads, order=order)
        got = out[0][0]
        if want == "nan":
            assert math.isnan(got)
        else:
            assert int(_f32_bits(got)) == int(want, 16), (name, order)


# ---------------------------------------------------------------- shard rule
@pytest.mark.parametrize("R", [1, 2, 3, 4, 7, 8, 16, 64])
def test_layout_matches_torch_chunk(orc, R):
    shapes = [(37, 16), (64, 64), (5,), (1,), (), (0, 3), (1001, 8), (6, 5), (3, 0)]
    s, m, off, S = orc.layout(shapes, R)
    pos = 0
    for p, shp in enumerate(shapes):
        full = torch.zeros(shp)
        shards = _chunk_shards(full, R)
        assert all(x.numel() == shards[0].numel() for x in shards)
        assert m[p] == shards[0].numel(), (shp, R)
        assert off[p] == pos
        pos += shards[0].numel()
    assert S == pos


def test_layout_alignment(orc):
    shapes = [(5,), (37, 16), (3, 3)]
    s, m, off, S = orc.layout(shapes, 4, align=8)
    assert list(m) == [2, 160, 3]
    assert list(off) == [0, 8, 168]
    assert S == 176


# ---------------------------------------------------------------- integer grid
INT_SHAPES = [(37, 16), (64, 64), (5,), (1001, 3), (7, 2, 3), (), (2,), (0, 4)]


@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 8, 17, 64])
@pytest.mark.parametrize("order", ["fixed", "tree"])
def test_integer_grid_exact(orc, R, order):
    """k*2^-10 inputs, |k| <= 127: every partial sum is exact in binary32
    (|sum| <= 64*127 < 2^24 ulps), so any order gives the integer sum.  The
    expected arenas are built from exact integer sums, torch.chunk and
    torch.cat, independently of the oracle's indexing."""
    shapes = INT_SHAPES
    grads = _draw(shapes, R, lambda a, q: synth.integer_grid_(a, 7000 + 31 * R + q))
    out = orc.rs(shapes, R, grads, order=order)
    for r in range(R):
        pieces = []
        for p, shp in enumerate(shapes):
            ks = sum(np.round(_widen(grads[q][p]).astype(np.float64) * 1024).astype(np.int64)
                     for q in range(R))
            full = torch.from_numpy(np.asarray(ks, np.int64).reshape(shp) if len(shp) else
                                    np.asarray(ks, np.int64).reshape(()))
            pieces.append(_chunk_shards(full, R)[r])
        want = torch.cat(pieces).to(torch.float64) / 1024.0
        np.testing.assert_array_equal(out[r], want.numpy().astype(np.float32))
        # +0.0 padding, not -0.0
        assert not np.any(_f32_bits(out[r]) == 0x80000000)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 7, 8, 16, 17, 32, 64])
@pytest.mark.parametrize("order", ["fixed", "tree"])
def test_identical_ranks_give_R_times_g(orc, R, order):
    """R copies of g sum to R*g exactly: R*g needs at most 8 + 6 significant
    bits, and with the fold starting from rank 0 every partial sum k*g is
    exact, so the result is the exact product (also for -0, subnormals)."""
    shapes = [(33, 8)]
    base = torch.empty(33 * 8, dtype=torch.bfloat16)
    synth.fill_normal_(base, 4242, 1.0)
    b = _bits16(base).copy()
    b[:6] = [0x8000, 0x0000, 0x0001, 0x807F, 0x3F80, 0x0080]
    grads = [[b] for _ in range(R)]
    out = orc.rs(shapes, R, grads, order=order)
    s = -(-33 // R)
    want = (_widen(b).astype(np.float64) * R).astype(np.float32)
    want = np.concatenate([want, np.zeros(R * s * 8 - want.size, np.float32)])
    got = np.concatenate([out[r][: s * 8] for r in range(R)])
    np.testing.assert_array_equal(_f32_bits(got), _f32_bits(want))


@pytest.mark.parametrize("R", [2, 3, 8, 16])
def test_one_hot_rank(orc, R):
    """Only rank h is nonzero: the result is f32(g_h) exactly."""
    shapes = [(19, 4)]
    for h in {0, R // 2, R - 1}:
        grads = []
        for q in range(R):
            t = torch.zeros(76, dtype=torch.bfloat16)
            if q == h:
                synth.fill_normal_(t, 99 + h, 1.0)
                t[t == 0] = 1.0
            grads.append([_bits16(t)])
        out = orc.rs(shapes, R, grads)
        s = -(-19 // R)
        got = np.concatenate([out[r][: s * 4] for r in range(R)])[:76]
        np.testing.assert_array_equal(_f32_bits(got), _f32_bits(_widen(grads[h][0])))


@pytest.mark.parametrize("R", [2, 4, 8, 64])
@pytest.mark.parametrize("order", ["fixed", "tree"])
def test_antisymmetric_pairs_cancel_to_plus_zero(orc, R, order):
    """Rank 2k+1 = -rank 2k: every pair cancels exactly; the fold ends at
    +0.0 (x + (-x) = +0 under round to nearest)."""
    shapes = [(40,)]
    grads = []
    for k in range(R // 2):
        t = torch.empty(40, dtype=torch.bfloat16)
        synth.fill_normal_(t, 500 + k, 1.0)
        grads.append([_bits16(t)])
        grads.append([_bits16(-t)])
    out = orc.rs(shapes, R, grads, order=order)
    for r in range(R):
        assert np.all(_f32_bits(out[r]) == 0)


def test_single_rank_is_exact_widening(orc):
    """R = 1: the shard is the bf16 tensor widened to fp32 (torch's exact
    bf16 -> fp32 conversion)."""
    t = torch.empty(517, dtype=torch.bfloat16)
    synth.bits_(t, 3)
    t[torch.isnan(t)] = 1.0
    out = orc.rs([(517,)], 1, [[_bits16(t)]])
    np.testing.assert_array_equal(_f32_bits(out[0]), _f32_bits(t.float().numpy()))


def test_two_ranks_round_once(orc):
    """R = 2: one IEEE add = the exact sum rounded once to binary32.  The
    exact sum is formed in fp64 and checked exact with Fraction."""
    a = torch.empty(2000, dtype=torch.bfloat16)
    b = torch.empty(2000, dtype=torch.bfloat16)
    synth.fill_normal_(a, 11, 1.0)
    synth.fill_normal_(b, 12, 3.0)
    out = orc.rs([(2000,)], 2, [[_bits16(a)], [_bits16(b)]])
    s64 = a.double().numpy() + b.double().numpy()
    for x, y, z in zip(a.double().numpy()[:200], b.double().numpy()[:200], s64[:200]):
        assert Fraction(x) + Fraction(y) == Fraction(z)
    want = s64.astype(np.float32)
    got = np.concatenate([out[0][:1000], out[1][:1000]])
    np.testing.assert_array_equal(_f32_bits(got), _f32_bits(want))


# ---------------------------------------------------------------- error bounds
@pytest.mark.parametrize("R", [3, 8, 16, 64])
def test_error_bounds(orc, R):
    """Recursive summation: |fixed - exact| <= gamma_{R-1} * sum|g|;
    pairwise: |tree - exact| <= gamma_{ceil(log2 R)} * sum|g| (Higham,
    Accuracy and Stability of Numerical Algorithms, ch. 4).  Also the
    tolerance 1e-6 * sum|g| for tree order.  The fixed and tree results must
    differ somewhere for random data when R >= 4 (for R <= 3 the two orders
    coincide: ((g0+g1)+g2))."""
    K = 4000
    gen = torch.Generator().manual_seed(R)
    # a wide exponent spread, so that partial sums round (bf16 values of one
    # magnitude add exactly in binary32 for small R)
    scale = torch.ldexp(torch.ones(K, R), torch.randint(-12, 13, (K, R), generator=gen))
    vals = (torch.randn(K, R, generator=gen) * 1e-3 * scale).to(torch.bfloat16)
    bits = _bits16(vals).reshape(K, R)
    fixed = orc.fold_points(bits, "fixed").astype(np.float64)
    tree = orc.fold_points(bits, "tree").astype(np.float64)
    w = _widen(bits).astype(np.float64)
    exact = np.asarray([math.fsum(row) for row in w])
    absum = np.abs(w).sum(axis=1)

    def gamma(n):
        return n * U / (1 - n * U)

    assert np.all(np.abs(fixed - exact) <= gamma(R - 1) * absum * (1 + 1e-12))
    assert np.all(np.abs(tree - exact) <= gamma(math.ceil(math.log2(R))) * absum * (1 + 1e-12))
    assert np.all(np.abs(tree - exact) <= 1e-6 * absum)
    if R >= 4:
        assert np.any(fixed != tree)
    else:
        np.testing.assert_array_equal(fixed, tree)


# ---------------------------------------------------------------- padding, gaps
def test_padding_written_gaps_untouched(orc):
    """Padding elements are written +0.0 (bits 0) over a NaN pre-fill;
    alignment gaps between shards keep their pre-fill."""
    shapes = [(5,), (37, 16), (3, 3)]
    R = 4
    grads = _draw(shapes, R, lambda a, q: synth.fill_normal_(a, 50 + q, 1.0))
    s, m, off, S = orc.layout(shapes, R, align=8)
    out = [np.full(S, np.nan, np.float32) for _ in range(R)]
    for r in range(R):
        out[r].view(np.uint32)[:] = 0xFFFFFFFF
    orc.rs(shapes, R, grads, align=8, out=out)
    for r in range(R):
        bits = out[r].view(np.uint32)
        for p in range(len(shapes)):
            n = int(np.prod(shapes[p]))
            shard = bits[off[p]:off[p] + m[p]]
            valid = max(0, min(m[p], n - r * m[p]))
            assert np.all(shard[valid:] == 0)
            assert not np.any(shard[:valid] == 0xFFFFFFFF)
            gap_end = off[p + 1] if p + 1 < len(shapes) else S
            assert np.all(bits[off[p] + m[p]:gap_end] == 0xFFFFFFFF)


# ---------------------------------------------------------------- all-gather
def _slots_from_fulls(fulls, R, sentinel=0xFFFF):
    """Build the rank-major gathered buffer with torch.chunk + pad + cat:
    slot r = concatenation over params of rank r's padded chunk; padding rows
    carry a sentinel so that trimming is visible."""
    slots = []
    for r in range(R):
        pieces = []
        for full in fulls:
            t = full if full.dim() else full.reshape(1)
            d0 = t.shape[0]
            s = -(-d0 // R)
            chunks = list(torch.chunk(t, R, dim=0)) if d0 > 0 else []
            ch = chunks[r] if r < len(chunks) else t[0:0]
            pad = torch.full((s - ch.shape[0],) + tuple(t.shape[1:]), sentinel, dtype=torch.int32)
            pieces.append(torch.cat([ch.to(torch.int32), pad]).reshape(-1))
        slots.append(torch.cat(pieces))
    return torch.cat(slots).numpy().astype(np.uint16)


@pytest.mark.parametrize("R", [1, 2, 3, 4, 8, 17])
def test_ag_round_trip_bits(orc, R):
    """Placement of slots sliced from T gives T back bit for bit (NaN
    payloads, -0, infinities included) and never copies the sentinel."""
    shapes = [(37, 16), (64, 64), (5,), (), (1001, 3), (0, 2), (2, 1, 3)]
    fulls = []
    for p, shp in enumerate(shapes):
        t = torch.empty(shp, dtype=torch.bfloat16)
        synth.bits_(t, 77 + p)
        if t.numel():
            t.view(-1).view(torch.int16)[t.view(-1).view(torch.int16) == -1] = 0x7FC1
        fulls.append(t.view(torch.int16).to(torch.int32) & 0xFFFF)
    gathered = _slots_from_fulls(fulls, R)
    _, _, _, S = orc.layout(shapes, R)
    assert gathered.size == R * S
    out = [np.full(int(np.prod(s)), 0xABCD, np.uint16) for s in shapes]
    orc.ag(shapes, R, gathered, out=out)
    for p in range(len(shapes)):
        np.testing.assert_array_equal(out[p], fulls[p].reshape(-1).numpy().astype(np.uint16))
        assert not np.any(out[p] == 0xFFFF)


@pytest.mark.parametrize("R", [2, 4, 8])
def test_ag_of_rs_equals_full_fold(orc, R):
    """AG(bf16(RS shards)) == bf16(fold of the full tensors): the shards the
    reduce-scatter writes are exactly the slots the placement reads."""
    shapes = [(37, 16), (5,), (64, 3)]
    grads = _draw(shapes, R, lambda a, q: synth.fill_normal_(a, 900 + q, 1.0))
    out = orc.rs(shapes, R, grads)
    gathered = np.concatenate([_bits16(torch.from_numpy(o).to(torch.bfloat16)) for o in out])
    placed = orc.ag(shapes, R, gathered)
    for p, shp in enumerate(shapes):
        n = int(np.prod(shp))
        full = orc.fold_points(np.stack([grads[q][p] for q in range(R)], axis=1))
        np.testing.assert_array_equal(placed[p], _bits16(torch.from_numpy(full).to(torch.bfloat16)))
        assert placed[p].size == n


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("seed", range(6))
def test_brute_force_random_shapes(orc, seed):
    rng = np.random.default_rng(seed)
    R = int(rng.integers(1, 10))
    P = int(rng.integers(1, 5))
    shapes = []
    for _ in range(P):
        nd = int(rng.integers(0, 3))
        shapes.append(tuple(int(rng.integers(0, 9)) for _ in range(nd)))
    grads = _draw(shapes, R, lambda a, q: synth.fill_normal_(a, 10 * seed + q, 1.0))
    out = orc.rs(shapes, R, grads)
    _, m, off, _ = orc.layout(shapes, R)
    want = rs_brute(shapes, R, grads)
    for (r, p), shard in want.items():
        np.testing.assert_array_equal(_f32_bits(out[r][off[p]:off[p] + m[p]]),
                                      _f32_bits(np.asarray(shard, np.float32)))


def test_tiny_workload_brute_force(orc):
    w = configs.get(1)
    grads = _draw(w.shapes, w.R,
                  lambda a, q: synth.fill_normal_(a, synth.SEED_STRIDE * w.key + q, w.sigma))
    out = orc.rs(w.shapes, w.R, grads)
    _, m, off, _ = orc.layout(w.shapes, w.R)
    want = rs_brute(w.shapes, w.R, grads)
    for (r, p), shard in want.items():
        np.testing.assert_array_equal(_f32_bits(out[r][off[p]:off[p] + m[p]]),
                                      _f32_bits(np.asarray(shard, np.float32)))


def test_fold_points_agrees_with_rs(orc):
    shapes = [(300, 7)]
    R = 6
    grads = _draw(shapes, R, lambda a, q: synth.fill_normal_(a, 321 + q, 1.0))
    for order in ("fixed", "tree"):
        out = orc.rs(shapes, R, grads, order=order)
        s = -(-300 // R)
        flat = np.concatenate([out[r][: s * 7] for r in range(R)])
        pts = orc.fold_points(np.stack([grads[q][0] for q in range(R)], axis=1), order)
        np.testing.assert_array_equal(_f32_bits(flat), _f32_bits(pts))


def test_ftz_daz_in_caller_do_not_leak(orc):
    """Subnormal sums stay subnormal even if the calling thread has
    flush-to-zero set (the oracle runs its arithmetic with IEEE settings)."""
    v = np.asarray([[0x0001, 0x0001]], np.uint16)
    assert int(_f32_bits(orc.fold_points(v)[0])) == 0x00020000


def test_rejects_bad_arguments(orc):
    with pytest.raises(ValueError):
        orc.layout([(3,)], 0)
    with pytest.raises(ValueError):
        orc.layout([(3,)], 2, align=0)
    with pytest.raises(ValueError):
        orc.rs([(3,)], 2, [[np.zeros(3, np.uint16)]])


def test_tiny_golden_regression(orc):
    """The oracle's tiny-workload outputs match the digests written by
    tests/golden/make_golden.py (inputs are checked first, so a change of
    torch's CPU generator is told apart from a change of the oracle)."""
    import json
    from tests.golden.make_golden import sha, split, tiny_inputs
    with open(os.path.join(GOLDEN, "tiny_oracle.json")) as fh:
        rec = json.load(fh)
    w, arenas, gathered = tiny_inputs()
    if [sha(a) for a in arenas] != rec["input_sha256"] or sha(gathered) != rec["gathered_sha256"]:
        pytest.skip("torch's CPU generator draws different tiny inputs here")
    grads = [split(a, w.shapes) for a in arenas]
    for order in ("fixed", "tree"):
        out = orc.rs(w.shapes, w.R, grads, order=order)
        assert [sha(o.view(np.uint32)) for o in out] == rec["rs_%s_sha256" % order]
    assert [sha(x) for x in orc.ag(w.shapes, w.R, gathered)] == rec["ag_sha256"]
