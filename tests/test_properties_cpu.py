"""Property tests on random shapes (hypothesis): the oracle against the
pure-Python brute force, the library's plan geometry against the oracle's,
and the plan's tile lists (partition of every shard, rank-outer order,
placement runs) on made-up addresses.  CPU only."""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from shard_placement_amd import api
from tests.brute import ag_brute, rs_brute
from tests.test_abi_cpu import _check_rs_tiles, _fake_ptrs, decode

SETTINGS = dict(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])

# params: 0-d, 1-D, 2-D and 3-D, dim0 in [0, 70], rows of 1..24 elements
shape = st.one_of(st.just(()),
                  st.tuples(st.integers(0, 70)),
                  st.tuples(st.integers(0, 70), st.integers(1, 24)),
                  st.tuples(st.integers(0, 20), st.integers(1, 6), st.integers(1, 4)))
shapes_st = st.lists(shape, min_size=1, max_size=3)


def _numel(s):
    return int(np.prod(s)) if len(s) else 1


def _bits(rng, n):
    """Finite bf16 bit patterns of both signs: zeros, subnormals, normals."""
    mag = rng.integers(0, 0x7F80, size=n, dtype=np.uint32)
    sign = rng.integers(0, 2, size=n, dtype=np.uint32) << 15
    return (mag | sign).astype(np.uint16)


@settings(**SETTINGS)
@given(shapes=shapes_st, R=st.integers(1, 17), seed=st.integers(0, 2 ** 32 - 1))
def test_oracle_rs_matches_brute_force(shapes, R, seed):
    rng = np.random.default_rng(seed)
    grads = [[_bits(rng, _numel(s)) for s in shapes] for _ in range(R)]
    out = oracle.rs(shapes, R, grads)
    _, m, off, _ = oracle.layout(shapes, R)
    want = rs_brute(shapes, R, grads)
    for (r, p), shard in want.items():
        got = out[r][int(off[p]):int(off[p]) + int(m[p])].view(np.uint32)
        np.testing.assert_array_equal(got, np.asarray(shard, np.float32).view(np.uint32))


@settings(**SETTINGS)
@given(shapes=shapes_st, R=st.integers(1, 17), seed=st.integers(0, 2 ** 32 - 1))
def test_oracle_ag_matches_brute_force(shapes, R, seed):
    rng = np.random.default_rng(seed)
    _, _, _, S = oracle.layout(shapes, R)
    gathered = _bits(rng, max(1, R * S))
    got = oracle.ag(shapes, R, gathered)
    want = ag_brute(shapes, R, gathered)
    for p in range(len(shapes)):
        np.testing.assert_array_equal(got[p], np.asarray(want[p], np.uint16))


@settings(**SETTINGS)
@given(shapes=shapes_st, R=st.integers(1, 64), align=st.sampled_from([1, 2, 4, 8, 64]))
def test_plan_geometry_matches_oracle(shapes, R, align):
    s, m, off, S = api.tide_desc_geometry(shapes, R, align)
    os_, om, ooff, oS = oracle.layout(shapes, R, align)
    assert list(s) == list(os_) and list(m) == list(om) and list(off) == list(ooff) and S == oS


@settings(**SETTINGS)
@given(shapes=shapes_st, R=st.integers(1, 33), gmis=st.sampled_from([0, 2, 6, 14]),
       omis=st.sampled_from([0, 4, 8]))
def test_plan_tiles_partition_in_rank_outer_order(shapes, R, gmis, omis):
    _, _, _, S = api.tide_desc_geometry(shapes, R)
    g, o, ga, f = _fake_ptrs(shapes, R, S, grad_misalign=gmis, out_misalign=omis)
    blob, _ = api.tide_desc_build(shapes, R, g, o, ga, f, rs_tile=2048)
    _check_rs_tiles(shapes, R, blob, g)
    _, _, _, rs, ag = decode(blob)
    # rank outer, then param, then index
    keys = [(int(t["r"]), int(t["p"]), int(t["j0"])) for t in rs]
    assert keys == sorted(keys)
    # placement tiles: every valid row range of every (param, rank) exactly once
    _, m, off, _ = api.tide_desc_geometry(shapes, R)
    cover = {}
    for t in ag:
        p = int(t["p"])
        cover.setdefault(p, []).append((int(t["dst"]), int(t["dst"] + t["len"]), int(t["src"])))
    for p, shp in enumerate(shapes):
        n = _numel(shp)
        runs = sorted(cover.get(p, []))
        pos = 0
        for a, b, src in runs:
            assert a == pos
            r, i = divmod(a, int(m[p])) if int(m[p]) else (0, 0)
            assert src == r * S + int(off[p]) + i
            pos = b
        assert pos == n
