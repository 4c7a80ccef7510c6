"""GPU parity of the fused reduce-scatter (tide_rs_bf16_to_fp32) against the
CPU oracle: bit for bit in fixed rank order, on small and ragged problems
in full and on the full-size workloads on sampled elements, plus properties
that hold at any size (summation bound for every element, +0.0 padding,
untouched guard bands, determinism)."""
import numpy as np
import pytest
import torch

from shard_placement_amd import api, configs, harness, synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def _wl(shapes, R, key=90, sigma=1.0, name="adhoc"):
    shapes = tuple(tuple(s) for s in shapes)
    return configs.Workload(key=key, name=name, R=R, names=tuple("p%d" % i for i in range(len(shapes))),
                            shapes=shapes, sigma=sigma)


def _run(st, order="fixed", max_wg=0):
    st.plan.rs(order=order, max_workgroups=max_wg)
    torch.cuda.synchronize()


@pytest.mark.parametrize("order", ["fixed", "tree"])
@pytest.mark.parametrize("flags", [0, 1, 2, 3])
def test_tiny_workload_bitwise(flags, order):
    w = configs.get(1)
    gu.say("tiny rs flags", flags, order)
    st = harness.setup(w, with_ag=False, gen_device="cpu", flags=flags)
    _run(st, order)
    gu.check_rs_full(st, order)


RANDOM_CASES = [
    (1, [(37, 16), (5,)]),
    (2, [(64, 64), (3,), ()]),
    (3, [(37, 16), (64, 64), (5,)]),
    (4, [(1001, 3), (0, 5), (2, 2, 2), (9,)]),
    (5, [(130, 24), (7, 1)]),
    (7, [(1, 1), (100, 40)]),
    (8, [(8192,), (1024, 64), (6, 40)]),
    (9, [(77, 33)]),
    (16, [(512, 48), (1,), (17, 8)]),
    (17, [(300, 16)]),
    (32, [(6, 5120), (5120,)]),
    (33, [(65, 32)]),
    (64, [(1001, 64), (128,), (3, 8)]),
]


@pytest.mark.parametrize("R,shapes", RANDOM_CASES, ids=[str(c[0]) for c in RANDOM_CASES])
@pytest.mark.parametrize("tile", [0, 2048])
@pytest.mark.parametrize("order", ["fixed", "tree"])
def test_ragged_shapes_bitwise(R, shapes, tile, order):
    w = _wl(shapes, R, key=100 + R)
    gu.say("ragged rs R", R, shapes, "tile", tile, order)
    st = harness.setup(w, with_ag=False, rs_tile=tile)
    _run(st, order)
    gu.check_rs_full(st, order)


SEPARATE_CASES = [(R, shapes, reuse) for R, shapes in RANDOM_CASES[::3] for reuse in (False, True)
                  if R >= 2 or not reuse]  # Slot-Reuse needs R >= 2


@pytest.mark.parametrize("R,shapes,slot_reuse", SEPARATE_CASES,
                         ids=["%d-%s" % (c[0], "reuse" if c[2] else "own") for c in SEPARATE_CASES])
def test_rank_arenas_allocated_separately(R, shapes, slot_reuse):
    """Every rank's gradient and output arena in an allocation of its own
    (the packed rows are the default): same bits."""
    w = _wl(shapes, R, key=100 + R)
    gu.say("separate arenas R", R, shapes, slot_reuse)
    st = harness.setup(w, with_ag=False, rank_layout="separate", slot_reuse=slot_reuse)
    _run(st)
    gu.check_rs_full(st, "fixed")


@pytest.mark.parametrize("R", [3, 5, 6, 7, 11, 13, 100, 129, 300])
def test_tree_order_odd_rank_counts(R):
    """Tree order for rank counts that are not powers of two (odd elements
    carried up at several levels), including R > 127 (the deeper stack)."""
    w = _wl([(R * 3 + 1, 24), (5,)], R, key=120 + R % 50)
    gu.say("tree R", R)
    st = harness.setup(w, with_ag=False, rs_tile=2048)
    _run(st, "tree")
    gu.check_rs_full(st, "tree")


@pytest.mark.parametrize("order", ["fixed", "tree"])
def test_largest_rank_count(order):
    """R = 4096, the library's limit (the tree's deepest stack): ragged and
    all-padding shards, whole arenas against the oracle."""
    R = 4096
    w = _wl([(R + 1, 2), (2 * R - 1,), ()], R, key=140)
    gu.say("R", R, order)
    st = harness.setup(w, with_ag=False)
    _run(st, order)
    gu.check_rs_full(st, order)


def _random_problem(seed):
    rng = np.random.default_rng(1000 + seed)
    R = int(rng.choice([1, 2, 3, 5, 8, 12, 16, 23, 32, 64, 70]))
    P = int(rng.integers(1, 7))
    shapes = []
    for _ in range(P):
        nd = int(rng.integers(0, 4))
        dims = [int(rng.integers(0, 200))] + [int(rng.integers(1, 40)) for _ in range(max(0, nd - 1))]
        shapes.append(tuple(dims[:nd]))
    align = int(rng.choice([1, 1, 2, 4, 8]))
    tile = int(rng.choice([0, 2048, 4096]))
    launch = int(rng.choice([0, -1, 1]))
    order = str(rng.choice(["fixed", "tree"]))
    return R, shapes, align, tile, launch, order


@pytest.mark.parametrize("seed", range(16))
def test_fuzz_random_problems(seed):
    """Seeded random problems (rank counts 1-70, 0-d/empty/ragged shapes,
    offset alignment, tile and launch sizes, both orders), compared with the
    oracle over whole arenas, gaps and guard bands included."""
    R, shapes, align, tile, launch, order = _random_problem(seed)
    gu.say("fuzz", seed, R, shapes, align, tile, launch, order)
    w = _wl(shapes, R, key=200 + seed)
    st = harness.setup(w, with_ag=False, align=align, rs_tile=tile, launch_mib=launch)
    _run(st, order)
    gu.check_rs_full(st, order)


@pytest.mark.parametrize("R", [8, 12, 16, 20, 24, 40, 64, 72])
@pytest.mark.parametrize("launch", ["reserving", "one"])
def test_rank_batching_variants_bitwise(R, launch):
    """Every rank-batching form of the fixed-order kernel against the oracle:
    R a multiple of 8 loads 4 ranks per batch in launches that reserve LDS
    (a small layer's default plan: at most 2 workgroups per CU) and 2 ranks
    per batch otherwise (one unrounded launch); other R load 8 per batch, the
    last batch re-reading a rank.  Ragged and all-padding shards included."""
    w = _wl([(2 * R + 3, 40), (R - 1, 8), (4096, 16)], R, key=260 + R, sigma=1e-3)
    gu.say("batching R", R, launch)
    st = harness.setup(w, with_ag=False, launch_mib=-1 if launch == "one" else 0)
    reserving = st.plan.info.rs_lds_bytes > 8192
    assert reserving == (launch == "reserving"), st.plan.info.rs_lds_bytes
    _run(st)
    gu.check_rs_full(st)


@pytest.mark.parametrize("R", [8, 16])
def test_skewed_launches_bitwise(R):
    """Launches of 2048 tiles or more at R a multiple of 8 (2 ranks per
    batch) run the skewed XCD mapping, in which the odd XCDs' spare
    workgroups take no tile: at R = 8 one skewed launch of 2425 tiles, at
    R = 16 (an explicit 160 MiB: the default makes one-round launches of
    1792) two of 2275 and a plain one of 299.  Whole arenas against the
    oracle; the per-tile trace stamps every tile exactly once with the same
    bits; a capped grid (no skew) gives the same bits."""
    w = _wl([(300 * R + 3, 2048), (R - 1, 8), (333, 40)], R, key=280 + R, sigma=1e-3)
    gu.say("skewed launches R", R)
    st = harness.setup(w, with_ag=False, launch_mib=160 if R == 16 else 0)
    info = st.plan.info
    assert info.rs_lds_bytes == 8192 and info.rs_launch_tiles >= 2048
    _run(st)
    gu.check_rs_full(st)
    ref = [o.clone() for o in st.out]

    def same():
        return all(torch.equal(a.view(torch.int32), b.view(torch.int32)) for a, b in zip(st.out, ref))

    for o in st.out:
        o.view(torch.int32).fill_(-1)
    census, stamps = st.plan.rs_trace()
    torch.cuda.synchronize()
    assert same()
    c, s = census.cpu().numpy(), stamps.cpu().numpy()
    assert c.size == info.rs_tiles and (c >= 0).all()
    assert (s[:, 0] > 0).all() and (s[:, 1] >= s[:, 0]).all()
    for o in st.out:
        o.view(torch.int32).fill_(-1)
    _run(st, max_wg=1000)
    assert same()


@pytest.mark.parametrize("align", [4, 8, 64])
def test_aligned_offsets_leave_gaps(align):
    w = _wl([(37, 16), (5,), (3, 3), (40, 8)], 4, key=131)
    gu.say("align", align)
    st = harness.setup(w, with_ag=False, align=align)
    _run(st)
    gu.check_rs_full(st)


def _custom(shapes, R, phases, out_shift=0, key=140):
    """Gradients as views at element offset phases[q] of a larger tensor, so
    ranks have different 16-byte phases (the element-wise path) or the same
    odd phase (scalar heads and tails around a vector body)."""
    w = _wl(shapes, R, key=key)
    n = synth.arena_numel(shapes)
    st = harness.Setup(w=w, device=torch.device("cuda"), arenas=[], grads=[], out=[], out_alloc=[])
    for q in range(R):
        big = torch.empty(n + 16, dtype=torch.bfloat16, device="cuda")
        synth.fill_normal_(big, 1000 * key + q, 1.0)
        a = big[phases[q]:phases[q] + n]
        st.arenas.append(big)
        st.grads.append(synth.views(a, shapes))
    _, _, _, S = api.tide_desc_geometry(shapes, R)
    st.S, st.guard = S, 8
    for r in range(R):
        buf = torch.empty(S + 16 + out_shift, dtype=torch.float32, device="cuda")
        buf.view(torch.int32).fill_(-1)
        st.out_alloc.append(buf)
        st.out.append(buf[8 + out_shift:8 + out_shift + S])
    st.plan = api.Plan(shapes, R, grads=st.grads, out=st.out)
    return st


@pytest.mark.parametrize("phases", [[0, 1, 2, 3], [3, 3, 3, 3], [5, 5, 5, 5], [0, 0, 4, 0]])
@pytest.mark.parametrize("out_shift", [0, 1, 2, 3])
def test_unaligned_sources_and_outputs(phases, out_shift):
    shapes = [(333, 24), (5,), (64, 7)]
    gu.say("unaligned", phases, out_shift)
    st = _custom(shapes, 4, phases, out_shift)
    _run(st)
    w = st.w
    want = [np.full(st.S, np.nan, np.float32) for _ in range(4)]
    for a in want:
        a.view(np.uint32)[:] = gu.NAN32
    import oracle
    oracle.rs(w.shapes, 4, gu.grads_np(st), out=want)
    for r in range(4):
        gu.assert_bits_equal(gu.bits32(st.out[r]), want[r].view(np.uint32), "rank %d" % r)
        a = gu.bits32(st.out_alloc[r])
        assert np.all(a[:8 + out_shift] == gu.NAN32) and np.all(a[8 + out_shift + st.S:] == gu.NAN32)


def test_special_values():
    """±0, subnormals, ±inf, NaN, bf16 max: identical to the oracle (a NaN
    matches any NaN)."""
    R = 5
    shapes = [(64, 40)]
    w = _wl(shapes, R, key=150)
    gu.say("special values")
    st = harness.setup(w, with_ag=False)
    vals = list(synth.SPECIAL_BF16.values())
    gen = torch.Generator(device="cpu").manual_seed(5)
    for q in range(R):
        pick = torch.randint(0, len(vals), (64 * 40,), generator=gen)
        bits = torch.tensor(vals, dtype=torch.int32)[pick].to(torch.int16)
        st.arenas[q].view(torch.int16).copy_(bits.to("cuda"))
    _run(st)
    gu.check_rs_full(st, nan_as_class=True)


@pytest.mark.parametrize("max_wg", [1, 3, 64, 1000])
@pytest.mark.parametrize("order", ["fixed", "tree"])
def test_capped_grid_same_bits(max_wg, order):
    w = _wl([(1001, 24), (5,), (64, 64)], 8, key=160)
    gu.say("max_wg", max_wg, order)
    st = harness.setup(w, with_ag=False, rs_tile=2048)
    _run(st, order, max_wg=max_wg)
    gu.check_rs_full(st, order)


@pytest.mark.parametrize("chunk", [1, 7, 64])
def test_chunked_launches_same_bits(chunk):
    """The reduce-scatter cut into tile ranges gives the same bits."""
    w = _wl([(1001, 24), (5,), (64, 64)], 8, key=165)
    st = harness.setup(w, with_ag=False, rs_tile=2048)
    n = st.plan.rs_chunked(chunk)
    torch.cuda.synchronize()
    assert n == -(-int(st.plan.info.rs_tiles) // chunk)
    gu.check_rs_full(st)


@pytest.mark.parametrize("R", [1, 3, 8, 64])
def test_one_call_per_rank_same_bits(R):
    """Each output rank's shards as one tile-range call (what one GPU of a
    real job would run), in any order of ranks: the same bits."""
    w = _wl([(1001, 24), (5,), (64, 64), ()], R, key=180 + R)
    st = harness.setup(w, with_ag=False)
    st.plan.rs()
    torch.cuda.synchronize()
    ref = [o.clone() for o in st.out]
    for o in st.out:
        o.view(torch.int32).fill_(-1)
    gu.say("per-rank calls", R)
    for r in reversed(range(R)):
        st.plan.rs_rank(r)
    torch.cuda.synchronize()
    for r in range(R):
        assert torch.equal(st.out[r].view(torch.int32), ref[r].view(torch.int32)), r
    gu.check_rs_full(st)


@pytest.mark.parametrize("launch_mib", [-1, 1, 4])
def test_launch_size_same_bits(launch_mib):
    """A call cut into many launches (or made in one) gives the same bits;
    so does the placement."""
    w = _wl([(1001, 96), (5,), (640, 64)], 8, key=166)
    st = harness.setup(w, rs_tile=2048, ag_tile=2048, launch_mib=launch_mib)
    assert st.plan.info.rs_launch_tiles >= 1
    st.plan.rs()
    st.plan.ag()
    torch.cuda.synchronize()
    gu.check_rs_full(st)
    gu.check_ag_full(st)


@pytest.mark.parametrize("order", ["fixed", "tree"])
@pytest.mark.parametrize("max_wg", [0, 3])
def test_lds_reserving_launches_same_bits(order, max_wg):
    """At R = 64 the default launches hold 512 tiles and each workgroup
    holds 64 KB of LDS (56 KB of it requested at launch, never touched).
    The bits are the oracle's and those of one launch without the
    reservation: 2241 tiles make four full launches and one of 193; with a
    capped grid each workgroup strides over tiles."""
    w = _wl([(1001, 64), (128,), (3, 8), (8192, 512)], 64, key=171, sigma=1e-3)
    gu.say("lds-reserving rs", order, "max_wg", max_wg)
    st = harness.setup(w, with_ag=False)
    info = st.plan.info
    assert info.rs_lds_bytes == 64 * 1024
    assert (info.rs_tiles, info.rs_launch_tiles) == (2241, 512)
    _run(st, order, max_wg)
    gu.check_rs_full(st, order)
    got = [o.clone() for o in st.out]
    one = api.Plan(w.shapes, w.R, grads=st.grads, out=st.out, launch_mib=-1)
    assert one.info.rs_lds_bytes == 8192
    for o in st.out:
        o.view(torch.int32).fill_(-1)
    one.rs(order=order)
    torch.cuda.synchronize()
    for a, b in zip(got, st.out):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_hip_graph_replays_match_eager():
    """One step (placement + reduce-scatter, several launches each) captured
    in a HIP graph: every replay, with eager work and synchronisation in
    between, gives the eager bits (the library records no memset and no
    allocation)."""
    w = _wl([(1001, 96), (5,), (640, 64)], 8, key=167)
    st = harness.setup(w, rs_tile=2048, ag_tile=2048, launch_mib=1)
    st.plan.ag()
    st.plan.rs()
    torch.cuda.synchronize()
    want_rs = [o.clone() for o in st.out]
    want_ag = st.full_arena.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        st.plan.ag()
        st.plan.rs()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in st.out:
            o.view(torch.int32).fill_(-1)
        st.full_arena.view(torch.int16).fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(want_rs, st.out):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), rep
        assert torch.equal(want_ag.view(torch.int16), st.full_arena.view(torch.int16)), rep
    gu.check_rs_full(st)


def test_cu_census_same_bits_and_counts():
    """The census call gives the same shards and names a compute unit for
    every tile; confined to a CU-masked stream it names at most that many."""
    w = _wl([(4096, 256), (7,)], 8, key=168, sigma=1e-3)
    st = harness.setup(w, with_ag=False)
    st.plan.rs()
    torch.cuda.synchronize()
    ref = [o.clone() for o in st.out]
    for o in st.out:
        o.view(torch.int32).fill_(-1)
    census = st.plan.rs_census()
    torch.cuda.synchronize()
    for a, b in zip(ref, st.out):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    c = census.cpu()
    assert int((c < 0).sum()) == 0
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    assert 1 <= len(set(c.tolist())) <= ncu
    s = api.tide_stream_create_cu_limited(8)
    try:
        c8 = st.plan.rs_census(stream=s)
        torch.cuda.synchronize()
        assert 1 <= len(set(c8.cpu().tolist())) <= 8
    finally:
        api.tide_stream_destroy(s)


@pytest.mark.parametrize("R,shapes,launch_mib", [(8, [(4096, 256), (7,), (130, 24)], 8),
                                                 (64, [(4096, 1024), (1001, 64), (128,)], 8),
                                                 (8, [(4096, 3072), (7,), (130, 24)], 80)],
                         ids=["8", "64", "8-skewed"])
def test_launches_dealt_over_streams_same_bits(R, shapes, launch_mib):
    """tide_rs_bf16_to_fp32_streams: the launches over 1, 2 or 3 CU-masked
    streams (hardware queues of their own) give the oracle's bits, also when
    the launches are skewed (2048 tiles each at R = 8 with 80 MiB)."""
    w = _wl(shapes, R, key=175 + R, sigma=1e-3)
    st = harness.setup(w, with_ag=False, guard=64, launch_mib=launch_mib)
    assert -(-int(st.plan.info.rs_tiles) // int(st.plan.info.rs_launch_tiles)) >= 3
    if launch_mib == 80:
        assert st.plan.info.rs_launch_tiles == 2048
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    extra = [api.tide_stream_create_cu_limited(ncu) for _ in range(3)]
    try:
        for k in (0, 1, 2):
            for o in st.out_alloc:
                o.view(torch.int32).fill_(-1)
            torch.cuda.synchronize()
            gu.say("rs over", k + 1, "streams, R", R)
            st.plan.rs_streams(extra[1:1 + k], stream=extra[0])
            torch.cuda.synchronize()
            gu.check_rs_full(st)
        # dealing launches onto the null stream is refused
        with pytest.raises(api.TideError):
            st.plan.rs_streams(extra[:1])
    finally:
        torch.cuda.synchronize()
        for s in extra:
            api.tide_stream_destroy(s)


def test_cu_limited_stream_bounds():
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    with pytest.raises(api.TideError):
        api.tide_stream_create_cu_limited(ncu + 1)
    s = api.tide_stream_create_cu_limited(ncu)
    api.tide_stream_destroy(s)


def test_deterministic_repeat():
    w = _wl([(4096, 256), (7,)], 16, key=170, sigma=1e-3)
    st = harness.setup(w, with_ag=False)
    _run(st)
    first = [o.clone() for o in st.out]
    for o in st.out:
        o.view(torch.int32).fill_(-1)
    _run(st)
    for a, b in zip(first, st.out):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("R", [2, 3, 8, 17, 64])
def test_identical_ranks_alias_one_tensor(R):
    """Every rank passes the same tensor: the result is R*g exactly."""
    shapes = [(100, 24), (3,)]
    w = _wl(shapes, R, key=180)
    n = synth.arena_numel(shapes)
    a = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    synth.fill_normal_(a, 181, 1.0)
    g = synth.views(a, shapes)
    _, m, off, S = api.tide_desc_geometry(shapes, R)
    out = [torch.full((S,), float("nan"), device="cuda") for _ in range(R)]
    plan = api.Plan(shapes, R, grads=[g] * R, out=out)
    plan.rs()
    torch.cuda.synchronize()
    for p, shp in enumerate(shapes):
        flat = torch.cat([out[r][int(off[p]):int(off[p]) + int(m[p])] for r in range(R)]).cpu()
        nn = gu.numel(shp)
        want = (g[p].reshape(-1).double() * R).float().cpu()
        assert torch.equal(flat[:nn].view(torch.int32), want.view(torch.int32))
        assert torch.all(flat[nn:].view(torch.int32) == 0)


@pytest.mark.parametrize("R", [2, 4, 8])
def test_slot_reuse_same_bits_no_allocation(R):
    w = _wl([(1001, 40), (5,), (64, 64)], R, key=190, sigma=1e-3)
    gu.say("slot reuse R", R)
    ref = harness.setup(w, with_ag=False, slot_reuse=False)
    _run(ref)
    st = harness.setup(w, with_ag=True, slot_reuse=True)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    st.plan.ag()   # the gathered buffer is used first ...
    st.plan.rs()   # ... then vacated and reused for the fp32 shards
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    for r in range(R):
        assert torch.equal(st.out[r].view(torch.int32), ref.out[r].view(torch.int32))
        gu.check_out_guards(st, r)
        assert st.out[r].data_ptr() == st.vacated[r].data_ptr()


# ------------------------------------------------------------ full size
def _free_gb():
    free, _ = torch.cuda.mem_get_info()
    return free / 1e9


def _need_gb(w, slot_reuse):
    n = w.numel()
    _, _, _, S = api.tide_desc_geometry(w.shapes, w.R)
    g = w.R * n * 2
    outs = w.R * 2 * S * w.R if slot_reuse else w.R * 4 * S
    return (g + outs + 2 * n + (0 if slot_reuse else 2 * w.R * S)) / 1e9 + 2


@pytest.mark.big
@pytest.mark.parametrize("key", [2, 3, 4, 5])
def test_full_size_workload(key):
    w = configs.get(key)
    need = _need_gb(w, w.slot_reuse)
    if _free_gb() < need:
        pytest.skip("needs %.0f GB of free HBM" % need)
    gu.say("full-size", w.name, "R", w.R, "need GB", round(need))
    st = harness.setup(w, guard=64)
    torch.cuda.synchronize()
    st.plan.ag()
    st.plan.rs()
    torch.cuda.synchronize()
    gu.say("sampled oracle check", w.name)
    n = gu.check_rs_sampled(st)
    assert n > 0
    gu.say("bound check over every element", w.name)
    gu.check_rs_bound_all(st)
    for r in range(w.R):
        gu.check_out_guards(st, r)
    # every element of every shard against the oracle, bit for bit (fixed
    # order), streamed param by param in blocks of flat indices
    assert gu.check_rs_whole(st) == w.numel()
    # tree order: sampled bit-exact vs the oracle's tree, and the tolerance
    # 1e-6 * sum|g| (plus the pairwise bound) for every element
    gu.say("tree order", w.name)
    st.plan.rs(order="tree")
    torch.cuda.synchronize()
    gu.check_rs_sampled(st, order="tree", per_shard=32, edge=8, seed=1)
    gu.check_rs_bound_all(st, order="tree")
    assert gu.check_rs_whole(st, order="tree") == w.numel()
    st.plan.rs()
    torch.cuda.synchronize()
    # determinism at full size
    snap = [o.clone() for o in st.out[:2]]
    st.plan.rs()
    torch.cuda.synchronize()
    for a, b in zip(snap, st.out[:2]):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    st.free()
    del snap
    torch.cuda.empty_cache()


@pytest.mark.big
def test_offsets_beyond_2_pow_31():
    """A ragged 2-D param of 2^31 + 98,304 elements (byte offsets past 4 GiB
    in the gradients, past 2^31 elements in the gathered buffer) at R = 3:
    rank 2 keeps 21,845 valid rows and 2 padding rows.  Elements straddling
    flat index 2^31 and every shard's edges against the oracle, every
    element within the summation bound, the placement in full."""
    w = _wl([(65539, 32768), (96,)], 3, key=990, sigma=1e-3, name="beyond-2^31")
    need = _need_gb(w, False)
    if _free_gb() < need:
        pytest.skip("needs %.0f GB of free HBM" % need)
    gu.say("offsets beyond 2^31: need GB", round(need))
    st = harness.setup(w, guard=64)
    torch.cuda.synchronize()
    st.plan.ag()
    st.plan.rs()
    torch.cuda.synchronize()
    n0 = 65539 * 32768
    pts = np.concatenate([np.arange(2 ** 31 - 64, 2 ** 31 + 64), np.arange(n0 - 64, n0),
                          np.arange(2 ** 30 - 8, 2 ** 30 + 8)])
    assert gu.check_rs_points(st, 0, pts) == pts.size
    gu.check_rs_sampled(st)
    gu.check_rs_bound_all(st)
    for r in range(w.R):
        gu.check_out_guards(st, r)
    gu.say("offsets beyond 2^31: placement")
    gu.check_ag_full(st)
    st.plan.rs(order="tree")
    torch.cuda.synchronize()
    gu.check_rs_points(st, 0, pts, order="tree")
    st.free()
    torch.cuda.empty_cache()
