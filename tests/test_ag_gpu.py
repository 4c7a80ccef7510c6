"""GPU parity of the all-gather placement (tide_ag_place on the compute
units, tide_ag_place_sdma on the copy engines) against the CPU oracle: bit
for bit, always (it is a pure move)."""
import numpy as np
import pytest
import torch

import oracle
from shard_placement_amd import api, configs, harness, synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _wl(shapes, R, key=300, sigma=1.0):
    shapes = tuple(tuple(s) for s in shapes)
    return configs.Workload(key=key, name="adhoc", R=R, names=tuple("p%d" % i for i in range(len(shapes))),
                            shapes=shapes, sigma=sigma)


def _place(plan, engine):
    if engine == "cu":
        plan.ag()
    elif engine == "dma":
        plan.ag_dma()
    else:
        plan.ag_sdma(engine_only=(engine == "sdma"))


@pytest.mark.parametrize("engine", ["cu", "sdma", "sdma-any", "dma"])
def test_tiny_workload_bitwise(engine):
    w = configs.get(1)
    gu.say("tiny ag", engine)
    st = harness.setup(w, with_rs=False, gen_device="cpu")
    _place(st.plan, engine)
    torch.cuda.synchronize()
    gu.check_ag_full(st)


CASES = [
    (1, [(37, 16), (5,)]),
    (3, [(37, 16), (64, 64), (5,), ()]),
    (4, [(1001, 3), (0, 5), (2, 2, 2), (9,)]),
    (8, [(8192,), (1024, 64), (6, 40)]),
    (17, [(300, 16), (1,)]),
    (32, [(6, 5120), (5120,)]),
    (64, [(1001, 64), (128,), (3, 8)]),
]


@pytest.mark.parametrize("R,shapes", CASES, ids=[str(c[0]) for c in CASES])
@pytest.mark.parametrize("engine,tile", [("cu", 0), ("cu", 2048), ("sdma", 0), ("dma", 0)])
def test_ragged_shapes_bitwise(R, shapes, engine, tile):
    """tile: the placement tile size of the compute-unit path (0: default);
    the copy-engine paths have no tiles."""
    w = _wl(shapes, R, key=310 + R)
    gu.say("ragged ag", R, shapes, engine, tile)
    st = harness.setup(w, with_rs=False, ag_tile=tile)
    _place(st.plan, engine)
    torch.cuda.synchronize()
    gu.check_ag_full(st)


@pytest.mark.parametrize("gshift", [1, 2, 3, 4, 5, 7])
@pytest.mark.parametrize("engine", ["cu", "sdma", "dma"])
def test_unaligned_gathered_buffer(gshift, engine):
    """The gathered buffer starts gshift elements into an allocation, so
    slots and full tensors disagree in 16-byte (or 4-byte) phase."""
    shapes = [(333, 24), (5,), (64, 7), (2048, 8)]
    R = 4
    _, _, _, S = api.tide_desc_geometry(shapes, R)
    big = torch.empty(R * S + 8, dtype=torch.bfloat16, device="cuda")
    synth.bits_(big, 400 + gshift)
    gathered = big[gshift:gshift + R * S]
    n = synth.arena_numel(shapes)
    fa = torch.empty(n + 32, dtype=torch.bfloat16, device="cuda")
    fa.view(torch.int16).fill_(-1)
    full = synth.views(fa[16:16 + n], shapes)
    plan = api.Plan(shapes, R, gathered=gathered, full=full)
    gu.say("unaligned ag", gshift, engine)
    _place(plan, engine)
    torch.cuda.synchronize()
    want = [np.full(gu.numel(s), gu.SENT16, np.uint16) for s in shapes]
    oracle.ag(shapes, R, gu.bits16(gathered), out=want)
    for p in range(len(shapes)):
        gu.assert_bits_equal(gu.bits16(full[p]), want[p], "full[%d]" % p)
    f = gu.bits16(fa)
    assert np.all(f[:16] == gu.SENT16) and np.all(f[16 + n:] == gu.SENT16)


@pytest.mark.parametrize("seed", range(12))
def test_fuzz_random_placements(seed):
    """Seeded random problems and gathered-buffer offsets, both engines,
    compared with the oracle bit for bit."""
    rng = np.random.default_rng(2000 + seed)
    R = int(rng.choice([1, 2, 3, 5, 8, 16, 33, 64]))
    P = int(rng.integers(1, 7))
    shapes = []
    for _ in range(P):
        nd = int(rng.integers(0, 4))
        dims = [int(rng.integers(0, 300))] + [int(rng.integers(1, 40)) for _ in range(max(0, nd - 1))]
        shapes.append(tuple(dims[:nd]))
    align = int(rng.choice([1, 2, 8]))
    gshift = int(rng.integers(0, 8))
    tile = int(rng.choice([0, 2048]))
    _, _, _, S = api.tide_desc_geometry(shapes, R, align)
    big = torch.empty(R * S + 16, dtype=torch.bfloat16, device="cuda")
    synth.bits_(big, 600 + seed)
    gathered = big[gshift:gshift + R * S]
    n = synth.arena_numel(shapes)
    fa = torch.empty(n + 32, dtype=torch.bfloat16, device="cuda")
    full = synth.views(fa[16:16 + n], shapes)
    gu.say("fuzz ag", seed, R, shapes, align, gshift, tile)
    want = [np.full(gu.numel(s), gu.SENT16, np.uint16) for s in shapes]
    oracle.ag(shapes, R, gu.bits16(gathered), align=align, out=want)
    for engine in ("cu", "sdma", "dma"):
        fa.view(torch.int16).fill_(-1)
        plan = api.Plan(shapes, R, gathered=gathered, full=full, align=align, ag_tile=tile)
        _place(plan, engine)
        torch.cuda.synchronize()
        for p in range(len(shapes)):
            gu.assert_bits_equal(gu.bits16(full[p]), want[p], "%s full[%d]" % (engine, p))
        f = gu.bits16(fa)
        assert np.all(f[:16] == gu.SENT16) and np.all(f[16 + n:] == gu.SENT16)


@pytest.mark.parametrize("engine", ["cu", "dma"])
def test_largest_rank_count(engine):
    """R = 4096, the library's limit: a gathered buffer of 4096 slots, ragged
    and empty ranks, placed in full and compared with the oracle."""
    R = 4096
    w = _wl([(R + 1, 2), (2 * R - 1,), ()], R, key=340)
    gu.say("ag R", R, engine)
    st = harness.setup(w, with_rs=False)
    _place(st.plan, engine)
    torch.cuda.synchronize()
    gu.check_ag_full(st)


def test_placement_of_rs_output_is_full_fold():
    """AG(bf16(RS shards)) equals bf16 of the full fold, all on the device."""
    shapes = [(1001, 24), (5,), (64, 64)]
    R = 8
    w = _wl(shapes, R, key=330)
    st = harness.setup(w, with_ag=False)
    st.plan.rs()
    _, _, _, S = api.tide_desc_geometry(shapes, R)
    gathered = torch.cat([o.to(torch.bfloat16) for o in st.out])
    n = synth.arena_numel(shapes)
    fa = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    full = synth.views(fa, shapes)
    plan = api.Plan(shapes, R, gathered=gathered, full=full)
    plan.ag()
    torch.cuda.synchronize()
    for p, shp in enumerate(shapes):
        folds = oracle.fold_points(np.stack([gu.bits16(st.grads[q][p]) for q in range(R)], axis=1))
        want = gu.bits16(torch.from_numpy(folds).to(torch.bfloat16))
        gu.assert_bits_equal(gu.bits16(full[p]), want, "param %d" % p)


def test_random_bit_patterns_round_trip():
    """Slots cut from random bit patterns (NaN payloads, -0, inf) with
    torch.chunk come back bit for bit; padding sentinels never appear."""
    shapes = [(37, 16), (64, 64), (5,), (1001, 3)]
    R = 4
    fulls = []
    for p, s in enumerate(shapes):
        t = torch.empty(s, dtype=torch.bfloat16)
        synth.bits_(t, 500 + p)
        t.view(torch.int16)[t.view(torch.int16) == -1] = 0x7FC1
        fulls.append(t)
    slots = []
    for r in range(R):
        pieces = []
        for t in fulls:
            d0 = t.shape[0]
            sr = -(-d0 // R)
            ch = list(torch.chunk(t, R, dim=0))
            c = ch[r] if r < len(ch) else t[0:0]
            pad = torch.full((sr - c.shape[0],) + tuple(t.shape[1:]), -1, dtype=torch.int16)
            pieces.append(torch.cat([c.view(torch.int16), pad]).reshape(-1))
        slots.append(torch.cat(pieces))
    gathered = torch.cat(slots).view(torch.bfloat16).to("cuda")
    n = synth.arena_numel(shapes)
    fa = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    full = synth.views(fa, shapes)
    for engine in ("cu", "sdma", "dma"):
        fa.view(torch.int16).fill_(0x1234)
        plan = api.Plan(shapes, R, gathered=gathered, full=full)
        _place(plan, engine)
        torch.cuda.synchronize()
        for p, t in enumerate(fulls):
            assert torch.equal(full[p].cpu().view(torch.int16), t.view(torch.int16)), (engine, p)


@pytest.mark.parametrize("n_streams", [1, 3, 8])
def test_copy_engine_placement_over_streams(n_streams):
    shapes = [(37, 16), (64, 64), (5,), (1001, 3), (8, 512)]
    R = 4
    w = _wl(shapes, R, key=340)
    st = harness.setup(w, with_rs=False)
    streams = [torch.cuda.Stream() for _ in range(n_streams)]
    ev = torch.cuda.Event()
    ev.record()
    for s in streams:
        s.wait_event(ev)
    st.plan.ag_sdma_streams(streams)
    torch.cuda.synchronize()
    gu.check_ag_full(st)


@pytest.mark.big
@pytest.mark.parametrize("key", [2, 3, 4, 5])
def test_full_size_placement(key):
    w = configs.get(key)
    gu.say("full-size ag", w.name)
    st = harness.setup(w, with_rs=False, guard=64)
    for engine in ("cu", "sdma", "dma"):
        st.full_arena.view(torch.int16).fill_(-1)
        gu.say("full-size ag", w.name, engine)
        _place(st.plan, engine)
        torch.cuda.synchronize()
        gu.say("oracle ag compare", w.name, engine)
        gu.check_ag_full(st)
    st.free()
    torch.cuda.empty_cache()
