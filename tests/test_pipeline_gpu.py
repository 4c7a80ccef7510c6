"""GPU parity of the two-phase pipeline emulation: phase 1 reduces chunks of
tiles into staging chunks, phase 2 moves them into the shard arenas; run on
two streams through a ring of staging chunks.  Bit for bit against the
oracle and against the in-place kernel."""
import pytest
import torch

from shard_placement_amd import api, configs, harness, pipeline
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _wl(shapes, R, key, sigma=1.0):
    shapes = tuple(tuple(s) for s in shapes)
    return configs.Workload(key=key, name="adhoc", R=R, names=tuple("p%d" % i for i in range(len(shapes))),
                            shapes=shapes, sigma=sigma)


CASES = [
    (1, [(37, 16), (5,)]),
    (3, [(37, 16), (64, 64), (5,), ()]),
    (4, [(1001, 3), (0, 5), (2, 2, 2), (9,)]),
    (8, [(8192,), (1024, 64), (6, 40)]),
    (17, [(300, 16)]),
    (32, [(6, 5120), (5120,)]),
    (64, [(1001, 64), (128,), (3, 8)]),
]


@pytest.mark.parametrize("R,shapes", CASES, ids=[str(c[0]) for c in CASES])
def test_phases_in_sequence_bitwise(R, shapes):
    """Phase 1 over all tiles into one staging chunk, then phase 2."""
    w = _wl(shapes, R, 900 + R)
    st = harness.setup(w, with_ag=False)
    n, T = int(st.plan.info.rs_tiles), int(st.plan.info.rs_tile_elems)
    stage = torch.empty(max(1, n) * T, dtype=torch.float32, device="cuda")
    gu.say("pipeline phases", R, shapes)
    api.tide_rs_tiles_to_stage(st.plan.blob, st.plan.d_blob, 0, n, stage)
    api.tide_rs_stage_to_shards(st.plan.blob, st.plan.d_blob, 0, n, stage)
    torch.cuda.synchronize()
    gu.check_rs_full(st)


@pytest.mark.parametrize("R", [8, 12, 16, 64])
@pytest.mark.parametrize("launch", ["reserving", "one"])
def test_phase1_rank_batching_variants_bitwise(R, launch):
    """Phase 1 in every rank-batching form (4 ranks per batch in launches
    that reserve LDS, 2 otherwise, 8 with a re-read rank when R is not a
    multiple of 8), then phase 2: the oracle's bits."""
    w = _wl([(2 * R + 3, 40), (R - 1, 8), (4096, 16)], R, 960 + R, sigma=1e-3)
    st = harness.setup(w, with_ag=False, launch_mib=-1 if launch == "one" else 0)
    assert (st.plan.info.rs_lds_bytes > 8192) == (launch == "reserving")
    n, T = int(st.plan.info.rs_tiles), int(st.plan.info.rs_tile_elems)
    stage = torch.empty(max(1, n) * T, dtype=torch.float32, device="cuda")
    gu.say("pipeline phase-1 batching", R, launch)
    api.tide_rs_tiles_to_stage(st.plan.blob, st.plan.d_blob, 0, n, stage)
    api.tide_rs_stage_to_shards(st.plan.blob, st.plan.d_blob, 0, n, stage)
    torch.cuda.synchronize()
    gu.check_rs_full(st)


@pytest.mark.parametrize("chunk,depth,phase2,cus", [(1, 1, "cu", 0), (7, 2, "cu", 0), (64, 3, "cu", 0),
                                                    (10 ** 6, 1, "cu", 0), (7, 2, "cu", 8),
                                                    (1, 2, "sdma", 0), (7, 2, "sdma", 0),
                                                    (64, 1, "sdma", 0)])
def test_two_streams_ring_bitwise(chunk, depth, phase2, cus):
    shapes = [(4096, 96), (96,), (1001, 24), (5,)]
    R = 8
    w = _wl(shapes, R, 950, sigma=1e-3)
    st = harness.setup(w, with_ag=False)
    st.plan.rs()
    torch.cuda.synchronize()
    ref = [o.clone() for o in st.out]
    for o in st.out:
        o.view(torch.int32).fill_(-1)
    tp = pipeline.TwoPhase(st.plan, chunk, depth, phase2, cus)
    try:
        gu.say("pipeline ring", chunk, depth, phase2, cus, tp.chunks())
        tp.run()
        torch.cuda.synchronize()
    finally:
        tp.close()
    for r in range(R):
        assert torch.equal(st.out[r].view(torch.int32), ref[r].view(torch.int32)), r
    gu.check_out_guards(st, 0)


@pytest.mark.big
@pytest.mark.parametrize("phase2", ["cu", "sdma"])
def test_full_size_pipeline_matches_in_place(phase2):
    w = configs.get(2)
    st = harness.setup(w, with_ag=False, guard=0)
    st.plan.rs()
    torch.cuda.synchronize()
    ref = [o.clone() for o in st.out]
    for o in st.out:
        o.view(torch.int32).fill_(-1)
    tp = pipeline.TwoPhase(st.plan, int(st.plan.info.rs_launch_tiles), 2, phase2)
    try:
        gu.say("full-size pipeline", w.name, phase2, tp.chunks())
        tp.run()
        torch.cuda.synchronize()
    finally:
        tp.close()
    for r in range(w.R):
        assert torch.equal(st.out[r].view(torch.int32), ref[r].view(torch.int32)), r
    del ref, tp
    st.free()
    torch.cuda.empty_cache()


def test_object_reused_across_calls_and_streams():
    """One pipeline object, two runs with a clearing of the arenas between
    them on the caller's stream, then a run on a side stream: the caller's
    work is ordered around each run (no host synchronisation in between)."""
    shapes = [(1001, 24), (4096, 96), (96,), (5,), ()]
    R = 5
    w = _wl(shapes, R, 960, sigma=1e-3)
    st = harness.setup(w, with_ag=False)
    st.plan.rs()
    torch.cuda.synchronize()
    ref = [o.clone() for o in st.out]
    tp = pipeline.TwoPhase(st.plan, 3, 2, "cu", 0)
    try:
        gu.say("pipeline reuse", tp.chunks())
        for o in st.out:
            o.view(torch.int32).fill_(-1)
        tp.run()
        for o in st.out:
            o.view(torch.int32).fill_(-1)
        tp.run()
        torch.cuda.synchronize()
        for r in range(R):
            assert torch.equal(st.out[r].view(torch.int32), ref[r].view(torch.int32)), r
        side = torch.cuda.Stream()
        with torch.cuda.stream(side):
            for o in st.out:
                o.view(torch.int32).fill_(-1)
            tp.run()
            for r in range(R):
                st.out[r].view(torch.int32).sub_(ref[r].view(torch.int32))
        torch.cuda.synchronize()
        for r in range(R):
            assert int(st.out[r].view(torch.int32).abs().max()) == 0, r
    finally:
        tp.close()
    gu.check_out_guards(st, 0)


def test_run_validates_before_issuing():
    shapes = [(4096, 96), (96,)]
    R = 4
    w = _wl(shapes, R, 961)
    st = harness.setup(w, with_ag=False)
    n, T = int(st.plan.info.rs_tiles), int(st.plan.info.rs_tile_elems)
    for o in st.out:
        o.view(torch.int32).fill_(-1)
    h = api.tide_pipeline_create(2, 0)
    h8 = api.tide_pipeline_create(2, 8)
    try:
        assert st.S >= 2 * T and n > 6
        ring = torch.empty(2 * 2 * T, dtype=torch.float32, device="cuda")
        with pytest.raises(api.TideError) as e:         # ring smaller than two slots of 3 tiles
            api.tide_pipeline_run(h, st.plan.blob, st.plan.d_blob, 3, ring)
        assert e.value.status == -1
        with pytest.raises(api.TideError) as e:         # the ring over rank 1's arena
            api.tide_pipeline_run(h, st.plan.blob, st.plan.d_blob, 1, st.out[1][: 2 * T])
        assert e.value.status == -3
        with pytest.raises(api.TideError) as e:         # copies on a CU-confined pipeline
            api.tide_pipeline_run(h8, st.plan.blob, st.plan.d_blob, 1, ring, phase2=1)
        assert e.value.status == -1
        with pytest.raises(api.TideError) as e:         # not 16-byte aligned
            api.tide_pipeline_run(h, st.plan.blob, st.plan.d_blob, 1, ring[1:])
        assert e.value.status == -2
        torch.cuda.synchronize()
        # nothing was issued: the arenas still hold the fill
        assert all(bool(o.view(torch.int32).eq(-1).all()) for o in st.out)
        gu.say("pipeline validation", n)
    finally:
        api.tide_pipeline_destroy(h)
        api.tide_pipeline_destroy(h8)


def test_prequeued_timing_of_a_pipelined_call():
    """The host-bound check behind the pipeline measurements: the same
    pipelined call timed as usual and queued behind a bounded spin kernel,
    on a stream of the checker's own; both give finite times of the same
    order, and the call's results are still the oracle's."""
    w = _wl([(4096, 96), (1001, 24), (5,)], 8, 951, sigma=1e-3)
    st = harness.setup(w, with_ag=False)
    for o in st.out:
        o.view(torch.int32).fill_(-1)
    pq = pipeline.Prequeued()
    assert pq.units_per_ms > 0
    gu.say("prequeued timing")
    with pipeline.TwoPhase(st.plan, 16, 2, "cu", 0) as tp:
        r = pq.compare(tp.run)
    assert r["plain_ms"] > 0 and r["host_issue_ms"] > 0
    assert r["prequeued_ms"] is not None
    assert 0.25 * r["plain_ms"] <= r["prequeued_ms"] <= 4.0 * r["plain_ms"] + 1.0, r
    gu.check_rs_full(st)


def test_ring_shared_by_calls_on_two_streams():
    """One pipeline object and one ring, two calls issued on two streams with
    nothing ordering them: each call's chunks wait for the phase 2 that last
    drained their slot, also the other call's, so both results are the
    oracle's (two plans over the same gradients with arenas of their own, so
    that a slot refilled too early would leave wrong words behind).  Phase 2
    on 8 CUs lags phase 1, which is what exposes a slot refilled while the
    other call still drains it: before each chunk waited for its slot's last
    drain from an earlier call too, this case left about a million wrong
    words in the first call's arenas."""
    shapes = [(16384, 1024)]
    R = 8
    w = _wl(shapes, R, 970, sigma=1e-3)
    st = harness.setup(w, with_ag=False)
    st.plan.rs()
    torch.cuda.synchronize()
    ref = [o.clone() for o in st.out]
    out2 = [torch.empty(st.S, dtype=torch.float32, device="cuda") for _ in range(R)]
    plan2 = api.Plan(w.shapes, R, grads=st.grads, out=out2)
    chunk, depth = 512, 2
    T = int(st.plan.info.rs_tile_elems)
    assert -(-int(st.plan.info.rs_tiles) // chunk) > 4 * depth
    ring = torch.empty(depth * chunk * T, dtype=torch.float32, device="cuda")
    h = api.tide_pipeline_create(depth, 8)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    try:
        for _ in range(3):
            for o in st.out + out2:
                o.view(torch.int32).fill_(-1)
            torch.cuda.synchronize()
            gu.say("ring shared by two streams")
            api.tide_pipeline_run(h, st.plan.blob, st.plan.d_blob, chunk, ring, 0, stream=sa)
            api.tide_pipeline_run(h, plan2.blob, plan2.d_blob, chunk, ring, 0, stream=sb)
            torch.cuda.synchronize()
            for r in range(R):
                assert torch.equal(st.out[r].view(torch.int32), ref[r].view(torch.int32)), r
                assert torch.equal(out2[r].view(torch.int32), ref[r].view(torch.int32)), r
    finally:
        torch.cuda.synchronize()
        api.tide_pipeline_destroy(h)
