"""The allocation-free two-phase call, tide_rs_two_phase_noalloc, through
the C ABI: its results must be those of the two-phase calls with a
caller-owned staging chunk (tide_rs_tiles_to_stage, then
tide_rs_stage_to_shards), bit for bit, on two calls in a row (the second on
a smaller layer, so the library's staging array still holds the first
call's values), and those of the oracle when a whole layer is run through it
chunk by chunk."""
import pytest
import torch

from shard_placement_amd import _lib, api, configs, harness
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

NAN = -1  # 0xFFFFFFFF as int32


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _wl(shapes, R, key):
    shapes = tuple(tuple(s) for s in shapes)
    return configs.Workload(key=key, name="noalloc", R=R,
                            names=tuple("p%d" % i for i in range(len(shapes))),
                            shapes=shapes, sigma=1.0)


def _reset(st):
    for o in st.out_alloc:
        o.view(torch.int32).fill_(NAN)


def _snapshot(st):
    return [o.view(torch.int32).clone() for o in st.out_alloc]


def _reference(st, b, cnt):
    """The same tiles through the two calls with a staging chunk of torch's."""
    plan = st.plan
    T = int(plan.info.rs_tile_elems)
    stage = torch.empty(max(1, cnt) * T, dtype=torch.float32, device="cuda")
    api.tide_rs_tiles_to_stage(plan.blob, plan.d_blob, b, cnt, stage)
    api.tide_rs_stage_to_shards(plan.blob, plan.d_blob, b, cnt, stage)
    torch.cuda.synchronize()
    del stage


def _noalloc_matches_reference(st, b, cnt):
    _reset(st)
    _reference(st, b, cnt)
    want = _snapshot(st)
    _reset(st)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    api.tide_rs_two_phase_noalloc(st.plan.blob, st.plan.d_blob, b, cnt)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    for r, (a, w) in enumerate(zip(_snapshot(st), want)):
        assert torch.equal(a, w), "rank %d arena differs from the two-phase calls" % r


def test_two_calls_in_a_row_second_smaller():
    T = 2048
    cap = _lib.SCRATCH_BYTES // (4 * T)
    # first call: the array's maximum, on a layer with vector, scalar-edge
    # and padding tiles
    big = _wl([(4001, 4096), (5,), (130, 24)], 8, key=301)
    gu.say("noalloc: first call", big.shapes, "tiles", cap)
    st = harness.setup(big, with_ag=False, guard=64, rs_tile=T)
    n = int(st.plan.info.rs_tiles)
    assert n > cap
    _noalloc_matches_reference(st, 100, cap)
    # tiles outside the range stay untouched
    b0, c0 = api.tide_plan_rank_tiles(st.plan.blob, 7)
    _reset(st)
    api.tide_rs_two_phase_noalloc(st.plan.blob, st.plan.d_blob, b0, c0)
    torch.cuda.synchronize()
    for r in range(7):
        assert bool(torch.all(st.out_alloc[r].view(torch.int32) == NAN)), r
    with pytest.raises(_lib.TideError) as e:
        api.tide_rs_two_phase_noalloc(st.plan.blob, st.plan.d_blob, 0, cap + 1)
    assert e.value.status == -4
    st.free()
    del st
    torch.cuda.empty_cache()
    # second call, smaller: another layer and R, fewer tiles than before
    small = _wl([(37, 16), (64, 64), (5,), (1001, 40)], 3, key=302)
    gu.say("noalloc: second call", small.shapes)
    st = harness.setup(small, with_ag=False, guard=64, gen_device="cpu")
    n = int(st.plan.info.rs_tiles)
    assert 0 < n < cap
    _noalloc_matches_reference(st, 0, n)
    gu.check_rs_full(st)


@pytest.mark.parametrize("R,shapes", [(4, [(1001, 3), (0, 5), (2, 2, 2), (9,)]),
                                      (64, [(1001, 64), (128,), (3, 8)]),
                                      (8, [(8192,), (1024, 64), (6, 40)])],
                         ids=["4", "64", "8"])
def test_whole_layer_in_chunks_matches_oracle(R, shapes):
    w = _wl(shapes, R, key=310 + R)
    gu.say("noalloc: whole layer in chunks", R, shapes)
    st = harness.setup(w, with_ag=False, guard=64, gen_device="cpu")
    n = int(st.plan.info.rs_tiles)
    chunk = max(1, n // 3)
    for b in range(0, n, chunk):
        api.tide_rs_two_phase_noalloc(st.plan.blob, st.plan.d_blob, b, min(chunk, n - b))
    torch.cuda.synchronize()
    gu.check_rs_full(st)
