"""GPU parity of the copy-engine-staged reduce-scatter: the DMA engines copy
every rank's slices into per-rank staging slots (tide_rs_stage_dma), a
kernel folds the slots (tide_rs_fold_staged).  Bit for bit against the
oracle (fixed and tree order) and against the in-place kernel."""
import numpy as np
import pytest
import torch

from shard_placement_amd import api, configs, harness
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
    (16, [(512, 48), (1,), (17, 8)]),
    (17, [(300, 16)]),
    (32, [(6, 5120), (5120,)]),
    (64, [(1001, 64), (128,), (3, 8)]),
]


def _staged(st, stage, order="fixed"):
    srs = api.StagedRS(st.plan, stage)
    srs.stage_dma()
    srs.fold(order)
    torch.cuda.synchronize()
    return srs


@pytest.mark.parametrize("order", ["fixed", "tree"])
def test_tiny_workload_bitwise(order):
    w = configs.get(1)
    gu.say("staged tiny", order)
    st = harness.setup(w, with_ag=False, gen_device="cpu")
    _staged(st, harness.stage_buffers(st), order)
    gu.check_rs_full(st, order)


@pytest.mark.parametrize("R,shapes", CASES, ids=[str(c[0]) for c in CASES])
@pytest.mark.parametrize("order", ["fixed", "tree"])
def test_ragged_shapes_bitwise(R, shapes, order):
    w = _wl(shapes, R, 800 + R)
    gu.say("staged ragged", R, shapes, order)
    st = harness.setup(w, with_ag=False)
    _staged(st, harness.stage_buffers(st), order)
    gu.check_rs_full(st, order)


@pytest.mark.parametrize("R", [8, 12, 16, 64])
@pytest.mark.parametrize("launch", ["reserving", "one"])
def test_fold_rank_batching_variants_bitwise(R, launch):
    """The fold in every rank-batching form (4 ranks per batch in launches
    that reserve LDS, 2 otherwise, 8 with a re-read rank when R is not a
    multiple of 8): the oracle's bits."""
    w = _wl([(2 * R + 3, 40), (R - 1, 8), (4096, 16)], R, 860 + R, sigma=1e-3)
    st = harness.setup(w, with_ag=False, launch_mib=-1 if launch == "one" else 0)
    assert (st.plan.info.rs_lds_bytes > 8192) == (launch == "reserving")
    gu.say("staged fold batching", R, launch)
    _staged(st, harness.stage_buffers(st))
    gu.check_rs_full(st)


@pytest.mark.parametrize("stride_extra,offset", [(13, 0), (0, 3), (64, 8)])
def test_unaligned_or_padded_slots(stride_extra, offset):
    """Slot strides that are not a multiple of 8 elements or buffers that do
    not start on 16 bytes take the element-wise fold; padded slots leave the
    gaps untouched."""
    shapes = [(1001, 24), (5,), (64, 64), (3, 7)]
    R = 8
    w = _wl(shapes, R, 830)
    gu.say("staged slots", stride_extra, offset)
    st = harness.setup(w, with_ag=False)
    stage = harness.stage_buffers(st, st.S + stride_extra, offset=offset)
    _staged(st, stage)
    gu.check_rs_full(st)


def test_fold_of_slots_staged_by_torch():
    """The fold alone: slots filled with torch copies (no DMA engines)."""
    shapes = [(1001, 24), (5,), (64, 64)]
    R = 8
    w = _wl(shapes, R, 840)
    st = harness.setup(w, with_ag=False)
    stage = harness.stage_buffers(st)
    s, m, off, S = api.tide_desc_geometry(shapes, R)
    for p, shp in enumerate(shapes):
        d0 = shp[0] if shp else 1
        c = int(np.prod(shp[1:])) if len(shp) > 1 else 1
        for r in range(R):
            v = max(0, min(int(s[p]), d0 - r * int(s[p])))
            for q in range(R):
                src = st.grads[q][p].reshape(-1)[r * int(m[p]): r * int(m[p]) + v * c]
                stage[r][q * S + int(off[p]): q * S + int(off[p]) + v * c].copy_(src)
    torch.cuda.synchronize()
    gu.say("fold of torch-staged slots")
    srs = api.StagedRS(st.plan, stage)
    srs.fold()
    torch.cuda.synchronize()
    gu.check_rs_full(st)


def test_staging_in_vacated_gathered_buffers():
    """Slot-Reuse as the pages describe it: gradients staged in each rank's
    vacated gathered buffer (R*S elements, slot stride S), fp32 shards in
    separate arenas."""
    shapes = [(1001, 24), (64, 64), (5,)]
    R = 8
    w = _wl(shapes, R, 850)
    st = harness.setup(w)
    st.plan.ag()
    _, _, _, S = api.tide_desc_geometry(shapes, R)
    vacated = [torch.empty(R * S, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    for v in vacated:
        v.copy_(st.gathered)  # every rank holds the same gathered data after an all-gather
    before = torch.cuda.memory_allocated()
    gu.say("staged into vacated buffers")
    _staged(st, vacated)
    assert torch.cuda.memory_allocated() == before
    gu.check_rs_full(st)


def test_same_bits_as_in_place_kernel_on_repeat():
    shapes = [(4096, 256), (256,), (100, 33)]
    R = 16
    w = _wl(shapes, R, 860, sigma=1e-3)
    st = harness.setup(w, with_ag=False)
    st.plan.rs()
    torch.cuda.synchronize()
    ref = [o.clone() for o in st.out]
    srs = api.StagedRS(st.plan, harness.stage_buffers(st))
    for rep in range(3):
        for o in st.out:
            o.view(torch.int32).fill_(-1)
        gu.say("staged repeat", rep)
        srs.stage_dma()
        srs.fold()
        torch.cuda.synchronize()
        for r in range(R):
            assert torch.equal(st.out[r].view(torch.int32), ref[r].view(torch.int32)), (rep, r)


def test_dma_engine_count():
    n = api.tide_dma_engine_count()
    gu.say("dma engines", n)
    assert n >= 1


@pytest.mark.big
@pytest.mark.parametrize("key", [2, 5])
def test_full_size_staged_matches_in_place(key):
    w = configs.get(key)
    gu.say("full-size staged", w.name)
    st = harness.setup(w, with_ag=False, slot_reuse=False, guard=0)
    st.plan.rs()
    torch.cuda.synchronize()
    ref = [o.clone() for o in st.out]
    for o in st.out:
        o.view(torch.int32).fill_(-1)
    stage = harness.stage_buffers(st)
    _staged(st, stage)
    for r in range(w.R):
        assert torch.equal(st.out[r].view(torch.int32), ref[r].view(torch.int32)), r
    del stage, ref
    st.free()
    torch.cuda.empty_cache()
