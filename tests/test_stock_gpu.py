"""The stock-FSDP2 analog on the GPU gives the same bits as the fused
kernels (fixed order) on small layers and on a full-size layer."""
import pytest
import torch

from shard_placement_amd import configs, harness, stock
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _wl(shapes, R, key):
    shapes = tuple(tuple(s) for s in shapes)
    return configs.Workload(key=key, name="adhoc", R=R, names=tuple("p%d" % i for i in range(len(shapes))),
                            shapes=shapes, sigma=1.0)


@pytest.mark.parametrize("R,shapes", [(4, [(37, 16), (64, 64), (5,)]),
                                      (8, [(1001, 24), (0, 5), (), (8192,)]),
                                      (16, [(768, 256), (256, 768), (128, 256)])])
def test_stock_matches_fused(R, shapes):
    w = _wl(shapes, R, 700 + R)
    gu.say("stock vs fused", R, shapes)
    st = harness.setup(w)
    st.plan.ag()
    st.plan.rs()
    sp = stock.StockPath.from_setup(st)
    sp.ag()
    sp.rs()
    torch.cuda.synchronize()
    assert sp.same_rs_bits(st.out)
    assert sp.same_ag_bits(st.full)
    gu.check_rs_full(st)


@pytest.mark.big
def test_stock_matches_fused_full_size():
    w = configs.get(2)
    gu.say("stock vs fused full size", w.name)
    st = harness.setup(w, guard=0)
    st.plan.ag()
    st.plan.rs()
    sp = stock.StockPath.from_setup(st)
    sp.ag()
    sp.rs()
    torch.cuda.synchronize()
    assert sp.same_rs_bits(st.out)
    assert sp.same_ag_bits(st.full)
    del sp
    st.free()
    torch.cuda.empty_cache()
