"""The stock-FSDP2 analog (pack with torch._chunk_cat, add in rank order,
copy out with torch.split_with_sizes_copy) run on the CPU and compared with
the oracle bit for bit: it is the comparison path the fused kernels are
timed against, so it must compute the same thing."""
import numpy as np
import pytest
import torch

import oracle
from shard_placement_amd import api, configs, stock, synth

CASES = [
    (4, [(37, 16), (64, 64), (5,)]),
    (3, [(37, 16), (64, 64), (5,), ()]),
    (4, [(1001, 3), (0, 5), (2, 2, 2), (9,)]),
    (8, [(8192,), (1024, 4), (6, 40)]),
    (17, [(300, 16), (1,)]),
    (32, [(6, 512), (512,)]),
]


def _wl(shapes, R):
    shapes = tuple(tuple(s) for s in shapes)
    return configs.Workload(key=900, name="adhoc", R=R, names=tuple("p%d" % i for i in range(len(shapes))),
                            shapes=shapes, sigma=1.0)


def _bits16(t):
    return t.reshape(-1).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("R,shapes", CASES, ids=[str(i) for i in range(len(CASES))])
def test_stock_analog_matches_oracle(R, shapes):
    w = _wl(shapes, R)
    n = synth.arena_numel(w.shapes)
    grads = []
    for q in range(R):
        a = torch.empty(n, dtype=torch.bfloat16)
        synth.fill_normal_(a, 9000 + q, 1.0)
        grads.append(synth.views(a, w.shapes))
    _, _, _, S = api.tide_desc_geometry(w.shapes, R)
    gathered = torch.empty(R * S, dtype=torch.bfloat16)
    synth.bits_(gathered, 77)
    sp = stock.StockPath(w, S, grads, gathered, "cpu")
    sp.rs()
    sp.ag()
    want = oracle.rs(w.shapes, R, [[_bits16(t) for t in grads[q]] for q in range(R)])
    for r in range(R):
        assert np.array_equal(sp.acc[r].numpy().view(np.uint32), want[r].view(np.uint32)), r
    full = oracle.ag(w.shapes, R, _bits16(gathered))
    for p, t in sp.unsharded:
        assert np.array_equal(_bits16(t), full[p]), p


def test_stock_traffic_formula():
    w = configs.get(2)
    _, _, _, S = api.tide_desc_geometry(w.shapes, w.R)
    n = w.numel()
    assert S * w.R == n  # no padding in the Llama layer at R = 8
    # pack: R*(2N + 4N); adds: (R-1)*12N
    assert stock.rs_traffic(w, S) == w.R * 6 * n + (w.R - 1) * 12 * n
