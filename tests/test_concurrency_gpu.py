"""Correctness under concurrency, on the GPU: each reduce-scatter path on
its own stream (CU-masked, so it has a hardware queue of its own) while a
train of single-wave bf16 GEMMs runs on another stream, its shards compared
with the oracle bit for bit and the GEMM's result with the GEMM run alone;
then the interference probe and the per-tile trace on a small multi-launch
layer.  Interference with concurrent compute is what the pages' design sets
out to cut (Abstract of "The Endgame of FSDP Communication",
weekinpapers.com)."""
import numpy as np
import pytest
import torch

from shard_placement_amd import api, configs, harness, pipeline, probe, profiling
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# R = 64 over ~9 M elements: about 4,400 tiles, nine launches of 512 tiles
LAYER = [(4096, 2048), (1001, 512), (128,), (6, 40)]
R = 64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def gemm():
    """A single-wave bf16 GEMM (256 workgroups of hipBLASLt's 256x256 tile)
    and its result computed alone."""
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    a = torch.randn(4096, 8192, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(8192, 4096, device="cuda", dtype=torch.bfloat16, generator=g)
    c = torch.empty(4096, 4096, device="cuda", dtype=torch.bfloat16)
    torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    return a, b, c, c.clone()


def _wl(key):
    shapes = tuple(tuple(s) for s in LAYER)
    return configs.Workload(key=key, name="concurrency", R=R,
                            names=tuple("p%d" % i for i in range(len(shapes))),
                            shapes=shapes, sigma=1e-3)


def _nan_outputs(st):
    for o in st.out_alloc:
        o.view(torch.int32).fill_(-1)


def _beside_gemms(gemm, issue, n_gemm=60):
    """Queue n_gemm GEMMs on a stream of their own, then `issue()` the
    reduce-scatter work on its streams; wait for both; check the GEMM's
    result against the one computed alone."""
    a, b, c, c_ref = gemm
    torch.cuda.synchronize()  # the outputs' NaN fill is done before any stream starts
    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(gs):
        for _ in range(n_gemm):
            torch.matmul(a, b, out=c)
    issue()
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), c_ref.view(torch.int16)), "GEMM result changed"


@pytest.mark.parametrize("n_cu", [0, 128])
def test_fused_rs_on_masked_stream_beside_gemms(gemm, n_cu):
    st = harness.setup(_wl(401), with_ag=False, guard=64)
    assert -(-int(st.plan.info.rs_tiles) // int(st.plan.info.rs_launch_tiles)) >= 4
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    s = api.tide_stream_create_cu_limited(n_cu or ncu)
    gu.say("fused RS beside GEMMs, CU mask", n_cu or ncu)
    try:
        _nan_outputs(st)

        def issue():
            for _ in range(20):
                st.plan.rs(stream=s)
        _beside_gemms(gemm, issue)
    finally:
        torch.cuda.synchronize()
        api.tide_stream_destroy(s)
    gu.check_rs_full(st)


def test_staged_fold_on_masked_stream_beside_gemms(gemm):
    st = harness.setup(_wl(402), with_ag=False, guard=64)
    stage = harness.stage_buffers(st)
    srs = api.StagedRS(st.plan, stage)
    srs.stage_dma()
    _nan_outputs(st)
    s = api.tide_stream_create_cu_limited(192)
    gu.say("staged fold beside GEMMs")
    try:
        def issue():
            for _ in range(10):
                srs.fold(stream=s)
        _beside_gemms(gemm, issue)
    finally:
        torch.cuda.synchronize()
        api.tide_stream_destroy(s)
    gu.check_rs_full(st)


@pytest.mark.parametrize("phase2_cus", [0, 8])
def test_pipeline_beside_gemms(gemm, phase2_cus):
    st = harness.setup(_wl(403), with_ag=False, guard=64)
    L = int(st.plan.info.rs_launch_tiles)
    _nan_outputs(st)
    gu.say("pipeline beside GEMMs, phase-2 CUs", phase2_cus)
    with pipeline.TwoPhase(st.plan, L, 2, "cu", phase2_cus) as tp:
        def issue():
            for _ in range(3):
                tp.run()
        _beside_gemms(gemm, issue)
    gu.check_rs_full(st)


def test_probe_smoke():
    """The interference probe on a small layer: a finite slowdown from GEMMs
    timed inside the reduce-scatter window, and sane bookkeeping."""
    w = _wl(404)
    st = harness.setup(w, with_ag=False, guard=0)
    gu.say("probe smoke")
    res = probe.run([("default launches", st.plan, 0, 0)], harness.rs_bytes(w), iters=12)
    m = res["modes"][0]
    assert res["t_gemm_alone_ms"] > 0 and m["t_gemm_alone_ms"] > 0
    assert m["gemm_inside"] >= 1
    # the GEMM train and the reduce-scatter calls overlapped in time (on
    # streams of different hardware queues), so the slowdown is measured
    assert m["ran_concurrently"], m
    assert isinstance(m["gemm_slowdown_pct"], float) and np.isfinite(m["gemm_slowdown_pct"])
    assert m["rs_alone_gbps"] > 0 and m["rs_concurrent_gbps"] > 0
    assert m["launches_per_rs"] == -(-int(st.plan.info.rs_tiles) // int(st.plan.info.rs_launch_tiles))
    census = st.plan.rs_census()
    torch.cuda.synchronize()
    assert len(set(census.cpu().tolist())) <= res["cus"]
    # the probe left the reduce-scatter's results as the oracle has them
    gu.check_rs_full(st)


def test_trace_same_bits_and_sane_stamps():
    """The timed census gives the reduce-scatter's bits, stamps every tile
    with start <= end, and its span agrees with the event-timed call (which
    checks the counter's assumed 100 MHz rate to within a factor of two)."""
    st = harness.setup(_wl(405), with_ag=False, guard=64)
    st.plan.rs()
    torch.cuda.synchronize()
    ref = [o.view(torch.int32).clone() for o in st.out]
    _nan_outputs(st)
    gu.say("trace")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st.plan.rs_trace()
    torch.cuda.synchronize()
    e0.record()
    census, stamps = st.plan.rs_trace()
    e1.record()
    torch.cuda.synchronize()
    for a, b in zip(ref, st.out):
        assert torch.equal(a, b.view(torch.int32))
    c = census.cpu().numpy()
    s = stamps.cpu().numpy()
    assert np.all(c >= 0) and np.all(s[:, 0] > 0) and np.all(s[:, 1] >= s[:, 0])
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    r = profiling.cu_time(c, s)
    assert 1 <= r["cus"] <= ncu
    assert r["held_cu_ms"] <= r["cus"] * r["span_ms"] * 1.0001
    assert r["held_cu_ms"] <= r["workgroup_ms_sum"] * 1.0001
    ev_ms = e0.elapsed_time(e1)
    assert 0.5 * ev_ms <= r["span_ms"] <= 2.0 * ev_ms, (r, ev_ms)
    # confined to 8 CUs: at most 8 distinct ids
    sm = api.tide_stream_create_cu_limited(8)
    try:
        c8, _ = st.plan.rs_trace(stream=sm)
        torch.cuda.synchronize()
        assert 1 <= len(set(c8.cpu().tolist())) <= 8
    finally:
        api.tide_stream_destroy(sm)


def test_probe_flags_serialised_streams(monkeypatch):
    """The probe's overlap check: with the reduce-scatter and the GEMM train
    on one stream (what two streams on one hardware queue amount to) no GEMM
    overlaps a reduce-scatter call, and the probe says so instead of
    reporting a slowdown that was never measured beside the reduce-scatter."""
    w = _wl(406)
    st = harness.setup(w, with_ag=False, guard=0)
    one = torch.cuda.Stream()
    monkeypatch.setattr(probe, "_new_stream", lambda: one)
    monkeypatch.setattr(probe.api, "tide_stream_create_cu_limited", lambda n: one)
    monkeypatch.setattr(probe.api, "tide_stream_destroy", lambda s: None)
    before = torch.cuda.current_stream()
    gu.say("probe on one stream")
    res = probe.run([("one stream", st.plan, 0, 0)], harness.rs_bytes(w), iters=12)
    torch.cuda.synchronize()
    m = res["modes"][0]
    assert m["gemms_overlapping_rs"] == 0, m
    assert not m["ran_concurrently"]
    gu.check_rs_full(st)
    assert torch.cuda.current_stream() == before
