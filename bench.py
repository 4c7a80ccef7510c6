"""Benchmark of the node-local data path of TIDE's layout-aware FSDP2
collectives on one MI355X.

One step = the whole hot path over one layer of synthetic gradients:
all-gather placement of the rank-major bf16 gathered buffer into the
per-parameter tensors, then the fused reduce-scatter of R ranks' bf16
gradients into fp32 dim-0 shards (the plan is built once per layer, before
timing, as in training).  Inputs are resident in HBM before the timed
region.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload 5] [--probe]

The default workload is the largest: one Llama-3.1-70B decoder layer plus a
ragged [1001, 8192] param at R = 64, its fp32 shards staged in the vacated
gathered buffers (Slot-Reuse), with the interference probe's single-wave
GEMM beside the reduce-scatter.  The other layers (R = 8, 16, 32) get a
compact record of their RS and AG rates at the end (--others).

Metric (bytes are algorithmic): RS GB/s = (R*N*2 + N*4) / t_RS and its
fraction of the 8 TB/s HBM peak; AG GB/s = 4*N / t_AG; GEMM slowdown of a
single-wave bf16 GEMM running beside the RS in the default launch
configuration (--probe adds other launch sizes, grid caps and CU masks).
``value`` is the whole step's algorithmic bytes over the step time.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import re
import sys
import time
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published

# The pages' own figures, measured on NVIDIA clusters (context only: other
# hardware, whole training steps, real networks).  Abstract of "The Endgame
# of FSDP Communication" (weekinpapers.com); kongchang.com article, sections
# "The Root of FSDP2 Communication Overhead" and "Performance: Step Time
# Reduction and Interference Cut".
PAGES_CONTEXT = {
    "hardware": "NVIDIA GPUs with NCCL; the system results on 64 GPUs (NVSwitch + RDMA), "
                "GPU count not stated for the two overhead figures",
    "layout_conversion_pct_of_step": 6.4,
    "layout_conversion_workload": "Llama-3.1 70B, 8K tokens per GPU",
    "gemm_slowdown_from_default_rs_pct": 69,
    "rs_sm_time_reduction_x": [12.5, 14.5],
    "interference_reduction": "up to about 10x",
    "step_time_reduction_pct": {"vs_stock_fsdp2": 27.1, "vs_fsdp2_symmmem": 6.0},
}

PROFILES = os.path.join(HERE, "profiles")
# what decides a kernel's launches: its source, the shared headers, and the
# plan builder (tile sizes, order, kinds)
RS_SOURCES = ["shard_placement_amd/csrc/rs.hip", "shard_placement_amd/csrc/plan_format.h",
              "shard_placement_amd/csrc/xcd_map.h", "shard_placement_amd/csrc/plan.cpp"]
AG_SOURCES = ["shard_placement_amd/csrc/ag.hip", "shard_placement_amd/csrc/plan_format.h",
              "shard_placement_amd/csrc/xcd_map.h", "shard_placement_amd/csrc/plan.cpp"]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """Source text without comments and blank lines (a comment edit does not
    change the kernel)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def src_hash(paths) -> str:
    """Hash of the kernel sources' code (comments ignored), recorded in the
    counter summaries so that stale counters are never reported."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(HERE, p)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str, sources) -> Optional[float]:
    """HBM bytes over algorithmic bytes for one launch, from a committed
    rocprofv3 counter summary, if it was taken on the current kernel source;
    else None."""
    path = os.path.join(PROFILES, "%s_%s_pmc.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_code_sha256_16 (comments stripped)") != src_hash(sources):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"]) / float(kv["algorithmic_bytes_per_launch"])
    except (KeyError, ValueError, ZeroDivisionError):
        return None


def _wall(fn, reps: int = 3) -> float:
    """Median wall time (ms) of a host-synchronous call."""
    import torch

    fn()
    ts = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        ts.append((time.perf_counter() - t0) * 1e3)
    return sorted(ts)[len(ts) // 2]


def dma_placement_leg(st, agb: int) -> dict:
    """Placement on the DMA engines through ROCr (engine-pinned 1-D copies,
    one per (param, rank) run), checked against the compute-unit placement."""
    import torch

    from shard_placement_amd import api

    st.plan.ag()
    torch.cuda.synchronize()
    ref = [f.clone() for f in st.full]
    ms = _wall(st.plan.ag_dma)
    same = all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(ref, st.full))
    del ref
    return {"engines": api.tide_dma_engine_count(), "ms": round(ms, 4),
            "GB/s": round(agb / (ms * 1e-3) / 1e9, 1), "same_bits": bool(same),
            "copies": "one engine-pinned 1-D copy per (param, rank) run, host-synchronous",
            "engine": "DMA engines through ROCr (no kernel is dispatched)"}


def staged_leg(st, rsb: int, fused_ms: float, reps: int = 3) -> dict:
    """Copy-engine-staged reduce-scatter: the DMA engines copy every rank's
    slice of every shard into per-rank staging slots, then a kernel folds
    the slots.  With Slot-Reuse the slots are the ranks' vacated gathered
    buffers and the fp32 shards go to arenas of their own; otherwise the
    staging buffers are allocated here.  Also times a single-wave GEMM while
    the engines stage (the compute units stay free for it)."""
    import torch

    from shard_placement_amd import api, harness, probe

    w = st.w
    if st.vacated is not None:
        out = [torch.empty(st.S, dtype=torch.float32, device="cuda") for _ in range(w.R)]
        plan = api.Plan(w.shapes, w.R, grads=st.grads, out=out)
        stage = [v[: w.R * st.S] for v in st.vacated]
        where = "vacated gathered buffers (slot stride S)"
    else:
        out = st.out
        plan = st.plan
        stage = harness.stage_buffers(st)
        where = "staging buffers of R*S bf16 per rank"
    st.plan.rs()  # the fused result, for the bit comparison
    torch.cuda.synchronize()
    ref = [o.clone() for o in st.out]
    srs = api.StagedRS(plan, stage)
    stage_ms = _wall(srs.stage_dma, reps)
    srs.fold()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        srs.fold()
    e1.record()
    torch.cuda.synchronize()
    fold_ms = e0.elapsed_time(e1) / reps
    same = all(torch.equal(a[: st.S].view(torch.int32), b[: st.S].view(torch.int32))
               for a, b in zip(out, ref))
    del ref
    # a single-wave GEMM train while the engines stage
    g = probe.gemm_during(lambda: srs.stage_dma(), stage_ms)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    staged_bytes = 2 * w.R * w.numel()
    rec = {"staging": where, "engines": api.tide_dma_engine_count(),
           "stage_ms": round(stage_ms, 3), "stage_copy_gbps": round(staged_bytes / (stage_ms * 1e-3) / 1e9, 1),
           "fold_ms": round(fold_ms, 4), "fold_gbps": round(rsb / (fold_ms * 1e-3) / 1e9, 1),
           "total_ms": round(stage_ms + fold_ms, 3), "fused_ms": round(fused_ms, 4),
           "fold_cu_ms": round(n_cu * fold_ms, 1), "fused_cu_ms": round(n_cu * fused_ms, 1),
           "stage_cu_ms": 0.0, "same_bits_as_fused": bool(same)}
    rec.update(g)
    del srs, stage, plan
    if st.vacated is not None:
        st.plan.rs()  # staging overwrote the Slot-Reuse arenas inside the vacated buffers
        torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def pipeline_leg(st, fused_ms: float) -> dict:
    """Two-phase pipeline emulation: each phase alone over the whole layer,
    then the two-stream ring for several chunk sizes (in launches of the
    plan's size), ring depths and phase-2 engines; checks the bits of the
    pipelined result against the in-place reduce-scatter."""
    import torch

    from shard_placement_amd import api, pipeline

    plan = st.plan
    n, T = int(plan.info.rs_tiles), int(plan.info.rs_tile_elems)
    L = int(plan.info.rs_launch_tiles) or n
    plan.rs()
    torch.cuda.synchronize()
    ref = [o[: st.S].clone() for o in st.out]

    def ev_time(fn, reps=2):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    full = torch.empty(n * T, dtype=torch.float32, device="cuda")
    t1 = ev_time(lambda: api.tide_rs_tiles_to_stage(plan.blob, plan.d_blob, 0, n, full))
    t2 = {"cu": ev_time(lambda: api.tide_rs_stage_to_shards(plan.blob, plan.d_blob, 0, n, full)),
          "sdma": ev_time(lambda: api.tide_rs_stage_to_shards_sdma(plan.blob, 0, n, full), reps=1)}
    # phase 2 confined to a few CUs: a consumer with a link's bandwidth (8
    # CUs) or with a quarter of the chip (64); in the pipeline phase 1 then
    # runs on the other CUs
    link = {"cu64": 64, "cu8": 8}
    # phase 1 alone on a stream of the pipeline's kind (CU-masked, all CUs)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    sm = api.tide_stream_create_cu_limited(n_cu)
    try:
        with torch.cuda.stream(sm):
            t1_masked = ev_time(lambda: api.tide_rs_tiles_to_stage(plan.blob, plan.d_blob, 0, n, full,
                                                                  stream=sm))
    finally:
        torch.cuda.synchronize()
        api.tide_stream_destroy(sm)
    for name, k in link.items():
        sk = api.tide_stream_create_cu_limited(k)
        try:
            with torch.cuda.stream(sk):
                t2[name] = ev_time(
                    lambda: api.tide_rs_stage_to_shards(plan.blob, plan.d_blob, 0, n, full, stream=sk),
                    reps=1)
        finally:
            torch.cuda.synchronize()
            api.tide_stream_destroy(sk)
    del full
    torch.cuda.empty_cache()
    runs = []
    same = True
    pq = pipeline.Prequeued()
    side = torch.cuda.Stream()
    for phase2 in ("cu", "sdma", "cu64", "cu8"):
        for mult, depth in ((0.25, 2), (1, 1), (1, 2), (1, 4), (4, 2)):
            chunk = max(1, int(L * mult))
            tp = pipeline.TwoPhase(plan, chunk, depth, "sdma" if phase2 == "sdma" else "cu",
                                   link.get(phase2, 0))
            try:
                # back to back on a stream of their own: on the null stream the
                # pipeline's blocking CU-masked streams wait on its pending work
                with torch.cuda.stream(side):
                    t = ev_time(tp.run, reps=2 if phase2 == "cu" else 1)
                    h0 = time.perf_counter()
                    tp.run()
                    host_ms = (time.perf_counter() - h0) * 1e3
                    torch.cuda.synchronize()
                cmp = pq.compare(tp.run)
            finally:
                tp.close()
            same = same and all(torch.equal(o[: st.S].view(torch.int32), r.view(torch.int32))
                                for o, r in zip(st.out, ref))
            serial = t1 + t2[phase2]
            runs.append({"phase2": phase2, "chunk_tiles": chunk, "depth": depth,
                         "staging_mib": round(tp.staging_bytes / 2 ** 20, 1), "ms": round(t, 3),
                         "host_issue_ms": round(host_ms, 3),
                         # on a stream of its own: the call as usual and
                         # queued before the device starts; slower than its
                         # pre-queued self, it waits for the host's issue
                         "own_stream_ms": round(cmp["plain_ms"], 3),
                         "own_stream_prequeued_ms": (None if cmp["prequeued_ms"] is None
                                                     else round(cmp["prequeued_ms"], 3)),
                         "host_bound": (None if cmp["prequeued_ms"] is None
                                        else bool(cmp["plain_ms"] > 1.1 * cmp["prequeued_ms"])),
                         "overlap": round((serial - t) / min(t1, t2[phase2]), 3)})
            del tp
    del ref
    torch.cuda.empty_cache()
    out = {"phase1_ms": round(t1, 4), "phase1_masked_stream_ms": round(t1_masked, 4)}
    out.update({"phase2_%s_ms" % k: round(v, 4) for k, v in t2.items()})
    out.update({"fused_ms": round(fused_ms, 4), "layer_staging_mib": round(n * T * 4 / 2 ** 20, 1),
                "runs": runs, "same_bits_as_fused": bool(same),
                "overlap_def": "(phase1 alone + phase2 alone - pipelined) / min(phase1, phase2)"})
    return out


def stock_leg(st, rsb: int, agb: int, reps: int = 3) -> dict:
    """Time the one-GPU analog of stock FSDP2's layout conversion (pack the
    ranks' gradients into a rank-major fp32 buffer, add in rank order, copy
    the gathered buffer out into padded parameter buffers; torch operators)
    on the same buffers, and check it gives the fused path's bits."""
    import torch

    from shard_placement_amd import stock

    sp = stock.StockPath.from_setup(st)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    st.plan.ag()  # the gathered buffer may have changed since the last placement
    ag_ms = timed(sp.ag)
    same_ag = sp.same_ag_bits(st.full)
    rs_ms = timed(sp.rs)
    same_rs = sp.same_rs_bits(st.out)
    pack_ms = timed(sp.pack)
    traffic = stock.rs_traffic(st.w, st.S)
    rec = {"ops": "torch._chunk_cat (cast+pack per rank) + add_ in rank order; "
                  "torch.split_with_sizes_copy into padded parameter buffers",
           "rs_ms": round(rs_ms, 4), "rs_effective_gbps": round(rsb / (rs_ms * 1e-3) / 1e9, 1),
           "rs_hbm_bytes": traffic, "rs_hbm_gbps": round(traffic / (rs_ms * 1e-3) / 1e9, 1),
           "pack_ms": round(pack_ms, 4),
           "ag_ms": round(ag_ms, 4), "ag_effective_gbps": round(agb / (ag_ms * 1e-3) / 1e9, 1),
           "same_bits_as_fused": bool(same_rs and same_ag)}
    del sp
    torch.cuda.empty_cache()
    return rec


def cpu_baseline(st, budget_s: float) -> dict:
    """Time the CPU oracle (all host threads) on the same workload: params
    in order, each read back in blocks of consecutive flat indices through
    pinned buffers (all R ranks' gradients of the block and the GPU's result
    words), each block reduced by the oracle as a 1-D problem of its own and
    compared bit for bit with the GPU.  Whole params are taken until about
    budget_s of oracle time (the whole layer when it fits).  The oracle's
    rate is the algorithmic bytes over its compute time; the copy time is
    reported beside it, not counted.  One thread is timed on one block."""
    import numpy as np

    import oracle
    from shard_placement_amd import harness

    w = st.w
    R = w.R
    _, m, off, _ = oracle.layout(w.shapes, R)
    reader = harness.BlockReader(st, m, off)
    used, nbytes, t_total, mism, first = [], 0, 0.0, 0, None
    t_wall = time.perf_counter()
    for p, shp in enumerate(w.shapes):
        for a, b, g, got in reader.blocks(p):
            L = b - a
            t0 = time.perf_counter()
            arenas = oracle.rs([(L,)], R, [[gq] for gq in g])
            t_total += time.perf_counter() - t0
            s = -(-L // R)
            want = np.concatenate([x[:s] for x in arenas])[:L].view(np.uint32)
            mism += int(np.count_nonzero(got != want))
            nbytes += R * L * 2 + L * 4
            if first is None:
                first = [gq.copy() for gq in g]
        used.append(p)
        if t_total >= budget_s:
            break
    t_wall = time.perf_counter() - t_wall
    cores = oracle.max_threads()
    # one thread on the first block, repeated for about a second
    L1 = first[0].size
    oracle.set_threads(1)
    try:
        reps, t_one = 0, 0.0
        while reps < 1 or (t_one < 1.0 and reps < 50):
            t0 = time.perf_counter()
            oracle.rs([(L1,)], R, [[gq] for gq in first])
            t_one += time.perf_counter() - t0
            reps += 1
    finally:
        oracle.set_threads(cores)
    whole = len(used) == w.P
    return {
        "value": round(nbytes / t_total / 1e9, 3), "unit": "GB/s",
        "cores": cores, "kind": "oracle",
        "one_thread": {"value": round(reps * (R * L1 * 2 + L1 * 4) / t_one / 1e9, 3),
                       "unit": "GB/s",
                       "sample": "one block of %d elements per rank, %d passes" % (L1, reps)},
        "sample": "reduce-scatter of %s of %s (R=%d, %.2f GB algorithmic), read back in blocks "
                  "of %d flat indices per rank, each reduced by the oracle (one pass, %.2f s of "
                  "oracle time; %.1f s waiting for device->host copies, %.1f s wall, not "
                  "counted); GPU shards of these params bit-exact: %s" % (
                      "every param" if whole else "params " + ",".join(w.names[p] for p in used),
                      w.name, R, nbytes / 1e9, reader.block, t_total, reader.copy_s, t_wall,
                      "yes" if mism == 0 else "NO (%d words differ)" % mism),
        "params_checked": len(used),
        "elements_checked": nbytes // (2 * R + 4),
        "parity_mismatches": mism,
    }


def two_queue_leg(st, rsb: int, fused_ms: float, probe_on: bool = True, reps: int = 10) -> dict:
    """The reduce-scatter with its launches dealt over two hardware queues
    (the current stream and a CU-masked stream of all CUs): its rate alone,
    its bits against the one-queue result, and the single-wave GEMM beside
    it (the launch boundaries that let a concurrent GEMM in are mostly
    lost)."""
    import torch

    from shard_placement_amd import api, probe

    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    # two CU-masked streams of all CUs, each with a hardware queue of its own
    # (not the null stream, which would serialise the launches)
    main = api.tide_stream_create_cu_limited(n_cu)
    extra = api.tide_stream_create_cu_limited(n_cu)
    try:
        st.plan.rs()
        torch.cuda.synchronize()
        ref = [o.view(torch.int32).clone() for o in st.out]
        st.plan.rs_streams([extra], stream=main)
        torch.cuda.synchronize()
        same = all(torch.equal(r, o.view(torch.int32)) for r, o in zip(ref, st.out))
        del ref
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(main)
        for _ in range(reps):
            st.plan.rs_streams([extra], stream=main)
        e1.record(main)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        rec = {"queues": 2, "rs_ms": round(ms, 4), "rs_gbps": round(rsb / (ms * 1e-3) / 1e9, 1),
               "rs_frac_hbm": round(rsb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "one_queue_rs_ms": round(fused_ms, 4), "same_bits": bool(same)}
        if probe_on:
            m = probe.run([("launches dealt over two queues", probe.DealtRS(st.plan, [extra]), 0, 0)],
                          rsb, iters=40)["modes"][0]
            # the probe deals over a stream of its own and `extra`: its rate
            # alone shows whether those two had hardware queues of their own
            rec.update({"t_gemm_alone_ms": m["t_gemm_alone_ms"],
                        "t_gemm_concurrent_ms": m["t_gemm_concurrent_ms"],
                        "gemm_slowdown_pct": m["gemm_slowdown_pct"],
                        "probe_rs_alone_gbps": m["rs_alone_gbps"],
                        "probe_ran_concurrently": m["ran_concurrently"]})
    finally:
        torch.cuda.synchronize()
        api.tide_stream_destroy(extra)
        api.tide_stream_destroy(main)
    return rec


def others_leg(keys, args, reps: int = 10) -> dict:
    """RS and AG rates of other workloads in the default launch
    configuration (event time on the launch stream, after two warm-up
    steps), one workload allocated at a time."""
    import torch

    from shard_placement_amd import configs, harness

    out = {}
    for k in keys:
        w = configs.get(k)
        st = harness.setup(w, guard=0, flags=args.flags, rank_layout=args.rank_layout)
        for _ in range(2):
            st.plan.ag()
            st.plan.rs()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        for _ in range(reps):
            st.plan.rs()
        ev[1].record()
        for _ in range(reps):
            st.plan.ag()
        ev[2].record()
        torch.cuda.synchronize()
        rs_ms = ev[0].elapsed_time(ev[1]) / reps
        ag_ms = ev[1].elapsed_time(ev[2]) / reps
        rsb, agb = harness.rs_bytes(w), harness.ag_bytes(w)
        info = st.plan.info
        out[w.name] = {
            "R": w.R, "P": w.P, "N": w.numel(), "slot_reuse": w.slot_reuse,
            "rs_ms": round(rs_ms, 4), "rs_gbps": round(rsb / (rs_ms * 1e-3) / 1e9, 1),
            "rs_frac_hbm": round(rsb / (rs_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "rs_launches": -(-int(info.rs_tiles) // max(1, int(info.rs_launch_tiles))),
            "ag_ms": round(ag_ms, 4), "ag_gbps": round(agb / (ag_ms * 1e-3) / 1e9, 1),
            "ag_frac_hbm": round(agb / (ag_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        log("other workload", w.name, out[w.name])
        st.free()
        del st
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def tree_leg(st, rsb: int) -> float:
    """The optional pairwise (tree) rank order, same tiles and launches: ms
    per call.  Leaves the fixed-order shards in place for later checks."""
    import torch

    st.plan.rs(order="tree")
    torch.cuda.synchronize()
    te0, te1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    te0.record()
    for _ in range(3):
        st.plan.rs(order="tree")
    te1.record()
    torch.cuda.synchronize()
    tree_ms = te0.elapsed_time(te1) / 3
    st.plan.rs()
    torch.cuda.synchronize()
    log("RS tree order: %.3f ms = %.0f GB/s" % (tree_ms, rsb / (tree_ms * 1e-3) / 1e9))
    return tree_ms


def graph_leg(step, steps: int) -> float:
    """The step captured once in a HIP graph and replayed (launch-bound host
    work removed; the device work is identical): ms per step."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    ge0, ge1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ge0.record()
    for _ in range(steps):
        g.replay()
    ge1.record()
    torch.cuda.synchronize()
    graph_ms = ge0.elapsed_time(ge1) / steps
    log("step as a HIP graph: %.3f ms" % graph_ms)
    return graph_ms


def sdma_leg(st, agb: int) -> dict:
    """The runtime's copy calls beside the kernel placement (1-D copies of
    the no-compute-unit kind, and 2-D copies), each checked against the
    kernel's result from the same gathered buffer."""
    import torch

    st.plan.ag()
    torch.cuda.synchronize()
    ref_full = [f.view(torch.int16).clone() for f in st.full]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        st.plan.ag()
    e1.record()
    torch.cuda.synchronize()
    t_kernel = e0.elapsed_time(e1) / 5
    sdma = {}
    forms = (
        ("copies_1d", True, "hipMemcpyDeviceToDeviceNoCU 1-D copies, one per (param, rank) run",
         "chosen by the HIP runtime (DMA engines or blit kernels; not checked in this run: "
         "ag_dma is the path that never uses a compute unit)"),
        ("copies_2d", False, "hipMemcpy2DAsync per param over the ranks with full shards, "
         "plus a 1-D copy for the partial rank",
         "the HIP runtime's blit kernels for 2-D copies (compute units)"),
    )
    for key, engine_only, copies, engine in forms:
        for f in st.full:
            f.view(torch.int16).fill_(-1)
        st.plan.ag_sdma(engine_only=engine_only)
        torch.cuda.synchronize()
        same = all(torch.equal(f.view(torch.int16), r) for f, r in zip(st.full, ref_full))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            st.plan.ag_sdma(engine_only=engine_only)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 5
        sdma[key] = {"ms": round(t, 4), "GB/s": round(agb / (t * 1e-3) / 1e9, 1),
                     "vs_kernel": round(t_kernel / t, 3), "same_bits": bool(same),
                     "copies": copies, "engine": engine}
        log("AG via %s: %.3f ms = %.0f GB/s (kernel %.3f ms), same bits %s" % (
            key, t, sdma[key]["GB/s"], t_kernel, same))
    sdma["kernel_ms"] = round(t_kernel, 4)
    del ref_full
    torch.cuda.empty_cache()
    return sdma


def trace_leg(st, max_wg: int):
    """Which compute units the reduce-scatter ran on, and for how long: one
    traced call outside the timed region (same launches; each tile records
    its CU's hardware id and its start and end on the real-time counter).
    Returns (CU-time record, distinct CUs, CUs per XCC)."""
    import torch

    from shard_placement_amd import profiling

    st.plan.rs_trace(max_workgroups=max_wg)
    torch.cuda.synchronize()
    te0, te1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    te0.record()
    census, stamps = st.plan.rs_trace(max_workgroups=max_wg)
    te1.record()
    torch.cuda.synchronize()
    ids = census.cpu().numpy()
    st_np = stamps.cpu().numpy()
    cu_rec = profiling.cu_time(ids, st_np)
    cu_rec["traced_call_ms_events"] = round(te0.elapsed_time(te1), 4)
    cu_rec["workgroup_us_by_xcc"] = profiling.workgroup_us_by_xcc(ids, st_np)
    per_xcc = {}
    for v in set(ids.tolist()):
        per_xcc[v >> 8] = per_xcc.get(v >> 8, 0) + 1
    log("census: %d distinct CUs over %d tiles; per XCC %s; CU time %s" % (
        cu_rec["cus"], len(ids), dict(sorted(per_xcc.items())), cu_rec))
    st.plan.rs()  # the untraced result for the checks that follow
    torch.cuda.synchronize()
    return cu_rec, cu_rec["cus"], per_xcc


def probe_leg(st, args, rsb: int) -> dict:
    """The single-wave GEMM beside the reduce-scatter in the default
    configuration; with --probe also launch sizes, a capped grid and CU
    masks."""
    from shard_placement_amd import api, probe

    w = st.w

    def plan_with(mib):
        return api.Plan(w.shapes, w.R, grads=st.grads, out=st.out, flags=args.flags,
                        rs_tile=args.rs_tile, launch_mib=mib)

    info = st.plan.info
    modes = [("default (%d MiB launches)" % (info.rs_launch_tiles * info.rs_tile_elems *
                                              (2 * w.R + 4) >> 20), st.plan, 0, 0)]
    if args.probe:
        one = plan_with(-1)
        modes += [("256 MiB launches", plan_with(256), 0, 0),
                  ("128 MiB launches", plan_with(128), 0, 0),
                  ("64 MiB launches", plan_with(64), 0, 0),
                  ("one launch", one, 0, 0),
                  ("one launch, grid 256", one, 256, 0),
                  ("one launch, CU mask 32", one, 0, 32)]
        # the default launches confined to part of the chip
        modes += [("default launches, CU mask %d" % n, st.plan, 0, n) for n in (128, 64, 32, 16)]
    res = probe.run(modes, rsb, iters=40)
    for m in res["modes"]:
        log("probe", m)
    return res


def pages_context(rec: dict, cu_rec: dict, stock_rec) -> dict:
    """The pages' figures (other hardware) beside this GPU's analogs."""
    import torch

    ctx = dict(PAGES_CONTEXT)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    ctx["one_gpu_analogs"] = {
        "gemm_slowdown_pct": rec["gemm_slowdown_pct"],
        "rs_cu_ms_fused": cu_rec["held_cu_ms"],
        # the analog's torch kernels have grids of far more than one
        # workgroup per CU: all CUs for its whole duration
        "rs_cu_ms_stock_analog": round(n_cu * stock_rec["rs_ms"], 1) if stock_rec else None,
        "rs_cu_time_stock_over_fused": (round(n_cu * stock_rec["rs_ms"] / cu_rec["held_cu_ms"], 2)
                                        if stock_rec and cu_rec.get("held_cu_ms") else None),
        "stock_analog_pack_pct_of_its_rs": (round(100 * stock_rec["pack_ms"] / stock_rec["rs_ms"], 1)
                                            if stock_rec else None),
        "fused_rs_speedup_over_stock_analog": stock_rec["fused_rs_speedup"] if stock_rec else None,
    }
    return ctx


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="5",
                    help="workload key or name (default: the Llama-3.1-70B layer plus a ragged "
                         "param at R=64 with Slot-Reuse)")
    ap.add_argument("--flags", type=int, default=-1, help="TIDE_FLAG_* access hints (-1: default)")
    ap.add_argument("--rs-tile", type=int, default=0)
    ap.add_argument("--launch-mib", type=int, default=0, help="MiB per kernel launch (0: default, -1: one launch)")
    ap.add_argument("--ag-tile", type=int, default=0)
    ap.add_argument("--max-wg", type=int, default=0, help="cap the RS grid (0: one workgroup per tile)")
    ap.add_argument("--rank-layout", choices=("packed", "separate"), default="packed",
                    help="simulated ranks' arenas as rows of one allocation, or one allocation each")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--probe", action="store_true",
                    help="full interference sweep (launch sizes, grid caps, CU masks)")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip even the default-configuration GEMM probe")
    ap.add_argument("--no-sdma", action="store_true", help="skip timing the copy-engine placement")
    ap.add_argument("--no-graph", action="store_true", help="skip timing the step as a HIP graph")
    ap.add_argument("--no-staged", action="store_true",
                    help="skip the copy-engine legs (DMA placement, copy-engine-staged RS)")
    ap.add_argument("--no-pipeline", action="store_true",
                    help="skip the two-phase pipeline emulation leg")
    ap.add_argument("--no-stock", action="store_true",
                    help="skip timing the stock-FSDP2 analog (pack, add, copy out in torch ops)")
    ap.add_argument("--no-two-queues", action="store_true",
                    help="skip the two-queue leg (launches dealt over two hardware queues)")
    ap.add_argument("--no-trace", action="store_true",
                    help="skip the traced call (CU census and per-tile timing)")
    ap.add_argument("--others", default="2,3,4",
                    help="other workload keys timed after the main one (RS and AG only); '' for none")
    ap.add_argument("--calib-copy-mib", type=int, default=1024,
                    help="size of a plain device copy run once (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: the library keeps all R simulated ranks in one "
              "GPU's HBM and has no multi-GPU mode; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from shard_placement_amd import configs, harness

    if not torch.cuda.is_available():
        print("no GPU visible: bench.py needs an MI355X", file=sys.stderr)
        sys.exit(1)
    w = configs.get(args.workload)
    log("workload", w.name, "R", w.R, "P", w.P, "N", w.numel())
    t0 = time.perf_counter()
    st = harness.setup(w, guard=0, flags=args.flags, rs_tile=args.rs_tile, ag_tile=args.ag_tile,
                       launch_mib=args.launch_mib, rank_layout=args.rank_layout)
    torch.cuda.synchronize()
    info = st.plan.info
    log("setup %.1f s; plan: %d RS tiles of %d (%d per launch), %d AG tiles of %d (%d per launch), "
        "blob %d B" % (time.perf_counter() - t0, info.rs_tiles, info.rs_tile_elems,
                       info.rs_launch_tiles, info.ag_tiles, info.ag_tile_elems,
                       info.ag_launch_tiles, info.blob_bytes))

    if args.calib_copy_mib > 0:
        # a plain elementwise kernel of known traffic (reads and writes
        # calib_copy_mib MiB each) for scaling the HBM byte counters
        src = torch.empty(args.calib_copy_mib << 19, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1.0)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    rsb, agb = harness.rs_bytes(w), harness.ag_bytes(w)

    # The heap is frozen after setup and the collector stays paused from here
    # on, as timeit does while timing: a full collection walks every tracked
    # object (~170 K here, 20-35 ms of one core) holding the interpreter lock,
    # so this thread stops issuing GPU work; the GPU idles, and kernels issued
    # after an idle stretch run slower for a while (the single-wave GEMM of
    # the interference probe by 10-25%); the host-timed legs (copy engines,
    # pipeline issue) would absorb its pauses too.
    gc.collect()
    gc.freeze()
    gc.disable()

    def step(ev=None):
        if ev:
            ev[0].record()
        st.plan.ag()
        if ev:
            ev[1].record()
        st.plan.rs(max_workgroups=args.max_wg)
        if ev:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ag_ms = [e[0].elapsed_time(e[1]) for e in evs]
    rs_ms = [e[1].elapsed_time(e[2]) for e in evs]
    ms_step = wall * 1e3 / args.steps
    rs_avg = sum(rs_ms) / len(rs_ms)
    ag_avg = sum(ag_ms) / len(ag_ms)
    rs_gbs = rsb / (rs_avg * 1e-3) / 1e9
    ag_gbs = agb / (ag_avg * 1e-3) / 1e9
    log("step %.3f ms; RS avg %.3f ms (min %.3f) = %.0f GB/s; AG avg %.3f ms = %.0f GB/s" % (
        ms_step, rs_avg, min(rs_ms), rs_gbs, ag_avg, ag_gbs))

    tree_ms = tree_leg(st, rsb)

    graph_ms = None if args.no_graph else graph_leg(step, args.steps)

    sdma = None if args.no_sdma else sdma_leg(st, agb)

    cu_rec, cus_measured, per_xcc = {"held_cu_ms": None}, None, {}
    if not args.no_trace:
        cu_rec, cus_measured, per_xcc = trace_leg(st, args.max_wg)

    dma_rec = staged_rec = None
    if not args.no_staged:
        dma_rec = dma_placement_leg(st, agb)
        log("placement on the DMA engines", dma_rec)
        staged_rec = staged_leg(st, rsb, rs_avg)
        log("copy-engine-staged RS", staged_rec)

    pipe_rec = None
    if not args.no_pipeline:
        pipe_rec = pipeline_leg(st, rs_avg)
        log("two-phase pipeline", pipe_rec)

    stock_rec = None
    if not args.no_stock:
        stock_rec = stock_leg(st, rsb, agb)
        stock_rec["fused_rs_speedup"] = round(stock_rec["rs_ms"] / rs_avg, 2)
        stock_rec["fused_ag_speedup"] = round(stock_rec["ag_ms"] / ag_avg, 2)
        log("stock-FSDP2 analog", stock_rec)

    probe = None if args.no_probe else probe_leg(st, args, rsb)

    two_q = None
    if not args.no_two_queues:
        two_q = two_queue_leg(st, rsb, rs_avg, probe_on=not args.no_probe)
        log("two queues", two_q)

    traffic_ratio = read_traffic("rs_fixed_kernel", w.name, RS_SOURCES)
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on the host cores")
        cpu = cpu_baseline(st, args.cpu_budget)
        log("cpu baseline", cpu)

    n_launch = -(-int(info.rs_tiles) // max(1, int(info.rs_launch_tiles)))
    algo_launch = rsb // n_launch
    # counters were read on full launches; scaled here to the average launch
    traffic = round(traffic_ratio * algo_launch) if traffic_ratio else None
    rec = {
        "metric": "RS bf16->fp32 shard GB/s & % of HBM peak; AG placement GB/s; GEMM slowdown %",
        "value": round((rsb + agb) / (ms_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: seeded bf16 N(0,%g) gradients shaped like %s" % (w.sigma, w.name),
        "config": {"workload": w.name, "R": w.R, "P": w.P, "N": w.numel(),
                   "step": "AG placement + fused RS", "slot_reuse": w.slot_reuse,
                   "rank_layout": args.rank_layout,
                   "rs_bytes": rsb, "ag_bytes": agb},
        "rs_gbps": round(rs_gbs, 1),
        "rs_frac_hbm": round(rs_gbs / HBM_PEAK_GBS, 4),
        "rs_ms": round(rs_avg, 4),
        "rs_ms_median": round(sorted(rs_ms)[len(rs_ms) // 2], 4),
        "rs_ms_min": round(min(rs_ms), 4),
        "rs_tree_gbps": round(rsb / (tree_ms * 1e-3) / 1e9, 1),
        "ag_gbps": round(ag_gbs, 1),
        "ag_frac_hbm": round(ag_gbs / HBM_PEAK_GBS, 4),
        "ag_ms": round(ag_avg, 4),
        "ag_ms_median": round(sorted(ag_ms)[len(ag_ms) // 2], 4),
        "ag_ms_min": round(min(ag_ms), 4),
        "ag_sdma": sdma,
        "graph_ms_per_step": round(graph_ms, 4) if graph_ms else None,
        "gemm_slowdown_pct": probe["modes"][0]["gemm_slowdown_pct"] if probe else None,
        "rs_launches": n_launch,
        "rs_lds_per_workgroup": int(info.rs_lds_bytes),
        "rs_cus": cus_measured,
        "rs_cus_per_xcc": {str(k): v for k, v in sorted(per_xcc.items())},
        # CU time the reduce-scatter held (per CU, the union of its tiles'
        # busy intervals, from the traced call), the one-GPU analog of the
        # pages' reduce-scatter "SM time"
        "rs_cu_ms": cu_rec["held_cu_ms"],
        "rs_cu_time": cu_rec if not args.no_trace else None,
        "ag_dma": dma_rec,
        "staged_rs": staged_rec,
        "pipeline": pipe_rec,
        "stock_analog": stock_rec,
        "rs_two_queues": two_q,
        "probe": probe,
        # per kernel launch: one reduce-scatter call is n_launch launches of
        # about rsb / n_launch algorithmic bytes; the event time per call
        # (divided by n_launch) includes the short gaps between launches
        "roofline": {"bound": "hbm", "achieved": round(rs_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(rs_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "rs_fixed_kernel",
                     "launches_per_call": n_launch,
                     "algorithmic_bytes_per_launch": algo_launch,
                     "traffic_over_algorithmic": round(traffic_ratio, 4) if traffic_ratio else None,
                     "avg_launch_ms": round(rs_avg / n_launch, 5),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE+WRITE_SIZE, "
                                     "copy-calibrated)"},
        "cpu_baseline": cpu,
        "env": {"device": torch.cuda.get_device_name(0), "torch": torch.__version__,
                "hip": torch.version.hip, "host_threads": len(os.sched_getaffinity(0))},
    }
    rec["pages_context"] = pages_context(rec, cu_rec, stock_rec)
    keys = [k for k in args.others.split(",") if k.strip() and configs.get(k).key != w.key]
    if keys:
        st.free()
        del st
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        rec["others"] = others_leg(keys, args)
    print(json.dumps(rec), flush=True)
    if cpu and cpu.get("parity_mismatches"):
        sys.exit(3)


if __name__ == "__main__":
    main()
