// pipeline.cpp -- CU-masked streams and the two-phase reduce-scatter
// pipeline, driven natively.
//
// The pages' reduce-scatter runs in two phases that overlap chunk by chunk:
// an intra-node reduction and a network phase that delivers partial results,
// with a staging buffer that stays nearly constant as the job grows
// [Abstract of "The Endgame of FSDP Communication", weekinpapers.com;
// "Performance" of the kongchang.com article].  On one GPU, phase 1 is the
// fixed-order reduction of a chunk of tiles into a slot of a ring of staging
// chunks (tide_rs_tiles_to_stage) and phase 2, the stand-in for the network,
// moves the slot into the shard arenas (tide_rs_stage_to_shards, or the
// copy-engine form tide_rs_stage_to_shards_sdma).
//
// The object holds two CU-masked streams (each gets a hardware queue of its
// own, so the phases really run side by side) and, per ring slot, a
// "produced" and a "drained" event.  Chunk i:
//   s1: wait drained[i % depth] (phase 2 of chunk i - depth left the slot)
//       phase 1 of chunk i into slot i % depth;  record produced[i % depth]
//   s2: wait produced[i % depth];  phase 2 of chunk i;  record drained[i % depth]
// A wait binds to the event's most recent record at the time the wait is
// issued, and every wait is issued after the record it needs, so events are
// reused across chunks and calls without a host synchronisation.  A slot
// drained by an earlier call is waited for in the next call too, so calls
// issued on different streams can share the ring.
// Host code only.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <cstring>
#include <new>
#include <vector>

#include "plan_format.h"
#include "stage_check.h"
#include "tide.h"

using namespace tide;

namespace {
constexpr int32_t kMaxPipelineDepth = 64;
}

struct tide_pipeline {
    int device = -1;
    int32_t depth = 0;
    int32_t phase2_cus = 0;
    hipStream_t s1 = nullptr, s2 = nullptr;
    hipEvent_t start = nullptr, done1 = nullptr, done2 = nullptr;
    std::vector<hipEvent_t> produced, drained;
    std::vector<char> drained_once;  // slot k's drained event has been recorded
};

namespace {

void release(tide_pipeline* p) {
    auto ev = [](hipEvent_t e) {
        if (e) (void)hipEventDestroy(e);
    };
    if (p->s1) (void)hipStreamSynchronize(p->s1);
    if (p->s2) (void)hipStreamSynchronize(p->s2);
    ev(p->start);
    ev(p->done1);
    ev(p->done2);
    for (hipEvent_t e : p->produced) ev(e);
    for (hipEvent_t e : p->drained) ev(e);
    if (p->s1) (void)hipStreamDestroy(p->s1);
    if (p->s2) (void)hipStreamDestroy(p->s2);
    delete p;
}

// Events that only order the two streams of one device need no system-scope
// fence: each kernel's own end-of-dispatch release makes its writes visible
// to the device's later kernels.
bool make_event(hipEvent_t* e, bool device_only = false) {
    unsigned flags = hipEventDisableTiming | (device_only ? hipEventDisableSystemFence : 0u);
    return hipEventCreateWithFlags(e, flags) == hipSuccess;
}

}  // namespace

// CU-masked streams: a stream created with a CU mask gets a hardware queue
// of its own, and its kernels' workgroups are placed only on the CUs whose
// mask bits are set.
extern "C" tide_status tide_stream_create_cu_range(int32_t first_cu, int32_t n_cu,
                                                   tide_stream_t* out) {
    if (!out || first_cu < 0 || n_cu < 1) return TIDE_EINVAL;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TIDE_EHIP;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return TIDE_EHIP;
    const int ncu = prop.multiProcessorCount;
    if (first_cu >= ncu || n_cu > ncu - first_cu) return TIDE_EINVAL;
    uint32_t mask[64] = {0};
    const int words = (ncu + 31) / 32;
    if (words > 64) return TIDE_EUNSUPPORTED;
    for (int i = first_cu; i < first_cu + n_cu; ++i) mask[i / 32] |= 1u << (i % 32);
    hipStream_t s = nullptr;
    if (hipExtStreamCreateWithCUMask(&s, (uint32_t)words, mask) != hipSuccess) return TIDE_EHIP;
    *out = reinterpret_cast<tide_stream_t>(s);
    return TIDE_OK;
}

extern "C" tide_status tide_stream_create_cu_limited(int32_t n_cu, tide_stream_t* out) {
    return tide_stream_create_cu_range(0, n_cu, out);
}

extern "C" tide_status tide_stream_destroy(tide_stream_t stream) {
    if (!stream) return TIDE_EINVAL;
    return hipStreamDestroy(reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? TIDE_OK : TIDE_EHIP;
}

extern "C" tide_status tide_pipeline_create(int32_t depth, int32_t phase2_cus,
                                            tide_pipeline_t* out) {
    if (!out || depth < 1 || depth > kMaxPipelineDepth || phase2_cus < 0) return TIDE_EINVAL;
    *out = nullptr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TIDE_EHIP;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return TIDE_EHIP;
    const int ncu = prop.multiProcessorCount;
    if (phase2_cus >= ncu) return TIDE_EINVAL;  // phase 1 needs CUs of its own
    tide_pipeline* p = new (std::nothrow) tide_pipeline;
    if (!p) return TIDE_EHIP;
    p->device = dev;
    p->depth = depth;
    p->phase2_cus = phase2_cus;
    p->drained_once.assign((size_t)depth, 0);
    // phase 2 confined to CUs [0, phase2_cus), phase 1 to the rest; with
    // phase2_cus == 0 both streams may use every CU
    tide_stream_t s1 = nullptr, s2 = nullptr;
    tide_status st = phase2_cus ? tide_stream_create_cu_range(phase2_cus, ncu - phase2_cus, &s1)
                                : tide_stream_create_cu_range(0, ncu, &s1);
    if (st == TIDE_OK) p->s1 = reinterpret_cast<hipStream_t>(s1);
    if (st == TIDE_OK) {
        st = tide_stream_create_cu_range(0, phase2_cus ? phase2_cus : ncu, &s2);
        if (st == TIDE_OK) p->s2 = reinterpret_cast<hipStream_t>(s2);
    }
    bool ok = st == TIDE_OK && make_event(&p->start) && make_event(&p->done1) &&
              make_event(&p->done2);
    for (int32_t k = 0; ok && k < depth; ++k) {
        hipEvent_t a = nullptr, b = nullptr;
        ok = make_event(&a, true);
        if (ok) p->produced.push_back(a);
        ok = ok && make_event(&b, true);
        if (ok) p->drained.push_back(b);
    }
    if (!ok) {
        release(p);
        return st == TIDE_OK ? TIDE_EHIP : st;
    }
    *out = p;
    return TIDE_OK;
}

extern "C" tide_status tide_pipeline_run(tide_pipeline_t p, const void* h_plan,
                                         const void* d_plan, int64_t chunk_tiles, float* ring,
                                         int64_t ring_elems, int32_t phase2,
                                         tide_stream_t stream) {
    if (!p || !d_plan || chunk_tiles < 1 || (phase2 != 0 && phase2 != 1)) return TIDE_EINVAL;
    if (phase2 == 1 && p->phase2_cus) return TIDE_EINVAL;  // copies take no CUs
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TIDE_EHIP;
    if (dev != p->device) return TIDE_EINVAL;
    PlanHeader h;
    if (!h_plan || !ring) return TIDE_EINVAL;
    std::memcpy(&h, h_plan, sizeof h);
    if (h.magic != kMagic || h.version != kVersion) return TIDE_EPLAN;
    if (!h.has_rs) return TIDE_EUNSUPPORTED;
    const int64_t n = h.n_rs_tiles, T = h.rs_tile;
    if (chunk_tiles > n && n > 0) chunk_tiles = n;
    // the whole ring is checked once (size, alignment, no overlap with any
    // gradient or arena), so that no chunk's call can fail validation halfway
    if (chunk_tiles > INT64_MAX / T / kMaxPipelineDepth) return TIDE_EINVAL;
    const int64_t slot = chunk_tiles * T;
    const int64_t chunks = n ? (n + chunk_tiles - 1) / chunk_tiles : 0;
    const int64_t need = slot * (chunks < p->depth ? chunks : p->depth);
    tide_status st = check_pipeline(h_plan, d_plan, 0, 0, ring, ring_elems, 0, &h);
    if (st != TIDE_OK) return st;
    if (ring_elems < need) return TIDE_EINVAL;
    const uint64_t lo = reinterpret_cast<uint64_t>(ring);
    if (overlaps_rs_buffers(h_plan, lo, lo + 4ull * (uint64_t)need)) return TIDE_EOVERLAP;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    tide_stream_t s1 = reinterpret_cast<tide_stream_t>(p->s1);
    tide_stream_t s2 = reinterpret_cast<tide_stream_t>(p->s2);
    if (hipEventRecord(p->start, s) != hipSuccess) return TIDE_EHIP;
    if (hipStreamWaitEvent(p->s1, p->start, 0) != hipSuccess ||
        hipStreamWaitEvent(p->s2, p->start, 0) != hipSuccess)
        return TIDE_EHIP;
    for (int64_t i = 0, b = 0; b < n && st == TIDE_OK; ++i, b += chunk_tiles) {
        const int64_t cnt = chunk_tiles < n - b ? chunk_tiles : n - b;
        const int32_t k = (int32_t)(i % p->depth);
        float* buf = ring + k * slot;
        if ((i >= p->depth || p->drained_once[k]) &&
            hipStreamWaitEvent(p->s1, p->drained[k], 0) != hipSuccess) {
            st = TIDE_EHIP;
            break;
        }
        // the ring and the tile range were checked above, once for all chunks
        st = issue_tiles_to_stage(h, d_plan, b, cnt, buf, 0, s1);
        if (st != TIDE_OK) break;
        if (hipEventRecord(p->produced[k], p->s1) != hipSuccess ||
            hipStreamWaitEvent(p->s2, p->produced[k], 0) != hipSuccess) {
            st = TIDE_EHIP;
            break;
        }
        st = phase2 == 0 ? issue_stage_to_shards(h, d_plan, b, cnt, buf, 0, s2)
                         : issue_stage_to_shards_sdma(h, h_plan, b, cnt, buf, s2);
        if (st != TIDE_OK) break;
        if (hipEventRecord(p->drained[k], p->s2) != hipSuccess)
            st = TIDE_EHIP;
        else
            p->drained_once[k] = 1;
    }
    // the caller's stream waits for both phases, also after a failure, so
    // that its later work never races whatever was issued
    if (hipEventRecord(p->done1, p->s1) != hipSuccess ||
        hipEventRecord(p->done2, p->s2) != hipSuccess ||
        hipStreamWaitEvent(s, p->done1, 0) != hipSuccess ||
        hipStreamWaitEvent(s, p->done2, 0) != hipSuccess)
        return TIDE_EHIP;
    return st;
}

extern "C" tide_status tide_pipeline_destroy(tide_pipeline_t p) {
    if (!p) return TIDE_EINVAL;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TIDE_EHIP;
    const int owner = p->device;
    if (dev != owner && hipSetDevice(owner) != hipSuccess) return TIDE_EHIP;
    release(p);
    if (dev != owner) (void)hipSetDevice(dev);
    return TIDE_OK;
}
