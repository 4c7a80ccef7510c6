// dma.cpp -- data movement on the DMA (SDMA) copy engines, issued through
// ROCr, for the two places where the pages move data without compute units:
// putting gathered shards into the parameter tensors, and staging gradients
// for a reduction that only brief compute work performs (the pages split the
// work between the copy engines and brief thread blocks, and keep the
// compute units out of transport and placement: Abstract of "The Endgame of
// FSDP Communication", weekinpapers.com; "TIDE's Design Approach" of the
// kongchang.com article).
//
// Every copy is a 1-D copy pinned to one engine; one call spreads its
// copies over all engines the device offers (largest first, each to the
// engine with the fewest bytes so far) and shares one completion signal
// among them, so a call costs about a microsecond of host work per copy
// and the engines run in parallel.  The runtime's own no-compute-unit copy
// kind takes ~12 us per copy on one queue and runs 2-D copies as a blit
// kernel, which is why this goes to ROCr directly.
//
// Calls are host-synchronous: they first wait for the caller's stream (so
// every earlier kernel on it has finished with the buffers), issue the
// copies and return when the engines are done.  The device's ROCr agent
// and engine list are looked up once per device and kept.
#include <hip/hip_runtime.h>
#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>

#include <algorithm>
#include <chrono>
#include <climits>
#include <cstring>
#include <mutex>
#include <thread>
#include <vector>

#include "bounded_wait.h"
#include "plan_format.h"
#include "stage_check.h"
#include "tide.h"

using namespace tide;

namespace {

struct Engines {
    bool looked_up = false;
    tide_status status = TIDE_EUNSUPPORTED;
    hsa_agent_t agent{};
    std::vector<hsa_amd_sdma_engine_id_t> ids;
};

constexpr int kMaxDevices = 64;
std::mutex g_mu;
Engines g_engines[kMaxDevices];

struct AgentQuery {
    uint32_t domain, bdf;
    bool found;
    hsa_agent_t agent;
};

hsa_status_t find_cpu(hsa_agent_t a, void* data) {
    hsa_device_type_t type;
    if (hsa_agent_get_info(a, HSA_AGENT_INFO_DEVICE, &type) == HSA_STATUS_SUCCESS &&
        type == HSA_DEVICE_TYPE_CPU) {
        *static_cast<hsa_agent_t*>(data) = a;
        return HSA_STATUS_INFO_BREAK;
    }
    return HSA_STATUS_SUCCESS;
}

// The device's copy engines.  Some ROCr versions answer the engine query
// only for host <-> device pairs (device-to-device: invalid agent); the
// engines they report there also run device-to-device copies when pinned.
uint32_t engine_mask(hsa_agent_t gpu) {
    uint32_t mask = 0;
    if (hsa_amd_memory_copy_engine_status(gpu, gpu, &mask) == HSA_STATUS_SUCCESS && mask) return mask;
    hsa_agent_t cpu{};
    if (hsa_iterate_agents(find_cpu, &cpu) != HSA_STATUS_INFO_BREAK) return 0;
    mask = 0;
    if (hsa_amd_memory_copy_engine_status(gpu, cpu, &mask) != HSA_STATUS_SUCCESS) return 0;
    return mask;
}

hsa_status_t match_agent(hsa_agent_t a, void* data) {
    AgentQuery* q = static_cast<AgentQuery*>(data);
    hsa_device_type_t type;
    if (hsa_agent_get_info(a, HSA_AGENT_INFO_DEVICE, &type) != HSA_STATUS_SUCCESS ||
        type != HSA_DEVICE_TYPE_GPU)
        return HSA_STATUS_SUCCESS;
    uint32_t bdf = 0, domain = 0;
    if (hsa_agent_get_info(a, static_cast<hsa_agent_info_t>(HSA_AMD_AGENT_INFO_BDFID), &bdf) !=
            HSA_STATUS_SUCCESS ||
        hsa_agent_get_info(a, static_cast<hsa_agent_info_t>(HSA_AMD_AGENT_INFO_DOMAIN), &domain) !=
            HSA_STATUS_SUCCESS)
        return HSA_STATUS_SUCCESS;
    // BDFID packs bus [15:8], device [7:3], function [2:0]
    if (domain == q->domain && (bdf & ~7u) == (q->bdf & ~7u)) {
        q->found = true;
        q->agent = a;
        return HSA_STATUS_INFO_BREAK;
    }
    return HSA_STATUS_SUCCESS;
}

// The current HIP device's agent and copy engines.
tide_status engines_of_current_device(const Engines** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TIDE_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return TIDE_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mu);
    Engines& e = g_engines[dev];
    if (!e.looked_up) {
        e.looked_up = true;
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            e.status = TIDE_EHIP;
        } else if (hsa_init() != HSA_STATUS_SUCCESS) {  // reference-counted; the runtime holds one
            e.status = TIDE_EHIP;
        } else {
            AgentQuery q{(uint32_t)prop.pciDomainID,
                         ((uint32_t)prop.pciBusID << 8) | ((uint32_t)prop.pciDeviceID << 3), false, {}};
            hsa_iterate_agents(match_agent, &q);
            const uint32_t mask = q.found ? engine_mask(q.agent) : 0;
            if (!q.found || mask == 0) {
                e.status = TIDE_EUNSUPPORTED;
            } else {
                e.agent = q.agent;
                for (int b = 0; b < 32; ++b)
                    if (mask & (1u << b)) e.ids.push_back(static_cast<hsa_amd_sdma_engine_id_t>(1u << b));
                e.status = TIDE_OK;
            }
        }
    }
    *out = &e;
    return e.status;
}

struct Copy {
    char* dst;
    const char* src;
    size_t bytes;
};

// Wait for the caller's stream to finish its earlier work, polling with
// short sleeps, for at most kStreamTimeoutNs.
tide_status drain_stream(tide_stream_t stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t last = hipSuccess;
    const bool done = wait_until(
        [&] {
            last = hipStreamQuery(s);
            return last != hipErrorNotReady;
        },
        [](uint64_t ns) {
            std::this_thread::sleep_for(std::chrono::nanoseconds(ns < 20000 ? ns : 20000));
        },
        kStreamTimeoutNs);
    return done && last == hipSuccess ? TIDE_OK : TIDE_EHIP;
}

// ROCr's wait takes its timeout hint in system timestamp ticks.
uint64_t ns_to_ticks(uint64_t ns) {
    static const uint64_t hz = [] {
        uint64_t f = 0;
        if (hsa_system_get_info(HSA_SYSTEM_INFO_TIMESTAMP_FREQUENCY, &f) != HSA_STATUS_SUCCESS || !f)
            f = 1000000000ull;
        return f;
    }();
    return (uint64_t)((double)ns * (double)hz * 1e-9) + 1;
}

// Issue the copies over all engines and wait for them (bounded: a call whose
// copies stop making progress returns TIDE_EHIP after copy_timeout_ns).
tide_status run_copies(std::vector<Copy>& copies, tide_stream_t stream) {
    if (drain_stream(stream) != TIDE_OK) return TIDE_EHIP;
    copies.erase(std::remove_if(copies.begin(), copies.end(), [](const Copy& c) { return c.bytes == 0; }),
                 copies.end());
    if (copies.empty()) return TIDE_OK;
    const Engines* eng = nullptr;
    tide_status st = engines_of_current_device(&eng);
    if (st != TIDE_OK) return st;
    std::stable_sort(copies.begin(), copies.end(),
                     [](const Copy& a, const Copy& b) { return a.bytes > b.bytes; });
    const size_t ne = eng->ids.size();
    std::vector<size_t> load(ne, 0);
    hsa_signal_t sig;
    if (hsa_signal_create((hsa_signal_value_t)copies.size(), 0, nullptr, &sig) != HSA_STATUS_SUCCESS)
        return TIDE_EHIP;
    size_t issued = 0;
    for (const Copy& c : copies) {
        const size_t k = std::min_element(load.begin(), load.end()) - load.begin();
        if (hsa_amd_memory_async_copy_on_engine(c.dst, eng->agent, c.src, eng->agent, c.bytes, 0,
                                                nullptr, sig, eng->ids[k], true) !=
            HSA_STATUS_SUCCESS) {
            st = TIDE_EHIP;
            break;
        }
        load[k] += c.bytes;
        ++issued;
    }
    if (issued < copies.size())  // the copies never issued will not decrement the signal
        hsa_signal_subtract_screlease(sig, (hsa_signal_value_t)(copies.size() - issued));
    uint64_t total = 0;
    for (const Copy& c : copies) total += c.bytes;
    const bool done = wait_until(
        [&] { return hsa_signal_load_scacquire(sig) == 0; },
        [&](uint64_t ns) {
            (void)hsa_signal_wait_scacquire(sig, HSA_SIGNAL_CONDITION_EQ, 0, ns_to_ticks(ns),
                                            HSA_WAIT_STATE_BLOCKED);
        },
        copy_timeout_ns(total));
    if (!done) {
        // Copies may still be in flight and will decrement the signal when
        // they end: it is left alive (a small leak) rather than destroyed
        // under them.
        return TIDE_EHIP;
    }
    hsa_signal_destroy(sig);
    return st;
}

bool read_header(const void* h_plan, PlanHeader* h) {
    std::memcpy(h, h_plan, sizeof *h);
    return h->magic == kMagic && h->version == kVersion;
}

struct Iv {
    uint64_t lo, hi;
};

}  // namespace

namespace tide {

tide_status check_stage(const void* h_plan, const uint64_t* h_stage, int64_t slot_stride,
                        bool* vec_ok) {
    if (!h_plan || !h_stage) return TIDE_EINVAL;
    PlanHeader h;
    if (!read_header(h_plan, &h)) return TIDE_EPLAN;
    if (!h.has_rs) return TIDE_EUNSUPPORTED;
    if (slot_stride < h.S || slot_stride > (INT64_MAX / 2) / (h.R > 0 ? h.R : 1)) return TIDE_EINVAL;
    const uint8_t* b = static_cast<const uint8_t*>(h_plan);
    const ParamDesc* ps = reinterpret_cast<const ParamDesc*>(b + h.off_params);
    const uint64_t* gptr = reinterpret_cast<const uint64_t*>(b + h.off_gptr);
    const uint64_t* obase = reinterpret_cast<const uint64_t*>(b + h.off_obase);
    const uint64_t span = 2ull * (uint64_t)h.R * (uint64_t)slot_stride;
    bool aligned = (2 * slot_stride) % 16 == 0;
    std::vector<Iv> stage;
    for (int32_t r = 0; r < h.R; ++r) {
        if (h_stage[r] == 0) return TIDE_EINVAL;
        if (h_stage[r] % 2) return TIDE_EALIGN;
        if (h_stage[r] % 16) aligned = false;
        if (span) stage.push_back({h_stage[r], h_stage[r] + span});
    }
    std::sort(stage.begin(), stage.end(), [](const Iv& x, const Iv& y) { return x.lo < y.lo; });
    for (size_t i = 1; i < stage.size(); ++i)
        if (stage[i].lo < stage[i - 1].hi) return TIDE_EOVERLAP;
    auto hits = [&](uint64_t lo, uint64_t hi) {
        if (lo >= hi) return false;
        // first staging buffer ending after lo
        auto it = std::upper_bound(stage.begin(), stage.end(), lo,
                                   [](uint64_t v, const Iv& x) { return v < x.hi; });
        return it != stage.end() && it->lo < hi;
    };
    for (int32_t p = 0; p < h.P; ++p) {
        ParamDesc d;
        std::memcpy(&d, ps + p, sizeof d);
        for (int32_t q = 0; q < h.R; ++q) {
            const uint64_t g = gptr[(int64_t)p * h.R + q];
            if (hits(g, g + 2ull * (uint64_t)d.n)) return TIDE_EOVERLAP;
        }
    }
    for (int32_t r = 0; r < h.R; ++r)
        if (hits(obase[r], obase[r] + 4ull * (uint64_t)h.S)) return TIDE_EOVERLAP;
    if (vec_ok) *vec_ok = aligned;
    return TIDE_OK;
}

}  // namespace tide

namespace tide {

bool overlaps_rs_buffers(const void* h_plan, uint64_t lo, uint64_t hi) {
    if (lo >= hi) return false;
    PlanHeader h;
    read_header(h_plan, &h);
    const uint8_t* b = static_cast<const uint8_t*>(h_plan);
    const ParamDesc* ps = reinterpret_cast<const ParamDesc*>(b + h.off_params);
    const uint64_t* gptr = reinterpret_cast<const uint64_t*>(b + h.off_gptr);
    const uint64_t* obase = reinterpret_cast<const uint64_t*>(b + h.off_obase);
    auto meets = [&](uint64_t a, uint64_t z) { return a < z && a < hi && lo < z; };
    for (int32_t p = 0; p < h.P; ++p) {
        ParamDesc d;
        std::memcpy(&d, ps + p, sizeof d);
        for (int32_t q = 0; q < h.R; ++q) {
            const uint64_t g = gptr[(int64_t)p * h.R + q];
            if (meets(g, g + 2ull * (uint64_t)d.n)) return true;
        }
    }
    for (int32_t r = 0; r < h.R; ++r)
        if (meets(obase[r], obase[r] + 4ull * (uint64_t)h.S)) return true;
    return false;
}

tide_status check_pipeline(const void* h_plan, const void* d_plan, int64_t tile_begin,
                           int64_t tile_count, const float* stage, int64_t stage_elems,
                           int32_t max_workgroups, PlanHeader* h) {
    if (!h_plan || !stage) return TIDE_EINVAL;
    if (!read_header(h_plan, h)) return TIDE_EPLAN;
    if (!h->has_rs) return TIDE_EUNSUPPORTED;
    if (max_workgroups < 0) return TIDE_EINVAL;
    if (tile_begin < 0 || tile_count < 0 || tile_begin > h->n_rs_tiles ||
        tile_count > h->n_rs_tiles - tile_begin)
        return TIDE_EINVAL;
    if (tile_count > INT64_MAX / h->rs_tile || stage_elems < tile_count * h->rs_tile)
        return TIDE_EINVAL;
    if (reinterpret_cast<uintptr_t>(stage) % 16 || reinterpret_cast<uintptr_t>(d_plan) % 16)
        return TIDE_EALIGN;
    const uint64_t lo = reinterpret_cast<uint64_t>(stage);
    if (overlaps_rs_buffers(h_plan, lo, lo + 4ull * (uint64_t)(tile_count * h->rs_tile)))
        return TIDE_EOVERLAP;
    return TIDE_OK;
}

}  // namespace tide

namespace tide {

tide_status issue_stage_to_shards_sdma(const PlanHeader& h, const void* h_plan,
                                       int64_t tile_begin, int64_t tile_count, const float* stage,
                                       tide_stream_t stream) {
    const uint8_t* b = static_cast<const uint8_t*>(h_plan);
    const RsTile* tiles = reinterpret_cast<const RsTile*>(b + h.off_rs);
    const uint64_t* obase = reinterpret_cast<const uint64_t*>(b + h.off_obase);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // merge tiles into runs contiguous both in the chunk (every tile but the
    // last of a run fills its T floats) and in the rank's arena
    int64_t t = tile_begin;
    const int64_t end = tile_begin + tile_count;
    while (t < end) {
        RsTile first;
        std::memcpy(&first, tiles + t, sizeof first);
        int64_t len = first.len;
        int64_t u = t + 1;
        while (u < end && len == (u - t) * (int64_t)h.rs_tile) {
            RsTile nx;
            std::memcpy(&nx, tiles + u, sizeof nx);
            if (nx.r != first.r || nx.o0 != first.o0 + len) break;
            len += nx.len;
            ++u;
        }
        char* dst = reinterpret_cast<char*>(obase[first.r]) + 4 * first.o0;
        const char* src = reinterpret_cast<const char*>(stage + (t - tile_begin) * h.rs_tile);
        if (hipMemcpyAsync(dst, src, (size_t)(4 * len), hipMemcpyDeviceToDeviceNoCU, s) !=
            hipSuccess)
            return TIDE_EHIP;
        t = u;
    }
    return TIDE_OK;
}

}  // namespace tide

extern "C" tide_status tide_rs_stage_to_shards_sdma(const void* h_plan, int64_t tile_begin,
                                                    int64_t tile_count, const float* stage,
                                                    int64_t stage_elems, tide_stream_t stream) {
    PlanHeader h;
    tide_status st = check_pipeline(h_plan, nullptr, tile_begin, tile_count, stage, stage_elems, 0,
                                    &h);
    if (st != TIDE_OK) return st;
    return issue_stage_to_shards_sdma(h, h_plan, tile_begin, tile_count, stage, stream);
}

extern "C" tide_status tide_dma_engine_count(int32_t* count) {
    if (!count) return TIDE_EINVAL;
    const Engines* eng = nullptr;
    tide_status st = engines_of_current_device(&eng);
    *count = st == TIDE_OK ? (int32_t)eng->ids.size() : 0;
    return st;
}

extern "C" tide_status tide_ag_place_dma(const void* h_plan, tide_stream_t stream) {
    if (!h_plan) return TIDE_EINVAL;
    PlanHeader h;
    if (!read_header(h_plan, &h)) return TIDE_EPLAN;
    if (!h.has_ag) return TIDE_EUNSUPPORTED;
    const uint8_t* b = static_cast<const uint8_t*>(h_plan);
    const ParamDesc* ps = reinterpret_cast<const ParamDesc*>(b + h.off_params);
    const uint64_t* full = reinterpret_cast<const uint64_t*>(b + h.off_full);
    const char* g = reinterpret_cast<const char*>(h.gathered);
    std::vector<Copy> copies;
    for (int32_t p = 0; p < h.P; ++p) {
        ParamDesc d;
        std::memcpy(&d, ps + p, sizeof d);
        if (d.n == 0) continue;
        char* dst = reinterpret_cast<char*>(full[p]);
        // rank r holds rows [r*s, r*s + v) of the param, v = clamp(d0 - r*s, 0, s)
        for (int64_t r = 0; r < h.R && r * d.s < d.d0; ++r) {
            const int64_t v = std::min(d.s, d.d0 - r * d.s);
            copies.push_back({dst + 2 * r * d.m, g + 2 * (r * h.S + d.off), (size_t)(2 * v * d.c)});
        }
    }
    return run_copies(copies, stream);
}

extern "C" tide_status tide_rs_stage_dma(const void* h_plan, const uint64_t* h_stage,
                                         int64_t slot_stride, tide_stream_t stream) {
    bool vec_ok = false;
    tide_status st = check_stage(h_plan, h_stage, slot_stride, &vec_ok);
    if (st != TIDE_OK) return st;
    PlanHeader h;
    read_header(h_plan, &h);
    const uint8_t* b = static_cast<const uint8_t*>(h_plan);
    const ParamDesc* ps = reinterpret_cast<const ParamDesc*>(b + h.off_params);
    const uint64_t* gptr = reinterpret_cast<const uint64_t*>(b + h.off_gptr);
    std::vector<Copy> copies;
    for (int32_t p = 0; p < h.P; ++p) {
        ParamDesc d;
        std::memcpy(&d, ps + p, sizeof d);
        if (d.n == 0) continue;
        // rank r's shard holds flat indices [r*m, r*m + v*c) of every rank's
        // gradient; padding rows are not staged (the fold writes them +0.0)
        for (int64_t r = 0; r < h.R && r * d.s < d.d0; ++r) {
            const int64_t v = std::min(d.s, d.d0 - r * d.s);
            char* slot0 = reinterpret_cast<char*>(h_stage[r]) + 2 * d.off;
            for (int32_t q = 0; q < h.R; ++q) {
                const char* src = reinterpret_cast<const char*>(gptr[(int64_t)p * h.R + q]);
                copies.push_back({slot0 + 2 * (int64_t)q * slot_stride, src + 2 * r * d.m,
                                  (size_t)(2 * v * d.c)});
            }
        }
    }
    return run_copies(copies, stream);
}
